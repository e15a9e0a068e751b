"""fp64 oracle of the AdamW step on a packed tail buffer.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" (arxivlens page), Abstract, and the gist.science summaries
("Méthodologie", part 1): vectors and the other tensors that are not 2D go,
grouped in one buffer, to tail owners and keep the ordinary AdamW optimizer.  The pages give no formula;
reading R11 takes textbook decoupled AdamW (Loshchilov & Hutter): weight decay
multiplies the parameter, moments are exponential averages, both are
bias-corrected with the step count t (t = 1 on the first step), and eps is
added outside the square root.
"""

from __future__ import annotations

import numpy as np


def adamw_tail(p, g, m, v, *, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, step: int):
    """One decoupled AdamW step on a packed 1D buffer (reading R11).

    In order:
      p  <- p * (1 - lr*wd)
      m' =  beta1*m + (1-beta1)*g
      v' =  beta2*v + (1-beta2)*g^2
      m_hat = m' / (1 - beta1^t),  v_hat = v' / (1 - beta2^t)
      p' =  p - lr * m_hat / (sqrt(v_hat) + eps)

    Returns (p', m', v') in float64.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new
