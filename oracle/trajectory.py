"""fp64 oracle of a trajectory of consecutive owner-local optimizer steps.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" (arxivlens page, Abstract): the owner's update equals
full-matrix Muon, step after step, with the momentum carried on the owner;
the gist.science summaries ("Résultats") check this over training by
comparing the loss curve with full-matrix DDP Muon.  The tail keeps its AdamW
moments and step count across steps.

Reading R19 (the pages say nothing about storage between steps): the state
lives in the storage dtype between steps, exactly as the caller's buffers hold
it.  After every step W' and M' are rounded to the storage dtype (bf16 or
fp32, round to nearest, ties to even) and the next step starts from the
rounded values; inside a step everything stays float64 (the single-step
oracle).  ``storage=None`` keeps float64 state (no rounding), which is what
the closed-form pins use.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .adamw_ref import adamw_tail
from .muon_ref import NS_EPS, muon_matrix_step


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    bfloat16 keeps 8 significant bits.  With x = f * 2**e, 0.5 <= |f| < 1,
    the nearest value with 8 significant bits is round(f * 2**8) * 2**(e-8),
    and numpy's round breaks ties to even.  Magnitudes below bf16's normal
    range (2**-126) and overflow are not handled: the optimizer states here
    are many orders of magnitude away from both.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.round(f * 256.0) / 256.0, e)


def round_to_f32(x) -> np.ndarray:
    """Nearest float32 value of each float64 (IEEE conversion, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _store(x, storage: Optional[str]) -> np.ndarray:
    if storage is None:
        return np.asarray(x, dtype=np.float64)
    if storage == "bf16":
        return round_to_bf16(x)
    if storage == "f32":
        return round_to_f32(x)
    raise ValueError(storage)


def muon_trajectory(weights: Sequence, momenta: Sequence, grads_per_step: Sequence[Sequence], *,
                    lr: float, beta: float, nesterov: bool, weight_decay: float,
                    ns_steps: int, abc: Sequence[float], storage: Optional[str],
                    scales: Optional[Sequence[float]] = None, eps: float = NS_EPS):
    """Run len(grads_per_step) owner-local Muon steps, carrying W and M.

    ``grads_per_step[t][k]`` is matrix k's gradient at step t.  Returns the
    list of states after each step: ``states[t] = (Ws, Ms)``, each a list of
    float64 arrays holding the stored (rounded, per ``storage``) values.
    """
    Ws = [_store(w, storage) for w in weights]
    Ms = [_store(m, storage) for m in momenta]
    states = []
    for grads in grads_per_step:
        new_w, new_m = [], []
        for k, (W, G, M) in enumerate(zip(Ws, grads, Ms)):
            s = None if scales is None else scales[k]
            w2, m2, _ = muon_matrix_step(W, G, M, lr=lr, beta=beta, nesterov=nesterov,
                                         weight_decay=weight_decay, ns_steps=ns_steps,
                                         abc=abc, scale=s, eps=eps)
            new_w.append(_store(w2, storage))
            new_m.append(_store(m2, storage))
        Ws, Ms = new_w, new_m
        states.append((list(Ws), list(Ms)))
    return states


def adamw_trajectory(p, m, v, grads_per_step: Sequence, *, lr: float, beta1: float,
                     beta2: float, eps: float, weight_decay: float, first_step: int = 1,
                     storage: Optional[str] = "f32") -> List[tuple]:
    """Run len(grads_per_step) AdamW steps on a packed tail, t = first_step, ...

    Returns ``states[t] = (p, m, v)`` after each step (stored values).
    """
    p, m, v = (_store(x, storage) for x in (p, m, v))
    states = []
    for i, g in enumerate(grads_per_step):
        p, m, v = adamw_tail(p, g, m, v, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                             weight_decay=weight_decay, step=first_step + i)
        p, m, v = (_store(x, storage) for x in (p, m, v))
        states.append((p, m, v))
    return states
