"""fp64 oracle of the owner-local Muon step on whole 2D matrices.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Source of the method: "MatrixFSDP: communication-free matrix optimizers under
ZeRO-3 parameter sharding" (arxivlens page), Abstract: Muon orthogonalizes
momentum-smoothed matrix updates with Newton-Schulz, which needs the complete
2D matrix; under owner-shaped placement the owner holds that matrix and runs
Newton-Schulz locally, and the resulting update is the same as full-matrix
Muon.  The gist.science summaries (section "Méthodologie", part 1) say the
same: after the gradient reduction the whole 2D gradient sits on the owner
rank, which performs the Newton-Schulz update without any matrix
communication.

The pages print no formula.  Readings used here (each one is a choice where the
pages are silent):

R1  momentum is the heavy-ball form  M' = beta*M + G;
R2  Nesterov input  U = G + beta*M'  (plain  U = M'  when Nesterov is off);
R3  Newton-Schulz starts from the Frobenius-normalized input
    X0 = U / (||U||_F + eps),  eps = 1e-7;
R5  a tall matrix (rows > cols) is iterated on its transpose and transposed
    back (exact in exact arithmetic -- it only changes the cost);
R6  the same coefficients (a, b, c) on every iteration;
R7  one iteration is  A = X X^T,  B = b A + c A A,  X <- a X + B X;
R8  the update scale s is an argument, default sqrt(max(1, rows/cols));
R9  decoupled, multiplicative weight decay with the same lr:
    W' = (1 - lr*wd) W - lr * s * O.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

#: Additive guard in the Frobenius normalization (reading R3).
NS_EPS = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def default_scale(rows: int, cols: int) -> float:
    """Update scale s = sqrt(max(1, rows/cols)) (reading R8; parity unpinned).

    The pages fix no update scale.  This is the convention of the original
    Muon write-up; the library carries s per matrix so any convention can be
    expressed.
    """
    return math.sqrt(max(1.0, rows / cols))


def momentum_nesterov(G, M, beta: float, nesterov: bool = True):
    """Momentum smoothing of the matrix gradient (readings R1, R2).

    The Abstract of the arxivlens page says only that Muon acts on
    momentum-smoothed updates.  Heavy-ball momentum  M' = beta*M + G; the
    Newton-Schulz input is  U = G + beta*M'  with Nesterov, else  U = M'.

    Returns (M', U) in float64.
    """
    G = _f64(G)
    M = _f64(M)
    M_new = beta * M + G
    U = G + beta * M_new if nesterov else M_new
    return M_new, U


def frobenius_normalize(U, eps: float = NS_EPS):
    """X0 = U / (||U||_F + eps) and nu = ||U||_F (reading R3).

    The Frobenius norm bounds the spectral norm, so every singular value of X0
    is at most 1, the interval on which the Newton-Schulz polynomial is tuned.
    The norm is a full float64 sum of squares.
    """
    U = _f64(U)
    nu = math.sqrt(float(np.sum(U * U)))
    return U / (nu + eps), nu


def newton_schulz(X0, steps: int, a: float, b: float, c: float):
    """Newton-Schulz orthogonalization of one whole matrix (readings R5-R7).

    The arxivlens Abstract names Newton-Schulz as the part of Muon that needs
    the complete matrix.  Each iteration applies the odd matrix polynomial
    X <- a X + (b A + c A^2) X with A = X X^T; a tall input is iterated on its
    transpose.  Dense float64 products; symmetry is not exploited.
    """
    X = _f64(X0)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if tall:
        X = X.T
    return np.ascontiguousarray(X)


def muon_matrix_step(W, G, M, *, lr: float, beta: float, nesterov: bool,
                     weight_decay: float, ns_steps: int,
                     abc: Sequence[float], scale: float | None = None,
                     eps: float = NS_EPS):
    """One owner-local Muon step on one whole matrix.

    The owner holds W, its gradient G and its momentum M whole (arxivlens
    Abstract; gist.science "Méthodologie", part 1), so the step is local:
    momentum (R1, R2), Frobenius normalization (R3), Newton-Schulz (R5-R7),
    then the decoupled-decay update (R8, R9).

    Returns (W', M', O) in float64, where O is the orthogonalized update
    before lr and scale.
    """
    W = _f64(W)
    rows, cols = W.shape
    if scale is None:
        scale = default_scale(rows, cols)
    a, b, c = abc
    M_new, U = momentum_nesterov(G, M, beta, nesterov)
    X0, _ = frobenius_normalize(U, eps)
    O = newton_schulz(X0, ns_steps, a, b, c)
    W_new = (1.0 - lr * weight_decay) * W - lr * scale * O
    return W_new, M_new, O


def muon_step(weights: Iterable, grads: Iterable, momenta: Iterable, *,
              lr: float, beta: float, nesterov: bool, weight_decay: float,
              ns_steps: int, abc: Sequence[float],
              scales: Sequence[float] | None = None, eps: float = NS_EPS):
    """Owner-local Muon step over the owner's list of whole matrices.

    Matrices are independent: the step is communication-free and each owned
    matrix is updated from its own gradient alone (arxivlens Abstract), so the
    list result is the list of per-matrix results.  An empty list (a rank that
    owns no matrix holds only empty shards) is a no-op.

    Returns three lists (W', M', O).
    """
    weights = list(weights)
    grads = list(grads)
    momenta = list(momenta)
    if not (len(weights) == len(grads) == len(momenta)):
        raise ValueError("weights, grads and momenta must have equal length")
    out_w, out_m, out_o = [], [], []
    for k, (W, G, M) in enumerate(zip(weights, grads, momenta)):
        s = None if scales is None else scales[k]
        w2, m2, o = muon_matrix_step(W, G, M, lr=lr, beta=beta,
                                     nesterov=nesterov,
                                     weight_decay=weight_decay,
                                     ns_steps=ns_steps, abc=abc, scale=s,
                                     eps=eps)
        out_w.append(w2)
        out_m.append(m2)
        out_o.append(o)
    return out_w, out_m, out_o
