"""Comparison rules of the parity tests (numpy only, no GPU).

Acceptance (relative Frobenius error, float64):
  * bf16 path: O and M' within 2e-2 per tensor; W' within
        ||W'_gpu - W'_ref||_F <= 2e-2 ||W'_ref - W||_F + 0.5 ||ulp_bf16(W'_ref)||_F
    (an update is only a few bf16 ulps of W, so the final rounding of W' is
    allowed for separately);
  * fp32 path: O, M' and W' - W within 1e-4 per tensor;
  * AdamW: p', m', v' within 1e-6.

A per-tensor norm averages an error over the whole matrix: a wrong value in
one 256 x 256 tile of a 2048 x 5632 matrix (176 tiles) is diluted by about
sqrt(176).  So the same rules are applied again per 256 x 256 tile of the
stored layout, with twice the per-tensor bar (each tile holds up to 65536
elements, so its error is a tight estimate of the per-tensor one when the
error is spread evenly; a tile whose error is twice the matrix-wide bar is
wrong).  The Newton-Schulz kernels write one 256 x 256 output tile per
workgroup and a tall matrix's tiles map one to one onto transposed stored
tiles, so every kernel tile is one checked tile.  Tiles with fewer than
TILE_MIN_ELEMS elements (the corner of a ragged matrix) are covered only by
the per-tensor bar: their few elements make the tile error a noisy estimate.

M' = beta*M + G is elementwise: each element is checked against one unit in
the last place of its storage dtype.  The reference of that check takes beta
as the float32 the C ABI receives (the oracle's float64 0.95 differs from it
by 1.2e-8 relative, which an element of M' that nearly cancels would magnify
past one ulp); the per-tensor check of M' uses the oracle's value as is.
"""

from __future__ import annotations

import numpy as np

BF16_TOL = 2e-2
F32_TOL = 1e-4
ADAMW_TOL = 1e-6
TILE = 256
TILE_FACTOR = 2.0
TILE_MIN_ELEMS = 1024


def rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(y)
    num = np.linalg.norm(x - y)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values (8 significant bits) at each |x|."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.where(ax > 0, np.exp2(e - 7), np.exp2(-133.0))


def ulp_f32(x: np.ndarray) -> np.ndarray:
    """Spacing of float32 values (24 significant bits) at each |x|."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.where(ax > 0, np.exp2(e - 23), np.exp2(-149.0))


def w_error_bf16(W_gpu, W_ref, W0) -> float:
    """Ratio of the W' error to its allowance (<= 1 passes)."""
    err = np.linalg.norm(np.asarray(W_gpu, np.float64) - W_ref)
    allow = BF16_TOL * np.linalg.norm(W_ref - W0) + 0.5 * np.linalg.norm(ulp_bf16(W_ref))
    return float(err / allow)


def _tiles(shape):
    r, c = shape
    for i in range(0, r, TILE):
        for j in range(0, c, TILE):
            sl = (slice(i, min(i + TILE, r)), slice(j, min(j + TILE, c)))
            if (sl[0].stop - sl[0].start) * (sl[1].stop - sl[1].start) >= TILE_MIN_ELEMS:
                yield (i // TILE, j // TILE), sl


def worst_tile_rel(x, y):
    """Largest per-tile relative Frobenius error of x against y, and its tile."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    worst, where = 0.0, None
    for t, sl in _tiles(y.shape):
        e = rel(x[sl], y[sl])
        if not e <= worst:          # NaN counts as worst
            worst, where = e, t
    return worst, where


def worst_tile_w_bf16(W_gpu, W_ref, W0):
    """Largest per-tile ratio of the W' error to its bf16 allowance."""
    W_gpu = np.asarray(W_gpu, np.float64)
    worst, where = 0.0, None
    for t, sl in _tiles(W_ref.shape):
        e = w_error_bf16(W_gpu[sl], W_ref[sl], W0[sl])
        if not e <= worst:
            worst, where = e, t
    return worst, where


def momentum_elementwise_ok(M_gpu, M0, G, beta: float, bf16: bool):
    """Every element of M' within one ulp (of its storage dtype) of
    beta*M0 + G, with beta as the float32 the library receives; returns
    (ok, worst ratio of |error| to that ulp)."""
    M_gpu = np.asarray(M_gpu, np.float64)
    b32 = float(np.float32(beta))
    M_ref = b32 * np.asarray(M0, np.float64) + np.asarray(G, np.float64)
    u = ulp_bf16(M_ref) if bf16 else ulp_f32(M_ref)
    ratio = np.abs(M_gpu - M_ref) / u
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(ratio <= 1.0)), worst


def compare_matrix(W0, G, M0, Wg, Mg, Og, ref, beta: float, bf16: bool):
    """All bars for one matrix: inputs W0, G, M0, GPU results Wg, Mg, Og (Og
    may be None), oracle results ref = (W', M', O).  Returns (ok, figures)."""
    W_ref, M_ref, O_ref = ref
    tol = BF16_TOL if bf16 else F32_TOL
    f = {}
    f["O"] = rel(Og, O_ref) if Og is not None else 0.0
    f["M"] = rel(Mg, M_ref)
    if bf16:
        f["W"] = w_error_bf16(Wg, W_ref, W0)
        w_ok = f["W"] <= 1.0
        f["W_tile"], f["W_tile_at"] = worst_tile_w_bf16(Wg, W_ref, W0)
        w_tile_ok = f["W_tile"] <= TILE_FACTOR
    else:
        dW_g = np.asarray(Wg, np.float64) - W0
        f["W"] = rel(dW_g, W_ref - W0)
        w_ok = f["W"] <= tol
        f["W_tile"], f["W_tile_at"] = worst_tile_rel(dW_g, W_ref - W0)
        w_tile_ok = f["W_tile"] <= TILE_FACTOR * tol
    if Og is not None:
        f["O_tile"], f["O_tile_at"] = worst_tile_rel(Og, O_ref)
    else:
        f["O_tile"], f["O_tile_at"] = 0.0, None
    m_elem_ok, f["M_ulp"] = momentum_elementwise_ok(Mg, M0, G, beta, bf16)
    finite = all(np.isfinite(f[k]) for k in ("O", "M", "W", "O_tile", "W_tile", "M_ulp"))
    ok = (finite and f["O"] <= tol and f["M"] <= tol and w_ok
          and f["O_tile"] <= TILE_FACTOR * tol and w_tile_ok and m_elem_ok)
    return ok, f
