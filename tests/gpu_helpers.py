"""Helpers shared by the GPU parity tests: run the HIP step, run the oracle on
the same host values, and compare with the acceptance bars.

Acceptance (relative Frobenius error, float64, per tensor):
  * bf16 path: O and M' within 2e-2; W' within
        ||W'_gpu - W'_ref||_F <= 2e-2 ||W'_ref - W||_F + 0.5 ||ulp_bf16(W'_ref)||_F
    (an update is only a few bf16 ulps of W, so the final rounding of W' is
    allowed for separately);
  * fp32 path: O, M' and W' - W within 1e-4;
  * AdamW: p', m', v' within 1e-6.
"""

from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

import matrix_optimizer_step_owner_amd as mf
import oracle

BF16_TOL = 2e-2
F32_TOL = 1e-4
ADAMW_TOL = 1e-6


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(y)
    num = np.linalg.norm(x - y)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.where(ax > 0, np.exp2(e - 7), np.exp2(-133.0))


def w_error_bf16(W_gpu, W_ref, W0) -> float:
    """Ratio of the W' error to its allowance (<= 1 passes)."""
    err = np.linalg.norm(np.asarray(W_gpu, np.float64) - W_ref)
    allow = BF16_TOL * np.linalg.norm(W_ref - W0) + 0.5 * np.linalg.norm(ulp_bf16(W_ref))
    return float(err / allow)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


class GpuStep:
    """Uploads host inputs; `run` calls mf.muon_step in place on the device."""

    def __init__(self, weights, grads, momenta, device="cuda:0",
                 update_mask: Optional[Sequence[bool]] = None):
        self.device = torch.device(device)
        self.W = [w.to(self.device) for w in weights]
        self.G = [g.to(self.device) for g in grads]
        self.M = [m.to(self.device) for m in momenta]
        self.U = [torch.full(w.shape, float("nan"), dtype=torch.float32, device=self.device)
                  if update_mask is None or update_mask[i] else None
                  for i, w in enumerate(weights)]

    def run(self, scales=None, **hp):
        mf.muon_step(self.W, self.G, self.M, update_out=self.U, scales=scales, **hp)
        torch.cuda.synchronize(self.device)


def muon_hparams(wl=None, **over):
    hp = dict(lr=0.02, beta=0.95, nesterov=True, weight_decay=0.01, ns_steps=5,
              abc=(3.4445, -4.7750, 2.0315))
    if wl is not None:
        hp.update(lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov,
                  weight_decay=wl.weight_decay, ns_steps=wl.ns_steps, abc=wl.abc)
    hp.update(over)
    return hp


def oracle_matrix(W, G, M, hp, scale=None):
    return oracle.muon_matrix_step(f64(W), f64(G), f64(M), lr=hp["lr"], beta=hp["beta"],
                                   nesterov=hp["nesterov"],
                                   weight_decay=hp["weight_decay"],
                                   ns_steps=hp["ns_steps"], abc=hp["abc"], scale=scale)


def check_matrix(idx, W0, Wg, Mg, Og, ref, dtype, label=""):
    """Compare one matrix's GPU results with the oracle's; returns errors."""
    W_ref, M_ref, O_ref = ref
    e_o = rel(Og, O_ref) if Og is not None else 0.0
    e_m = rel(Mg, M_ref)
    if dtype == torch.bfloat16:
        e_w = w_error_bf16(Wg, W_ref, W0)
        ok = e_o <= BF16_TOL and e_m <= BF16_TOL and e_w <= 1.0
    else:
        e_w = rel(np.asarray(Wg) - W0, W_ref - W0)
        ok = e_o <= F32_TOL and e_m <= F32_TOL and e_w <= F32_TOL
    msg = f"{label} matrix {idx} {tuple(W0.shape)}: rel O={e_o:.3e} M={e_m:.3e} W={e_w:.3e}"
    say(msg)
    assert np.isfinite(e_o) and np.isfinite(e_m) and np.isfinite(e_w), msg
    assert ok, msg
    return e_o, e_m, e_w


def run_and_check(weights, grads, momenta, hp, dtype, label="", scales=None,
                  check_idx: Optional[List[int]] = None):
    """Full GPU step on all matrices, oracle on `check_idx` (default all)."""
    W0 = [f64(w) for w in weights]
    idxs = list(range(len(weights))) if check_idx is None else list(check_idx)
    mask = [i in set(idxs) for i in range(len(weights))]
    st = GpuStep(weights, grads, momenta, update_mask=mask)
    st.run(scales=scales, **hp)
    out = []
    for i in idxs:
        s = None if scales is None else scales[i]
        ref = oracle_matrix(weights[i], grads[i], momenta[i], hp, scale=s)
        out.append(check_matrix(i, W0[i], f64(st.W[i]), f64(st.M[i]), f64(st.U[i]), ref,
                                dtype, label))
    return st, out
