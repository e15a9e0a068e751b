"""Helpers shared by the GPU parity tests: run the HIP step, run the oracle on
the same host values, and compare with the acceptance bars of
tests/parity_checks.py (per tensor, per 256 x 256 tile, and elementwise for
the momentum).
"""

from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

import matrix_optimizer_step_owner_amd as mf
import oracle

from parity_checks import (ADAMW_TOL, BF16_TOL, F32_TOL, compare_matrix, rel,  # noqa: F401
                           ulp_bf16, w_error_bf16)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


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


def check_matrix(idx, W0, G, M0, Wg, Mg, Og, ref, dtype, beta, label=""):
    """Compare one matrix's GPU results with the oracle's (every bar of
    parity_checks.compare_matrix); returns (rel O, rel M', W' figure)."""
    ok, f = compare_matrix(W0, G, M0, Wg, Mg, Og, ref, beta, dtype == torch.bfloat16)
    msg = (f"{label} matrix {idx} {tuple(W0.shape)}: rel O={f['O']:.3e} M={f['M']:.3e} "
           f"W={f['W']:.3e}; worst tile O={f['O_tile']:.3e} at {f['O_tile_at']}, "
           f"W={f['W_tile']:.3e} at {f['W_tile_at']}; M' worst {f['M_ulp']:.2f} ulp")
    say(msg)
    assert ok, msg
    return f["O"], f["M"], f["W"]


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
        out.append(check_matrix(i, W0[i], f64(grads[i]), f64(momenta[i]), f64(st.W[i]),
                                f64(st.M[i]), f64(st.U[i]), ref, dtype, hp["beta"], label))
    return st, out
