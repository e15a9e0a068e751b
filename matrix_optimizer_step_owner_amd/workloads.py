"""Seeded synthetic workloads for the owner-local optimizer step.

This module only draws numbers: it holds none of the optimizer's arithmetic.
The same host arrays feed the HIP library and the float64 oracle, so both sides
start from bit-identical inputs.

Recipe (the pages name no dataset; every input is synthetic):

* one ``numpy.random.default_rng(seed)`` (PCG64) per workload, seed 0 unless
  stated;
* for each matrix in listing order: draw W, then G, then M when it is random;
  afterwards the tail parameter (when random) and the tail gradient;
* normals are drawn in float32 (``standard_normal(dtype=float32)``), scaled in
  float32 and rounded to the storage dtype with round-to-nearest-even (torch's
  conversion);
* "N(0, x)" means standard deviation x.

The five workloads mirror the owner shares of the pages' transformer models:
one tiny fp32 correctness case, one d=2048 block, four Llama-3-8B-shaped
blocks, 512 small MoE-expert-like matrices, and a 32B-class d=5120 share.
Matrices are stored row-major as (out_features, in_features).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

# Quintic Newton-Schulz coefficients used by every workload.
NS_ABC = (3.4445, -4.7750, 2.0315)


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    description: str
    dtype: torch.dtype
    matrices: Tuple[MatrixSpec, ...]
    w_std: float
    g_kind: str                 # "normal" or "row_loguniform"
    g_std: float                # std of G (normal) or of z (row_loguniform)
    m_std: Optional[float]      # None: momentum starts at zero
    tail_n: int
    tail_p: str                 # "ones" or "normal"
    tail_p_std: float
    tail_g_std: float
    lr: float = 0.02
    beta: float = 0.95
    nesterov: bool = True
    weight_decay: float = 0.01
    ns_steps: int = 5
    abc: Tuple[float, float, float] = NS_ABC
    adam_beta1: float = 0.9
    adam_beta2: float = 0.95
    adam_eps: float = 1e-8
    adam_lr: float = 0.02
    adam_weight_decay: float = 0.01
    adam_step: int = 1

    @property
    def n_elements(self) -> int:
        return sum(s.rows * s.cols for s in self.matrices)


def _block_d2048() -> Tuple[MatrixSpec, ...]:
    d, f = 2048, 5632
    return (MatrixSpec("wq", d, d), MatrixSpec("wk", d, d),
            MatrixSpec("wv", d, d), MatrixSpec("wo", d, d),
            MatrixSpec("gate", f, d), MatrixSpec("up", f, d),
            MatrixSpec("down", d, f))


def _llama_block(i: int, d: int, kv: int, f: int) -> List[MatrixSpec]:
    return [MatrixSpec(f"b{i}.wq", d, d), MatrixSpec(f"b{i}.wo", d, d),
            MatrixSpec(f"b{i}.wk", kv, d), MatrixSpec(f"b{i}.wv", kv, d),
            MatrixSpec(f"b{i}.gate", f, d), MatrixSpec(f"b{i}.up", f, d),
            MatrixSpec(f"b{i}.down", d, f)]


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        key="tiny_fp32",
        description="3 fp32 matrices 64x128, 128x64, 96x96 + 512-float AdamW tail",
        dtype=torch.float32,
        matrices=(MatrixSpec("a", 64, 128), MatrixSpec("b", 128, 64),
                  MatrixSpec("c", 96, 96)),
        w_std=0.02, g_kind="normal", g_std=1e-3, m_std=None,
        tail_n=512, tail_p="normal", tail_p_std=0.02, tail_g_std=1e-3),
    "block_d2048": Workload(
        key="block_d2048",
        description="one d=2048 transformer block owner share in bf16 "
                    "(Wq/Wk/Wv/Wo 2048x2048, gate/up 5632x2048, down 2048x5632)"
                    " + 2x2048 RMSNorm-gain tail",
        dtype=torch.bfloat16,
        matrices=_block_d2048(),
        w_std=0.02, g_kind="normal", g_std=1e-3, m_std=1e-3,
        tail_n=2 * 2048, tail_p="ones", tail_p_std=0.0, tail_g_std=1e-3),
    "llama3_8b_4blocks": Workload(
        key="llama3_8b_4blocks",
        description="4 Llama-3-8B-shaped blocks in bf16 (d=4096, GQA kv=1024, "
                    "ffn=14336), per-row log-uniform gradient scale + 8x4096 tail",
        dtype=torch.bfloat16,
        matrices=tuple(s for i in range(4)
                       for s in _llama_block(i, 4096, 1024, 14336)),
        w_std=0.02, g_kind="row_loguniform", g_std=1.0, m_std=None,
        tail_n=8 * 4096, tail_p="ones", tail_p_std=0.0, tail_g_std=1e-3),
    "many_small": Workload(
        key="many_small",
        description="256 matrices 512x512 + 256 matrices 512x1536 in bf16, no tail",
        dtype=torch.bfloat16,
        matrices=tuple([MatrixSpec(f"sq{i}", 512, 512) for i in range(256)] +
                       [MatrixSpec(f"ex{i}", 512, 1536) for i in range(256)]),
        w_std=0.02, g_kind="normal", g_std=1e-3, m_std=None,
        tail_n=0, tail_p="normal", tail_p_std=0.02, tail_g_std=1e-3),
    "d5120_2blocks": Workload(
        key="d5120_2blocks",
        description="2 blocks of a 32B-class model in bf16 (d=5120, kv=1024, "
                    "ffn=27648) + 1M-element packed fp32 tail",
        dtype=torch.bfloat16,
        matrices=tuple(s for i in range(2)
                       for s in _llama_block(i, 5120, 1024, 27648)),
        w_std=0.02, g_kind="normal", g_std=1e-3, m_std=None,
        tail_n=1 << 20, tail_p="normal", tail_p_std=0.02, tail_g_std=1e-3),
}

#: Listing order of the five workloads (small correctness case first).
WORKLOAD_ORDER = ("tiny_fp32", "block_d2048", "llama3_8b_4blocks",
                  "many_small", "d5120_2blocks")


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    return x


def _to_storage(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(x).to(dtype)


@dataclasses.dataclass
class Inputs:
    """Host tensors of one workload in their storage dtypes."""
    workload: Workload
    weights: List[torch.Tensor]
    grads: List[torch.Tensor]
    momenta: List[torch.Tensor]
    tail_p: torch.Tensor
    tail_g: torch.Tensor
    tail_m: torch.Tensor
    tail_v: torch.Tensor


def draw_matrix(rng: np.random.Generator, wl: Workload, spec: MatrixSpec):
    """Draw (W, G, M) for one matrix, in that order, as storage-dtype tensors."""
    r, c = spec.rows, spec.cols
    W = _to_storage(_normal(rng, (r, c), wl.w_std), wl.dtype)
    if wl.g_kind == "normal":
        G = _to_storage(_normal(rng, (r, c), wl.g_std), wl.dtype)
    elif wl.g_kind == "row_loguniform":
        expo = rng.uniform(-4.0, -2.0, size=(r, 1))
        scale = np.power(10.0, expo).astype(np.float32)
        z = _normal(rng, (r, c), wl.g_std)
        z *= scale
        G = _to_storage(z, wl.dtype)
    else:
        raise ValueError(wl.g_kind)
    if wl.m_std is None:
        M = torch.zeros((r, c), dtype=wl.dtype)
    else:
        M = _to_storage(_normal(rng, (r, c), wl.m_std), wl.dtype)
    return W, G, M


def draw_tail(rng: np.random.Generator, wl: Workload):
    n = wl.tail_n
    if wl.tail_p == "ones":
        p = np.ones(n, dtype=np.float32)
    else:
        p = _normal(rng, (n,), wl.tail_p_std)
    g = _normal(rng, (n,), wl.tail_g_std)
    z = np.zeros(n, dtype=np.float32)
    return (torch.from_numpy(p), torch.from_numpy(g),
            torch.from_numpy(z.copy()), torch.from_numpy(z.copy()))


def generate(key: str, seed: int = 0,
             matrix_indices: Optional[List[int]] = None) -> Inputs:
    """Generate a workload's inputs on the host.

    ``matrix_indices`` keeps only some matrices; the random stream is still
    consumed for every matrix in listing order, so a kept matrix has the same
    values as in the full workload.
    """
    wl = WORKLOADS[key]
    rng = np.random.default_rng(seed)
    Ws, Gs, Ms = [], [], []
    keep = None if matrix_indices is None else set(matrix_indices)
    for i, spec in enumerate(wl.matrices):
        W, G, M = draw_matrix(rng, wl, spec)
        if keep is None or i in keep:
            Ws.append(W)
            Gs.append(G)
            Ms.append(M)
    p, g, m, v = draw_tail(rng, wl)
    return Inputs(wl, Ws, Gs, Ms, p, g, m, v)


def random_matrix_inputs(shapes, dtype: torch.dtype, seed: int,
                         w_std: float = 0.02, g_std: float = 1e-3,
                         m_std: Optional[float] = 1e-3):
    """(W, G, M) lists for arbitrary shapes (ragged-shape and edge cases)."""
    rng = np.random.default_rng(seed)
    Ws, Gs, Ms = [], [], []
    for (r, c) in shapes:
        Ws.append(_to_storage(_normal(rng, (r, c), w_std), dtype))
        Gs.append(_to_storage(_normal(rng, (r, c), g_std), dtype))
        if m_std is None:
            Ms.append(torch.zeros((r, c), dtype=dtype))
        else:
            Ms.append(_to_storage(_normal(rng, (r, c), m_std), dtype))
    return Ws, Gs, Ms


def random_tail_state(n: int, seed: int, p_std: float = 0.02,
                      g_std: float = 1e-3, m_std: float = 1e-3,
                      v_std: float = 1e-3):
    """A non-fresh AdamW tail state: m ~ N(0, m_std), v = (N(0, v_std))^2."""
    rng = np.random.default_rng(seed)
    p = _normal(rng, (n,), p_std)
    g = _normal(rng, (n,), g_std)
    m = _normal(rng, (n,), m_std)
    v = _normal(rng, (n,), v_std)
    v = v * v
    return (torch.from_numpy(p), torch.from_numpy(g), torch.from_numpy(m),
            torch.from_numpy(v))


def trajectory_gradients(shapes, dtype: torch.dtype, steps: int, seed: int,
                         g_std: float = 1e-3, tail_n: int = 0, tail_g_std: float = 1e-3):
    """Per-step gradients of a multi-step run: step t draws, from
    ``default_rng([seed, t])``, one G per shape (listing order) and then the
    tail gradient.  Returns ``[(Gs, tail_g), ...]`` with one entry per step."""
    out = []
    for t in range(steps):
        rng = np.random.default_rng([seed, t])
        Gs = [_to_storage(_normal(rng, tuple(s), g_std), dtype) for s in shapes]
        g = torch.from_numpy(_normal(rng, (tail_n,), tail_g_std))
        out.append((Gs, g))
    return out


def describe(key: str) -> str:
    wl = WORKLOADS[key]
    return (f"{wl.key}: {len(wl.matrices)} matrices, {wl.n_elements:,} "
            f"elements, tail {wl.tail_n:,}")
