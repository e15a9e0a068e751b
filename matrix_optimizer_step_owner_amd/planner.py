"""Balance-aware owner planning for a model's optimizer state.

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" -- arxivlens page, Methodology (ownership assigned by a
balance-aware planner, by bytes and by work); gist.science summaries,
"Méthodologie", part 2, first mechanism (resident bytes and optimizer work
balanced across the ranks), part 1 (1D and other non-2D tensors grouped on a tail
owner).

Every 2D weight is an item owned whole by one rank; every non-matrix tensor
is an item of that rank's packed tail.  Each item has a predicted step time
(its cost) and resident bytes; ``mfsdp_plan_owners`` assigns them (greedy
longest-processing-time first under a byte cap, in C++).  Costs come from
times measured per distinct shape on this GPU (``measure_shape_ms``, a
single-matrix ``mfsdp_muon_step`` each) or, without a GPU, from an analytic
model whose rates are stated arguments.

``python -m matrix_optimizer_step_owner_amd.planner --workload
llama3_8b_4blocks --ranks 8 [--measure]`` prints the plan and the predicted
per-rank step time.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import time
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import plan_owners, tail_layout

#: resident bytes per element of an owned matrix: weight, gradient and
#: momentum in the storage dtype
MATRIX_STATES = 3
#: resident bytes per element of a tail tensor: fp32 parameter, gradient and
#: the two AdamW moments
TAIL_BYTES_PER_ELEM = 16
#: algorithmic HBM bytes per element of the elementwise work of a matrix step
#: (momentum: read G, M, write M' and U; apply: read and write W), per storage
#: byte, and of AdamW per tail element
MATRIX_EW_BYTES_PER_STORAGE_BYTE = 6
TAIL_EW_BYTES_PER_ELEM = 28


def ns_flops(rows: int, cols: int, ns_steps: int = 5) -> float:
    """Algorithmic Newton-Schulz flops of one matrix (symmetric products once)."""
    m, n = min(rows, cols), max(rows, cols)
    return ns_steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


@dataclasses.dataclass
class CostModel:
    """Analytic step time: NS flops at a sustained rate, elementwise bytes at
    a sustained HBM rate, plus a fixed per-matrix cost (launch share, small-
    matrix inefficiency).  Rates are arguments, e.g. measured ones."""
    ns_tflops: float = 800.0
    hbm_gbs: float = 5000.0
    per_matrix_us: float = 20.0

    def matrix_ms(self, rows: int, cols: int, storage_bytes: int, ns_steps: int = 5) -> float:
        t = ns_flops(rows, cols, ns_steps) / (self.ns_tflops * 1e12)
        t += rows * cols * storage_bytes * MATRIX_EW_BYTES_PER_STORAGE_BYTE / (self.hbm_gbs * 1e9)
        return 1e3 * t + self.per_matrix_us * 1e-3

    def tail_ms(self, numel: int) -> float:
        return 1e3 * numel * TAIL_EW_BYTES_PER_ELEM / (self.hbm_gbs * 1e9)


def measure_shape_ms(shapes: Sequence[Tuple[int, int]], dtype=torch.bfloat16,
                     reps: int = 5, device: str = "cuda:0") -> Dict[Tuple[int, int], float]:
    """Median ms of a single-matrix owner-local Muon step per distinct shape."""
    from . import muon_step
    out = {}
    dev = torch.device(device)
    for shape in sorted(set(tuple(s) for s in shapes)):
        W = [torch.randn(shape, device=dev).to(dtype) * 0.02]
        G = [torch.randn(shape, device=dev).to(dtype) * 1e-3]
        M = [torch.zeros(shape, device=dev, dtype=dtype)]
        muon_step(W, G, M, lr=0.02, weight_decay=0.01)
        torch.cuda.synchronize(dev)
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            muon_step(W, G, M, lr=0.02, weight_decay=0.01)
            e1.record()
            torch.cuda.synchronize(dev)
            ts.append(e0.elapsed_time(e1))
        out[shape] = sorted(ts)[len(ts) // 2]
        del W, G, M
    return out


@dataclasses.dataclass
class OwnerPlan:
    n_ranks: int
    matrix_owner: List[int]
    tail_owner: List[int]
    tail_offsets: List[int]          # element offset in its owner's packed tail
    tail_numel_per_rank: List[int]   # packed tail length per rank
    rank_ms: List[float]             # predicted optimizer-step ms per rank
    rank_bytes: List[int]            # resident optimizer bytes per rank

    def matrices_of(self, rank: int) -> List[int]:
        return [i for i, r in enumerate(self.matrix_owner) if r == rank]

    def tails_of(self, rank: int) -> List[int]:
        return [i for i, r in enumerate(self.tail_owner) if r == rank]


def plan(matrices: Sequence[Tuple[int, int]], tails: Sequence[int], n_ranks: int,
         storage_bytes: int = 2, shape_ms: Optional[Dict[Tuple[int, int], float]] = None,
         model: Optional[CostModel] = None, byte_slack: float = 0.1,
         ns_steps: int = 5) -> OwnerPlan:
    """Assign every matrix and tail tensor to an owner; lay out each owner's
    packed tail.  Costs: ``shape_ms`` where it has the shape, else ``model``."""
    model = model or CostModel()
    cost, nbytes = [], []
    for r, c in matrices:
        ms = shape_ms.get((r, c)) if shape_ms else None
        cost.append(ms if ms is not None else model.matrix_ms(r, c, storage_bytes, ns_steps))
        nbytes.append(MATRIX_STATES * storage_bytes * r * c)
    for k in tails:
        cost.append(model.tail_ms(k))
        nbytes.append(TAIL_BYTES_PER_ELEM * k)
    owner, rank_ms, rank_bytes = plan_owners(cost, nbytes, n_ranks, byte_slack)
    nm = len(matrices)
    m_owner, t_owner = owner[:nm], owner[nm:]
    t_off = [0] * len(tails)
    t_len = [0] * n_ranks
    for rank in range(n_ranks):
        mine = [i for i, r in enumerate(t_owner) if r == rank]
        offs, total = tail_layout([tails[i] for i in mine])
        for i, o in zip(mine, offs):
            t_off[i] = o
        t_len[rank] = total
    return OwnerPlan(n_ranks, m_owner, t_owner, t_off, t_len, rank_ms, rank_bytes)


def main(argv=None) -> None:
    from . import workloads as wlm
    ap = argparse.ArgumentParser(prog="python -m matrix_optimizer_step_owner_amd.planner")
    ap.add_argument("--workload", default="llama3_8b_4blocks", choices=list(wlm.WORKLOADS))
    ap.add_argument("--ranks", type=int, default=8)
    ap.add_argument("--tail-tensors", type=int, default=0,
                    help="split the workload's tail into this many equal tensors (default: "
                         "one per 4096 elements)")
    ap.add_argument("--repeat", type=int, default=1,
                    help="plan this many copies of the workload's matrices and tail (a "
                         "whole model from a few blocks)")
    ap.add_argument("--measure", action="store_true", help="measure per-shape ms on the GPU")
    ap.add_argument("--byte-slack", type=float, default=0.1)
    a = ap.parse_args(argv)
    wl = wlm.WORKLOADS[a.workload]
    mats = [(s.rows, s.cols) for s in wl.matrices] * a.repeat
    nt = a.tail_tensors or max(1, wl.tail_n // 4096) if wl.tail_n else 0
    tails = ([wl.tail_n // nt] * nt if nt else []) * a.repeat
    es = 2 if wl.dtype == torch.bfloat16 else 4
    shape_ms = None
    if a.measure:
        t0 = time.perf_counter()
        shape_ms = measure_shape_ms(mats, wl.dtype)
        print(f"measured {len(shape_ms)} shapes in {time.perf_counter() - t0:.1f} s: "
              + ", ".join(f"{r}x{c}={ms:.3f}ms" for (r, c), ms in shape_ms.items()), flush=True)
    p = plan(mats, tails, a.ranks, es, shape_ms=shape_ms, byte_slack=a.byte_slack)
    total = sum(p.rank_ms)
    print(json.dumps({
        "workload": a.workload, "repeat": a.repeat, "matrices": len(mats),
        "tail_tensors": len(tails), "ranks": a.ranks,
        "costs": "measured per shape" if shape_ms else "analytic model",
        "predicted_step_ms_per_rank": [round(x, 4) for x in p.rank_ms],
        "max_rank_ms": round(max(p.rank_ms), 4),
        "balance_max_over_mean": round(max(p.rank_ms) / (total / a.ranks), 4) if total else None,
        "resident_gb_per_rank": [round(b / 1e9, 3) for b in p.rank_bytes],
        "matrices_per_rank": [len(p.matrices_of(r)) for r in range(a.ranks)],
        "tail_elements_per_rank": p.tail_numel_per_rank,
    }), flush=True)


if __name__ == "__main__":
    main()
