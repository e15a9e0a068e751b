"""Plain references of the owner planner and the packed-tail layout.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" -- arxivlens page, Methodology (ownership is assigned by a
balance-aware planner, by bytes and by work); gist.science summaries,
"Méthodologie", part 2, first mechanism (resident bytes and optimizer work
balanced across ranks) and part 1 (1D and other non-2D tensors grouped on a tail
owner).  The pages give no algorithm.  Reading R20: greedy
longest-processing-time-first (Graham 1969) under a per-owner byte cap, with
the tie rules written below; tails packed in order with 16-byte aligned
segments, gaps zero.
"""

from __future__ import annotations

import itertools
import math
from typing import List, Sequence, Tuple

import numpy as np


def byte_cap(nbytes: Sequence[int], n_ranks: int, slack: float) -> int:
    """ceil((1 + slack) * max(total / R, largest item))."""
    total = sum(nbytes)
    largest = max(nbytes) if len(nbytes) else 0
    return int(math.ceil(max(total / n_ranks, largest) * (1.0 + slack)))


def lpt_owners(cost: Sequence[float], nbytes: Sequence[int], n_ranks: int,
               slack: float) -> Tuple[List[int], List[float], List[int]]:
    """Greedy LPT: items by decreasing cost (then more bytes, then lower index);
    each to the least-loaded owner (lowest rank on ties) among those that keep
    their bytes within the cap, else to the owner with the fewest bytes."""
    n = len(cost)
    cap = byte_cap(nbytes, n_ranks, slack)
    order = sorted(range(n), key=lambda i: (-cost[i], -nbytes[i], i))
    load = [0.0] * n_ranks
    used = [0] * n_ranks
    owner = [-1] * n
    for i in order:
        fits = [r for r in range(n_ranks) if used[r] + nbytes[i] <= cap]
        if fits:
            r = min(fits, key=lambda k: (load[k], k))
        else:
            r = min(range(n_ranks), key=lambda k: (used[k], k))
        owner[i] = r
        load[r] += cost[i]
        used[r] += nbytes[i]
    return owner, load, used


def optimal_makespan(cost: Sequence[float], n_ranks: int) -> float:
    """Smallest achievable maximum owner load, by trying every assignment."""
    best = math.inf
    for assign in itertools.product(range(n_ranks), repeat=len(cost)):
        load = [0.0] * n_ranks
        for i, r in enumerate(assign):
            load[r] += cost[i]
        best = min(best, max(load))
    return best


def tail_layout(numel: Sequence[int]) -> Tuple[List[int], int]:
    """Offsets of tensors packed in order, each on a 4-element boundary."""
    offs, off = [], 0
    for k in numel:
        offs.append(off)
        off += (k + 3) // 4 * 4
    return offs, off


def tail_pack(arrays: Sequence[np.ndarray]) -> Tuple[np.ndarray, List[int]]:
    """Packed float32 tail: each flattened array at its offset, zeros between."""
    offs, total = tail_layout([a.size for a in arrays])
    out = np.zeros(total, dtype=np.float32)
    for a, o in zip(arrays, offs):
        out[o:o + a.size] = np.asarray(a, dtype=np.float32).ravel()
    return out, offs
