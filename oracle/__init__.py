"""Plain fp64 CPU oracle of the owner-local optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and imports
nothing from it.

What it computes (source: "MatrixFSDP: communication-free matrix optimizers
under ZeRO-3 parameter sharding", arxivlens page, Abstract; and the
gist.science technical summaries, section "Méthodologie" / "Metodologia",
part 1 "Owner-shaped placement"):

* every 2D weight lives whole on one owner, whose optimizer step runs Muon on
  the whole matrix -- a momentum-smoothed update orthogonalized by a
  Newton-Schulz iteration -- with no communication;
* every tensor that is not a 2D matrix goes, packed, to a tail owner, where
  AdamW updates it.

The pages give no formula for either step, so each arithmetic choice is a
reading stated in the docstring where it is made.  The oracle is written in
numpy, in float64, one matrix at a time, using dense products only (no
symmetry, blocking or fusion).

Parity status of each function (what pins it, see ``tests/test_oracle_pins.py``):

* ``momentum_nesterov``      pinned (special cases M=0 / G=0 / no Nesterov, torch.optim.Muon)
* ``frobenius_normalize``    pinned (norm of the result, scale invariance)
* ``newton_schulz``          pinned (SVD closed form, cubic -> polar factor, invariants)
* ``muon_matrix_step``       pinned (torch.optim.Muon with this NS plugged in, zero-grad decay)
* ``muon_step``              pinned (order independence, equals per-matrix steps)
* ``adamw_tail``             pinned (torch.optim.AdamW in float64, constant-gradient invariant)
* ``quintic_scalar_exact``   pinned (it is the scalar map the SVD closed form composes)
* ``default_scale``          parity unpinned: the pages fix no update scale; the
                             value follows the common original-Muon convention.
* ``round_to_bf16``          pinned (torch's float32 -> bfloat16 conversion, hand-worked ties)
* ``muon_trajectory``        pinned (one step = the single-step oracle; momentum closed form)
* ``adamw_trajectory``       pinned (constant-gradient closed form over many steps)
* ``shampoo_stats``          pinned (Frobenius/trace identity, rank-1 closed form, shared
                             nonzero spectrum of G G^T and G^T G, triple-loop definition)
* ``planner_ref``            the LPT rule pinned by a hand-worked schedule and Graham's
                             4/3 - 1/(3R) bound against brute-force optima; the
                             tail layout by hand-worked offsets
"""

from .muon_ref import (
    NS_EPS,
    default_scale,
    frobenius_normalize,
    momentum_nesterov,
    muon_matrix_step,
    muon_step,
    newton_schulz,
)
from .adamw_ref import adamw_tail
from .ns_scalar import quintic_scalar_exact, quintic_scalar_float
from .trajectory import adamw_trajectory, muon_trajectory, round_to_bf16, round_to_f32
from . import planner_ref
from .shampoo_ref import shampoo_stats

__all__ = [
    "NS_EPS",
    "adamw_tail",
    "adamw_trajectory",
    "default_scale",
    "frobenius_normalize",
    "momentum_nesterov",
    "muon_matrix_step",
    "muon_step",
    "muon_trajectory",
    "newton_schulz",
    "planner_ref",
    "quintic_scalar_exact",
    "quintic_scalar_float",
    "round_to_bf16",
    "round_to_f32",
    "shampoo_stats",
]
