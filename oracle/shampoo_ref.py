"""fp64 oracle of Shampoo-type preconditioner statistics on the owner.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" -- gist.science summaries (French and Portuguese pages),
"Problématique" (Shampoo and SOAP, like Muon, take the whole 2D gradient as
input) and "Contributions clés", item "Généralité" (the owner-shaped layout is
not tied to one optimizer: Muon, Shampoo and SOAP all run on it).  The arxivlens
page names only Muon.  The pages give no formulas.
Reading R21: the textbook Shampoo statistics (Gupta, Koren and Singer 2018),
L += G G^T and R += G^T G, with SOAP's moving-average form
L <- beta L + alpha G G^T (alpha = 1 - beta) as the general case.
"""

from __future__ import annotations

import numpy as np


def shampoo_stats(G, L, R, *, beta: float, alpha: float):
    """Return (L', R') = (beta L + alpha G G^T, beta R + alpha G^T G) in float64.

    With beta == 0 the old statistics are not read (L' = alpha G G^T), so
    they may hold anything.  R may be None (no right statistic).
    """
    G = np.asarray(G, dtype=np.float64)
    GGt = G @ G.T
    L_new = alpha * GGt if beta == 0 else beta * np.asarray(L, np.float64) + alpha * GGt
    if R is None:
        return L_new, None
    GtG = G.T @ G
    R_new = alpha * GtG if beta == 0 else beta * np.asarray(R, np.float64) + alpha * GtG
    return L_new, R_new
