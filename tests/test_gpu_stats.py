"""Shampoo-type statistics on the GPU against the float64 oracle.

Bar: relative Frobenius error <= 2e-5 per statistic.  Derivation: the
gradient values are exact in both paths (the oracle upcasts the stored bf16 /
fp32 values), every product of two bf16 values is exact in fp32, and the fp32
accumulation of K terms errs by about sqrt(K) * 2^-24 relative in the typical
(random-sign) case: 4.5e-6 at K = 5632, the largest K here, plus one rounding
of beta*L + alpha*GG^T; 2e-5 leaves a four-fold margin.  The statistics are
also exactly symmetric (upper tiles mirrored).
"""

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
from matrix_optimizer_step_owner_amd import workloads as wlm
import oracle

from gpu_helpers import f64, rel, say

pytestmark = pytest.mark.gpu

TOL = 2e-5
SHAPES = [(300, 1000), (1000, 300), (256, 256), (17, 33), (1, 300), (513, 257),
          (2048, 5632)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _spd(n, rng):
    a = rng.standard_normal((n, min(n, 64))).astype(np.float32) * 1e-3
    return (a @ a.T).astype(np.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("beta,alpha", [(0.0, 1.0), (0.95, 0.05), (1.0, 1.0)])
def test_stats_parity(dtype, beta, alpha):
    shapes = SHAPES if dtype == torch.bfloat16 else SHAPES[:-1]
    _, Gs, _ = wlm.random_matrix_inputs(shapes, dtype, seed=11, m_std=None)
    rng = np.random.default_rng(12)
    L0 = [np.full((r, r), np.nan, np.float32) if beta == 0 else _spd(r, rng) for r, _ in shapes]
    R0 = [np.full((c, c), np.nan, np.float32) if beta == 0 else _spd(c, rng) for _, c in shapes]
    dev = torch.device("cuda:0")
    G = [g.to(dev) for g in Gs]
    L = [torch.from_numpy(x).to(dev) for x in L0]
    # the third matrix has no right statistic
    R = [None if i == 2 else torch.from_numpy(x).to(dev) for i, x in enumerate(R0)]
    mf.shampoo_stats(G, L, R, beta=beta, alpha=alpha)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (r, c) in enumerate(shapes):
        Lr, Rr = oracle.shampoo_stats(f64(Gs[i]), L0[i].astype(np.float64),
                                      None if R[i] is None else R0[i].astype(np.float64),
                                      beta=beta, alpha=alpha)
        Lg = f64(L[i])
        assert np.array_equal(Lg, Lg.T), f"L of {r}x{c} not symmetric"
        e = rel(Lg, Lr)
        worst = max(worst, e)
        assert e <= TOL, (r, c, "L", e)
        if R[i] is not None:
            Rg = f64(R[i])
            assert np.array_equal(Rg, Rg.T)
            e = rel(Rg, Rr)
            worst = max(worst, e)
            assert e <= TOL, (r, c, "R", e)
    say(f"stats {dtype} beta={beta} alpha={alpha}: worst rel {worst:.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_stats_unaligned_gradient(dtype):
    # rows of a whole number of 16-byte vectors, but the gradient starts one
    # element past a 16-byte boundary: the element-wise copy path, against the
    # same statistics from an aligned copy of the same values and the oracle
    r, c = 96, 320
    dev = torch.device("cuda:0")
    _, Gs, _ = wlm.random_matrix_inputs([(r, c)], dtype, seed=13, m_std=None)
    buf = torch.zeros(r * c + 8, dtype=dtype, device=dev)
    buf[1:1 + r * c] = Gs[0].reshape(-1).to(dev)
    G_off = buf[1:1 + r * c].view(r, c)
    assert G_off.data_ptr() % 16 != 0
    G_al = Gs[0].to(dev).contiguous()
    assert G_al.data_ptr() % 16 == 0
    outs = []
    for G in (G_off, G_al):
        L = torch.zeros(r, r, device=dev)
        R = torch.zeros(c, c, device=dev)
        mf.shampoo_stats([G], [L], [R], beta=0.0, alpha=1.0)
        outs.append((L, R))
    torch.cuda.synchronize()
    Lr, Rr = oracle.shampoo_stats(f64(Gs[0]), np.zeros((r, r)), np.zeros((c, c)),
                                  beta=0.0, alpha=1.0)
    for L, R in outs:
        assert rel(f64(L), Lr) <= TOL and rel(f64(R), Rr) <= TOL
    # both copy paths feed the same product kernel the same operands
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
