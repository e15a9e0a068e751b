"""The comparison rules of the parity tests catch the faults they are meant to
(CPU only; every mistake is planted in an oracle result, never on a GPU).

A float64 oracle step of a 1280 x 768 (tall) matrix stands in for a GPU
result.  Relative noise of 1e-2 spread over every element (the size of the
bf16 path's rounding error) passes every bar.  Each planted fault passes the
per-tensor bar and must fail the per-tile or elementwise one:
* one 256 x 256 tile 5% off (2.5 times the bf16 bar, diluted below it over
  the 15 tiles of the matrix);
* one tile's mirror image (its transpose) stored instead of the tile;
* one row band of 32 rows sign-flipped inside one tile;
* one element of M' off by two bf16 ulps.
"""

import numpy as np
import pytest

import oracle
from parity_checks import (BF16_TOL, TILE_FACTOR, compare_matrix, rel, ulp_bf16,
                           worst_tile_rel)

HP = dict(lr=0.02, beta=0.95, nesterov=True, weight_decay=0.01, ns_steps=5,
          abc=(3.4445, -4.7750, 2.0315))


def _bf16(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(7)
    r, c = 1280, 768
    W0 = _bf16(rng.standard_normal((r, c)) * 0.02)
    G = _bf16(rng.standard_normal((r, c)) * 1e-3)
    M0 = _bf16(rng.standard_normal((r, c)) * 1e-3)
    ref = oracle.muon_matrix_step(W0, G, M0, **HP)
    W_ref, M_ref, O_ref = ref
    # uniform relative noise of standard deviation 1.5e-2 / sqrt(3) = 0.87e-2
    O_g = O_ref * (1 + rng.uniform(-1.5e-2, 1.5e-2, O_ref.shape))
    # W' as the GPU stores it: the noisy update applied, rounded to bf16
    decay = 1 - HP["lr"] * HP["weight_decay"]
    s = oracle.default_scale(r, c)
    W_g = _bf16(decay * W0 - HP["lr"] * s * O_g)
    M_g = _bf16(float(np.float32(HP["beta"])) * M0 + G)
    return W0, G, M0, ref, W_g, M_g, O_g


def _run(case, W_g=None, M_g=None, O_g=None):
    W0, G, M0, ref, Wg0, Mg0, Og0 = case
    return compare_matrix(W0, G, M0, Wg0 if W_g is None else W_g, Mg0 if M_g is None else M_g,
                          Og0 if O_g is None else O_g, ref, HP["beta"], True)


def test_clean_noise_passes(case):
    ok, f = _run(case)
    assert ok, f
    assert 0 < f["O"] < BF16_TOL and f["O_tile"] < TILE_FACTOR * BF16_TOL
    assert f["M_ulp"] <= 1.0


def test_one_tile_off_by_5_percent(case):
    O = case[6].copy()
    O[512:768, 256:512] *= 1.05
    assert rel(O, case[3][2]) < BF16_TOL          # per tensor: passes
    ok, f = _run(case, O_g=O)
    assert not ok and f["O_tile_at"] == (2, 1)


def test_mirror_stored_instead_of_tile(case):
    O = case[6].copy()
    O[256:512, 0:256] = O[256:512, 0:256].T.copy()
    ok, f = _run(case, O_g=O)
    assert not ok and f["O_tile_at"] == (1, 0)


def test_row_band_sign_flip(case):
    O = case[6].copy()
    O[1024 + 64:1024 + 96, 512:768] *= -1.0
    t, at = worst_tile_rel(O, case[3][2])
    assert t > TILE_FACTOR * BF16_TOL and at == (4, 2)
    ok, _ = _run(case, O_g=O)
    assert not ok


def test_weight_tile_fault(case):
    W0, _, _, ref, W_g, _, _ = case
    W = W_g.copy()
    # one tile of W' given the update twice: its error is the whole update
    W[0:256, 0:256] += ref[0][0:256, 0:256] - W0[0:256, 0:256]
    ok, f = _run(case, W_g=W)
    assert not ok and f["W_tile_at"] == (0, 0)


def test_momentum_element_two_ulps_off(case):
    M = case[5].copy()
    M[100, 200] += 2 * ulp_bf16(M[100, 200])
    assert rel(M, case[3][1]) < BF16_TOL
    ok, f = _run(case, M_g=M)
    assert not ok and f["M_ulp"] > 1.0
