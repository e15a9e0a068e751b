"""Pins of the statistics oracle (CPU only).

* trace(G G^T) = trace(G^T G) = ||G||_F^2;
* rank one G = u v^T: G G^T = ||v||^2 u u^T and G^T G = ||u||^2 v v^T;
* G G^T and G^T G share their nonzero eigenvalues, the squared singular values;
* a triple-loop definition on a tiny matrix;
* the beta/alpha form: beta = 0 ignores the old value (even NaN), beta = 1 and
  alpha = 1 accumulate.
"""

import numpy as np

import oracle


def test_trace_identity_and_spectrum():
    rng = np.random.default_rng(0)
    G = rng.standard_normal((7, 12))
    L, R = oracle.shampoo_stats(G, None, np.zeros((12, 12)), beta=0.0, alpha=1.0)
    fro2 = np.sum(G * G)
    assert abs(np.trace(L) - fro2) < 1e-12 * fro2
    assert abs(np.trace(R) - fro2) < 1e-12 * fro2
    s = np.linalg.svd(G, compute_uv=False)
    eL = np.sort(np.linalg.eigvalsh(L))[::-1]
    eR = np.sort(np.linalg.eigvalsh(R))[::-1]
    np.testing.assert_allclose(eL, s ** 2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(eR[:7], s ** 2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(eR[7:], 0.0, atol=1e-12)


def test_rank_one_closed_form():
    rng = np.random.default_rng(1)
    u, v = rng.standard_normal(5), rng.standard_normal(9)
    G = np.outer(u, v)
    L, R = oracle.shampoo_stats(G, None, np.zeros((9, 9)), beta=0.0, alpha=1.0)
    np.testing.assert_allclose(L, (v @ v) * np.outer(u, u), rtol=1e-12)
    np.testing.assert_allclose(R, (u @ u) * np.outer(v, v), rtol=1e-12)


def test_triple_loop_definition_and_beta_alpha():
    rng = np.random.default_rng(2)
    G = rng.standard_normal((3, 4))
    L0 = rng.standard_normal((3, 3))
    R0 = rng.standard_normal((4, 4))
    L, R = oracle.shampoo_stats(G, L0, R0, beta=0.9, alpha=0.1)
    for i in range(3):
        for j in range(3):
            want = 0.9 * L0[i, j] + 0.1 * sum(G[i, k] * G[j, k] for k in range(4))
            assert abs(L[i, j] - want) < 1e-14
    for i in range(4):
        for j in range(4):
            want = 0.9 * R0[i, j] + 0.1 * sum(G[k, i] * G[k, j] for k in range(3))
            assert abs(R[i, j] - want) < 1e-14
    Ln, _ = oracle.shampoo_stats(G, np.full((3, 3), np.nan), None, beta=0.0, alpha=2.0)
    assert np.all(np.isfinite(Ln))
    La, _ = oracle.shampoo_stats(G, L0, None, beta=1.0, alpha=1.0)
    np.testing.assert_allclose(La, L0 + G @ G.T, rtol=1e-14, atol=1e-14)
