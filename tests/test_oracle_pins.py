"""Pins of the float64 oracle against what the mathematics fixes.

None of these compare the oracle with itself: each one checks it against a
closed form, an invariant, an exact-arithmetic value or an independent library
routine (numpy's SVD, scipy's polar decomposition, torch.optim.Muon,
torch.optim.AdamW), chosen so that a dropped term, a wrong sign, a swapped
coefficient or a transposed operand in the oracle fails at least one test.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import (NS_EPS, adamw_tail, default_scale, frobenius_normalize,
                    momentum_nesterov, muon_matrix_step, muon_step,
                    newton_schulz, quintic_scalar_exact, quintic_scalar_float)

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ns_scalar.json")


def rel(x, y):
    return float(np.linalg.norm(np.asarray(x) - np.asarray(y)) /
                 np.linalg.norm(np.asarray(y)))


def spectral_ns(U, steps, abc, eps=NS_EPS):
    """Closed form: P diag(p^k(sigma / (nu + eps))) Q^T from numpy's SVD."""
    P, s, Qt = np.linalg.svd(np.asarray(U, np.float64), full_matrices=False)
    nu = math.sqrt(float(np.sum(s * s)))   # Frobenius norm from the spectrum
    f = np.array([quintic_scalar_float(x / (nu + eps), steps, abc) for x in s])
    return (P * f) @ Qt


# --------------------------------------------------------------------------
# Scalar map (exact arithmetic) and the golden table it wrote.
# --------------------------------------------------------------------------

def test_scalar_map_matches_independent_values():
    # p(1) = a + b + c, and values of p composed five times derived
    # independently of this code base (worked by hand / separate script).
    assert float(quintic_scalar_exact(1, 1, QUINTIC)) == pytest.approx(0.7010, abs=1e-12)
    assert float(quintic_scalar_exact(1, 5, QUINTIC)) == pytest.approx(0.696436409469752, rel=1e-13)
    for s, want in [(0.5, 0.76544), (0.1, 0.71212), (0.01, 0.69892),
                    (1e-3, 0.47054), (1e-4, 0.048473)]:
        got = float(quintic_scalar_exact(s, 5, QUINTIC))
        assert got == pytest.approx(want, rel=2e-4), (s, got)
    # The cubic map fixes 1 and maps (0, 1) into itself, increasing.
    assert quintic_scalar_exact(1, 7, CUBIC) == 1
    assert quintic_scalar_exact(Fraction(1, 2), 1, CUBIC) == Fraction(11, 16)


def test_scalar_float_agrees_with_exact():
    for s in [1.0, 0.5, 0.1, 0.01, 1e-3, 1e-4, 0.9, 0.3]:
        for k in range(6):
            e = float(quintic_scalar_exact(s, k, QUINTIC))
            assert quintic_scalar_float(s, k, QUINTIC) == pytest.approx(e, rel=1e-13)


def test_golden_table_consistent():
    with open(GOLDEN) as f:
        g = json.load(f)["values"]
    for name, abc in (("quintic", QUINTIC), ("cubic", CUBIC)):
        for s, row in g[name]["by_sigma"].items():
            assert row[0] == pytest.approx(float(s), rel=1e-15)
            for k, val in enumerate(row):
                assert quintic_scalar_float(float(s), k, abc) == pytest.approx(val, rel=1e-12, abs=1e-300)
    assert g["quintic"]["by_sigma"]["1"][5] == pytest.approx(0.696436409469752, rel=1e-13)


# --------------------------------------------------------------------------
# Newton-Schulz: SVD closed form, polar factor, invariants.
# --------------------------------------------------------------------------

SHAPES = [(64, 128), (128, 64), (96, 96), (17, 33), (33, 17), (1, 7), (7, 1)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_ns_spectral_closed_form(shape, steps):
    rng = np.random.default_rng(hash(shape) % 1000 + steps)
    U = rng.standard_normal(shape) * 1e-3
    X0, nu = frobenius_normalize(U)
    O = newton_schulz(X0, steps, *QUINTIC)
    want = spectral_ns(U, steps, QUINTIC)
    assert rel(O, want) < 1e-12


def test_ns_closed_form_with_spread_spectrum():
    # Prescribed singular values spanning 1e-4..1 relative to the norm.
    rng = np.random.default_rng(7)
    m, n = 40, 90
    P, _ = np.linalg.qr(rng.standard_normal((m, m)))
    Q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    s = np.logspace(0, -4, m)
    U = (P * s) @ Q.T
    O = newton_schulz(frobenius_normalize(U)[0], 5, *QUINTIC)
    assert rel(O, spectral_ns(U, 5, QUINTIC)) < 1e-11
    # The spectrum of the output is the scalar map of the input's.
    so = np.linalg.svd(O, compute_uv=False)
    nu = np.linalg.norm(s)
    want = np.sort([quintic_scalar_float(x / (nu + NS_EPS), 5, QUINTIC) for x in s])[::-1]
    assert np.allclose(np.sort(so)[::-1], want, rtol=1e-9, atol=1e-12)


def test_ns_rank_one_closed_form():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(24)
    v = rng.standard_normal(40)
    U = np.outer(u, v)
    O = newton_schulz(frobenius_normalize(U)[0], 5, *QUINTIC)
    want = 0.696436409469752 * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert rel(O, want) < 1e-6   # sigma/(nu+eps) = 1 - O(1e-7)


@pytest.mark.parametrize("shape", [(8, 8), (6, 6), (8, 4), (4, 8)])
def test_cubic_converges_to_polar_factor(shape):
    rng = np.random.default_rng(11)
    U = rng.standard_normal(shape)
    O = newton_schulz(frobenius_normalize(U)[0], 60, *CUBIC)
    P, _, Qt = np.linalg.svd(U, full_matrices=False)
    assert np.abs(O - P @ Qt).max() < 1e-12
    if shape[0] == shape[1]:
        polar_u, _ = scipy.linalg.polar(U)
        assert np.abs(O - polar_u).max() < 1e-12


def test_ns_invariants():
    rng = np.random.default_rng(5)
    U = rng.standard_normal((20, 36)) * 1e-3
    X0 = frobenius_normalize(U)[0]
    O = newton_schulz(X0, 5, *QUINTIC)
    # odd
    assert rel(newton_schulz(-X0, 5, *QUINTIC), -O) < 1e-14
    # transpose equivariance
    assert rel(newton_schulz(X0.T, 5, *QUINTIC), O.T) < 1e-13
    # orthogonal equivariance
    Q1, _ = np.linalg.qr(rng.standard_normal((20, 20)))
    Q2, _ = np.linalg.qr(rng.standard_normal((36, 36)))
    O2 = newton_schulz(Q1 @ X0 @ Q2, 5, *QUINTIC)
    assert rel(O2, Q1 @ O @ Q2) < 1e-12
    # zero steps returns the normalized input; the zero matrix stays zero
    assert np.array_equal(newton_schulz(X0, 0, *QUINTIC), X0)
    assert not newton_schulz(np.zeros((5, 9)), 5, *QUINTIC).any()


def test_ns_is_not_symmetric_in_operand_order():
    # A = X^T X (instead of X X^T) on a square non-normal X changes the result:
    # the closed form above would catch it, this documents that it is visible.
    rng = np.random.default_rng(9)
    X = frobenius_normalize(rng.standard_normal((12, 12)))[0]
    a, b, c = QUINTIC
    A = X.T @ X
    wrong = a * X + (b * A + c * A @ A) @ X
    right = newton_schulz(X, 1, *QUINTIC)
    assert rel(wrong, right) > 1e-3


# --------------------------------------------------------------------------
# Normalization.
# --------------------------------------------------------------------------

def test_frobenius_normalize():
    rng = np.random.default_rng(1)
    U = rng.standard_normal((13, 29)) * 1e-2
    X0, nu = frobenius_normalize(U)
    s = np.linalg.svd(U, compute_uv=False)
    assert nu == pytest.approx(math.sqrt(np.sum(s * s)), rel=1e-13)
    assert np.linalg.norm(X0) == pytest.approx(nu / (nu + NS_EPS), rel=1e-13)
    # scale invariance up to eps
    O1 = newton_schulz(X0, 5, *QUINTIC)
    O2 = newton_schulz(frobenius_normalize(37.0 * U)[0], 5, *QUINTIC)
    assert rel(O1, O2) < 1e-5
    X00, nu0 = frobenius_normalize(np.zeros((3, 4)))
    assert nu0 == 0.0 and not X00.any()


# --------------------------------------------------------------------------
# Momentum.
# --------------------------------------------------------------------------

def test_momentum_hand_worked_example():
    # beta = 0.5: M' = 0.5*[0.5, 4] + [1, -2] = [1.25, 0];
    # U = G + 0.5*M' = [1.625, -2].
    M_new, U = momentum_nesterov([[1.0, -2.0]], [[0.5, 4.0]], 0.5, True)
    assert M_new.tolist() == [[1.25, 0.0]]
    assert U.tolist() == [[1.625, -2.0]]
    M_new, U = momentum_nesterov([[1.0, -2.0]], [[0.5, 4.0]], 0.5, False)
    assert U.tolist() == [[1.25, 0.0]]


def test_momentum_special_cases():
    rng = np.random.default_rng(2)
    G = rng.standard_normal((4, 6))
    M = rng.standard_normal((4, 6))
    beta = 0.95
    Mn, U = momentum_nesterov(G, np.zeros_like(G), beta, True)
    assert np.array_equal(Mn, G)
    assert np.allclose(U, (1 + beta) * G, rtol=1e-15)
    Mn, U = momentum_nesterov(np.zeros_like(M), M, beta, True)
    assert np.allclose(Mn, beta * M, rtol=1e-15)
    assert np.allclose(U, beta * beta * M, rtol=1e-15)


# --------------------------------------------------------------------------
# Whole Muon step against torch.optim.Muon.
# --------------------------------------------------------------------------

def _torch_muon_steps(W, grads, lr, wd, beta, abc, ns_steps, eps, patch_ns):
    import torch.optim._muon as tm
    p = torch.nn.Parameter(torch.tensor(W, dtype=torch.float64))
    opt = torch.optim.Muon([p], lr=lr, weight_decay=wd, momentum=beta,
                           nesterov=True, ns_coefficients=abc, eps=eps,
                           ns_steps=ns_steps, adjust_lr_fn="original")
    saved = tm._zeropower_via_newtonschulz
    if patch_ns:
        def ns64(g, coeffs, steps, e):
            X0, _ = frobenius_normalize(g.numpy(), e)
            return torch.from_numpy(newton_schulz(X0, steps, *coeffs))
        tm._zeropower_via_newtonschulz = ns64
    try:
        for g in grads:
            p.grad = torch.tensor(g, dtype=torch.float64)
            opt.step()
    finally:
        tm._zeropower_via_newtonschulz = saved
    return p.detach().numpy(), opt.state[p]["momentum_buffer"].numpy()


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32)])
def test_muon_step_matches_torch_muon_conventions(shape):
    # torch.optim.Muon keeps an EMA momentum buffer, (1-beta) times the
    # heavy-ball buffer; Newton-Schulz is scale invariant, so with eps = 0 the
    # parameter trajectories coincide.  Its NS routine is swapped for the
    # float64 one so that only momentum / Nesterov / decay / lr scaling are
    # compared.
    rng = np.random.default_rng(4)
    W = rng.standard_normal(shape) * 0.02
    grads = [rng.standard_normal(shape) for _ in range(3)]
    lr, wd, beta = 0.02, 0.01, 0.95
    Wt, buf = _torch_muon_steps(W, grads, lr, wd, beta, QUINTIC, 5, 0.0, True)
    Wo, M = W.copy(), np.zeros(shape)
    for g in grads:
        Wo, M, _ = muon_matrix_step(Wo, g, M, lr=lr, beta=beta, nesterov=True,
                                    weight_decay=wd, ns_steps=5, abc=QUINTIC,
                                    eps=0.0)
    assert rel(Wt - W, Wo - W) < 1e-12
    assert rel(buf, (1 - beta) * M) < 1e-14


def test_muon_update_matches_torch_bf16_newton_schulz():
    # Unpatched torch.optim.Muon runs Newton-Schulz in bfloat16; the float64
    # update must agree with it to bf16 accuracy.  A swapped coefficient or a
    # missing normalization would be off by O(1).
    rng = np.random.default_rng(8)
    shape = (48, 80)
    W = rng.standard_normal(shape) * 0.02
    g = rng.standard_normal(shape) * 1e-3
    lr, wd = 0.02, 0.0
    Wt, _ = _torch_muon_steps(W, [g], lr, wd, 0.95, QUINTIC, 5, 1e-7, False)
    _, _, O = muon_matrix_step(W, g, np.zeros(shape), lr=lr, beta=0.95,
                               nesterov=True, weight_decay=wd, ns_steps=5,
                               abc=QUINTIC)
    O_torch = (W - Wt) / (lr * default_scale(*shape))
    assert rel(O_torch, O) < 3e-2


def test_muon_zero_gradient_is_decay_only():
    W = np.arange(12.0).reshape(3, 4) / 7
    Wn, Mn, O = muon_matrix_step(W, np.zeros((3, 4)), np.zeros((3, 4)), lr=0.1,
                                 beta=0.9, nesterov=True, weight_decay=0.5,
                                 ns_steps=5, abc=QUINTIC)
    assert not O.any() and not Mn.any()
    assert np.allclose(Wn, 0.95 * W, rtol=1e-15)


def test_muon_update_sign_and_scale():
    # wd = 0: W' - W = -lr * s * O with O from the SVD closed form.
    rng = np.random.default_rng(12)
    W = rng.standard_normal((30, 10))
    G = rng.standard_normal((30, 10))
    lr = 0.05
    Wn, _, _ = muon_matrix_step(W, G, np.zeros_like(G), lr=lr, beta=0.9,
                                nesterov=True, weight_decay=0.0, ns_steps=5,
                                abc=QUINTIC)
    O = spectral_ns((1 + 0.9) * G, 5, QUINTIC)
    assert rel(Wn - W, -lr * math.sqrt(3.0) * O) < 1e-12
    assert default_scale(30, 10) == pytest.approx(math.sqrt(3.0))
    assert default_scale(10, 30) == 1.0


def test_muon_list_is_per_matrix_and_order_free():
    rng = np.random.default_rng(6)
    shapes = [(8, 12), (12, 8), (10, 10)]
    Ws = [rng.standard_normal(s) for s in shapes]
    Gs = [rng.standard_normal(s) for s in shapes]
    Ms = [rng.standard_normal(s) for s in shapes]
    kw = dict(lr=0.02, beta=0.95, nesterov=True, weight_decay=0.01,
              ns_steps=5, abc=QUINTIC)
    w1, m1, o1 = muon_step(Ws, Gs, Ms, **kw)
    perm = [2, 0, 1]
    w2, m2, o2 = muon_step([Ws[i] for i in perm], [Gs[i] for i in perm],
                           [Ms[i] for i in perm], **kw)
    for j, i in enumerate(perm):
        assert np.array_equal(w1[i], w2[j]) and np.array_equal(o1[i], o2[j])
    assert muon_step([], [], [], **kw) == ([], [], [])


# --------------------------------------------------------------------------
# AdamW tail.
# --------------------------------------------------------------------------

def test_adamw_matches_torch_adamw():
    rng = np.random.default_rng(10)
    n = 257
    p0 = rng.standard_normal(n) * 0.02
    gs = [rng.standard_normal(n) * 1e-3 for _ in range(6)]
    kw = dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01)
    p = torch.nn.Parameter(torch.tensor(p0))
    opt = torch.optim.AdamW([p], lr=kw["lr"], betas=(kw["beta1"], kw["beta2"]),
                            eps=kw["eps"], weight_decay=kw["weight_decay"],
                            foreach=False)
    po, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(gs, start=1):
        p.grad = torch.tensor(g)
        opt.step()
        po, m, v = adamw_tail(po, g, m, v, step=t, **kw)
    st = opt.state[p]
    assert rel(po, p.detach().numpy()) < 1e-14
    assert rel(m, st["exp_avg"].numpy()) < 1e-14
    assert rel(v, st["exp_avg_sq"].numpy()) < 1e-14


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(13)
    p = rng.standard_normal(100)
    g = rng.standard_normal(100) * 1e-3
    lr, wd, eps = 0.02, 0.01, 1e-8
    pn, m, v = adamw_tail(p, g, np.zeros(100), np.zeros(100), lr=lr, beta1=0.9,
                          beta2=0.95, eps=eps, weight_decay=wd, step=1)
    assert np.allclose(pn, p * (1 - lr * wd) - lr * g / (np.abs(g) + eps),
                       rtol=1e-13, atol=1e-16)
    assert np.allclose(m, 0.1 * g, rtol=1e-14)
    assert np.allclose(v, 0.05 * g * g, rtol=1e-14)


def test_adamw_constant_gradient_invariant():
    # With a constant gradient from a fresh state, bias correction makes
    # m_hat = g and v_hat = g^2 exactly at every step.
    g = np.array([1e-3, -2e-3, 5e-4])
    p = np.zeros(3)
    m = np.zeros(3)
    v = np.zeros(3)
    lr, eps = 0.01, 1e-8
    for t in range(1, 30):
        p_prev = p
        p, m, v = adamw_tail(p, g, m, v, lr=lr, beta1=0.9, beta2=0.99, eps=eps,
                             weight_decay=0.0, step=t)
        assert np.allclose(p_prev - p, lr * g / (np.abs(g) + eps), rtol=1e-9)


def test_adamw_rejects_step_zero():
    with pytest.raises(ValueError):
        adamw_tail(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), lr=0.1,
                   beta1=0.9, beta2=0.9, eps=1e-8, weight_decay=0.0, step=0)


def test_oracle_exports():
    for name in oracle.__all__:
        assert hasattr(oracle, name)
