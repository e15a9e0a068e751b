"""Pins of the trajectory oracle (CPU only).

* round_to_bf16: torch's float32 -> bfloat16 conversion (round to nearest,
  ties to even) on many float32 values, and hand-worked ties;
* round_to_f32: torch's float64 -> float32 conversion on many float64 values,
  exact float32 midpoints and their neighbours, and hand-worked ties;
* muon_trajectory: one step equals the single-step oracle; with float64
  state the carried momentum has the closed form
  M_T = beta^T M_0 + sum_k beta^(T-1-k) G_k;
* adamw_trajectory: with a constant gradient g and fresh moments, the bias
  corrections make m_hat = g and v_hat = g^2 at every step, so
  p_T = d^T p_0 - lr * g/(|g|+eps) * (1 + d + ... + d^(T-1)), d = 1 - lr*wd.
"""

import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=0.02, beta=0.95, nesterov=True, weight_decay=0.01, ns_steps=5,
          abc=(3.4445, -4.7750, 2.0315))


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    # plus exact midpoints between neighbouring bf16 values (ties)
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    mids = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, mids])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("x,want", [
    (1.0 + 2.0 ** -8, 1.0),                       # tie, rounds to even (down)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),       # tie, rounds to even (up)
    (-(1.0 + 2.0 ** -8), -1.0),
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above the tie
    (3.0, 3.0),
    (0.0, 0.0),
])
def test_round_to_bf16_hand_cases(x, want):
    assert oracle.round_to_bf16(np.array([x]))[0] == want


def test_round_to_f32_matches_torch_on_float64_values():
    # float64 values over a wide exponent range, plus the exact midpoints
    # between neighbouring float32 values (ties: to even) and points one
    # float64 ulp either side of them
    rng = np.random.default_rng(2)
    x = rng.standard_normal(200_000) * np.exp(rng.uniform(-60, 60, 200_000))
    f = x[:2000].astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf), dtype=np.float32)
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2.0
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    want = torch.from_numpy(x).to(torch.float32).double().numpy()
    got = oracle.round_to_f32(x)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("x,want", [
    (1.0 + 2.0 ** -24, 1.0),                          # tie, rounds to even (down)
    (1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -22),         # tie, rounds to even (up)
    (-(1.0 + 2.0 ** -24), -1.0),
    (1.0 + 2.0 ** -24 + 2.0 ** -50, 1.0 + 2.0 ** -23),  # just above the tie
    (0.1, 0.100000001490116119384765625),             # nearest float32 to 0.1
    (0.0, 0.0),
])
def test_round_to_f32_hand_cases(x, want):
    assert oracle.round_to_f32(np.array([x]))[0] == want


def _mats(seed, shapes):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) * 0.02 for s in shapes]


def test_one_step_trajectory_is_the_single_step_oracle():
    shapes = [(12, 20), (20, 12), (9, 9)]
    W, M, G = _mats(0, shapes), _mats(1, shapes), _mats(2, shapes)
    st = oracle.muon_trajectory(W, M, [G], storage=None, **HP)
    w1, m1, _ = oracle.muon_step(W, G, M, **HP)
    for a, b in zip(st[0][0], w1):
        assert np.array_equal(a, b)
    for a, b in zip(st[0][1], m1):
        assert np.array_equal(a, b)
    # with bf16 storage the result is the rounded single step
    st = oracle.muon_trajectory(W, M, [G], storage="bf16", **HP)
    w1, m1, _ = oracle.muon_step([oracle.round_to_bf16(w) for w in W], G,
                                 [oracle.round_to_bf16(m) for m in M], **HP)
    for a, b in zip(st[0][0], w1):
        assert np.array_equal(a, oracle.round_to_bf16(b))


def test_momentum_closed_form_over_steps():
    shapes = [(8, 16), (16, 8)]
    T, beta = 6, HP["beta"]
    W, M0 = _mats(3, shapes), _mats(4, shapes)
    Gs = [_mats(10 + t, shapes) for t in range(T)]
    st = oracle.muon_trajectory(W, M0, Gs, storage=None, **HP)
    for k in range(len(shapes)):
        want = beta ** T * M0[k] + sum(beta ** (T - 1 - t) * Gs[t][k] for t in range(T))
        np.testing.assert_allclose(st[-1][1][k], want, rtol=1e-13, atol=1e-18)


def test_adamw_constant_gradient_closed_form():
    lr, wd, eps, T = 0.02, 0.01, 1e-8, 25
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal(64) * 0.02
    g = rng.standard_normal(64) * 1e-3
    z = np.zeros(64)
    st = oracle.adamw_trajectory(p0, z, z, [g] * T, lr=lr, beta1=0.9, beta2=0.95, eps=eps,
                                 weight_decay=wd, storage=None)
    d = 1.0 - lr * wd
    want = d ** T * p0 - lr * g / (np.abs(g) + eps) * sum(d ** k for k in range(T))
    np.testing.assert_allclose(st[-1][0], want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(st[-1][1], (1 - 0.9 ** T) * g, rtol=1e-12)
    np.testing.assert_allclose(st[-1][2], (1 - 0.95 ** T) * g * g, rtol=1e-12)
