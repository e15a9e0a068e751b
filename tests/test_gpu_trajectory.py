"""Multi-step trajectory parity: consecutive owner-local steps carrying the
optimizer state (Muon momentum; AdamW m, v and the step count) against the
float64 trajectory oracle run of the same steps from the same inputs.

The oracle keeps its own state (it is never reset to the GPU's values), so
any error the HIP path makes is carried forward and the per-step numbers show
how it grows.  Both sides store the state in the storage dtype between steps
(oracle reading R19).

Bars, at every step t = 1..T:
  * fp32 (50 steps): rel(W_t - W_0), rel(M_t) within 1e-4;
  * bf16 (10 steps): rel(M_t) within 2e-2, and
        ||W_t,gpu - W_t,ref||_F <= 2e-2 ||W_t,ref - W_0||_F
                                   + 0.5 sqrt(t) ||ulp_bf16(W_t,ref)||_F
    -- the single-step W' bar with one half-ulp allowance per step for the
    stored rounding, the t disagreements being independent (added in
    quadrature);
  * AdamW tail (fp32, 20 steps from t = 1): rel(p), rel(m), rel(v) within 1e-6.
"""

import math

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
from matrix_optimizer_step_owner_amd import workloads as wlm
import oracle

from gpu_helpers import ADAMW_TOL, BF16_TOL, F32_TOL, f64, rel, say, ulp_bf16

pytestmark = pytest.mark.gpu

HP = dict(lr=0.02, beta=0.95, nesterov=True, weight_decay=0.01, ns_steps=5,
          abc=wlm.NS_ABC)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_trajectory(shapes, dtype, steps, seed):
    dev = torch.device("cuda:0")
    W0, _, M0 = wlm.random_matrix_inputs(shapes, dtype, seed=seed, m_std=1e-3)
    grads = wlm.trajectory_gradients(shapes, dtype, steps, seed=seed + 1)
    W = [w.to(dev) for w in W0]
    M = [m.to(dev) for m in M0]
    gpu_states = []
    for Gs, _ in grads:
        G = [g.to(dev) for g in Gs]
        mf.muon_step(W, G, M, **HP)
        torch.cuda.synchronize()
        gpu_states.append(([f64(w) for w in W], [f64(m) for m in M]))
    storage = "bf16" if dtype == torch.bfloat16 else "f32"
    ref_states = oracle.muon_trajectory([f64(w) for w in W0], [f64(m) for m in M0],
                                        [[f64(g) for g in Gs] for Gs, _ in grads],
                                        storage=storage, **HP)
    return [f64(w) for w in W0], gpu_states, ref_states


def test_fp32_trajectory_50_steps():
    # the tiny workload's shapes (the small-matrix kernel) and two that take
    # the tiled MFMA path (m = 200 and 130 exceed the small kernel's bound)
    shapes = [(64, 128), (128, 64), (96, 96), (300, 200), (130, 130)]
    T = 50
    W0, gpu, ref = run_trajectory(shapes, torch.float32, T, seed=100)
    worst = 0.0
    for t in range(T):
        for k in range(len(shapes)):
            ew = rel(gpu[t][0][k] - W0[k], ref[t][0][k] - W0[k])
            em = rel(gpu[t][1][k], ref[t][1][k])
            worst = max(worst, ew, em)
            assert ew <= F32_TOL and em <= F32_TOL, (t + 1, k, ew, em)
        if (t + 1) % 10 == 0:
            say(f"fp32 step {t + 1}: worst rel so far {worst:.2e}")


def test_bf16_trajectory_10_steps():
    # a tall, a wide and a square matrix; 384 is a tile and a half (ragged);
    # 120 x 96 takes the small-matrix kernel
    shapes = [(512, 256), (256, 768), (384, 384), (120, 96)]
    T = 10
    W0, gpu, ref = run_trajectory(shapes, torch.bfloat16, T, seed=200)
    for t in range(T):
        ratios, ems = [], []
        for k in range(len(shapes)):
            Wr, Wg = ref[t][0][k], gpu[t][0][k]
            err = np.linalg.norm(Wg - Wr)
            allow = (BF16_TOL * np.linalg.norm(Wr - W0[k])
                     + 0.5 * math.sqrt(t + 1) * np.linalg.norm(ulp_bf16(Wr)))
            ratios.append(err / allow)
            ems.append(rel(gpu[t][1][k], ref[t][1][k]))
        say(f"bf16 step {t + 1}: W error / allowance {max(ratios):.3f}, "
            f"rel(W_t - W_0) {max(rel(gpu[t][0][k] - W0[k], ref[t][0][k] - W0[k]) for k in range(len(shapes))):.2e}, "
            f"rel(M_t) {max(ems):.2e}")
        assert max(ratios) <= 1.0, (t + 1, ratios)
        assert max(ems) <= BF16_TOL, (t + 1, ems)


def test_bf16_trajectory_block_d2048_3_steps():
    # The d=2048 block at its real shapes and launch configuration (two
    # Newton-Schulz stream groups), three consecutive steps, same bars.
    shapes = [(s.rows, s.cols) for s in wlm.WORKLOADS["block_d2048"].matrices]
    T = 3
    W0, gpu, ref = run_trajectory(shapes, torch.bfloat16, T, seed=400)
    for t in range(T):
        ratios, ems = [], []
        for k in range(len(shapes)):
            Wr, Wg = ref[t][0][k], gpu[t][0][k]
            err = np.linalg.norm(Wg - Wr)
            allow = (BF16_TOL * np.linalg.norm(Wr - W0[k])
                     + 0.5 * math.sqrt(t + 1) * np.linalg.norm(ulp_bf16(Wr)))
            ratios.append(err / allow)
            ems.append(rel(gpu[t][1][k], ref[t][1][k]))
        say(f"d=2048 block bf16 step {t + 1}: W error / allowance {max(ratios):.3f}, "
            f"rel(M_t) {max(ems):.2e}")
        assert max(ratios) <= 1.0, (t + 1, ratios)
        assert max(ems) <= BF16_TOL, (t + 1, ems)


def test_adamw_trajectory_20_steps():
    n, T = 4099, 20
    p0, _, m0, v0 = wlm.random_tail_state(n, seed=300)
    m0.zero_()
    v0.zero_()
    grads = wlm.trajectory_gradients([], torch.float32, T, seed=301, tail_n=n)
    dev = torch.device("cuda:0")
    P, Mt, Vt = p0.to(dev), m0.to(dev), v0.to(dev)
    hp = dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01)
    gpu = []
    for t, (_, g) in enumerate(grads):
        mf.adamw_tail(P, g.to(dev), Mt, Vt, step=t + 1, **hp)
        torch.cuda.synchronize()
        gpu.append((f64(P), f64(Mt), f64(Vt)))
    ref = oracle.adamw_trajectory(f64(p0), f64(m0), f64(v0), [f64(g) for _, g in grads],
                                  first_step=1, storage="f32", **hp)
    for t in range(T):
        ep, em, ev = (rel(gpu[t][i], ref[t][i]) for i in range(3))
        assert max(ep, em, ev) <= ADAMW_TOL, (t + 1, ep, em, ev)
    say(f"adamw {T} steps: rel p {ep:.2e} m {em:.2e} v {ev:.2e}")
