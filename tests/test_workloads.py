"""Host-side checks of the seeded workload generator (no GPU)."""

import numpy as np
import torch

from matrix_optimizer_step_owner_amd import workloads as wlmod


def test_shapes_and_counts():
    W = wlmod.WORKLOADS
    assert [(s.rows, s.cols) for s in W["tiny_fp32"].matrices] == [(64, 128), (128, 64), (96, 96)]
    assert len(W["block_d2048"].matrices) == 7
    assert W["block_d2048"].n_elements == 4 * 2048 * 2048 + 3 * 5632 * 2048
    assert len(W["llama3_8b_4blocks"].matrices) == 28
    assert W["llama3_8b_4blocks"].n_elements == 4 * (2 * 4096 ** 2 + 2 * 1024 * 4096 + 3 * 14336 * 4096)
    assert len(W["many_small"].matrices) == 512 and W["many_small"].tail_n == 0
    assert len(W["d5120_2blocks"].matrices) == 14 and W["d5120_2blocks"].tail_n == 1 << 20
    assert set(wlmod.WORKLOAD_ORDER) == set(W)


def test_tiny_is_deterministic_and_typed():
    a = wlmod.generate("tiny_fp32", seed=0)
    b = wlmod.generate("tiny_fp32", seed=0)
    for x, y in zip(a.weights + a.grads, b.weights + b.grads):
        assert x.dtype == torch.float32 and torch.equal(x, y)
    assert not any(m.any() for m in a.momenta)
    assert a.tail_p.shape == (512,) and not a.tail_m.any() and not a.tail_v.any()
    # standard deviations are as stated
    g = torch.cat([x.flatten() for x in a.grads]).double()
    assert 0.9e-3 < g.std().item() < 1.1e-3
    c = wlmod.generate("tiny_fp32", seed=1)
    assert not torch.equal(a.grads[0], c.grads[0])


def test_subset_matches_full_stream():
    full = wlmod.generate("tiny_fp32", seed=0)
    sub = wlmod.generate("tiny_fp32", seed=0, matrix_indices=[2])
    assert torch.equal(sub.weights[0], full.weights[2])
    assert torch.equal(sub.grads[0], full.grads[2])
    assert torch.equal(sub.tail_g, full.tail_g)


def test_bf16_inputs_are_rounded_storage():
    Ws, Gs, Ms = wlmod.random_matrix_inputs([(5, 7)], torch.bfloat16, seed=3)
    assert Ws[0].dtype == torch.bfloat16
    # upcasting and re-rounding is the identity (values are representable)
    assert torch.equal(Gs[0].double().to(torch.bfloat16), Gs[0])
    p, g, m, v = wlmod.random_tail_state(64, seed=1)
    assert (v.numpy() >= 0).all() and np.isfinite(v.numpy()).all()
