"""GPU parity of the HIP owner-local step against the float64 oracle.

Every test runs the library through its C ABI (Python ctypes binding) on
cuda:0 and compares with ``oracle`` on the same host values.  Bars: see
tests/gpu_helpers.py.
"""

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
from matrix_optimizer_step_owner_amd import workloads as wlm
import oracle

from gpu_helpers import (ADAMW_TOL, BF16_TOL, F32_TOL, GpuStep, check_matrix,
                         f64, muon_hparams, oracle_matrix, rel, run_and_check, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------------------
# AdamW tail
# ---------------------------------------------------------------------------

def adamw_check(p, g, m, v, step, lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.01,
                label=""):
    dev = torch.device("cuda:0")
    P, Gd, Md, Vd = (t.to(dev) for t in (p, g, m, v))
    mf.adamw_tail(P, Gd, Md, Vd, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                  weight_decay=wd, step=step)
    torch.cuda.synchronize()
    pr, mr, vr = oracle.adamw_tail(f64(p), f64(g), f64(m), f64(v), lr=lr, beta1=beta1,
                                   beta2=beta2, eps=eps, weight_decay=wd, step=step)
    ep, em, ev = rel(f64(P), pr), rel(f64(Md), mr), rel(f64(Vd), vr)
    edp = rel(f64(P) - f64(p), pr - f64(p))
    say(f"adamw {label} n={p.numel()} t={step}: rel p={ep:.2e} m={em:.2e} v={ev:.2e} "
        f"(dp {edp:.2e})")
    assert ep <= ADAMW_TOL and em <= ADAMW_TOL and ev <= ADAMW_TOL


@pytest.mark.parametrize("key", ["tiny_fp32", "block_d2048", "llama3_8b_4blocks",
                                 "d5120_2blocks"])
def test_adamw_workload_tails(key):
    wl = wlm.WORKLOADS[key]
    rng = np.random.default_rng(0)
    p, g, m, v = wlm.draw_tail(rng, wl)
    adamw_check(p, g, m, v, wl.adam_step, lr=wl.adam_lr, beta1=wl.adam_beta1,
                beta2=wl.adam_beta2, eps=wl.adam_eps, wd=wl.adam_weight_decay, label=key)


@pytest.mark.parametrize("n", [1, 3, 5, 255, 1023, 4097, 1 << 20, (1 << 23) - 1, (1 << 23) + 3])
def test_adamw_ragged_and_warm_state(n):
    p, g, m, v = wlm.random_tail_state(n, seed=n)
    adamw_check(p, g, m, v, step=10, label="warm")


def test_adamw_large_tail_sampled():
    # 2^28 + 3 elements (4 GiB of state, the bench's informational size, with
    # a ragged end): the unrolled, fully streamed kernel, four 16-byte groups
    # per thread, indices past 2^28; sampled elements, both ends included,
    # against the oracle, and the step is deterministic.
    n = (1 << 28) + 3
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    P, Gd, Md, Vd = (torch.randn(n, generator=gen, device=dev) * s
                     for s in (0.02, 1e-3, 1e-3, 1e-3))
    Vd.mul_(Vd)
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                    rng.integers(0, n, 200_000)]))
    it = torch.from_numpy(idx).to(dev)
    before = [f64(t[it]) for t in (P, Gd, Md, Vd)]
    hp = dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01, step=10)
    P2, M2, V2 = P.clone(), Md.clone(), Vd.clone()
    mf.adamw_tail(P, Gd, Md, Vd, **hp)
    mf.adamw_tail(P2, Gd, M2, V2, **hp)
    torch.cuda.synchronize()
    assert torch.equal(P, P2) and torch.equal(Md, M2) and torch.equal(Vd, V2)
    del P2, M2, V2
    pr, mr, vr = oracle.adamw_tail(*before, **hp)
    ep, em, ev = rel(f64(P[it]), pr), rel(f64(Md[it]), mr), rel(f64(Vd[it]), vr)
    say(f"adamw large n={n} sampled {idx.size}: rel p={ep:.2e} m={em:.2e} v={ev:.2e}")
    assert ep <= ADAMW_TOL and em <= ADAMW_TOL and ev <= ADAMW_TOL


def test_adamw_empty_tail():
    z = torch.zeros(0, device="cuda:0")
    mf.adamw_tail(z, z, z, z, lr=0.02, step=1)


# ---------------------------------------------------------------------------
# Muon: small cases against the oracle
# ---------------------------------------------------------------------------

def test_tiny_fp32_workload():
    inp = wlm.generate("tiny_fp32", seed=0)
    hp = muon_hparams(inp.workload)
    run_and_check(inp.weights, inp.grads, inp.momenta, hp, torch.float32, label="tiny")
    wl = inp.workload
    adamw_check(inp.tail_p, inp.tail_g, inp.tail_m, inp.tail_v, 1, lr=wl.adam_lr,
                beta1=wl.adam_beta1, beta2=wl.adam_beta2, eps=wl.adam_eps,
                wd=wl.adam_weight_decay, label="tiny")


RAGGED = [(1, 1), (1, 300), (300, 1), (17, 33), (33, 17), (127, 129), (129, 127),
          (300, 1000), (1000, 300), (256, 256), (257, 513)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_shapes(dtype):
    Ws, Gs, Ms = wlm.random_matrix_inputs(RAGGED, dtype, seed=1)
    run_and_check(Ws, Gs, Ms, muon_hparams(), dtype, label=f"ragged {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("variant", ["ns0", "ns1", "cubic", "no_nesterov", "custom_scale",
                                     "zero_wd"])
def test_variants(dtype, variant):
    shapes = [(64, 200), (200, 64), (130, 130)]
    Ws, Gs, Ms = wlm.random_matrix_inputs(shapes, dtype, seed=2)
    hp = muon_hparams()
    scales = None
    if variant == "ns0":
        hp["ns_steps"] = 0
    elif variant == "ns1":
        hp["ns_steps"] = 1
    elif variant == "cubic":
        hp["abc"] = (1.5, -0.5, 0.0)
        hp["ns_steps"] = 12
    elif variant == "no_nesterov":
        hp["nesterov"] = False
    elif variant == "custom_scale":
        scales = [0.7, 2.5, 1.0]
    elif variant == "zero_wd":
        hp["weight_decay"] = 0.0
    run_and_check(Ws, Gs, Ms, hp, dtype, label=variant, scales=scales)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_gradient_is_decay_only(dtype):
    shapes = [(40, 70), (70, 40)]
    Ws, _, _ = wlm.random_matrix_inputs(shapes, dtype, seed=3)
    Gs = [torch.zeros_like(w) for w in Ws]
    Ms = [torch.zeros_like(w) for w in Ws]
    st = GpuStep(Ws, Gs, Ms)
    hp = muon_hparams()
    st.run(**hp)
    # the library forms 1 - lr*wd in fp32 from fp32 arguments
    decay = np.float32(1.0) - np.float32(hp["lr"]) * np.float32(hp["weight_decay"])
    for i, w in enumerate(Ws):
        assert not st.U[i].any().item()
        assert not st.M[i].any().item()
        want = (w.to(torch.float32) * torch.tensor(decay)).to(dtype)
        assert torch.equal(st.W[i].cpu(), want)


# ---------------------------------------------------------------------------
# The d=2048 block: every matrix against the oracle
# ---------------------------------------------------------------------------

def test_block_d2048_full_workload():
    inp = wlm.generate("block_d2048", seed=0)
    wl = inp.workload
    run_and_check(inp.weights, inp.grads, inp.momenta, muon_hparams(wl), torch.bfloat16,
                  label="block_d2048")
    adamw_check(inp.tail_p, inp.tail_g, inp.tail_m, inp.tail_v, wl.adam_step,
                lr=wl.adam_lr, beta1=wl.adam_beta1, beta2=wl.adam_beta2, eps=wl.adam_eps,
                wd=wl.adam_weight_decay, label="block_d2048")


# ---------------------------------------------------------------------------
# List semantics: determinism, grouping and order independence, resume
# ---------------------------------------------------------------------------

def _subset_inputs():
    shapes = [(512, 512), (1536, 512), (512, 1536), (300, 700), (2048, 2048)]
    return wlm.random_matrix_inputs(shapes, torch.bfloat16, seed=4)


def test_bitwise_determinism_and_grouping():
    Ws, Gs, Ms = _subset_inputs()
    hp = muon_hparams()
    a = GpuStep(Ws, Gs, Ms)
    a.run(**hp)
    b = GpuStep(Ws, Gs, Ms)
    b.run(**hp)
    for i in range(len(Ws)):
        assert torch.equal(a.W[i], b.W[i]) and torch.equal(a.M[i], b.M[i])
        assert torch.equal(a.U[i], b.U[i])
    # one matrix per call
    for i in range(len(Ws)):
        s = GpuStep([Ws[i]], [Gs[i]], [Ms[i]])
        s.run(**hp)
        assert torch.equal(s.W[0], a.W[i]) and torch.equal(s.U[0], a.U[i]), i
    # reversed list
    r = GpuStep(Ws[::-1], Gs[::-1], Ms[::-1])
    r.run(**hp)
    for i in range(len(Ws)):
        j = len(Ws) - 1 - i
        assert torch.equal(r.W[j], a.W[i]) and torch.equal(r.U[j], a.U[i]), i


def test_stream_group_count_is_bitwise_invariant(monkeypatch):
    # 1 to 4 Newton-Schulz stream groups (the library picks 2 for this list)
    Ws, Gs, Ms = _subset_inputs()
    hp = muon_hparams()
    ref = None
    for groups in ("1", "2", "3", "4"):
        monkeypatch.setenv("MFSDP_NS_GROUPS", groups)
        st = GpuStep(Ws, Gs, Ms)
        st.run(**hp)
        if ref is None:
            ref = st
            continue
        for i in range(len(Ws)):
            assert torch.equal(st.W[i], ref.W[i]) and torch.equal(st.U[i], ref.U[i]), (groups, i)
            assert torch.equal(st.M[i], ref.M[i]), (groups, i)


def test_caller_stream_orders_every_group():
    # The whole d=2048 block (two stream groups) on a non-default caller
    # stream: copies of W and M made on that stream right after the call
    # see the finished step, bitwise equal to the same step on the default
    # stream, so both groups were joined back into the caller's stream.
    inp = wlm.generate("block_d2048", seed=0)
    hp = muon_hparams(inp.workload)
    dev = torch.device("cuda:0")

    def run(side):
        W = [t.to(dev) for t in inp.weights]
        G = [t.to(dev) for t in inp.grads]
        M = [t.to(dev) for t in inp.momenta]
        torch.cuda.synchronize()
        s = torch.cuda.Stream(device=dev) if side else torch.cuda.current_stream(dev)
        with torch.cuda.stream(s):
            mf.muon_step(W, G, M, **hp)
            out = [t.clone() for t in W + M]
        torch.cuda.synchronize()
        return out

    ref = run(False)
    got = run(True)
    say(f"caller stream: {len(got)} tensors compared")
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), i


def test_resume_equals_continuous():
    Ws, Gs, Ms = _subset_inputs()
    hp = muon_hparams()
    cont = GpuStep(Ws, Gs, Ms)
    cont.run(**hp)
    cont.run(**hp)
    first = GpuStep(Ws, Gs, Ms)
    first.run(**hp)
    saved_w = [w.cpu() for w in first.W]
    saved_m = [m.cpu() for m in first.M]
    del first
    torch.cuda.empty_cache()
    again = GpuStep(saved_w, Gs, saved_m)
    again.run(**hp)
    for i in range(len(Ws)):
        assert torch.equal(again.W[i], cont.W[i]) and torch.equal(again.M[i], cont.M[i])


def test_prepared_step_object_equals_function():
    # mf.MuonStep validates once and reuses its descriptors: two steps of it
    # equal two calls of mf.muon_step, bitwise
    Ws, Gs, Ms = _subset_inputs()
    hp = muon_hparams()
    a = GpuStep(Ws, Gs, Ms, update_mask=[False] * len(Ws))
    for _ in range(2):
        a.run(**hp)
    b = GpuStep(Ws, Gs, Ms, update_mask=[False] * len(Ws))
    obj = mf.MuonStep(b.W, b.G, b.M)
    kw = {k: v for k, v in hp.items()}
    for _ in range(2):
        obj.step(**kw)
    torch.cuda.synchronize()
    for i in range(len(Ws)):
        assert torch.equal(a.W[i], b.W[i]) and torch.equal(a.M[i], b.M[i]), i


@pytest.mark.parametrize("groups", ["1", "2", "small"])
def test_nan_gradient_stays_in_its_matrix(monkeypatch, groups):
    # Non-finite inputs propagate and nothing checks them, but matrices are
    # independent: a NaN in one matrix's gradient must leave every other
    # matrix of the same grouped call bitwise equal to a clean run, on one
    # stream and with two Newton-Schulz stream groups.  In the poisoned
    # matrix, M' differs from the clean M' only at the NaN element, and its
    # norm (hence every NS iterate, O and W') is NaN.
    # "small": small-matrix kernels (one workgroup each) beside a tiled one
    if groups == "small":
        Ws, Gs, Ms = wlm.random_matrix_inputs([(64, 128), (120, 96), (512, 256), (33, 17)],
                                              torch.bfloat16, seed=5)
        k, (r, c) = 1, (70, 33)
    else:
        monkeypatch.setenv("MFSDP_NS_GROUPS", groups)
        Ws, Gs, Ms = _subset_inputs()
        k, (r, c) = 1, (700, 33)
    hp = muon_hparams()
    clean = GpuStep(Ws, Gs, Ms)
    clean.run(**hp)
    Gbad = [g.clone() for g in Gs]
    Gbad[k][r, c] = float("nan")
    bad = GpuStep(Ws, Gbad, Ms)
    bad.run(**hp)
    for i in range(len(Ws)):
        if i == k:
            continue
        assert torch.equal(bad.W[i], clean.W[i]) and torch.equal(bad.M[i], clean.M[i]), i
        assert torch.equal(bad.U[i], clean.U[i]), i
    nan_m = torch.isnan(bad.M[k])
    assert nan_m.sum().item() == 1 and nan_m[r, c].item()
    keep = ~nan_m
    assert torch.equal(bad.M[k][keep], clean.M[k][keep])
    assert torch.isnan(bad.U[k]).all().item() and torch.isnan(bad.W[k]).all().item()
    say(f"NaN in matrix {k} ({tuple(Ws[k].shape)}), groups={groups}: "
        f"{len(Ws) - 1} other matrices bitwise clean")


def test_two_caller_streams_run_independently():
    # Two lists on two caller streams, enqueued alternately so that their
    # Newton-Schulz groups overlap on the GPU: each caller stream has its own
    # auxiliary streams, and each result is bitwise equal to the same list
    # stepped alone on the default stream.
    dev = torch.device("cuda:0")
    A = wlm.random_matrix_inputs([(512, 1536), (1536, 512), (1024, 1024), (300, 700)],
                                 torch.bfloat16, seed=11)
    B = wlm.random_matrix_inputs([(2048, 2048), (768, 256), (256, 2304)],
                                 torch.bfloat16, seed=12)
    hp = muon_hparams()

    def dev_copy(lists):
        return [[t.to(dev) for t in ts] for ts in lists]

    refs = []
    for lists in (A, B):
        W, G, M = dev_copy(lists)
        for _ in range(2):
            mf.muon_step(W, G, M, **hp)
        torch.cuda.synchronize()
        refs.append((W, M))
    (Wa, Ga, Ma), (Wb, Gb, Mb) = dev_copy(A), dev_copy(B)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    for _ in range(2):
        with torch.cuda.stream(s1):
            mf.muon_step(Wa, Ga, Ma, **hp)
        with torch.cuda.stream(s2):
            mf.muon_step(Wb, Gb, Mb, **hp)
    torch.cuda.synchronize()
    for (W, M), (Wr, Mr) in zip(((Wa, Ma), (Wb, Mb)), refs):
        for i in range(len(W)):
            assert torch.equal(W[i], Wr[i]) and torch.equal(M[i], Mr[i]), i
    say("two caller streams: both lists bitwise equal to their default-stream runs")


def test_graph_capture_is_refused():
    # The step uploads its launch tables from host memory that is freed when
    # the call returns, so a captured copy would replay a dangling pointer:
    # the library refuses a capturing stream before enqueueing anything, and
    # the capture around it stays valid.
    dev = torch.device("cuda:0")
    Ws, Gs, Ms = wlm.random_matrix_inputs([(256, 512)], torch.bfloat16, seed=13)
    W, G, M = (t[0].to(dev) for t in (Ws, Gs, Ms))
    ws = torch.empty(mf.muon_workspace_size([(256, 512)], torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    W0 = W.clone()
    x = torch.zeros(1024, device=dev)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.capture_begin()
        x.add_(1.0)
        with pytest.raises(mf.MfsdpError) as err:
            mf.muon_step([W], [G], [M], lr=0.02, workspace=ws)
        g.capture_end()
    assert err.value.status == 2          # MFSDP_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(W, W0)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
    assert torch.all(x == 3.0).item()
    say(f"graph capture refused: {err.value}")


def test_launch_plan_log(monkeypatch, capfd):
    monkeypatch.setenv("MFSDP_LOG", "1")
    Ws, Gs, Ms = _subset_inputs()
    GpuStep(Ws, Gs, Ms).run(**muon_hparams())
    err = capfd.readouterr().err
    assert "mfsdp_muon_step: 5 matrices, bf16, ns_steps 5" in err, err
    assert "group 0 on the caller's stream" in err and "2048x2048*1" in err, err


SMALL_MIX = [(64, 128), (128, 64), (96, 96), (1, 5), (7, 300), (100, 100), (100, 200),
             (130, 130), (512, 256)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_small_matrices_mixed_with_tiled_ones(dtype):
    # Matrices with m <= 128 whose iterate and products fit in LDS run their
    # whole Newton-Schulz chain in one workgroup; the others (100 x 200,
    # 130 x 130, 512 x 256 here) take the tiled MFMA path.  Every matrix against the
    # oracle, and the path depends on the shape alone: each matrix stepped
    # alone gives bitwise the result it gets in the mixed call.
    Ws, Gs, Ms = wlm.random_matrix_inputs(SMALL_MIX, dtype, seed=31)
    hp = muon_hparams()
    st, _ = run_and_check(Ws, Gs, Ms, hp, dtype, label=f"small mix {dtype}")
    for i in range(len(SMALL_MIX)):
        one = GpuStep([Ws[i]], [Gs[i]], [Ms[i]])
        one.run(**hp)
        assert torch.equal(one.W[0], st.W[i]) and torch.equal(one.U[0], st.U[i]), i


@pytest.mark.parametrize("variant", ["ns1", "cubic", "no_nesterov"])
def test_small_matrix_variants(variant):
    shapes = [(64, 128), (96, 96), (33, 17)]
    Ws, Gs, Ms = wlm.random_matrix_inputs(shapes, torch.float32, seed=32)
    hp = muon_hparams()
    if variant == "ns1":
        hp["ns_steps"] = 1
    elif variant == "cubic":
        hp["abc"] = (1.5, -0.5, 0.0)
        hp["ns_steps"] = 12
    else:
        hp["nesterov"] = False
    run_and_check(Ws, Gs, Ms, hp, torch.float32, label=f"small {variant}")


EXTREME = [(200, 8192), (8192, 200), (129, 2000), (700, 3000), (3000, 700), (1100, 1300)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_extreme_aspect_ratios(dtype):
    # Tiled-path matrices far from square: one 256-row panel with a K = 8192
    # Gram and 32 update tile columns (200 x 8192 and its transpose), m just
    # above the small-matrix limit (129 x 2000), and matrices with several
    # ragged row panels in both directions.  Every matrix against the oracle,
    # and each one stepped alone bitwise equal to its result in the list.
    Ws, Gs, Ms = wlm.random_matrix_inputs(EXTREME, dtype, seed=51)
    hp = muon_hparams()
    st, _ = run_and_check(Ws, Gs, Ms, hp, dtype, label=f"extreme {dtype}")
    for i in range(len(EXTREME)):
        one = GpuStep([Ws[i]], [Gs[i]], [Ms[i]])
        one.run(**hp)
        assert torch.equal(one.W[0], st.W[i]) and torch.equal(one.U[0], st.U[i]), i


def _random_shapes(n, seed, lo=1, hi=1500):
    rng = np.random.default_rng(seed)
    dims = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(n, 2))).astype(int)
    return [(int(r), int(c)) for r, c in np.clip(dims, lo, hi)]


def test_random_shapes_fp32():
    # Sixteen seeded shapes, log-uniform in 1..1500 on each side: small-path
    # and tiled matrices, wide, tall and ragged in both directions, in one
    # grouped call, every matrix against the oracle at the fp32 bar.  (In
    # bf16 the rounding of the iterates alone can approach the 2e-2 bar for
    # matrices whose singular values share a narrow band, so the random
    # sweep uses the dtype whose bar every shape meets.)
    shapes = _random_shapes(16, seed=61)
    Ws, Gs, Ms = wlm.random_matrix_inputs(shapes, torch.float32, seed=62)
    run_and_check(Ws, Gs, Ms, muon_hparams(), torch.float32, label="random fp32")


def test_mfma_probe_runs_and_sums_are_finite():
    # the measurement kernel that bench.py times as the sustained MFMA ceiling
    dev = torch.device("cuda:0")
    out = torch.full((16 * 8,), float("nan"), dtype=torch.float32, device=dev)
    mf.mfma_probe(out, iters=50)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool((out > 0).all())


def _random_shapes_bf16(n, seed, lo=129, hi=1500, max_aspect=4.0):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        r, c = np.exp(rng.uniform(np.log(lo), np.log(hi), size=2)).astype(int)
        if max(r, c) / min(r, c) <= max_aspect:
            out.append((int(r), int(c)))
    return out


def test_random_shapes_bf16():
    # Twelve seeded tiled-path shapes (129..1500 per side, aspect ratio at
    # most 4, ragged in both directions) in one grouped bf16 call, each against
    # the oracle at the bf16 bars.  The range keeps the rounding of the bf16
    # iterates itself, as a CPU emulation of the defined iteration gives it
    # for these very inputs (0.88-1.05e-2), well inside the 2e-2 bar.
    shapes = _random_shapes_bf16(12, seed=63)
    Ws, Gs, Ms = wlm.random_matrix_inputs(shapes, torch.bfloat16, seed=64)
    run_and_check(Ws, Gs, Ms, muon_hparams(), torch.bfloat16, label="random bf16")
