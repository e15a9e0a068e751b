"""Benchmark of the owner-local Muon + AdamW-tail step on one MI355X.

One step = mfsdp_muon_step over every owned matrix of the workload (momentum,
Nesterov, Frobenius normalization, 5 quintic Newton-Schulz iterations, apply)
followed by mfsdp_adamw_tail over the packed tail, on one HIP stream, with all
inputs resident in HBM.  W warm-up steps, then exactly K timed steps between
two device synchronizations.

Prints one JSON line.  ``value`` is the Newton-Schulz algorithmic TFLOP/s of
the whole step (NS flops per step / wall time per step); ``ms_per_step`` is
the step time.  The timed region runs the library exactly as a caller would
(its Newton-Schulz stream groups included) with no per-kernel instrumentation.

``cold_cache`` times single steps (hipEvents on the current stream) after
overwriting 512 MiB, twice the MALL, so that no operand survives in cache from
the step before; it gives the median and the minimum over up to 20 steps.

``roofline`` describes the dominant kernel (most GPU time per step).  It comes
from a second pass of the same K steps right after the timed region, with the
Newton-Schulz work on ONE stream (MFSDP_NS_GROUPS=1) so that no two kernels of
the library overlap; the library records hipEvents around each of its launches
on the launch stream, and ``achieved`` is the kernel's algorithmic flops (or
bytes) per launch over its average launch duration.  A Newton-Schulz kernel is
priced against the MFMA peak when its flops per algorithmic byte (operands read
once, results written once) reach the ridge of the chip (peak flops over 8 TB/s),
else against HBM; ``mfma_frac`` and ``hbm_frac`` give both.  ``kernels`` holds the
same per-kind figures.  ``traffic`` is the kernel's measured HBM bytes per
launch (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy) read from
profiles/, or null when the kernel sources changed since it was measured.
``mfma_loop`` is the sustained bf16 MFMA rate of the same GPU with no memory
traffic (mfsdp_mfma_probe, timed in the same run): under sustained MFMA load
the clock settles well below the one at which the dense peak is quoted, so
``roofline.frac_of_mfma_loop`` gives the dominant kernel against what the chip
sustains, beside ``frac`` against the published peak.
``cpu_baseline`` is the float64 oracle on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "owner-local Muon step ms and Newton-Schulz TFLOP/s (% bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs x 128 FMA lanes x 2.4 GHz)
KINDS = ("momentum", "norm", "gram", "poly", "update", "final", "apply", "adamw", "small")
#: cold-cache pass: bytes overwritten before each timed step (2x the 256 MB
#: MALL) and the most steps it times
FLUSH_BYTES = 512 << 20
COLD_REPS = 20


def small_path(m, n):
    """Whether the library runs a matrix's Newton-Schulz chain whole in one
    workgroup (the rule of ns_small.hpp: m <= 128, the iterate and both m x m
    products, rows padded to an odd number of 16-byte chunks, within 38400
    LDS floats, at most 1024 four-by-four output blocks: two per thread)."""
    def pitch(c):
        return 4 * (((c + 3) // 4) | 1)
    m4 = (m + 3) // 4 * 4
    return (m <= 128 and m4 * (pitch(n) + 2 * pitch(m)) <= 38400
            and ((m + 3) // 4) * ((n + 3) // 4) <= 1024)


def ns_flops_by_kind(shapes):
    """Algorithmic flops of ONE launch of each Newton-Schulz kernel kind.

    With m = min(r, c), n = max(r, c): gram A = X X^T counts its upper triangle
    m(m+1)n; poly A A the same way m^2(m+1); update B X 2 m^2 n.
    """
    g = p = u = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        g += m * (m + 1) * n
        p += m * m * (m + 1)
        u += 2 * m * m * n
    return {"gram": g, "poly": p, "update": u}


def ns_bytes_by_kind(shapes, es):
    """Algorithmic HBM bytes of ONE launch of each Newton-Schulz kernel kind,
    every operand read once and every result written once (storage dtype of
    es bytes): gram reads X (m x n) and writes A (m x m); poly reads A and
    writes B'; update reads B' and X and writes X'.  One iteration moves
    3mn + 4m^2 elements.
    """
    g = p = u = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        g += (m * n + m * m) * es
        p += 2 * m * m * es
        u += (m * m + 2 * m * n) * es
    return {"gram": g, "poly": p, "update": u}


def ns_roofline(flops, nbytes, sec, peak_tflops):
    """Roofline of one Newton-Schulz launch: algorithmic flops and bytes per
    launch over its duration.  Its bound is the MFMA peak when the launch's
    intensity (flops per algorithmic byte) is at or above the chip's ridge,
    else HBM; both fractions are given either way."""
    ai = flops / nbytes
    ridge = peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)
    tflops = flops / sec / 1e12
    gbs = nbytes / sec / 1e9
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak_tflops, "unit": "TFLOP/s",
                "frac": tflops / peak_tflops}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
    roof.update({"flop_per_byte": round(ai, 1), "ridge_flop_per_byte": round(ridge, 1),
                 "mfma_frac": tflops / peak_tflops, "hbm_frac": gbs / PEAK_HBM_GBS})
    return roof


def mfma_ceiling(dev, reps=5, iters=20000, blocks=1024):
    """Sustained bf16 MFMA rate of this GPU with no memory traffic
    (mfsdp_mfma_probe, each launch timed alone with hipEvents on the current
    stream): the practical ceiling under the power cap, reported beside the
    published peak.  Median and maximum TFLOP/s over `reps` launches."""
    import matrix_optimizer_step_owner_amd as mf
    out = torch.empty(blocks * 8, dtype=torch.float32, device=dev)
    flops = blocks * 8 * 8 * iters * 2.0 * 32 * 32 * 16
    mf.mfma_probe(out, iters)
    torch.cuda.synchronize()
    tf = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        mf.mfma_probe(out, iters)
        e1.record()
        torch.cuda.synchronize()
        tf.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("MFMA probe produced non-finite sums")
    tf.sort()
    return {"tflops_median": round(tf[len(tf) // 2], 1), "tflops_max": round(tf[-1], 1),
            "reps": reps, "blocks": blocks, "iters": iters,
            "flops_per_launch": flops}


def elementwise_bytes(shapes, es, tail_n):
    """Algorithmic HBM bytes of one launch of the elementwise kernels."""
    elems = sum(r * c for r, c in shapes)
    return {"momentum": elems * 4 * es,      # read G, M; write M', U
            "adamw": tail_n * 7 * 4}         # read p, g, m, v; write p, m, v


def cpu_sample_order(wl):
    """Matrix indices in order of increasing Newton-Schulz work (the oracle's
    bounded sample takes them smallest first)."""
    return sorted(range(len(wl.matrices)),
                  key=lambda i: ns_flops_by_kind([(wl.matrices[i].rows,
                                                   wl.matrices[i].cols)])["update"])


def cpu_baseline(key, sample, budget_s=20.0):
    """Time the float64 oracle on a bounded sample of the workload.

    ``sample`` is a list of (index, W, G, M) host tensors, smallest first, taken
    from the bench's own inputs; matrices are stepped until ``budget_s`` of
    oracle time is spent."""
    import oracle
    from matrix_optimizer_step_owner_amd import workloads as wlm
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    wl = wlm.WORKLOADS[key]
    done_flops = 0
    done = []
    t_total = 0.0
    for i, Wt, Gt, Mt in sample:
        W, G, M = (t.double().numpy() for t in (Wt, Gt, Mt))
        t0 = time.perf_counter()
        oracle.muon_matrix_step(W, G, M, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov,
                                weight_decay=wl.weight_decay, ns_steps=wl.ns_steps,
                                abc=wl.abc)
        t_total += time.perf_counter() - t0
        f = ns_flops_by_kind([(wl.matrices[i].rows, wl.matrices[i].cols)])
        done_flops += wl.ns_steps * sum(f.values())
        done.append(f"{wl.matrices[i].name} {wl.matrices[i].rows}x{wl.matrices[i].cols}")
        if t_total > budget_s:
            break
    return {"value": done_flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 numpy oracle Muon step on {len(done)} matrices of "
                      f"{key} ({', '.join(done)}), {t_total:.1f} s, NS algorithmic flops "
                      f"{done_flops:.3e}",
            "host": host_description()}


def host_description():
    """CPU model and the BLAS numpy uses (the oracle's matrix products)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # older numpy: no dict form
        pass
    return {"cpu": model, "blas": blas}


def stats_bench(args, wl, dev):
    """Time mfsdp_shampoo_stats over the workload's gradients (one line of JSON).

    Algorithmic work: the symmetric products counted once, r(r+1)c flops for L
    and c(c+1)r for R per r x c gradient.  The dominant kernel is the
    statistics product (kind "syrk"); its roofline is the dtype's MFMA peak.
    """
    import matrix_optimizer_step_owner_amd as mf
    from matrix_optimizer_step_owner_amd import workloads as wlm
    inp = wlm.generate(args.workload, seed=0)
    G = [t.to(dev) for t in inp.grads]
    del inp
    L = [torch.zeros(g.shape[0], g.shape[0], device=dev) for g in G]
    R = [torch.zeros(g.shape[1], g.shape[1], device=dev) for g in G]
    flops = sum(r * (r + 1) * c + c * (c + 1) * r for r, c in (g.shape for g in G))
    hp = dict(beta=0.95, alpha=0.05)
    for _ in range(args.warmup):
        mf.shampoo_stats(G, L, R, **hp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mf.shampoo_stats(G, L, R, **hp)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    mf.timing.reset()
    mf.timing.enable(True)
    for _ in range(args.steps):
        mf.shampoo_stats(G, L, R, **hp)
    torch.cuda.synchronize()
    mf.timing.enable(False)
    kern = {}
    for k in ("stats_prep", "syrk"):
        tot, cnt = mf.timing.read(k)
        if cnt:
            kern[k] = {"avg_ms": round(tot / cnt, 5)}
    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    ach = flops / (kern["syrk"]["avg_ms"] * 1e-3) / 1e12
    print(json.dumps({
        "metric": "Shampoo-type statistics update L,R (TFLOP/s, symmetric products once)",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": args.workload, "matrices": len(G), "flops_per_step": flops},
        "kernels": kern,
        "roofline": {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                     "frac": ach / peak, "kernel": "syrk", "traffic": None},
    }), flush=True)


def adamw_cpu_baseline(n_sample, hp):
    """The float64 AdamW oracle on an n_sample-element tail on the host cores."""
    import oracle
    rng = np.random.default_rng(1)
    p, g, m = (rng.standard_normal(n_sample) * s for s in (0.02, 1e-3, 1e-3))
    v = (rng.standard_normal(n_sample) * 1e-3) ** 2
    reps, t_total = 0, 0.0
    while t_total < 5.0 and reps < 50:
        t0 = time.perf_counter()
        oracle.adamw_tail(p, g, m, v, **hp)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * n_sample * 28 / t_total / 1e9, 2), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"float64 numpy AdamW oracle on a {n_sample}-element tail, {reps} reps, "
                      f"{t_total:.1f} s, 28 algorithmic bytes per element"}


def adamw_bench(args, dev):
    """Time mfsdp_adamw_tail alone on an n-element packed fp32 tail (one JSON line).

    Algorithmic bytes: 28 per element (read p, g, m, v; write p, m, v).  The
    tail state is a warm one: p ~ N(0, 0.02), g, m ~ N(0, 1e-3), v = N(0, 1e-3)^2,
    drawn on the device from a seeded generator, step 10.
    """
    import matrix_optimizer_step_owner_amd as mf
    n = args.adamw_elements
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    P, Gt, Mt, Vt = (torch.randn(n, generator=gen, device=dev) * s
                     for s in (0.02, 1e-3, 1e-3, 1e-3))
    Vt.mul_(Vt)
    hp = dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01, step=10)

    def step():
        mf.adamw_tail(P, Gt, Mt, Vt, **hp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    mf.timing.reset()
    mf.timing.enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    mf.timing.enable(False)
    tot, cnt = mf.timing.read("adamw")
    avg_ms = tot / cnt
    nbytes = 28 * n
    ach = nbytes / (avg_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "AdamW tail GB/s (28 algorithmic bytes per element)",
        "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"adamw_tail_{n}", "elements": n, "step": hp["step"]},
        "kernels": {"adamw": {"avg_ms": round(avg_ms, 5), "gbs": round(ach, 1)}},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "kernel": "adamw", "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else adamw_cpu_baseline(
            min(n, 1 << 24), hp),
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d5120_2blocks",
                    help="workload key (default: the 32B-class d=5120 two-block share, "
                         "the largest owner share that fits one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the run, copy this many MiB device-to-device with a plain "
                         "copy kernel (reference point for HBM byte counters)")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with measured HBM bytes per launch of the dominant kernel "
                         "(default: profiles/<kernel>_<workload>_traffic.json)")
    ap.add_argument("--shampoo-stats", action="store_true",
                    help="measure the Shampoo-type statistics update (L += G G^T, "
                         "R += G^T G) on the workload's gradients instead of the Muon step")
    ap.add_argument("--adamw-elements", type=int, default=0,
                    help="measure mfsdp_adamw_tail alone on a packed fp32 tail of this many "
                         "elements instead of the Muon step")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="measure only the sustained bf16 MFMA rate with no memory traffic "
                         "(mfsdp_mfma_probe) and print it")
    ap.add_argument("--mfma-iters", type=int, default=20000,
                    help="iterations per wave of each MFMA-ceiling launch (20000: ~30 ms, "
                         "long enough for the clock to settle)")
    ap.add_argument("--ns-groups", type=int, default=0,
                    help="Newton-Schulz stream groups in the timed region (0: the library's "
                         "own choice)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the owner-local step on one GPU only; "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import matrix_optimizer_step_owner_amd as mf
    from matrix_optimizer_step_owner_amd import profiling
    from matrix_optimizer_step_owner_amd import workloads as wlm

    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.mfma_ceiling:
        print(json.dumps({"mfma_loop": mfma_ceiling(dev, reps=max(args.steps, 1),
                                                     iters=args.mfma_iters)}), flush=True)
        return
    if args.adamw_elements > 0:
        adamw_bench(args, dev)
        return
    wl = wlm.WORKLOADS[args.workload]
    if args.shampoo_stats:
        stats_bench(args, wl, dev)
        return
    t_setup = time.perf_counter()
    inp = wlm.generate(args.workload, seed=0)
    setup_gen_s = time.perf_counter() - t_setup
    shapes = [(s.rows, s.cols) for s in wl.matrices]
    # host copies of the oracle's sample (smallest matrices first)
    sample = [] if args.no_cpu_baseline else [
        (i, inp.weights[i], inp.grads[i], inp.momenta[i]) for i in cpu_sample_order(wl)[:8]]
    W = [t.to(dev) for t in inp.weights]
    G = [t.to(dev) for t in inp.grads]
    M = [t.to(dev) for t in inp.momenta]
    P, Gt, Mt, Vt = (t.to(dev) for t in (inp.tail_p, inp.tail_g, inp.tail_m, inp.tail_v))
    del inp
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    es = 2 if wl.dtype == torch.bfloat16 else 4
    ws = torch.empty(mf.muon_workspace_size(shapes, wl.dtype), dtype=torch.uint8, device=dev)
    hp = dict(lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, weight_decay=wl.weight_decay,
              ns_steps=wl.ns_steps, abc=wl.abc)

    muon = mf.MuonStep(W, G, M)

    def step():
        muon.step(workspace=ws, **hp)
        mf.adamw_tail(P, Gt, Mt, Vt, lr=wl.adam_lr, beta1=wl.adam_beta1,
                      beta2=wl.adam_beta2, eps=wl.adam_eps,
                      weight_decay=wl.adam_weight_decay, step=wl.adam_step)

    if args.ns_groups > 0:
        os.environ["MFSDP_NS_GROUPS"] = str(args.ns_groups)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # cold-cache pass: each step timed alone with hipEvents on the current
    # stream after overwriting a 512 MiB buffer (twice the 256 MB MALL), so
    # no operand is cache-resident from the step before; median and minimum
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(min(args.steps, COLD_REPS)):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold.sort()

    # roofline pass: the same steps with the Newton-Schulz work on one stream
    saved = os.environ.get("MFSDP_NS_GROUPS")
    os.environ["MFSDP_NS_GROUPS"] = "1"
    mf.timing.reset()
    mf.timing.enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    mf.timing.enable(False)
    if saved is None:
        del os.environ["MFSDP_NS_GROUPS"]
    else:
        os.environ["MFSDP_NS_GROUPS"] = saved
    per_kind = {}
    for k in KINDS:
        tot, cnt = mf.timing.read(k)
        if cnt:
            per_kind[k] = {"avg_ms": tot / cnt, "launches": cnt,
                           "ms_per_step": tot / args.steps}

    small = [(r, c) for r, c in shapes if small_path(min(r, c), max(r, c))]
    flops = ns_flops_by_kind([s for s in shapes if s not in small])
    # one launch of the small-matrix kernel runs every iteration
    flops["small"] = wl.ns_steps * sum(ns_flops_by_kind(small).values())
    ns_flops_step = wl.ns_steps * sum(ns_flops_by_kind(shapes).values())
    ns_kernel_ms = sum(per_kind[k]["ms_per_step"]
                       for k in ("gram", "poly", "update", "final", "small") if k in per_kind)
    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    dominant = max(per_kind, key=lambda k: per_kind[k]["ms_per_step"])
    ew = elementwise_bytes(shapes, es, wl.tail_n)
    if dominant == "small":   # fp32 dot products on the vector ALUs, either dtype
        achieved = flops["small"] / (per_kind["small"]["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS}
    elif dominant in flops:
        nsb = ns_bytes_by_kind([s for s in shapes if s not in small], es)
        roof = ns_roofline(flops[dominant], nsb[dominant], per_kind[dominant]["avg_ms"] * 1e-3,
                           peak)
    else:
        achieved = ew[dominant] / (per_kind[dominant]["avg_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof["kernel"] = dominant
    roof["launches_per_step"] = per_kind[dominant]["launches"] // args.steps
    roof["avg_launch_ms"] = round(per_kind[dominant]["avg_ms"], 5)
    roof["pass"] = "one stream, the K steps after the timed region"
    roof["traffic"] = None
    tpath = args.traffic or os.path.join(ROOT, "profiles",
                                         f"{dominant}_kernel_{args.workload}_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if (tr.get("kernel") == dominant and tr.get("workload") == args.workload
                and tr.get("source_sha256") == profiling.kernel_source_hash(dominant)):
            roof["traffic"] = tr.get("bytes_per_launch")

    # the practical MFMA ceiling of this GPU, measured in the same run
    mfma_loop = None
    if roof["bound"] == "mfma" and wl.dtype == torch.bfloat16:
        mfma_loop = mfma_ceiling(dev, iters=args.mfma_iters)
        roof["mfma_loop_tflops"] = mfma_loop["tflops_median"]
        roof["frac_of_mfma_loop"] = roof["achieved"] / mfma_loop["tflops_median"]

    kernels = {}
    for k, v in per_kind.items():
        e = {"avg_ms": round(v["avg_ms"], 5), "ms_per_step": round(v["ms_per_step"], 5)}
        if k in flops:
            e["tflops"] = round(flops[k] / (v["avg_ms"] * 1e-3) / 1e12, 2)
        if k in ew:
            e["gbs"] = round(ew[k] / (v["avg_ms"] * 1e-3) / 1e9, 1)
        if k == "final":
            # the last update (2 m^2 n per matrix) split over the wide-matrix and
            # tall-matrix launches: per step, not per launch
            e["tflops_per_step"] = round(flops["update"] / (v["ms_per_step"] * 1e-3) / 1e12, 2)
        kernels[k] = e

    out = {
        "metric": METRIC,
        "value": round(ns_flops_step / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "ns_groups": int(os.environ.get("MFSDP_NS_GROUPS", "0")) or "library",
        "config": {"workload": args.workload, "matrices": len(shapes),
                   "elements": wl.n_elements, "tail": wl.tail_n, "ns_steps": wl.ns_steps,
                   "ns_flops_per_step": ns_flops_step},
        "ns_tflops_kernels": round(ns_flops_step / (ns_kernel_ms * 1e-3) / 1e12, 2)
        if ns_kernel_ms else None,
        "pct_bf16_peak_step": round(100 * ns_flops_step / (ms_per_step * 1e-3) / 1e12 / peak, 2),
        "kernels": kernels,
        "cold_cache": {"reps": len(cold), "flush_bytes": FLUSH_BYTES,
                       "ms_median": round(cold[len(cold) // 2], 4), "ms_min": round(cold[0], 4)},
        "roofline": roof,
        "mfma_loop": mfma_loop,
        "setup_s": {"generate": round(setup_gen_s, 1), "generate_and_upload": round(setup_s, 1)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(args.workload, sample,
                                                                      args.cpu_budget),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
