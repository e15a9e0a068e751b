"""bench.py on the host (no GPU): the refusal of more than one GPU, and the
module-level names the timed run uses."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr


def test_module_constants_and_kinds():
    import bench
    from matrix_optimizer_step_owner_amd import _lib
    assert bench.FLUSH_BYTES == 512 << 20 and bench.COLD_REPS == 20
    assert set(bench.KINDS) <= set(_lib.KERNEL_KINDS)
    # the small-matrix rule: the tiny workload's three matrices take it, a
    # 2048-wide block's do not
    assert all(bench.small_path(m, n) for m, n in ((64, 128), (64, 128), (96, 96)))
    assert not bench.small_path(2048, 2048) and not bench.small_path(130, 130)
    f = bench.ns_flops_by_kind([(2, 3)])
    assert f == {"gram": 2 * 3 * 3, "poly": 4 * 3, "update": 2 * 4 * 3}


def test_newton_schulz_bytes_and_roofline_bound():
    import bench
    # one iteration moves 3mn + 4m^2 elements (each operand read once)
    b = bench.ns_bytes_by_kind([(3, 5)], 2)
    assert b == {"gram": (15 + 9) * 2, "poly": 18 * 2, "update": (9 + 30) * 2}
    assert sum(b.values()) == (3 * 3 * 5 + 4 * 9) * 2
    # many 512 x 512 updates sit below the bf16 ridge (312.5 flop/B): HBM-bound
    f = bench.ns_flops_by_kind([(512, 512)])["update"]
    u = bench.ns_bytes_by_kind([(512, 512)], 2)["update"]
    r = bench.ns_roofline(f, u, 1e-3, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - u / 1e-3 / 1e9) < 1e-9 and abs(r["frac"] - r["hbm_frac"]) < 1e-12
    # a 5120 x 27648 update is far above it: MFMA-bound
    f = bench.ns_flops_by_kind([(5120, 27648)])["update"]
    u = bench.ns_bytes_by_kind([(5120, 27648)], 2)["update"]
    r = bench.ns_roofline(f, u, 1e-3, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "mfma" and r["flop_per_byte"] > 2000 and r["ridge_flop_per_byte"] == 312.5
