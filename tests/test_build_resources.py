"""Resource guards of the gfx950 kernels (host-side compile, no GPU).

The Newton-Schulz kernels must keep their 128 fp32 accumulators per wave and
their epilogue inputs in registers (no scratch: a dynamically indexed accumulator
array, a spill, or an array passed by reference to an outlined helper moves
to scratch memory and costs several times in speed) and stay well inside the
64 KB instruction cache that two CUs share (the once-per-tile epilogue is
fetched cold for every tile otherwise).
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "matrix_optimizer_step_owner_amd", "csrc", "mfsdp.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
LLVM = "/opt/rocm/llvm/bin"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

CODE_LIMIT = 48 * 1024   # bytes of code per steady-state NS kernel


@pytest.fixture(scope="module")
def device_build():
    tmp = tempfile.mkdtemp()
    obj = os.path.join(tmp, "dev.o")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-o", obj, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    yield obj, res.stderr
    shutil.rmtree(tmp, ignore_errors=True)


def kernel_usage(remarks):
    usage, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1).strip()] = int(m.group(2))
    return usage


def test_ns_kernels_use_no_scratch(device_build):
    # every mode (gram, poly, update, wide and tall apply, statistics) in both dtypes
    _, remarks = device_build
    usage = kernel_usage(remarks)
    ns = {k: v for k, v in usage.items() if "ns_gemm_kernel" in k}
    assert len(ns) == 12, list(usage)
    for k, v in ns.items():
        assert v.get("ScratchSize", 0) == 0, (k, v)
        assert v.get("VGPRs Spill", 0) == 0, (k, v)


def test_small_matrix_kernel_uses_no_scratch(device_build):
    # the whole-chain kernel of small matrices keeps its output blocks in
    # registers (both dtypes) and its LDS within the 160 KB of a CU
    _, remarks = device_build
    usage = kernel_usage(remarks)
    small = {k: v for k, v in usage.items() if "small_ns_kernel" in k}
    assert len(small) == 2, list(usage)
    for k, v in small.items():
        assert v.get("ScratchSize", 0) == 0, (k, v)
        assert v.get("LDS Size", 0) <= 160 * 1024, (k, v)


def test_steady_state_ns_kernels_fit_the_instruction_cache(device_build):
    obj, _ = device_build
    bundler = os.path.join(LLVM, "clang-offload-bundler")
    readelf = os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(bundler) and os.path.exists(readelf)):
        pytest.skip("llvm tools not available")
    gfx = obj + ".gfx950"
    subprocess.run([bundler, "--unbundle", "--type=o", f"--input={obj}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={gfx}"],
                   check=True)
    out = subprocess.run([readelf, "-s", gfx], capture_output=True, text=True,
                         check=True).stdout
    sizes = {}
    for line in out.splitlines():
        parts = line.split()
        if len(parts) >= 8 and parts[3] == "FUNC":
            sizes[parts[7]] = int(parts[2])
    ns = {k: v for k, v in sizes.items() if re.search(r"ns_gemm_kernelINS_8ElemBF16ELi[012]E", k)}
    assert len(ns) == 3, sorted(sizes)
    for k, v in ns.items():
        assert v < CODE_LIMIT, (k, v)
