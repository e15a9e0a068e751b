"""C-ABI checks that run without a GPU.

The library validates every argument before it makes any HIP call, so invalid
arguments and empty lists can be exercised on the host: the pointers below are
never dereferenced (each call returns before anything is enqueued).  No test
here launches a kernel.
"""

import ctypes
import os
import re

import pytest

from matrix_optimizer_step_owner_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfsdp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmfsdp.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mfsdp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = header_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTED) == names


def test_status_strings():
    lib = _lib.load()
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.mfsdp_status_string(code).decode() == name
    assert lib.mfsdp_status_string(99).decode() == "MFSDP_UNKNOWN_STATUS"


FAKE = 1 << 40   # a 16-byte aligned address that is never dereferenced


def mats(shapes, base=FAKE, es=2, upd=False, stride=None):
    arr = (_lib.MfsdpMatrix * max(len(shapes), 1))()
    off = base
    for i, (r, c) in enumerate(shapes):
        nb = r * c * es
        step = stride if stride is not None else ((nb + 4095) // 4096) * 4096
        arr[i].weight = off
        arr[i].grad = off + step
        arr[i].momentum = off + 2 * step
        arr[i].update_out = (off + 3 * step) if upd else None
        arr[i].rows, arr[i].cols, arr[i].scale = r, c, 1.0
        off += 4 * step + (((r * c * 4 + 4095) // 4096) * 4096 if upd else 0)
    return arr, off


def ws_size(arr, n, dtype=_lib.DTYPE_BF16):
    out = ctypes.c_size_t(0)
    st = _lib.load().mfsdp_muon_workspace_size(arr, n, dtype, ctypes.byref(out))
    return st, out.value


def step(arr, n, ws, wsb, dtype=_lib.DTYPE_BF16, lr=0.02, beta=0.95, ns=5,
         abc=(3.4445, -4.775, 2.0315), wd=0.01):
    return _lib.load().mfsdp_muon_step(arr, n, dtype, lr, beta, 1, wd, ns, *abc,
                                       ws, wsb, None)


def test_workspace_size_values():
    arr, _ = mats([(2048, 2048), (5632, 2048)])
    st, nb = ws_size(arr, 2)
    assert st == 0
    # two iterate buffers m_pad*n_pad and two m_pad^2 buffers per matrix, bf16
    want = 2 * 2 * (2048 * 2048 + 2048 * 2048) + 2 * 2 * (2048 * 5632 + 2048 * 2048)
    assert want <= nb <= want + (1 << 20)
    st32, nb32 = ws_size(arr, 2, _lib.DTYPE_F32)
    assert st32 == 0 and nb32 > nb
    # padding to the 256 tile: a 17 x 33 matrix uses 256 x 256 buffers
    arr1, _ = mats([(17, 33)])
    st, nb = ws_size(arr1, 1)
    assert st == 0 and nb >= 4 * 256 * 256 * 2
    assert ws_size(arr, 0) == (0, 0)


def test_workspace_size_errors():
    lib = _lib.load()
    arr, _ = mats([(0, 5)])
    assert ws_size(arr, 1)[0] == 1
    arr, _ = mats([(4, 4)])
    assert ws_size(arr, 1, dtype=7)[0] == 2
    assert lib.mfsdp_muon_workspace_size(arr, 1, 1, None) == 1
    assert ws_size(arr, -1)[0] == 1
    arr, _ = mats([(1 << 20, 1 << 20)])
    assert ws_size(arr, 1)[0] == 2


def test_empty_list_is_noop():
    assert step(None, 0, None, 0) == 0
    assert step(None, -1, None, 0) == 1


def test_step_validation_errors():
    lib = _lib.load()
    arr, end = mats([(64, 128), (128, 64)])
    st, need = ws_size(arr, 2)
    assert st == 0
    ws = (end + 4095) // 4096 * 4096 + (1 << 20)
    ws = (ws + 255) // 256 * 256
    # workspace too small / misaligned / null
    assert step(arr, 2, ws, need - 1) == 3
    assert step(arr, 2, ws + 16, need) == 3
    assert step(arr, 2, None, need) == 3
    # bad hyperparameters
    assert step(arr, 2, ws, need, ns=-1) == 1
    assert step(arr, 2, ws, need, ns=101) == 1
    assert step(arr, 2, ws, need, lr=float("nan")) == 1
    assert step(arr, 2, ws, need, abc=(float("inf"), 0.0, 0.0)) == 1
    assert step(arr, 2, ws, need, dtype=9) == 2
    # null pointer
    arr[1].grad = None
    assert step(arr, 2, ws, need) == 1
    assert b"null" in lib.mfsdp_last_error()
    # misaligned pointer
    arr, end = mats([(64, 128), (128, 64)])
    arr[0].momentum += 2
    assert step(arr, 2, ws, need) == 1
    # bad scale
    arr, end = mats([(64, 128), (128, 64)])
    arr[1].scale = 0.0
    assert step(arr, 2, ws, need) == 1
    arr[1].scale = float("nan")
    assert step(arr, 2, ws, need) == 1


def test_step_alias_errors():
    arr, end = mats([(64, 128), (128, 64)])
    st, need = ws_size(arr, 2)
    ws = (end + (1 << 20)) // 256 * 256
    # grad of matrix 1 inside weight of matrix 0
    arr[1].grad = arr[0].weight + 64
    assert step(arr, 2, ws, need) == 4
    # workspace overlapping a momentum buffer
    arr, end = mats([(64, 128), (128, 64)])
    ws = (arr[1].momentum // 256) * 256
    assert step(arr, 2, ws, need) == 4
    # a big range that swallows a later small one (non-adjacent overlap)
    arr, end = mats([(512, 512), (4, 4)], stride=1 << 20)
    arr[1].weight = arr[0].weight + 4096
    arr[1].grad = end + (1 << 22)
    arr[1].momentum = end + (1 << 23)
    st, need = ws_size(arr, 2)
    assert step(arr, 2, end + (1 << 24), need) == 4


def test_adamw_validation():
    lib = _lib.load()
    f = lib.mfsdp_adamw_tail
    P = FAKE
    n = 1024
    args = lambda **kw: dict(dict(p=P, g=P + 8192, m=P + 16384, v=P + 24576, n=n,
                                  lr=0.02, b1=0.9, b2=0.95, eps=1e-8, wd=0.01,
                                  step=1), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["p"], a["g"], a["m"], a["v"], a["n"], a["lr"], a["b1"], a["b2"],
                 a["eps"], a["wd"], a["step"], None)

    assert call(n=0) == 0
    assert call(n=0, p=None, g=None, m=None, v=None) == 0
    assert call(n=-1) == 1
    assert call(step=0) == 1
    assert call(b1=1.0) == 1
    assert call(b2=-0.1) == 1
    assert call(eps=-1.0) == 1
    assert call(lr=float("inf")) == 1
    assert call(g=None) == 1
    assert call(m=P + 8192 + 4) == 1            # misaligned
    assert call(n=(1 << 40) + 4) == 2           # MFSDP_ERR_UNSUPPORTED, before any launch
    assert call(m=P + 8192) == 4                # overlaps g
    assert call(v=P + 100 * 16) == 4            # overlaps p


def test_timing_api_without_launches():
    lib = _lib.load()
    assert lib.mfsdp_timing_enable(0) == 0
    ms = ctypes.c_double(-1)
    cnt = ctypes.c_int64(-1)
    assert lib.mfsdp_timing_read(2, ctypes.byref(ms), ctypes.byref(cnt)) == 0
    assert cnt.value == 0
    assert lib.mfsdp_timing_read(99, ctypes.byref(ms), ctypes.byref(cnt)) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    import matrix_optimizer_step_owner_amd as mf
    W = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mf.muon_step([W], [W.clone()], [W.clone()], lr=0.1)
    p = torch.zeros(8)
    with pytest.raises(ValueError):
        mf.adamw_tail(p, p.clone(), p.clone(), p.clone(), lr=0.1)
    mf.muon_step([], [], [], lr=0.1)   # non-owner: no-op


def test_stats_workspace_and_validation():
    lib = _lib.load()
    M = _lib.MfsdpStatsMatrix
    arr = (M * 2)()
    arr[0].grad, arr[0].left, arr[0].right, arr[0].rows, arr[0].cols = 0x100000, 0x200000, 0x300000, 300, 1000
    arr[1].grad, arr[1].left, arr[1].right, arr[1].rows, arr[1].cols = 0x400000, 0x500000, None, 17, 33
    out = ctypes.c_size_t(0)
    assert lib.mfsdp_stats_workspace_size(arr, 2, _lib.DTYPE_BF16, ctypes.byref(out)) == 0
    # two padded copies per gradient: 512 x 1024 and 256 x 256, bf16
    want = 2 * 2 * (512 * 1024 + 256 * 256)
    assert want <= out.value <= want + (1 << 20)
    assert lib.mfsdp_stats_workspace_size(arr, 0, _lib.DTYPE_BF16, ctypes.byref(out)) == 0
    assert out.value == 0
    # invalid calls return before any device work (fake addresses never used)
    ws = 0x10000000
    assert lib.mfsdp_shampoo_stats(arr, 2, _lib.DTYPE_BF16, 1.0, 1.0, ws, 16, None) == 3  # small ws
    arr[1].left = None
    assert lib.mfsdp_shampoo_stats(arr, 2, _lib.DTYPE_BF16, 1.0, 1.0, ws, 1 << 30, None) == 1
    arr[1].left = 0x100000 + 8   # inside matrix 0's gradient
    assert lib.mfsdp_shampoo_stats(arr, 2, _lib.DTYPE_BF16, 1.0, 1.0, ws, 1 << 30, None) == 4
    arr[1].left = 0x500000
    assert lib.mfsdp_shampoo_stats(arr, 2, _lib.DTYPE_BF16, float("nan"), 1.0, ws, 1 << 30,
                                   None) == 1
    arr[1].rows = 0
    assert lib.mfsdp_stats_workspace_size(arr, 2, _lib.DTYPE_BF16, ctypes.byref(out)) == 1


def test_fp32_iterate_byte_limit():
    # 32768 x 32768 fp32 iterates would need 2^32-byte offsets: refused; bf16 fits
    arr, _ = mats([(32768, 32768)])
    st, _ = ws_size(arr, 1, _lib.DTYPE_F32)
    assert st == 2
    st, nb = ws_size(arr, 1, _lib.DTYPE_BF16)
    assert st == 0 and nb > 0


def test_noalloc_step_refuses_a_list_beyond_its_scratch():
    # refused before the device is touched: the size check comes first
    lib = _lib.load()
    arr, _ = mats([(8192, 8192)])
    assert ws_size(arr, 1)[1] > _lib.NOALLOC_SCRATCH_BYTES
    abc = (3.4445, -4.775, 2.0315)
    st = lib.mfsdp_muon_step_noalloc(arr, 1, _lib.DTYPE_BF16, 0.02, 0.95, 1, 0.01, 5, *abc,
                                     None)
    assert st == 3 and b"static scratch" in lib.mfsdp_last_error()
    # an empty list is a no-op; its hyperparameters are still validated
    assert lib.mfsdp_muon_step_noalloc(None, 0, _lib.DTYPE_BF16, 0.02, 0.95, 1, 0.01, 5,
                                       *abc, None) == 0
    assert lib.mfsdp_muon_step_noalloc(None, 0, _lib.DTYPE_BF16, float("nan"), 0.95, 1,
                                       0.01, 5, *abc, None) == 1
    assert lib.mfsdp_muon_step_noalloc(None, 0, 9, 0.02, 0.95, 1, 0.01, 5, *abc, None) == 2


def test_mfma_probe_validation():
    # refused before any launch (no device needed)
    lib = _lib.load()
    assert lib.mfsdp_mfma_probe(None, 8, 10, None) == 1
    assert lib.mfsdp_mfma_probe(FAKE, 0, 10, None) == 1
    assert lib.mfsdp_mfma_probe(FAKE, (1 << 16) + 1, 10, None) == 1
    assert lib.mfsdp_mfma_probe(FAKE, 8, 0, None) == 1
    assert lib.mfsdp_mfma_probe(FAKE, 65536, 1 << 20, None) == 1
    assert b"2^28" in lib.mfsdp_last_error()
    assert lib.mfsdp_mfma_probe(FAKE + 2, 8, 10, None) == 1
    assert b"aligned" in lib.mfsdp_last_error()
