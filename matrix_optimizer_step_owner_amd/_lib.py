"""ctypes view of the C ABI in include/mfsdp.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
import threading

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmfsdp.so")

MFSDP_OK = 0
STATUS_NAMES = {0: "MFSDP_OK", 1: "MFSDP_ERR_INVALID_ARGUMENT",
                2: "MFSDP_ERR_UNSUPPORTED", 3: "MFSDP_ERR_WORKSPACE",
                4: "MFSDP_ERR_ALIAS", 5: "MFSDP_ERR_HIP"}
DTYPE_F32 = 0
DTYPE_BF16 = 1
NS_EPS = 1e-7
#: size of the static device scratch of mfsdp_muon_step_noalloc (bytes)
NOALLOC_SCRATCH_BYTES = 256 << 20
KERNEL_KINDS = {"momentum": 0, "norm": 1, "gram": 2, "poly": 3, "update": 4,
                "apply": 5, "adamw": 6, "final": 7, "stats_prep": 8, "syrk": 9,
                "small": 10}

#: Every symbol include/mfsdp.h declares.
EXPORTED = ("mfsdp_muon_workspace_size", "mfsdp_muon_step", "mfsdp_muon_step_noalloc",
            "mfsdp_adamw_tail",
            "mfsdp_plan_owners", "mfsdp_tail_layout", "mfsdp_tail_pack",
            "mfsdp_tail_unpack", "mfsdp_stats_workspace_size", "mfsdp_shampoo_stats",
            "mfsdp_status_string", "mfsdp_last_error",
            "mfsdp_timing_enable", "mfsdp_timing_reset", "mfsdp_timing_read",
            "mfsdp_mfma_probe")


class MfsdpMatrix(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p),
                ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p),
                ("update_out", ctypes.c_void_p),
                ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64),
                ("scale", ctypes.c_float)]


class MfsdpStatsMatrix(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p),
                ("left", ctypes.c_void_p),
                ("right", ctypes.c_void_p),
                ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class MfsdpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {detail}")


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load libmfsdp.so; raise if it has not been built (no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m matrix_optimizer_step_owner_amd.build` "
                "(the optimizer step has no non-HIP implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        c = ctypes
        lib.mfsdp_muon_workspace_size.argtypes = [
            c.POINTER(MfsdpMatrix), c.c_int64, c.c_int, c.POINTER(c.c_size_t)]
        lib.mfsdp_muon_workspace_size.restype = c.c_int
        lib.mfsdp_muon_step.argtypes = [
            c.POINTER(MfsdpMatrix), c.c_int64, c.c_int, c.c_float, c.c_float,
            c.c_int, c.c_float, c.c_int, c.c_float, c.c_float, c.c_float,
            c.c_void_p, c.c_size_t, c.c_void_p]
        lib.mfsdp_muon_step.restype = c.c_int
        lib.mfsdp_muon_step_noalloc.argtypes = [
            c.POINTER(MfsdpMatrix), c.c_int64, c.c_int, c.c_float, c.c_float,
            c.c_int, c.c_float, c.c_int, c.c_float, c.c_float, c.c_float, c.c_void_p]
        lib.mfsdp_muon_step_noalloc.restype = c.c_int
        lib.mfsdp_adamw_tail.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64,
            c.c_float, c.c_float, c.c_float, c.c_float, c.c_float, c.c_int64,
            c.c_void_p]
        lib.mfsdp_adamw_tail.restype = c.c_int
        lib.mfsdp_plan_owners.argtypes = [
            c.POINTER(c.c_double), c.POINTER(c.c_int64), c.c_int64, c.c_int32, c.c_double,
            c.POINTER(c.c_int32), c.POINTER(c.c_double), c.POINTER(c.c_int64)]
        lib.mfsdp_plan_owners.restype = c.c_int
        lib.mfsdp_tail_layout.argtypes = [c.POINTER(c.c_int64), c.c_int64,
                                          c.POINTER(c.c_int64), c.POINTER(c.c_int64)]
        lib.mfsdp_tail_layout.restype = c.c_int
        lib.mfsdp_tail_pack.argtypes = [
            c.POINTER(c.c_void_p), c.POINTER(c.c_int64), c.POINTER(c.c_int64), c.c_int64,
            c.c_void_p, c.c_int64, c.c_void_p]
        lib.mfsdp_tail_pack.restype = c.c_int
        lib.mfsdp_tail_unpack.argtypes = [
            c.c_void_p, c.c_int64, c.POINTER(c.c_void_p), c.POINTER(c.c_int64),
            c.POINTER(c.c_int64), c.c_int64, c.c_void_p]
        lib.mfsdp_tail_unpack.restype = c.c_int
        lib.mfsdp_stats_workspace_size.argtypes = [
            c.POINTER(MfsdpStatsMatrix), c.c_int64, c.c_int, c.POINTER(c.c_size_t)]
        lib.mfsdp_stats_workspace_size.restype = c.c_int
        lib.mfsdp_shampoo_stats.argtypes = [
            c.POINTER(MfsdpStatsMatrix), c.c_int64, c.c_int, c.c_float, c.c_float,
            c.c_void_p, c.c_size_t, c.c_void_p]
        lib.mfsdp_shampoo_stats.restype = c.c_int
        lib.mfsdp_status_string.argtypes = [c.c_int]
        lib.mfsdp_status_string.restype = c.c_char_p
        lib.mfsdp_last_error.argtypes = []
        lib.mfsdp_last_error.restype = c.c_char_p
        lib.mfsdp_timing_enable.argtypes = [c.c_int]
        lib.mfsdp_timing_enable.restype = c.c_int
        lib.mfsdp_timing_reset.argtypes = []
        lib.mfsdp_timing_reset.restype = c.c_int
        lib.mfsdp_timing_read.argtypes = [c.c_int, c.POINTER(c.c_double),
                                          c.POINTER(c.c_int64)]
        lib.mfsdp_timing_read.restype = c.c_int
        lib.mfsdp_mfma_probe.argtypes = [c.c_void_p, c.c_int64, c.c_int, c.c_void_p]
        lib.mfsdp_mfma_probe.restype = c.c_int
        _lib = lib
        return lib


def check(status: int) -> None:
    if status != MFSDP_OK:
        detail = load().mfsdp_last_error().decode(errors="replace")
        raise MfsdpError(status, detail)
