"""Owner-local optimizer step of MatrixFSDP on MI355X (gfx950).

Python binding of ``libmfsdp.so`` (C ABI in ``include/mfsdp.h``).  The
functions here only marshal torch tensors into the C structures and pass
torch's current HIP stream; every step of the computation runs in the HIP
kernels of the library, and a missing library is an error (there is no
fallback).

Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
parameter sharding" (arxivlens page, Abstract): the owner of whole 2D weights
runs Muon -- momentum, Newton-Schulz orthogonalization, update -- locally, and
packed non-matrix tail tensors take AdamW.
"""

from __future__ import annotations

import ctypes
import math
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import MfsdpError, NOALLOC_SCRATCH_BYTES, NS_EPS

__all__ = ["muon_step", "muon_step_noalloc", "MuonStep", "adamw_tail", "muon_workspace_size",
           "default_scale", "plan_owners", "tail_layout", "tail_pack", "tail_unpack",
           "shampoo_stats", "mfma_probe", "timing", "MfsdpError", "NS_EPS", "NOALLOC_SCRATCH_BYTES",
           "library_path"]

library_path = _lib.LIB_PATH

_DTYPES = {torch.float32: _lib.DTYPE_F32, torch.bfloat16: _lib.DTYPE_BF16}


def default_scale(rows: int, cols: int) -> float:
    """Update scale sqrt(max(1, rows/cols)), the original-Muon convention."""
    return math.sqrt(max(1.0, rows / cols))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_matrix(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _build_descs(weights, grads, momenta, scales, update_out):
    n = len(weights)
    arr = (_lib.MfsdpMatrix * max(n, 1))()
    for i in range(n):
        W = weights[i]
        r, c = W.shape
        arr[i].weight = W.data_ptr()
        arr[i].grad = grads[i].data_ptr()
        arr[i].momentum = momenta[i].data_ptr()
        arr[i].update_out = _ptr(None if update_out is None else update_out[i])
        arr[i].rows = r
        arr[i].cols = c
        arr[i].scale = default_scale(r, c) if scales is None else float(scales[i])
    return arr


def muon_workspace_size(shapes: Sequence[Tuple[int, int]], dtype: torch.dtype) -> int:
    """Workspace bytes of a muon_step over matrices of these shapes."""
    lib = _lib.load()
    n = len(shapes)
    arr = (_lib.MfsdpMatrix * max(n, 1))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows = r
        arr[i].cols = c
        arr[i].scale = 1.0
    out = ctypes.c_size_t(0)
    _lib.check(lib.mfsdp_muon_workspace_size(arr, n, _DTYPES[dtype], ctypes.byref(out)))
    return int(out.value)


# One cached workspace per (device, stream): calls on one stream are ordered,
# so they can share it.
_WS_CACHE: Dict[Tuple[int, int], torch.Tensor] = {}


def _workspace(device: torch.device, stream_ptr: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream_ptr)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        _WS_CACHE.pop(key, None)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS_CACHE[key] = ws
    return ws


def muon_step(weights: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
              momenta: Sequence[torch.Tensor], *, lr: float, beta: float = 0.95,
              nesterov: bool = True, weight_decay: float = 0.0,
              ns_steps: int = 5, abc=(3.4445, -4.7750, 2.0315),
              scales: Optional[Sequence[float]] = None,
              update_out: Optional[Sequence[torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None) -> None:
    """Owner-local Muon step on whole matrices, in place (mfsdp_muon_step).

    weights / grads / momenta: 2D contiguous tensors on one GPU, all bf16 or
    all fp32.  ``update_out``: optional list (entries may be None) of fp32
    tensors that receive the orthogonalized update O.  ``scales``: per-matrix update scale, default
    sqrt(max(1, rows/cols)).  Runs on torch's current stream.
    """
    lib = _lib.load()
    n = len(weights)
    if not (len(grads) == n and len(momenta) == n):
        raise ValueError("weights, grads and momenta must have the same length")
    if scales is not None and len(scales) != n:
        raise ValueError("scales must have one entry per matrix")
    if update_out is not None and len(update_out) != n:
        raise ValueError("update_out must have one entry per matrix")
    if n == 0:
        return
    dtype = weights[0].dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    device = weights[0].device
    if device.type != "cuda":
        raise ValueError("muon_step needs GPU tensors")
    for i in range(n):
        if weights[i].dim() != 2:
            raise ValueError(f"weights[{i}] must be 2D")
        _check_matrix(weights[i], f"weights[{i}]", dtype, device)
        _check_matrix(grads[i], f"grads[{i}]", dtype, device, weights[i].shape)
        _check_matrix(momenta[i], f"momenta[{i}]", dtype, device, weights[i].shape)
        if update_out is not None and update_out[i] is not None:
            _check_matrix(update_out[i], f"update_out[{i}]", torch.float32, device,
                          weights[i].shape)
    arr = _build_descs(weights, grads, momenta, scales, update_out)
    code = _DTYPES[dtype]
    need = ctypes.c_size_t(0)
    _lib.check(lib.mfsdp_muon_workspace_size(arr, n, code, ctypes.byref(need)))
    stream = torch.cuda.current_stream(device).cuda_stream
    if workspace is None:
        workspace = _workspace(device, stream, need.value)
    a, b, c = abc
    _lib.check(lib.mfsdp_muon_step(arr, n, code, lr, beta, 1 if nesterov else 0,
                                   weight_decay, ns_steps, a, b, c,
                                   workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   stream))


def muon_step_noalloc(weights: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                      momenta: Sequence[torch.Tensor], *, lr: float, beta: float = 0.95,
                      nesterov: bool = True, weight_decay: float = 0.0,
                      ns_steps: int = 5, abc=(3.4445, -4.7750, 2.0315),
                      scales: Optional[Sequence[float]] = None,
                      update_out: Optional[Sequence[torch.Tensor]] = None) -> None:
    """Owner-local Muon step with the library's static device scratch as its
    workspace (mfsdp_muon_step_noalloc): no device memory is allocated, by the
    library or here.  Lists needing more than NOALLOC_SCRATCH_BYTES of
    workspace are refused; calls that overlap on one GPU race on the shared
    scratch.  Same arguments and results as ``muon_step``."""
    lib = _lib.load()
    n = len(weights)
    if not (len(grads) == n and len(momenta) == n):
        raise ValueError("weights, grads and momenta must have the same length")
    if scales is not None and len(scales) != n:
        raise ValueError("scales must have one entry per matrix")
    if update_out is not None and len(update_out) != n:
        raise ValueError("update_out must have one entry per matrix")
    if n == 0:
        return
    dtype = weights[0].dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    device = weights[0].device
    if device.type != "cuda":
        raise ValueError("muon_step_noalloc needs GPU tensors")
    for i in range(n):
        if weights[i].dim() != 2:
            raise ValueError(f"weights[{i}] must be 2D")
        _check_matrix(weights[i], f"weights[{i}]", dtype, device)
        _check_matrix(grads[i], f"grads[{i}]", dtype, device, weights[i].shape)
        _check_matrix(momenta[i], f"momenta[{i}]", dtype, device, weights[i].shape)
        if update_out is not None and update_out[i] is not None:
            _check_matrix(update_out[i], f"update_out[{i}]", torch.float32, device,
                          weights[i].shape)
    arr = _build_descs(weights, grads, momenta, scales, update_out)
    stream = torch.cuda.current_stream(device).cuda_stream
    a, b, c = abc
    _lib.check(lib.mfsdp_muon_step_noalloc(arr, n, _DTYPES[dtype], lr, beta,
                                           1 if nesterov else 0, weight_decay, ns_steps,
                                           a, b, c, stream))


class MuonStep:
    """A validated, reusable owner-local Muon step over a fixed list of
    matrices (mfsdp_muon_step without per-call marshalling).

    The tensors are checked and their descriptors built once; each ``step``
    call only passes the hyperparameters, torch's current stream and the
    workspace to the C ABI.  The tensors must stay alive and in place (the same
    storage) for the object's lifetime; their contents change freely.
    """

    def __init__(self, weights: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                 momenta: Sequence[torch.Tensor],
                 scales: Optional[Sequence[float]] = None,
                 update_out: Optional[Sequence[torch.Tensor]] = None):
        n = len(weights)
        if not (len(grads) == n and len(momenta) == n):
            raise ValueError("weights, grads and momenta must have the same length")
        if scales is not None and len(scales) != n:
            raise ValueError("scales must have one entry per matrix")
        if update_out is not None and len(update_out) != n:
            raise ValueError("update_out must have one entry per matrix")
        self._n = n
        self._keep = (list(weights), list(grads), list(momenta),
                      None if update_out is None else list(update_out))
        if n == 0:
            return
        dtype = weights[0].dtype
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}")
        device = weights[0].device
        if device.type != "cuda":
            raise ValueError("MuonStep needs GPU tensors")
        for i in range(n):
            if weights[i].dim() != 2:
                raise ValueError(f"weights[{i}] must be 2D")
            _check_matrix(weights[i], f"weights[{i}]", dtype, device)
            _check_matrix(grads[i], f"grads[{i}]", dtype, device, weights[i].shape)
            _check_matrix(momenta[i], f"momenta[{i}]", dtype, device, weights[i].shape)
            if update_out is not None and update_out[i] is not None:
                _check_matrix(update_out[i], f"update_out[{i}]", torch.float32, device,
                              weights[i].shape)
        self._device = device
        self._code = _DTYPES[dtype]
        self._arr = _build_descs(weights, grads, momenta, scales, update_out)
        need = ctypes.c_size_t(0)
        _lib.check(_lib.load().mfsdp_muon_workspace_size(self._arr, n, self._code,
                                                         ctypes.byref(need)))
        self._need = need.value

    def step(self, *, lr: float, beta: float = 0.95, nesterov: bool = True,
             weight_decay: float = 0.0, ns_steps: int = 5, abc=(3.4445, -4.7750, 2.0315),
             workspace: Optional[torch.Tensor] = None) -> None:
        if self._n == 0:
            return
        stream = torch.cuda.current_stream(self._device).cuda_stream
        if workspace is None:
            workspace = _workspace(self._device, stream, self._need)
        a, b, c = abc
        _lib.check(_lib.load().mfsdp_muon_step(
            self._arr, self._n, self._code, lr, beta, 1 if nesterov else 0, weight_decay,
            ns_steps, a, b, c, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), stream))


def adamw_tail(p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
               *, lr: float, beta1: float = 0.9, beta2: float = 0.95,
               eps: float = 1e-8, weight_decay: float = 0.0, step: int = 1) -> None:
    """Decoupled AdamW on a packed fp32 tail, in place (mfsdp_adamw_tail)."""
    lib = _lib.load()
    n = p.numel()
    if n == 0:
        _lib.check(lib.mfsdp_adamw_tail(None, None, None, None, 0, lr, beta1, beta2,
                                        eps, weight_decay, step, None))
        return
    device = p.device
    if device.type != "cuda":
        raise ValueError("adamw_tail needs GPU tensors")
    for name, t in (("p", p), ("g", g), ("m", m), ("v", v)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != device \
                or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} "
                             f"elements on {device}")
    stream = torch.cuda.current_stream(device).cuda_stream
    _lib.check(lib.mfsdp_adamw_tail(p.data_ptr(), g.data_ptr(), m.data_ptr(),
                                    v.data_ptr(), n, lr, beta1, beta2, eps,
                                    weight_decay, step, stream))


def shampoo_stats(grads: Sequence[torch.Tensor], lefts: Sequence[torch.Tensor],
                  rights: Optional[Sequence[Optional[torch.Tensor]]] = None, *,
                  beta: float = 1.0, alpha: float = 1.0,
                  workspace: Optional[torch.Tensor] = None) -> None:
    """Preconditioner statistics in place (mfsdp_shampoo_stats):
    L <- beta*L + alpha*G G^T and, where given, R <- beta*R + alpha*G^T G.

    grads: 2D contiguous bf16 or fp32 tensors on one GPU; lefts / rights:
    contiguous fp32 (rows x rows) / (cols x cols).  Runs on torch's current
    stream."""
    lib = _lib.load()
    n = len(grads)
    if len(lefts) != n or (rights is not None and len(rights) != n):
        raise ValueError("one left (and right) statistic per gradient")
    if n == 0:
        return
    dtype = grads[0].dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    device = grads[0].device
    if device.type != "cuda":
        raise ValueError("shampoo_stats needs GPU tensors")
    arr = (_lib.MfsdpStatsMatrix * n)()
    for i, G in enumerate(grads):
        if G.dim() != 2:
            raise ValueError(f"grads[{i}] must be 2D")
        r, c = G.shape
        _check_matrix(G, f"grads[{i}]", dtype, device)
        _check_matrix(lefts[i], f"lefts[{i}]", torch.float32, device, (r, r))
        R = None if rights is None else rights[i]
        if R is not None:
            _check_matrix(R, f"rights[{i}]", torch.float32, device, (c, c))
        arr[i].grad = G.data_ptr()
        arr[i].left = lefts[i].data_ptr()
        arr[i].right = None if R is None else R.data_ptr()
        arr[i].rows = r
        arr[i].cols = c
    code = _DTYPES[dtype]
    need = ctypes.c_size_t(0)
    _lib.check(lib.mfsdp_stats_workspace_size(arr, n, code, ctypes.byref(need)))
    stream = torch.cuda.current_stream(device).cuda_stream
    if workspace is None:
        workspace = _workspace(device, stream, need.value)
    _lib.check(lib.mfsdp_shampoo_stats(arr, n, code, beta, alpha, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), stream))


def plan_owners(cost_ms: Sequence[float], nbytes: Sequence[int], n_ranks: int,
                byte_slack: float = 0.1):
    """Balance-aware owner assignment of whole items (mfsdp_plan_owners).

    Returns (owner per item, predicted ms per rank, resident bytes per rank).
    Host only.
    """
    lib = _lib.load()
    n = len(cost_ms)
    if len(nbytes) != n:
        raise ValueError("cost_ms and nbytes must have the same length")
    c = (ctypes.c_double * max(n, 1))(*[float(x) for x in cost_ms])
    b = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in nbytes])
    owner = (ctypes.c_int32 * max(n, 1))()
    rms = (ctypes.c_double * max(n_ranks, 1))()
    rbytes = (ctypes.c_int64 * max(n_ranks, 1))()
    _lib.check(lib.mfsdp_plan_owners(c, b, n, n_ranks, byte_slack, owner, rms, rbytes))
    return ([int(owner[i]) for i in range(n)], [float(rms[r]) for r in range(n_ranks)],
            [int(rbytes[r]) for r in range(n_ranks)])


def tail_layout(numels: Sequence[int]):
    """Offsets of tensors packed in order into one fp32 tail, each segment on a
    16-byte boundary (mfsdp_tail_layout).  Returns (offsets, total)."""
    lib = _lib.load()
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    off = (ctypes.c_int64 * max(n, 1))()
    total = ctypes.c_int64(0)
    _lib.check(lib.mfsdp_tail_layout(arr, n, off, ctypes.byref(total)))
    return [int(off[i]) for i in range(n)], int(total.value)


def _tail_args(tensors, offsets):
    n = len(tensors)
    if len(offsets) != n:
        raise ValueError("one offset per tensor")
    ptrs = (ctypes.c_void_p * max(n, 1))()
    nums = (ctypes.c_int64 * max(n, 1))()
    offs = (ctypes.c_int64 * max(n, 1))(*[int(o) for o in offsets])
    for i, t in enumerate(tensors):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"tail tensor {i} must be a contiguous fp32 tensor")
        ptrs[i] = t.data_ptr() if t.numel() else None
        nums[i] = t.numel()
    return ptrs, nums, offs


def tail_pack(tensors: Sequence[torch.Tensor], packed: Optional[torch.Tensor] = None,
              offsets: Optional[Sequence[int]] = None):
    """Gather fp32 tensors (any shape, contiguous) into a packed tail
    (mfsdp_tail_pack).  Returns (packed, offsets)."""
    lib = _lib.load()
    if offsets is None:
        offsets, total = tail_layout([t.numel() for t in tensors])
    else:
        total = max([o + (t.numel() + 3) // 4 * 4 for o, t in zip(offsets, tensors)] or [0])
    if packed is None:
        device = tensors[0].device if tensors else torch.device("cuda")
        packed = torch.empty(total, dtype=torch.float32, device=device)
    if packed.dtype != torch.float32 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous fp32 tensor")
    if len(tensors) == 0:
        return packed, list(offsets)
    ptrs, nums, offs = _tail_args(tensors, offsets)
    stream = torch.cuda.current_stream(packed.device).cuda_stream
    _lib.check(lib.mfsdp_tail_pack(ptrs, nums, offs, len(tensors), packed.data_ptr(),
                                   packed.numel(), stream))
    return packed, list(offsets)


def tail_unpack(packed: torch.Tensor, tensors: Sequence[torch.Tensor],
                offsets: Sequence[int]) -> None:
    """Scatter a packed fp32 tail back into its tensors (mfsdp_tail_unpack)."""
    lib = _lib.load()
    if len(tensors) == 0:
        return
    if packed.dtype != torch.float32 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous fp32 tensor")
    ptrs, nums, offs = _tail_args(tensors, offsets)
    stream = torch.cuda.current_stream(packed.device).cuda_stream
    _lib.check(lib.mfsdp_tail_unpack(packed.data_ptr(), packed.numel(), ptrs, nums, offs,
                                     len(tensors), stream))


def mfma_probe(out: torch.Tensor, iters: int) -> None:
    """Enqueue the MFMA-only measurement kernel (mfsdp_mfma_probe) on torch's
    current stream: out.numel() // 8 workgroups of 8 waves, 8 * iters bf16
    MFMAs of 32768 flops per wave; out is a contiguous fp32 device tensor."""
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() % 8:
        raise ValueError("out must be a contiguous fp32 tensor of 8 floats per workgroup")
    stream = torch.cuda.current_stream(out.device).cuda_stream
    _lib.check(_lib.load().mfsdp_mfma_probe(out.data_ptr(), out.numel() // 8, int(iters), stream))


class timing:
    """Per-kernel-kind launch timing through the library's hipEvents."""

    @staticmethod
    def enable(on: bool = True) -> None:
        _lib.check(_lib.load().mfsdp_timing_enable(1 if on else 0))

    @staticmethod
    def reset() -> None:
        _lib.check(_lib.load().mfsdp_timing_reset())

    @staticmethod
    def read(kind: str) -> Tuple[float, int]:
        ms = ctypes.c_double(0.0)
        cnt = ctypes.c_int64(0)
        _lib.check(_lib.load().mfsdp_timing_read(_lib.KERNEL_KINDS[kind],
                                                 ctypes.byref(ms), ctypes.byref(cnt)))
        return ms.value, int(cnt.value)
