"""Gated delta rule layer core on MI355X (gfx950): a thin Python binding.

Everything numeric runs in the HIP kernels of libgdn.so, reached through its
C ABI (include/gdn.h).  This module only marshals torch tensors (device
memory and the current HIP stream) into that ABI: it checks devices, dtypes
and contiguity, allocates outputs and the workspace, and raises GdnError on a
non-OK status.  There is no CPU fallback: if libgdn.so is missing or cannot
be loaded, every call raises.

    o, S = chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None)
    o    = decode_step(state, q, k, v, log_alpha, beta)      # state updated in place
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["GdnError", "chunk_fwd", "chunk_fwd_noalloc", "decode_step", "chunk_bwd", "chunk_fwd_workspace_size",
           "chunk_bwd_workspace_size", "chunk_fwd_check", "load", "lib_path", "profile", "CHUNK"]

HERE = os.path.dirname(os.path.abspath(__file__))
CHUNK = 64

GDN_FP32, GDN_BF16, GDN_FP16 = 0, 1, 2
GDN_QK_L2NORM = 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES in gdn.h
_DT = {torch.float32: GDN_FP32, torch.bfloat16: GDN_BF16, torch.float16: GDN_FP16}
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
           5: "GDN_ERR_UNSUPPORTED", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP", 8: "GDN_ERR_ALIAS",
           9: "GDN_ERR_DEVICE_INPUT"}


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = _STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


class ChunkDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


def lib_path() -> str:
    return os.environ.get("GDN_LIB", os.path.join(HERE, "libgdn.so"))


_lib = None


def load():
    """Load libgdn.so (raises if it is absent: build it with
    `python -m gated_delta_rule_24_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    p = lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m gated_delta_rule_24_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.gdn_abi_version.restype = ctypes.c_int
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_last_error_message.restype = ctypes.c_char_p
    lib.gdn_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.POINTER(sz)]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd.argtypes = [ctypes.POINTER(ChunkDesc)] + [vp] * 16 + [sz, vp]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_check.restype = ctypes.c_int
    lib.gdn_chunk_fwd_check.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_profile_enable.restype = ctypes.c_int
    lib.gdn_profile_enable.argtypes = [i32]
    lib.gdn_profile_count.restype = ctypes.c_int
    lib.gdn_profile_count.argtypes = [ctypes.POINTER(i32)]
    lib.gdn_profile_read.restype = ctypes.c_int
    lib.gdn_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double)]
    if lib.gdn_abi_version() != 5:
        raise RuntimeError(f"{p}: unexpected ABI version {lib.gdn_abi_version()}")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise GdnError(status, load().gdn_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, device, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _desc(B, T, H, dk, dv, N, in_dt, out_dt, chunk=CHUNK, flags=0):
    return ChunkDesc(B, T, H, dk, dv, N, chunk, in_dt, out_dt, flags)


def chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype=torch.bfloat16, out_dtype=torch.float32,
                             chunk=CHUNK) -> int:
    d = _desc(B, T, H, dk, dv, num_seqs, _DT[in_dtype], _DT[out_dtype], chunk)
    n = ctypes.c_size_t(0)
    _check(load().gdn_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def _chunk_call_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out_dtype, o, final_state, chunk,
                     qk_l2norm):
    """Checks and marshals the arguments shared by chunk_fwd and chunk_fwd_noalloc.
    Returns (descriptor, o, final_state or None, the leading pointer arguments)."""
    load()
    dev = q.device
    dts = (torch.float32, torch.bfloat16, torch.float16)
    _need(q, "q", dts, dev, 4)
    B, T, H, dk = q.shape
    _need(k, "k", (q.dtype,), dev, 4)
    _need(v, "v", (q.dtype,), dev, 4)
    dv = v.shape[3]
    if tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _need(log_alpha, "log_alpha", (torch.float32,), dev, 3)
    _need(beta, "beta", (torch.float32,), dev, 3)
    if tuple(log_alpha.shape) != (B, T, H) or tuple(beta.shape) != (B, T, H):
        raise ValueError("log_alpha and beta must be [B, T, H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if init_state is not None:
        _need(init_state, "init_state", (torch.float32,), dev, 4)
        if tuple(init_state.shape) != (N, H, dv, dk):
            raise ValueError(f"init_state must be {(N, H, dv, dk)}, got {tuple(init_state.shape)}")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(o, "o", (torch.float32, torch.bfloat16, torch.float16), dev, 4)
        if tuple(o.shape) != (B, T, H, dv):
            raise ValueError("o has the wrong shape")
    if final_state is True:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    elif final_state is not None:
        _need(final_state, "final_state", (torch.float32,), dev, 4)
        if tuple(final_state.shape) != (N, H, dv, dk):
            raise ValueError("final_state has the wrong shape")
    desc = _desc(B, T, H, dk, dv, N, _DT[q.dtype], _DT[o.dtype], chunk, GDN_QK_L2NORM if qk_l2norm else 0)
    ptrs = [_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu_seqlens), _ptr(o),
            _ptr(final_state)]
    return desc, o, final_state, ptrs


def chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, *, out_dtype=torch.float32,
              o=None, final_state=True, workspace=None, chunk=CHUNK, qk_l2norm=False):
    """Chunkwise-parallel prefill.

    q, k [B,T,H,dk], v [B,T,H,dv] (fp32/bf16/fp16, same dtype);
    log_alpha, beta [B,T,H] fp32; init_state [N,H,dv,dk] fp32 or None;
    cu_seqlens int32 [N+1] (packed batch, B == 1) or None.
    final_state: True (allocate), False/None (not returned) or a tensor to
    write (it may be init_state itself).  qk_l2norm: normalise q and k per
    (token, head) inside the kernels.  Returns (o, final_state or None).
    """
    lib = load()
    desc, o, final_state, ptrs = _chunk_call_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out_dtype, o,
                                                  final_state, chunk, qk_l2norm)
    need = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(int(need.value), dtype=torch.uint8, device=q.device)
    _check(lib.gdn_chunk_fwd(ctypes.byref(desc), *ptrs, _ptr(workspace),
                             ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(q.device)))
    return o, final_state


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, *, out_dtype=torch.float32,
                      o=None, final_state=True, chunk=CHUNK, qk_l2norm=False):
    """chunk_fwd through gdn_chunk_fwd_noalloc: the library's per-GPU scratch
    array (NOALLOC_SCRATCH_BYTES) stands in for the workspace, so with `o` and
    `final_state` passed in (or final_state=False) nothing is allocated.
    Calls that overlap in time on one GPU race on the scratch array."""
    lib = load()
    desc, o, final_state, ptrs = _chunk_call_args(q, k, v, log_alpha, beta, init_state, cu_seqlens, out_dtype, o,
                                                  final_state, chunk, qk_l2norm)
    _check(lib.gdn_chunk_fwd_noalloc(ctypes.byref(desc), *ptrs, _stream(q.device)))
    return o, final_state


def chunk_bwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype=torch.bfloat16, chunk=CHUNK,
                             qk_l2norm=False) -> int:
    d = _desc(B, T, H, dk, dv, num_seqs, _DT[in_dtype], GDN_FP32, chunk, GDN_QK_L2NORM if qk_l2norm else 0)
    n = ctypes.c_size_t(0)
    _check(load().gdn_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def chunk_bwd(q, k, v, log_alpha, beta, d_o, init_state=None, d_final=None, cu_seqlens=None, *,
              d_init=True, workspace=None, chunk=CHUNK, qk_l2norm=False):
    """Gradients of chunk_fwd's o and final state with respect to its inputs.

    q, k, v, log_alpha, beta, init_state, cu_seqlens, qk_l2norm as for
    chunk_fwd; d_o [B,T,H,dv] fp32; d_final [N,H,dv,dk] fp32 or None (zeros).
    d_init: True (allocate and return dL/d init_state) or False.
    Returns (dq, dk, dv, dlog_alpha, dbeta, d_init or None), all fp32.
    """
    lib = load()
    dev = q.device
    dts = (torch.float32, torch.bfloat16, torch.float16)
    _need(q, "q", dts, dev, 4)
    B, T, H, dk = q.shape
    _need(k, "k", (q.dtype,), dev, 4)
    _need(v, "v", (q.dtype,), dev, 4)
    dv = v.shape[3]
    if tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _need(log_alpha, "log_alpha", (torch.float32,), dev, 3)
    _need(beta, "beta", (torch.float32,), dev, 3)
    if tuple(log_alpha.shape) != (B, T, H) or tuple(beta.shape) != (B, T, H):
        raise ValueError("log_alpha and beta must be [B, T, H]")
    _need(d_o, "d_o", (torch.float32,), dev, 4)
    if tuple(d_o.shape) != (B, T, H, dv):
        raise ValueError(f"d_o must be {(B, T, H, dv)}, got {tuple(d_o.shape)}")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    for name, t in (("init_state", init_state), ("d_final", d_final)):
        if t is not None:
            _need(t, name, (torch.float32,), dev, 4)
            if tuple(t.shape) != (N, H, dv, dk):
                raise ValueError(f"{name} must be {(N, H, dv, dk)}, got {tuple(t.shape)}")
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk_, dv_ = torch.empty((B, T, H, dk), **f32), torch.empty((B, T, H, dk), **f32), torch.empty((B, T, H, dv), **f32)
    dla, db = torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32)
    di = torch.empty((N, H, dv, dk), **f32) if d_init else None
    desc = _desc(B, T, H, dk, dv, N, _DT[q.dtype], _DT[torch.float32], chunk, GDN_QK_L2NORM if qk_l2norm else 0)
    need = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    _check(lib.gdn_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                             _ptr(init_state), _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final), _ptr(dq), _ptr(dk_),
                             _ptr(dv_), _ptr(dla), _ptr(db), _ptr(di), _ptr(workspace),
                             ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev)))
    return dq, dk_, dv_, dla, db, di


def chunk_fwd_check(workspace: torch.Tensor) -> int:
    """Synchronise and return the device-side cu_seqlens check code of the last
    chunk_fwd that used `workspace` (0 = valid)."""
    code = ctypes.c_int32(0)
    st = load().gdn_chunk_fwd_check(_ptr(workspace), _stream(workspace.device), ctypes.byref(code))
    if st not in (0, 9):
        _check(st)
    return int(code.value)


def decode_step(state, q, k, v, log_alpha, beta, *, out_dtype=torch.float32, o=None, qk_l2norm=False):
    """One decode step, in place on `state` [N,H,dv,dk] fp32.
    q, k [N,H,dk], v [N,H,dv]; log_alpha, beta [N,H] fp32.  qk_l2norm:
    normalise q and k inside the kernel.  Returns o [N,H,dv]."""
    lib = load()
    dev = state.device
    _need(state, "state", (torch.float32,), dev, 4)
    N, H, dv, dk = state.shape
    dts = (torch.float32, torch.bfloat16, torch.float16)
    _need(q, "q", dts, dev, 3)
    _need(k, "k", (q.dtype,), dev, 3)
    _need(v, "v", (q.dtype,), dev, 3)
    if tuple(q.shape) != (N, H, dk) or tuple(k.shape) != (N, H, dk) or tuple(v.shape) != (N, H, dv):
        raise ValueError("q, k must be [N,H,dk] and v [N,H,dv] matching state")
    _need(log_alpha, "log_alpha", (torch.float32,), dev, 2)
    _need(beta, "beta", (torch.float32,), dev, 2)
    if tuple(log_alpha.shape) != (N, H) or tuple(beta.shape) != (N, H):
        raise ValueError("log_alpha and beta must be [N, H]")
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(o, "o", dts, dev, 3)
    _check(lib.gdn_decode_step(N, H, dk, dv, _DT[q.dtype], _DT[o.dtype], GDN_QK_L2NORM if qk_l2norm else 0,
                               _ptr(state), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(log_alpha), _ptr(beta), _ptr(o), _stream(dev)))
    return o


class profile:
    """Context manager collecting per-kernel launch times recorded by the
    library (HIP events around each launch, on the launch stream).

        with profile() as p:
            ...
        p.results  ->  {kernel name: (launches, total ms)}
    """

    def __enter__(self):
        _check(load().gdn_profile_enable(1))
        self.results = {}
        return self

    def __exit__(self, *exc):
        lib = load()
        _check(lib.gdn_profile_enable(0))
        n = ctypes.c_int32(0)
        _check(lib.gdn_profile_count(ctypes.byref(n)))
        for i in range(n.value):
            name, cnt, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
            _check(lib.gdn_profile_read(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)))
            self.results[name.value.decode()] = (int(cnt.value), float(ms.value))
        return False
