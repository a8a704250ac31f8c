"""ctypes binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, turned into raw device pointers and handed to the library with the
current HIP stream.  Every step of the computation runs in the library's
kernels; there is no fallback of any kind.  If libgdn.so is missing the import
of this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
GDN_ERR_CHECK = 4   # the debug library libgdn_check.so only
GDN_F32, GDN_BF16 = 0, 1
GDN_GATES_SCALAR, GDN_GATES_CHANNEL = 0, 1
ABI_VERSION = 9


class GdnFwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class GdnRawGates(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("ld_a", ctypes.c_int64), ("ld_b", ctypes.c_int64), ("ld_w", ctypes.c_int64)]


class GdnVarlenDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("total_T", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class GdnDecodeDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("scale", ctypes.c_float)]


class GdnBwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("scale", ctypes.c_float)]


class GdnBwdVarlenDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("total_T", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("scale", ctypes.c_float)]


class GdnConvDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("total_T", ctypes.c_int64), ("ld_x", ctypes.c_int64),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class GdnGateDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("ld_a", ctypes.c_int64), ("ld_b", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("H_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("gate_dtype", ctypes.c_int32)]


class GdnNormDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("ld_z", ctypes.c_int64),
                ("H_v", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python gated_delta_rule_gdn_amd/build.py` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.gdn_chunk_fwd.argtypes = [ctypes.POINTER(GdnFwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdn_chunk_fwd_gated.argtypes = [ctypes.POINTER(GdnFwdDesc), vp, vp, vp,
                                        ctypes.POINTER(GdnRawGates), vp, vp, vp, vp]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_varlen.argtypes = [ctypes.POINTER(GdnVarlenDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp]
    lib.gdn_chunk_fwd_varlen.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [ctypes.POINTER(GdnDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_backward_workspace_size.argtypes = [ctypes.POINTER(GdnBwdDesc)]
    lib.gdn_backward_workspace_size.restype = ctypes.c_size_t
    lib.gdn_backward.argtypes = [ctypes.POINTER(GdnBwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 vp, ctypes.c_size_t, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_backward.restype = ctypes.c_int
    lib.gdn_backward_saved.argtypes = lib.gdn_backward.argtypes
    lib.gdn_backward_saved.restype = ctypes.c_int
    lib.gdn_chunk_fwd_save.argtypes = [ctypes.POINTER(GdnFwdDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd_save.restype = ctypes.c_int
    lib.gdn_backward_noalloc.argtypes = [ctypes.POINTER(GdnBwdDesc), vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_backward_noalloc.restype = ctypes.c_int
    lib.gdn_backward_noalloc_max_bytes.argtypes = []
    lib.gdn_backward_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.gdn_backward_varlen_workspace_size.argtypes = [ctypes.POINTER(GdnBwdVarlenDesc)]
    lib.gdn_backward_varlen_workspace_size.restype = ctypes.c_size_t
    lib.gdn_backward_varlen.argtypes = [ctypes.POINTER(GdnBwdVarlenDesc), vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp, vp,
                                        vp, vp, vp]
    lib.gdn_backward_varlen.restype = ctypes.c_int
    lib.gdn_backward_varlen_saved.argtypes = lib.gdn_backward_varlen.argtypes
    lib.gdn_backward_varlen_saved.restype = ctypes.c_int
    lib.gdn_chunk_fwd_varlen_save.argtypes = [ctypes.POINTER(GdnVarlenDesc), vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd_varlen_save.restype = ctypes.c_int
    lib.gdn_short_conv.argtypes = [ctypes.POINTER(GdnConvDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_short_conv.restype = ctypes.c_int
    lib.gdn_gates.argtypes = [ctypes.POINTER(GdnGateDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_gates.restype = ctypes.c_int
    lib.gdn_output_gate.argtypes = [ctypes.POINTER(GdnNormDesc), vp, vp, vp, vp, vp]
    lib.gdn_output_gate.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_check_selftest.argtypes = [vp, vp]
    lib.gdn_check_selftest.restype = ctypes.c_int
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    if lib.gdn_abi_version() != ABI_VERSION:
        raise ImportError("libgdn.so ABI version mismatch")
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.gdn_status_string(int(status)).decode()


def abi_version() -> int:
    return lib.gdn_abi_version()


def check_selftest(out64, stream=None) -> int:
    """gdn_check_selftest: the raw status (GDN_OK from the debug library when
    its LDS checks fire, GDN_ERR_UNSUPPORTED from libgdn.so); out64 is a
    64-element fp32 device tensor."""
    _check(out64, "out64", shape=(64,), dtype=torch.float32)
    return lib.gdn_check_selftest(_ptr(out64), _stream(stream))


_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(t, name, shape=None, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _fwd_desc(q, k, v, beta_or_b, w, g, state_in, state_out, o, scale, chunk):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    io = q.dtype
    if io not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    gdt = beta_or_b.dtype
    channel = w is not None
    gshape = (B, T, Hv, dk) if channel else (B, T, Hv)
    _check(q, "q", (B, T, Hk, dk), io)
    _check(k, "k", (B, T, Hk, dk), io)
    _check(v, "v", (B, T, Hv, dv), io)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    _check(w, "w", (B, T, Hv, dv), gdt)
    _check(g, "g", gshape, gdt)
    _check(state_in, "state_in", (B, Hv, dk, dv), torch.float32)
    _check(state_out, "state_out", (B, Hv, dk, dv), torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=io, device=q.device)
    _check(o, "o", (B, T, Hv, dv), io)
    if gdt not in _DT:
        raise ValueError("gates must be float32 or bfloat16")
    desc = GdnFwdDesc(B, T, Hk, Hv, dk, dv, _DT[io], _DT[gdt],
                      GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, chunk, float(scale))
    return desc, o


def gdn_chunk_fwd(q, k, v, beta_or_b, w=None, g=None, state_in=None, state_out=None, o=None,
                  scale: float = 1.0, chunk: int = 64, stream=None):
    """Chunkwise forward (see include/gdn.h).  Returns (o, state_out).

    q, k [B,T,Hk,dk]; v [B,T,Hv,dv]; beta_or_b [B,T,Hv] (scalar gates) or
    [B,T,Hv,dk] (channel gates, then w [B,T,Hv,dv] is required); g like
    beta_or_b or None; state_in/state_out [B,Hv,dk,dv] fp32 or None.  o is
    allocated when not given.
    """
    desc, o = _fwd_desc(q, k, v, beta_or_b, w, g, state_in, state_out, o, scale, chunk)
    st = lib.gdn_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b),
                           _ptr(w), _ptr(g), _ptr(state_in), _ptr(state_out), _ptr(o),
                           _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, state_out


def _workspace(workspace, need, device):
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace, workspace.numel() * workspace.element_size()


def gdn_chunk_fwd_save(q, k, v, beta_or_b, w=None, g=None, state_in=None, state_out=None,
                       o=None, scale: float = 1.0, chunk: int = 64, workspace=None, stream=None):
    """gdn_chunk_fwd that also fills a backward workspace for gdn_backward_saved
    (see include/gdn.h).  Returns (o, state_out, workspace); the workspace is
    allocated (gdn_backward_workspace_size bytes) when not given."""
    desc, o = _fwd_desc(q, k, v, beta_or_b, w, g, state_in, state_out, o, scale, chunk)
    need = gdn_backward_workspace_size(q, v, beta_or_b, w, scale)
    workspace, nbytes = _workspace(workspace, need, q.device)
    st = lib.gdn_chunk_fwd_save(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b),
                                _ptr(w), _ptr(g), _ptr(state_in), _ptr(state_out), _ptr(o),
                                _ptr(workspace), ctypes.c_size_t(nbytes), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_save")
    return o, state_out, workspace


def gdn_chunk_fwd_gated(q, k, v, b_raw, a_raw=None, w_raw=None, A_log=None, dt_bias=None,
                        state_in=None, state_out=None, o=None, scale: float = 1.0, chunk: int = 64,
                        stream=None):
    """Chunkwise forward on raw gate projections, the activations applied in
    the kernel (see include/gdn.h).  Returns (o, state_out).

    q, k [B,T,Hk,dk]; v [B,T,Hv,dv]; b_raw, a_raw [B*T, >= Hv] (scalar gates)
    or [B*T, >= Hv dk] (channel gates, then w_raw [B*T, >= Hv dv] is
    required): column blocks of a projection output are fine.  a_raw None
    means alpha = 1.  A_log, dt_bias fp32 [columns of a] or None.
    """
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    io = q.dtype
    gdt = b_raw.dtype
    channel = w_raw is not None
    rows = B * T
    ncol = Hv * dk if channel else Hv
    _check(q, "q", (B, T, Hk, dk), io)
    _check(k, "k", (B, T, Hk, dk), io)
    _check(v, "v", (B, T, Hv, dv), io)
    ld_b = _check_rows(b_raw, "b_raw", rows, ncol, gdt)
    ld_a = _check_rows(a_raw, "a_raw", rows, ncol, gdt) if a_raw is not None else 0
    ld_w = _check_rows(w_raw, "w_raw", rows, Hv * dv, gdt) if channel else 0
    _check(A_log, "A_log", (ncol,), torch.float32)
    _check(dt_bias, "dt_bias", (ncol,), torch.float32)
    _check(state_in, "state_in", (B, Hv, dk, dv), torch.float32)
    _check(state_out, "state_out", (B, Hv, dk, dv), torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=io, device=q.device)
    _check(o, "o", (B, T, Hv, dv), io)
    if io not in _DT or gdt not in _DT:
        raise ValueError("q and the projections must be float32 or bfloat16")
    desc = GdnFwdDesc(B, T, Hk, Hv, dk, dv, _DT[io], _DT[gdt],
                      GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, chunk, float(scale))
    gates = GdnRawGates(_ptr(a_raw), _ptr(b_raw), _ptr(w_raw), _ptr(A_log), _ptr(dt_bias),
                        ld_a, ld_b, ld_w)
    st = lib.gdn_chunk_fwd_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(gates),
                                 _ptr(state_in), _ptr(state_out), _ptr(o), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_gated")
    return o, state_out


def _varlen_fwd_desc(q, k, v, beta_or_b, cu_seqlens, w, g, state_in, state_out, o, scale, chunk):
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    io = q.dtype
    if io not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    gdt = beta_or_b.dtype
    channel = w is not None
    gshape = (T, Hv, dk) if channel else (T, Hv)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64)
    _check(q, "q", (T, Hk, dk), io)
    _check(k, "k", (T, Hk, dk), io)
    _check(v, "v", (T, Hv, dv), io)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    _check(w, "w", (T, Hv, dv), gdt)
    _check(g, "g", gshape, gdt)
    _check(state_in, "state_in", (N, Hv, dk, dv), torch.float32)
    _check(state_out, "state_out", (N, Hv, dk, dv), torch.float32)
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=io, device=q.device)
    _check(o, "o", (T, Hv, dv), io)
    if gdt not in _DT:
        raise ValueError("gates must be float32 or bfloat16")
    desc = GdnVarlenDesc(N, T, Hk, Hv, dk, dv, _DT[io], _DT[gdt],
                         GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, chunk, float(scale))
    return desc, o


def gdn_chunk_fwd_varlen(q, k, v, beta_or_b, cu_seqlens, w=None, g=None, state_in=None,
                         state_out=None, o=None, scale: float = 1.0, chunk: int = 64,
                         stream=None):
    """Chunkwise forward over packed sequences (see include/gdn.h).
    Returns (o, state_out).

    q, k [total_T,Hk,dk]; v [total_T,Hv,dv]; beta_or_b [total_T,Hv] or
    [total_T,Hv,dk] (then w [total_T,Hv,dv]); g like beta_or_b or None;
    cu_seqlens int64 device tensor [N+1] of token offsets; state_in/state_out
    [N,Hv,dk,dv] fp32 or None.  o is allocated when not given.
    """
    desc, o = _varlen_fwd_desc(q, k, v, beta_or_b, cu_seqlens, w, g, state_in, state_out, o,
                               scale, chunk)
    st = lib.gdn_chunk_fwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(beta_or_b), _ptr(w), _ptr(g), _ptr(state_in),
                                  _ptr(state_out), _ptr(o), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_varlen")
    return o, state_out


def gdn_chunk_fwd_varlen_save(q, k, v, beta_or_b, cu_seqlens, w=None, g=None, state_in=None,
                              state_out=None, o=None, scale: float = 1.0, chunk: int = 64,
                              workspace=None, stream=None):
    """gdn_chunk_fwd_varlen that also fills a backward workspace for
    gdn_backward_varlen_saved (see include/gdn.h).  Returns (o, state_out,
    workspace); the workspace is allocated when not given."""
    desc, o = _varlen_fwd_desc(q, k, v, beta_or_b, cu_seqlens, w, g, state_in, state_out, o,
                               scale, chunk)
    bdesc = GdnBwdVarlenDesc(desc.N, desc.total_T, desc.H_k, desc.H_v, desc.d_k, desc.d_v,
                             desc.io_dtype, desc.gate_dtype, desc.gate_mode, desc.scale)
    need = int(lib.gdn_backward_varlen_workspace_size(ctypes.byref(bdesc)))
    workspace, nbytes = _workspace(workspace, need, q.device)
    st = lib.gdn_chunk_fwd_varlen_save(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(beta_or_b), _ptr(w), _ptr(g),
                                       _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(workspace),
                                       ctypes.c_size_t(nbytes), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_varlen_save")
    return o, state_out, workspace


def gdn_decode_step(q, k, v, beta_or_b, state, w=None, g=None, o=None, scale: float = 1.0,
                    stream=None):
    """One decode step, state updated in place (see include/gdn.h).  Returns o.

    q, k [N,Hk,dk]; v [N,Hv,dv]; beta_or_b [N,Hv] or [N,Hv,dk]; w [N,Hv,dv]
    or None; g like beta_or_b or None; state [N,Hv,dk,dv] fp32.
    """
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    io = q.dtype
    if io not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    gdt = beta_or_b.dtype
    channel = w is not None
    gshape = (N, Hv, dk) if channel else (N, Hv)
    _check(q, "q", (N, Hk, dk), io)
    _check(k, "k", (N, Hk, dk), io)
    _check(v, "v", (N, Hv, dv), io)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    _check(w, "w", (N, Hv, dv), gdt)
    _check(g, "g", gshape, gdt)
    _check(state, "state", (N, Hv, dk, dv), torch.float32)
    if o is None:
        o = torch.empty((N, Hv, dv), dtype=io, device=q.device)
    _check(o, "o", (N, Hv, dv), io)
    if gdt not in _DT:
        raise ValueError("gates must be float32 or bfloat16")
    desc = GdnDecodeDesc(N, Hk, Hv, dk, dv, _DT[io], _DT[gdt],
                         GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, float(scale))
    st = lib.gdn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b),
                             _ptr(w), _ptr(g), _ptr(state), _ptr(o), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_step")
    return o


def _check_rows(t, name, rows, min_cols, dtype):
    """A 2-d device tensor of `rows` rows with unit column stride (a column
    block of a wider buffer is fine).  Returns its row stride in elements."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < min_cols:
        raise ValueError(f"{name} must be [{rows}, >= {min_cols}], got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if rows > 1 else max(t.stride(0), t.shape[1])


def gdn_short_conv(x, conv_w, H_k, H_v, d_k, d_v, N=None, cu_seqlens=None, conv_state_in=None,
                   conv_state_out=None, q=None, k=None, v=None, eps: float = 1e-6, stream=None):
    """q, k, v branch: causal conv (kernel 4) + SiLU + L2 norm of q, k (see
    include/gdn.h).  Returns (q, k, v, conv_state_out).

    x [total_T, >= C] (C = 2 H_k d_k + H_v d_v; a column block of the
    projection output is fine); conv_w [C, 4] fp32; cu_seqlens int64 device
    [N+1] or None for N sequences of total_T / N tokens (N defaults to 1);
    conv states [N, 3, C] in x's dtype or None.  q, k [total_T, H_k, d_k] and
    v [total_T, H_v, d_v] are allocated when not given.
    """
    io = x.dtype
    if io not in _DT:
        raise ValueError("x must be float32 or bfloat16")
    T = x.shape[0]
    C = 2 * H_k * d_k + H_v * d_v
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-d tensor of N + 1 offsets")
        N = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64)
    elif N is None:
        N = 1
    ld_x = _check_rows(x, "x", T, C, io)
    _check(conv_w, "conv_w", (C, 4), torch.float32)
    _check(conv_state_in, "conv_state_in", (N, 3, C), io)
    _check(conv_state_out, "conv_state_out", (N, 3, C), io)
    dev = x.device
    if q is None:
        q = torch.empty((T, H_k, d_k), dtype=io, device=dev)
    if k is None:
        k = torch.empty((T, H_k, d_k), dtype=io, device=dev)
    if v is None:
        v = torch.empty((T, H_v, d_v), dtype=io, device=dev)
    _check(q, "q", (T, H_k, d_k), io)
    _check(k, "k", (T, H_k, d_k), io)
    _check(v, "v", (T, H_v, d_v), io)
    desc = GdnConvDesc(N, T, ld_x, H_k, H_v, d_k, d_v, _DT[io], float(eps))
    st = lib.gdn_short_conv(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(x), _ptr(conv_w),
                            _ptr(conv_state_in), _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v),
                            _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_short_conv")
    return q, k, v, conv_state_out


def gdn_gates(a_raw, b_raw, H_v, w_raw=None, A_log=None, dt_bias=None, d_k=None, d_v=None,
              gate_dtype=None, g=None, beta_or_b=None, w=None, stream=None):
    """Gate activations (see include/gdn.h).  Returns (g, beta_or_b, w).

    Scalar gates (w_raw None): a_raw, b_raw [rows, >= H_v] -> g, beta [rows, H_v].
    Channel gates: a_raw, b_raw [rows, >= H_v d_k], w_raw [rows, >= H_v d_v] ->
    g, b [rows, H_v, d_k], w [rows, H_v, d_v].  Raw inputs may be column blocks
    of one projection output.  A_log, dt_bias fp32 [columns of a] or None.
    """
    io = a_raw.dtype
    if io not in _DT:
        raise ValueError("a_raw must be float32 or bfloat16")
    gdt = io if gate_dtype is None else gate_dtype
    if gdt not in _DT:
        raise ValueError("gate_dtype must be float32 or bfloat16")
    rows = a_raw.shape[0]
    channel = w_raw is not None
    if channel and (d_k is None or d_v is None):
        raise ValueError("channel gates need d_k and d_v")
    n_ab = H_v * d_k if channel else H_v
    ld_a = _check_rows(a_raw, "a_raw", rows, n_ab, io)
    ld_b = _check_rows(b_raw, "b_raw", rows, n_ab, io)
    ld_w = _check_rows(w_raw, "w_raw", rows, H_v * d_v, io) if channel else 0
    _check(A_log, "A_log", (n_ab,), torch.float32)
    _check(dt_bias, "dt_bias", (n_ab,), torch.float32)
    gshape = (rows, H_v, d_k) if channel else (rows, H_v)
    dev = a_raw.device
    if g is None:
        g = torch.empty(gshape, dtype=gdt, device=dev)
    if beta_or_b is None:
        beta_or_b = torch.empty(gshape, dtype=gdt, device=dev)
    if channel and w is None:
        w = torch.empty((rows, H_v, d_v), dtype=gdt, device=dev)
    _check(g, "g", gshape, gdt)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    if channel:
        _check(w, "w", (rows, H_v, d_v), gdt)
    desc = GdnGateDesc(rows, ld_a, ld_b, ld_w, H_v, d_k or 0, d_v or 0,
                       GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, _DT[io], _DT[gdt])
    st = lib.gdn_gates(ctypes.byref(desc), _ptr(a_raw), _ptr(b_raw), _ptr(w_raw), _ptr(A_log),
                       _ptr(dt_bias), _ptr(g), _ptr(beta_or_b), _ptr(w), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_gates")
    return g, beta_or_b, w


def gdn_output_gate(o, z, weight, eps: float = 1e-6, y=None, stream=None):
    """RMS norm of each value head's output times swish(z) (see include/gdn.h).
    Returns y.

    o [rows, H_v, d_v]; z [rows, >= H_v d_v] (a column block of the projection
    output is fine); weight [d_v] fp32; y like o (allocated when not given; may
    be o itself).
    """
    rows, Hv, dv = o.shape
    io = o.dtype
    if io not in _DT:
        raise ValueError("o must be float32 or bfloat16")
    _check(o, "o", (rows, Hv, dv), io)
    ld_z = _check_rows(z, "z", rows, Hv * dv, io)
    _check(weight, "weight", (dv,), torch.float32)
    if y is None:
        y = torch.empty_like(o)
    _check(y, "y", (rows, Hv, dv), io)
    desc = GdnNormDesc(rows, ld_z, Hv, dv, _DT[io], float(eps))
    st = lib.gdn_output_gate(ctypes.byref(desc), _ptr(o), _ptr(z), _ptr(weight), _ptr(y),
                             _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_output_gate")
    return y


def _bwd_desc(q, v, beta_or_b, w, scale):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if q.dtype not in _DT or beta_or_b.dtype not in _DT:
        raise ValueError("inputs must be float32 or bfloat16")
    return GdnBwdDesc(B, T, Hk, Hv, dk, dv, _DT[q.dtype], _DT[beta_or_b.dtype],
                      GDN_GATES_CHANNEL if w is not None else GDN_GATES_SCALAR, float(scale))


def gdn_backward_workspace_size(q, v, beta_or_b, w=None, scale: float = 1.0) -> int:
    """Workspace bytes gdn_backward needs for these shapes (see include/gdn.h)."""
    return int(lib.gdn_backward_workspace_size(ctypes.byref(_bwd_desc(q, v, beta_or_b, w, scale))))


def _bwd_outputs(q, k, v, beta_or_b, d_o, w, g, state_in, d_state_out, need_dg,
                 need_d_state_in, grads):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    io = q.dtype
    gdt = beta_or_b.dtype
    channel = w is not None
    gshape = (B, T, Hv, dk) if channel else (B, T, Hv)
    _check(q, "q", (B, T, Hk, dk), io)
    _check(k, "k", (B, T, Hk, dk), io)
    _check(v, "v", (B, T, Hv, dv), io)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    _check(w, "w", (B, T, Hv, dv), gdt)
    _check(g, "g", gshape, gdt)
    _check(state_in, "state_in", (B, Hv, dk, dv), torch.float32)
    _check(d_o, "d_o", (B, T, Hv, dv), io)
    _check(d_state_out, "d_state_out", (B, Hv, dk, dv), torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = {"dq": (B, T, Hk, dk), "dk": (B, T, Hk, dk), "dv": (B, T, Hv, dv), "db": gshape,
              "dw": (B, T, Hv, dv) if channel else None,
              "dg": gshape if (g is not None and need_dg) else None,
              "d_state_in": (B, Hv, dk, dv) if need_d_state_in else None}
    out = {} if grads is None else dict(grads)
    for name, shp in shapes.items():
        if shp is None:
            out[name] = None
            continue
        if out.get(name) is None:
            out[name] = torch.empty(shp, **f32)
        _check(out[name], name, shp, torch.float32)
    return out


def gdn_backward(q, k, v, beta_or_b, d_o, w=None, g=None, state_in=None, d_state_out=None,
                 scale: float = 1.0, workspace=None, need_dg: bool = True,
                 need_d_state_in: bool = True, grads=None, stream=None):
    """Gradients of the chunk forward (see include/gdn.h).  Returns a dict of
    fp32 tensors dq, dk, dv, db, dw (None for scalar gates), dg (None when g
    is None or need_dg is False), d_state_in (None unless need_d_state_in).

    Shapes as for gdn_chunk_fwd; d_o like o; d_state_out like the state or
    None.  `workspace` is a device uint8 tensor of at least
    gdn_backward_workspace_size(...) bytes (allocated when None); `grads` may
    hold preallocated outputs under the same keys.
    """
    return _backward_call(lib.gdn_backward, "gdn_backward", q, k, v, beta_or_b, d_o, w, g,
                          state_in, d_state_out, scale, workspace, need_dg, need_d_state_in,
                          grads, stream)


def _backward_call(fn, name, q, k, v, beta_or_b, d_o, w, g, state_in, d_state_out, scale,
                   workspace, need_dg, need_d_state_in, grads, stream):
    out = _bwd_outputs(q, k, v, beta_or_b, d_o, w, g, state_in, d_state_out, need_dg,
                       need_d_state_in, grads)
    desc = _bwd_desc(q, v, beta_or_b, w, scale)
    need = int(lib.gdn_backward_workspace_size(ctypes.byref(desc)))
    workspace, nbytes = _workspace(workspace, need, q.device)
    st = fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b), _ptr(w), _ptr(g),
            _ptr(state_in), _ptr(d_o), _ptr(d_state_out), _ptr(workspace),
            ctypes.c_size_t(nbytes), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
            _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dg"]), _ptr(out["d_state_in"]),
            _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, name)
    return out


def gdn_backward_saved(q, k, v, beta_or_b, d_o, workspace, w=None, g=None, state_in=None,
                       d_state_out=None, scale: float = 1.0, need_dg: bool = True,
                       need_d_state_in: bool = True, grads=None, stream=None):
    """gdn_backward over a workspace that gdn_chunk_fwd_save filled for the same
    inputs (see include/gdn.h): only the reverse walk runs.  Returns the same
    dict as gdn_backward."""
    if workspace is None:
        raise ValueError("gdn_backward_saved needs the workspace gdn_chunk_fwd_save filled")
    return _backward_call(lib.gdn_backward_saved, "gdn_backward_saved", q, k, v, beta_or_b, d_o,
                          w, g, state_in, d_state_out, scale, workspace, need_dg,
                          need_d_state_in, grads, stream)


def gdn_backward_noalloc_max_bytes() -> int:
    """Bytes of the static workspace gdn_backward_noalloc uses on each GPU."""
    return int(lib.gdn_backward_noalloc_max_bytes())


def gdn_backward_noalloc(q, k, v, beta_or_b, d_o, w=None, g=None, state_in=None,
                         d_state_out=None, scale: float = 1.0, need_dg: bool = True,
                         need_d_state_in: bool = True, grads=None, stream=None):
    """gdn_backward on the library's static workspace (see include/gdn.h): no
    workspace argument; with every output passed in `grads`, the library
    allocates nothing.  Raises GdnError(GDN_ERR_UNSUPPORTED) when the shapes
    need more than gdn_backward_noalloc_max_bytes() of workspace."""
    out = _bwd_outputs(q, k, v, beta_or_b, d_o, w, g, state_in, d_state_out, need_dg,
                       need_d_state_in, grads)
    desc = _bwd_desc(q, v, beta_or_b, w, scale)
    st = lib.gdn_backward_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b),
                                  _ptr(w), _ptr(g), _ptr(state_in), _ptr(d_o), _ptr(d_state_out),
                                  _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                  _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dg"]),
                                  _ptr(out["d_state_in"]), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_backward_noalloc")
    return out


def gdn_backward_varlen(q, k, v, beta_or_b, d_o, cu_seqlens, w=None, g=None, state_in=None,
                        d_state_out=None, scale: float = 1.0, workspace=None,
                        need_dg: bool = True, need_d_state_in: bool = True, grads=None,
                        stream=None):
    """Gradients over packed sequences (see include/gdn.h).  Shapes as for
    gdn_chunk_fwd_varlen ([total_T, ...] packed, states [N, ...]); returns the
    same dict of fp32 tensors as gdn_backward."""
    return _backward_varlen_call(lib.gdn_backward_varlen, "gdn_backward_varlen", q, k, v,
                                 beta_or_b, d_o, cu_seqlens, w, g, state_in, d_state_out, scale,
                                 workspace, need_dg, need_d_state_in, grads, stream)


def gdn_backward_varlen_saved(q, k, v, beta_or_b, d_o, cu_seqlens, workspace, w=None, g=None,
                              state_in=None, d_state_out=None, scale: float = 1.0,
                              need_dg: bool = True, need_d_state_in: bool = True, grads=None,
                              stream=None):
    """gdn_backward_varlen over a workspace that gdn_chunk_fwd_varlen_save
    filled for the same inputs (see include/gdn.h): only the reverse walk
    runs."""
    if workspace is None:
        raise ValueError("gdn_backward_varlen_saved needs the workspace "
                         "gdn_chunk_fwd_varlen_save filled")
    return _backward_varlen_call(lib.gdn_backward_varlen_saved, "gdn_backward_varlen_saved", q,
                                 k, v, beta_or_b, d_o, cu_seqlens, w, g, state_in, d_state_out,
                                 scale, workspace, need_dg, need_d_state_in, grads, stream)


def _backward_varlen_call(fn, fname, q, k, v, beta_or_b, d_o, cu_seqlens, w, g, state_in,
                          d_state_out, scale, workspace, need_dg, need_d_state_in, grads,
                          stream):
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    io = q.dtype
    gdt = beta_or_b.dtype
    if io not in _DT or gdt not in _DT:
        raise ValueError("inputs must be float32 or bfloat16")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    channel = w is not None
    gshape = (T, Hv, dk) if channel else (T, Hv)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int64)
    _check(q, "q", (T, Hk, dk), io)
    _check(k, "k", (T, Hk, dk), io)
    _check(v, "v", (T, Hv, dv), io)
    _check(beta_or_b, "beta_or_b", gshape, gdt)
    _check(w, "w", (T, Hv, dv), gdt)
    _check(g, "g", gshape, gdt)
    _check(state_in, "state_in", (N, Hv, dk, dv), torch.float32)
    _check(d_o, "d_o", (T, Hv, dv), io)
    _check(d_state_out, "d_state_out", (N, Hv, dk, dv), torch.float32)
    desc = GdnBwdVarlenDesc(N, T, Hk, Hv, dk, dv, _DT[io], _DT[gdt],
                            GDN_GATES_CHANNEL if channel else GDN_GATES_SCALAR, float(scale))
    need = int(lib.gdn_backward_varlen_workspace_size(ctypes.byref(desc)))
    workspace, nbytes = _workspace(workspace, need, q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = {"dq": (T, Hk, dk), "dk": (T, Hk, dk), "dv": (T, Hv, dv), "db": gshape,
              "dw": (T, Hv, dv) if channel else None,
              "dg": gshape if (g is not None and need_dg) else None,
              "d_state_in": (N, Hv, dk, dv) if need_d_state_in else None}
    out = {} if grads is None else dict(grads)
    for name, shp in shapes.items():
        if shp is None:
            out[name] = None
            continue
        if out.get(name) is None:
            out[name] = torch.empty(shp, **f32)
        _check(out[name], name, shp, torch.float32)
    st = fn(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(beta_or_b),
            _ptr(w), _ptr(g), _ptr(state_in), _ptr(d_o), _ptr(d_state_out), _ptr(workspace),
            ctypes.c_size_t(nbytes), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
            _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dg"]), _ptr(out["d_state_in"]),
            _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, fname)
    return out
