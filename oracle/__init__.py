"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``gated_delta_rule_gdn_amd``) never imports, links or falls back to it, and
this package imports nothing from the product library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double); this module
only marshals numpy arrays into it through ctypes.  Every input is converted
to float64 exactly (bf16 and fp32 values are exactly representable), so the
oracle sees the very values handed to the GPU.

Functions (each follows the passages cited in ``gdn_oracle.c``):
  recurrent  -- token-by-token recurrence ("Gated DeltaNet-2", Methodologie §1,
                update equation; read-out o_t = S_t^T q_t).
  chunkwise  -- naive chunkwise form (same page, §3, decay absorption and
                (I+T)^{-1} solve).  Used only to check the decomposition.
  decode     -- one token per sequence, state updated in place.
  backward   -- gradients of the recurrence (reverse mode, token by token).

The operations around the recurrence in a Gated DeltaNet block (short causal
convolution, SiLU, L2 norm, gate activations, output norm and swish gate) are
in ``oracle.layer`` (numpy, float64).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    common = [ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
              ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_double]
    lib.gdn_ref_recurrent.argtypes = common + [_dp, _dp, _dp, ctypes.c_int]
    lib.gdn_ref_recurrent.restype = ctypes.c_int
    lib.gdn_ref_chunkwise.argtypes = common + [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int]
    lib.gdn_ref_chunkwise.restype = ctypes.c_int
    lib.gdn_ref_decode.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp,
                                   ctypes.c_double, _dp, _dp, ctypes.c_int]
    lib.gdn_ref_decode.restype = ctypes.c_int
    lib.gdn_ref_backward.argtypes = common + [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                              ctypes.c_int]
    lib.gdn_ref_backward.restype = ctypes.c_int
    lib.gdn_oracle_abi.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> numpy, exact up-conversion
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _threads(nthreads):
    if nthreads:
        return int(nthreads)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _shapes(q, v, beta_or_b, w):
    if q.ndim != 4 or v.ndim != 4:
        raise ValueError("q/k must be [B,T,Hk,dk] and v [B,T,Hv,dv]")
    B, T, Hk, dk = q.shape
    _, _, Hv, dv = v.shape
    gate_mode = 1 if w is not None else 0
    if gate_mode == 0 and beta_or_b.shape != (B, T, Hv):
        raise ValueError("scalar gates must be [B,T,Hv]")
    if gate_mode == 1 and beta_or_b.shape != (B, T, Hv, dk):
        raise ValueError("erase gate must be [B,T,Hv,dk]")
    return B, T, Hk, Hv, dk, dv, gate_mode


def recurrent(q, k, v, beta_or_b, w=None, g=None, scale=1.0, state_in=None, nthreads=None):
    """Token-by-token fp64 recurrence.  Returns (o, state_out) as float64."""
    q, k, v, bb, w, g, s0 = map(_f64, (q, k, v, beta_or_b, w, g, state_in))
    B, T, Hk, Hv, dk, dv, mode = _shapes(q, v, bb, w)
    o = np.zeros((B, T, Hv, dv), np.float64)
    s1 = np.zeros((B, Hv, dk, dv), np.float64)
    rc = _load().gdn_ref_recurrent(B, T, Hk, Hv, dk, dv, mode, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(bb), _ptr(w), _ptr(g), float(scale), _ptr(s0),
                                   _ptr(s1), _ptr(o), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, s1


def chunkwise(q, k, v, beta_or_b, w=None, g=None, scale=1.0, state_in=None, chunk=64,
              nthreads=None):
    """Naive chunkwise fp64 form.  Returns (o, state_out) as float64."""
    q, k, v, bb, w, g, s0 = map(_f64, (q, k, v, beta_or_b, w, g, state_in))
    B, T, Hk, Hv, dk, dv, mode = _shapes(q, v, bb, w)
    o = np.zeros((B, T, Hv, dv), np.float64)
    s1 = np.zeros((B, Hv, dk, dv), np.float64)
    rc = _load().gdn_ref_chunkwise(B, T, Hk, Hv, dk, dv, mode, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(bb), _ptr(w), _ptr(g), float(scale), _ptr(s0),
                                   _ptr(s1), _ptr(o), int(chunk), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, s1


def decode(q, k, v, beta_or_b, state, w=None, g=None, scale=1.0, nthreads=None):
    """One decode step.  q, k [N,Hk,dk]; v [N,Hv,dv]; state [N,Hv,dk,dv].

    Returns (o, new_state) as float64; the input array is not modified.
    """
    q, k, v, bb, w, g = map(_f64, (q, k, v, beta_or_b, w, g))
    st = _f64(state).copy()
    N, Hk, dk = q.shape
    _, Hv, dv = v.shape
    mode = 1 if w is not None else 0
    o = np.zeros((N, Hv, dv), np.float64)
    rc = _load().gdn_ref_decode(N, Hk, Hv, dk, dv, mode, _ptr(q), _ptr(k), _ptr(v), _ptr(bb),
                                _ptr(w), _ptr(g), float(scale), _ptr(st), _ptr(o),
                                _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, st


def backward(q, k, v, beta_or_b, d_o, w=None, g=None, scale=1.0, state_in=None,
             d_state_out=None, nthreads=None):
    """Gradients of the token recurrence (reverse mode, fp64).

    Returns a dict with dq, dk [B,T,Hk,dk], dv [B,T,Hv,dv], db (shape of
    beta_or_b), dw (shape of w, or None), dg (shape of beta_or_b, or None when
    g is None) and d_state_in [B,Hv,dk,dv], all float64.  Keeps every state
    of a head, so it is meant for small T.
    """
    q, k, v, bb, w, g, s0, do, dsT = map(_f64, (q, k, v, beta_or_b, w, g, state_in, d_o,
                                                d_state_out))
    B, T, Hk, Hv, dk, dv, mode = _shapes(q, v, bb, w)
    out = {"dq": np.zeros(q.shape), "dk": np.zeros(q.shape), "dv": np.zeros(v.shape),
           "db": np.zeros(bb.shape), "dw": None if w is None else np.zeros(w.shape),
           "dg": None if g is None else np.zeros(bb.shape),
           "d_state_in": np.zeros((B, Hv, dk, dv))}
    rc = _load().gdn_ref_backward(B, T, Hk, Hv, dk, dv, mode, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(bb), _ptr(w), _ptr(g), float(scale), _ptr(s0), _ptr(do),
                                  _ptr(dsT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                  _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dg"]),
                                  _ptr(out["d_state_in"]), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def abi_version():
    return _load().gdn_oracle_abi()
