"""CPU oracle for the operations around the recurrence in a Gated DeltaNet
block -- TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
use it; the product library never does).

Plain numpy in float64.  Every input is converted to float64 exactly, so the
oracle sees the values handed to the GPU.

The block is described by the notes page "Gated DeltaNet" (docsaid.org),
§Architecture et versions hybrides and its Figure 1 (right-hand block), and by
the architecture notes page "Gated DeltaNet" (mkdocs.reaper.mx), §La
convolution causale and §La porte de sortie:

  * q, k and v each go through a short causal convolution and SiLU; q and k
    are then L2-normalised (per head).                     -> short_conv_block
  * alpha and beta come from a plain projection; alpha follows the Mamba-2
    parameterisation.                                       -> gates
  * the recurrence output is normalised, then multiplied by swish(z), the
    output-gate branch (swish(x) = x sigmoid(x)).           -> output_gate

Readings where the pages leave a step open (each is stated again where it is
used):
  * convolution: depthwise, kernel 4, no bias (the architecture notes count
    exactly 4 parameters per channel); tap 3 multiplies the current token and
    tap 0 the token three back; before a sequence's first token the window
    holds the carried conv state (the 3 previous inputs) or zeros.
  * L2 norm: x / sqrt(sum(x^2) + eps) over the d_k channels of a head.
  * beta = sigmoid(raw)   (the pages put beta in ]0,1[);
    Mamba-2 decay: g = log(alpha) = -exp(A_log) * softplus(raw + dt_bias),
    so alpha = exp(g) is in ]0,1[ (the pages put alpha in ]0,1[).  In GDN-2
    mode the same maps apply channel by channel, and the write gate is
    w = sigmoid(raw) (the GDN-2 gates lie in [0,1]).
  * output norm: RMS norm over the d_v channels of each value head, with one
    weight vector of length d_v shared by all heads (the architecture notes
    count 128 = d_v normalisation parameters per layer):
    y = o / sqrt(mean(o^2) + eps) * weight * swish(z).
"""
from __future__ import annotations

import numpy as np

KERNEL = 4


def _f64(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(x):
    """SiLU (= swish): x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def softplus(x):
    """log(1 + e^x), written so that it neither overflows nor loses small values."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def l2_normalize(x, eps):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _ranges(total_T, N, cu_seqlens):
    """[start, end) of every sequence: N equal sequences, or the packed offsets
    (each range clamped into [0, total_T], a reversed range is empty)."""
    if cu_seqlens is None:
        if N == 0:
            return []
        T = total_T // N
        return [(n * T, (n + 1) * T) for n in range(N)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    out = []
    for n in range(N):
        a0 = min(max(cu[n], 0), total_T)
        a1 = min(max(cu[n + 1], a0), total_T)
        out.append((a0, a1))
    return out


def causal_conv(x, weight, N=1, cu_seqlens=None, state_in=None):
    """Depthwise causal convolution of kernel 4 along the token axis of every
    sequence (architecture notes "Gated DeltaNet", §La convolution causale: the
    output at a token combines that token's input with the inputs of the
    three tokens before it).

    x          [total_T, C]  the packed inputs of N sequences
    weight     [C, 4]        tap 3 multiplies the current token
    state_in   [N, 3, C]     inputs before each sequence's first token, oldest
                             first; None = zeros
    Returns (y [total_T, C], state_out [N, 3, C]) with state_out[n] the last
    three inputs of sequence n (taken from state_in where the sequence is
    shorter than three tokens).
    """
    x = _f64(x)
    weight = _f64(weight)
    total_T, C = x.shape
    assert weight.shape == (C, KERNEL)
    s_in = np.zeros((N, KERNEL - 1, C)) if state_in is None else _f64(state_in)
    y = np.zeros_like(x)
    s_out = np.zeros((N, KERNEL - 1, C))
    for n, (a, b) in enumerate(_ranges(total_T, N, cu_seqlens)):
        # the sequence's inputs with its carried history in front
        hist = np.concatenate([s_in[n], x[a:b]], axis=0)       # [3 + L, C]
        L = b - a
        for t in range(L):
            acc = np.zeros(C)
            for j in range(KERNEL):
                acc += weight[:, j] * hist[t + j]                # hist[t + 3] is token t
            y[a + t] = acc
        s_out[n] = hist[L:L + KERNEL - 1]
    return y, s_out


def short_conv_block(x, weight, H_k, H_v, d_k, d_v, N=1, cu_seqlens=None, state_in=None,
                     eps=1e-6):
    """The q, k, v branch of the block (notes "Gated DeltaNet", Figure 1):
    causal conv, SiLU, then a per-head L2 norm for q and k.

    x  [total_T, C]: columns [0, H_k d_k) are q, the next H_k d_k are k, the
       next H_v d_v are v (extra trailing columns, e.g. the z branch, are
       ignored).
    Returns (q [total_T, H_k, d_k], k [total_T, H_k, d_k], v [total_T, H_v, d_v],
    conv state_out [N, 3, C]).
    """
    x = _f64(x)
    cq = H_k * d_k
    C = 2 * cq + H_v * d_v
    y, s_out = causal_conv(x[:, :C], weight, N, cu_seqlens, state_in)
    a = silu(y)
    T = x.shape[0]
    q = l2_normalize(a[:, :cq].reshape(T, H_k, d_k), eps)
    k = l2_normalize(a[:, cq:2 * cq].reshape(T, H_k, d_k), eps)
    v = a[:, 2 * cq:C].reshape(T, H_v, d_v)
    return q, k, v, s_out


def gates(a_raw, b_raw, A_log=None, dt_bias=None, w_raw=None):
    """Gate activations (notes "Gated DeltaNet", §Architecture: alpha with the
    Mamba-2 parameterisation; architecture notes: alpha and beta in ]0,1[).

    a_raw, b_raw  [rows, n]   projections for the decay and the erase/write rate
    A_log, dt_bias [n]        per-column parameters (None = 0)
    w_raw         [rows, m]   GDN-2 write-gate projection, or None
    Returns (g = log(alpha) [rows, n], beta_or_b [rows, n], w [rows, m] or None).
    """
    a_raw = _f64(a_raw)
    b_raw = _f64(b_raw)
    n = a_raw.shape[-1]
    A_log = np.zeros(n) if A_log is None else _f64(A_log)
    dt_bias = np.zeros(n) if dt_bias is None else _f64(dt_bias)
    g = -np.exp(A_log) * softplus(a_raw + dt_bias)
    beta = sigmoid(b_raw)
    w = None if w_raw is None else sigmoid(_f64(w_raw))
    return g, beta, w


def output_gate(o, z, weight, eps=1e-6):
    """Output normalisation and gate (notes "Gated DeltaNet", Figure 1: the
    output is normalised, then gated; architecture notes §La porte de sortie:
    y = o (.) swish(z)).

    o       [rows, H_v, d_v]
    z       [rows, H_v, d_v]
    weight  [d_v]            shared by all heads
    """
    o = _f64(o)
    z = _f64(z)
    weight = _f64(weight)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * weight * silu(z)
