"""Pins for the block-level CPU oracle (``oracle.layer``): the short causal
convolution, SiLU and L2 norm of the q/k/v branch, the gate activations and
the output norm with its swish gate.

No GPU is involved.  Each test checks the oracle against something other than
itself: closed forms, the convolution's impulse response, textbook and library
routines that compute the same special case (numpy's convolve, torch's CPU
conv1d, softplus, sigmoid, rms_norm), invariants (causality, state carry-over,
unit norm), and the notes' remark that a unit-norm key with beta = 1 erases
exactly.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layer


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# causal convolution
# ----------------------------------------------------------------------------

def test_conv_impulse_response_is_the_reversed_kernel():
    """A unit impulse at token t0 of channel c comes out as w[c, 3], w[c, 2],
    w[c, 1], w[c, 0] at tokens t0 .. t0+3 and nothing anywhere else."""
    rng = _rng(1)
    T, C, t0, c = 12, 5, 4, 3
    w = rng.standard_normal((C, 4))
    x = np.zeros((T, C))
    x[t0, c] = 1.0
    y, _ = layer.causal_conv(x, w)
    expect = np.zeros((T, C))
    for i in range(4):
        expect[t0 + i, c] = w[c, 3 - i]
    assert np.array_equal(y, expect)


def test_conv_matches_numpy_convolve():
    rng = _rng(2)
    T, C = 37, 6
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    y, _ = layer.causal_conv(x, w)
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:T]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


def test_conv_matches_torch_depthwise_conv1d():
    """torch's depthwise conv1d (cross-correlation, kernel 4, left padding 3)
    on the CPU in float64, with the carried state as the padding."""
    rng = _rng(3)
    T, C = 50, 8
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    s0 = rng.standard_normal((1, 3, C))
    y, s1 = layer.causal_conv(x, w, state_in=s0)
    inp = torch.from_numpy(np.concatenate([s0[0], x], 0).T[None])      # [1, C, 3 + T]
    ref = F.conv1d(inp, torch.from_numpy(w)[:, None, :], groups=C)[0].T.numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(s1[0], x[-3:])


def test_conv_is_causal():
    rng = _rng(4)
    T, C = 20, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    y0, _ = layer.causal_conv(x, w)
    x2 = x.copy()
    x2[9:] += rng.standard_normal((T - 9, C))
    y1, _ = layer.causal_conv(x2, w)
    assert np.array_equal(y0[:9], y1[:9])
    assert not np.allclose(y0[9:], y1[9:])


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_conv_state_carries_across_a_split(split):
    """Running a sequence in two calls, the second starting from the first's
    state, gives the one-call result."""
    rng = _rng(5)
    T, C = 11, 3
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    s0 = rng.standard_normal((1, 3, C))
    y, s = layer.causal_conv(x, w, state_in=s0)
    ya, sa = layer.causal_conv(x[:split], w, state_in=s0)
    yb, sb = layer.causal_conv(x[split:], w, state_in=sa)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-14)
    assert np.array_equal(sb, s)


def test_conv_state_of_short_sequences():
    """With fewer than three tokens the new state keeps the tail of the old."""
    rng = _rng(6)
    C = 2
    s0 = rng.standard_normal((1, 3, C))
    x = rng.standard_normal((2, C))
    _, s1 = layer.causal_conv(x[:1], np.ones((C, 4)), state_in=s0)
    assert np.array_equal(s1[0], np.stack([s0[0, 1], s0[0, 2], x[0]]))
    _, s2 = layer.causal_conv(x, np.ones((C, 4)), state_in=s0)
    assert np.array_equal(s2[0], np.stack([s0[0, 2], x[0], x[1]]))
    _, s3 = layer.causal_conv(x[:0], np.ones((C, 4)), state_in=s0)
    assert np.array_equal(s3, s0)


def test_conv_packed_sequences_equal_separate_runs():
    rng = _rng(7)
    lengths = [5, 0, 1, 9, 2]
    C = 3
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = rng.standard_normal((int(cu[-1]), C))
    w = rng.standard_normal((C, 4))
    s0 = rng.standard_normal((len(lengths), 3, C))
    y, s = layer.causal_conv(x, w, N=len(lengths), cu_seqlens=cu, state_in=s0)
    for n in range(len(lengths)):
        yn, sn = layer.causal_conv(x[cu[n]:cu[n + 1]], w, state_in=s0[n:n + 1])
        assert np.array_equal(y[cu[n]:cu[n + 1]], yn)
        assert np.array_equal(s[n], sn[0])


def test_conv_equal_length_batch_equals_packed():
    rng = _rng(8)
    N, T, C = 3, 6, 2
    x = rng.standard_normal((N * T, C))
    w = rng.standard_normal((C, 4))
    y0, s0 = layer.causal_conv(x, w, N=N)
    y1, s1 = layer.causal_conv(x, w, N=N, cu_seqlens=np.arange(N + 1) * T)
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


# ----------------------------------------------------------------------------
# pointwise maps
# ----------------------------------------------------------------------------

def test_silu_closed_forms():
    assert layer.silu(0.0) == 0.0
    # sigmoid(1) = e / (1 + e)
    assert abs(float(layer.silu(1.0)) - math.e / (1.0 + math.e)) < 1e-16
    x = _rng(9).standard_normal(100) * 5
    # x sigmoid(-x) = x - x sigmoid(x)  =>  silu(-x) = silu(x) - x
    np.testing.assert_allclose(layer.silu(-x), layer.silu(x) - x, rtol=1e-12, atol=1e-12)
    assert float(layer.silu(-800.0)) == 0.0 and float(layer.silu(800.0)) == 800.0


def test_sigmoid_softplus_match_torch():
    x = np.concatenate([_rng(10).standard_normal(200) * 8, [-60.0, -30.0, 0.0, 30.0, 60.0]])
    t = torch.from_numpy(x)
    np.testing.assert_allclose(layer.sigmoid(x), torch.sigmoid(t).numpy(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(layer.softplus(x), torch.log1p(torch.exp(t)).numpy(),
                               rtol=1e-14, atol=1e-300)
    assert layer.softplus(0.0) == math.log(2.0)
    # softplus(x) - softplus(-x) = x
    np.testing.assert_allclose(layer.softplus(x) - layer.softplus(-x), x, rtol=1e-12, atol=1e-12)


def test_l2_normalize_unit_norm_and_eps():
    rng = _rng(11)
    x = rng.standard_normal((7, 4, 128)) * 3
    u = layer.l2_normalize(x, 0.0)
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(layer.l2_normalize(5.0 * x, 0.0), u, rtol=1e-13)
    # with eps the norm is n / sqrt(n^2 + eps)
    n = np.linalg.norm(x, axis=-1)
    eps = 0.5
    np.testing.assert_allclose(np.linalg.norm(layer.l2_normalize(x, eps), axis=-1),
                               n / np.sqrt(n * n + eps), rtol=1e-13)
    assert np.array_equal(layer.l2_normalize(np.zeros(8), 1e-6), np.zeros(8))


# ----------------------------------------------------------------------------
# q, k, v branch
# ----------------------------------------------------------------------------

def test_short_conv_block_matches_torch_composition():
    rng = _rng(12)
    Hk, Hv, dk, dv, T, N = 2, 4, 16, 8, 30, 2
    C = 2 * Hk * dk + Hv * dv
    x = rng.standard_normal((N * T, C + 5))          # 5 trailing columns are ignored
    w = rng.standard_normal((C, 4))
    s0 = rng.standard_normal((N, 3, C))
    q, k, v, s1 = layer.short_conv_block(x, w, Hk, Hv, dk, dv, N=N, state_in=s0, eps=1e-6)
    for n in range(N):
        xs = np.concatenate([s0[n], x[n * T:(n + 1) * T, :C]], 0)
        y = F.conv1d(torch.from_numpy(xs.T[None]), torch.from_numpy(w)[:, None, :], groups=C)[0].T
        a = F.silu(y)
        qr = a[:, :Hk * dk].reshape(T, Hk, dk)
        kr = a[:, Hk * dk:2 * Hk * dk].reshape(T, Hk, dk)
        qr = qr / torch.sqrt((qr * qr).sum(-1, keepdim=True) + 1e-6)
        kr = kr / torch.sqrt((kr * kr).sum(-1, keepdim=True) + 1e-6)
        sl = slice(n * T, (n + 1) * T)
        np.testing.assert_allclose(q[sl], qr.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(k[sl], kr.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(v[sl], a[:, 2 * Hk * dk:].reshape(T, Hv, dv).numpy(),
                                   rtol=1e-12, atol=1e-13)
        assert np.array_equal(s1[n], x[(n + 1) * T - 3:(n + 1) * T, :C])


def test_unit_norm_keys_from_the_branch_erase_exactly():
    """The notes' remark: with a key of norm 1 and beta = 1, I - k k^T removes
    the component along k exactly.  Keys from the branch (eps = 0) written with
    beta = 1, alpha = 1 are recalled exactly by the recurrence."""
    rng = _rng(13)
    Hk = Hv = 1
    dk = dv = 16
    T = 6
    C = 2 * dk + dv
    x = rng.standard_normal((T, C))
    q, k, v, _ = layer.short_conv_block(x, rng.standard_normal((C, 4)), Hk, Hv, dk, dv, eps=0.0)
    # overwrite the key of token 3 at token 5 with a new value: recall gives the new value
    k[5] = k[3]
    qq = k.copy()
    beta = np.ones((1, T, Hv))
    o, S = oracle.recurrent(qq[None], k[None], v[None], beta)
    np.testing.assert_allclose(o[0, 5, 0], v[5, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0].T @ k[3, 0], v[5, 0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# gates
# ----------------------------------------------------------------------------

def test_gates_closed_forms():
    # A_log = 0, raw + dt_bias = 0: g = -softplus(0) = -log 2, alpha = 1/2
    g, beta, w = layer.gates(np.zeros((1, 3)), np.zeros((1, 3)))
    assert np.array_equal(g, -math.log(2.0) * np.ones((1, 3)))
    assert np.array_equal(np.exp(g), 0.5 * np.ones((1, 3)))
    assert np.array_equal(beta, 0.5 * np.ones((1, 3))) and w is None
    # dt_bias shifts the raw input; A_log = log 2 doubles the log-decay
    a = _rng(14).standard_normal((4, 3))
    g1, _, _ = layer.gates(a, a, A_log=np.full(3, math.log(2.0)), dt_bias=np.full(3, 0.25))
    g0, _, _ = layer.gates(a + 0.25, a)
    np.testing.assert_allclose(g1, 2.0 * g0, rtol=1e-14)


def test_gates_ranges_and_monotonicity():
    rng = _rng(15)
    a = np.sort(rng.standard_normal(400) * 6)[None]
    b = rng.standard_normal((1, 400)) * 6
    wr = rng.standard_normal((1, 64)) * 6
    g, beta, w = layer.gates(a, b, A_log=np.full(400, 0.3), dt_bias=np.full(400, -0.7), w_raw=wr)
    alpha = np.exp(g)
    assert np.all((alpha > 0) & (alpha < 1))
    assert np.all(np.diff(alpha[0]) < 0)            # larger raw input -> faster decay
    assert np.all((beta > 0) & (beta < 1)) and np.all((w > 0) & (w < 1))
    # torch's softplus and sigmoid on the CPU
    ta = torch.from_numpy(a + (-0.7))
    np.testing.assert_allclose(g, (-math.exp(0.3) * F.softplus(ta)).numpy(), rtol=1e-13)
    np.testing.assert_allclose(w, torch.sigmoid(torch.from_numpy(wr)).numpy(), rtol=1e-14)


# ----------------------------------------------------------------------------
# output norm and gate
# ----------------------------------------------------------------------------

def test_output_gate_closed_forms():
    dv = 8
    eps = 1e-3
    c = 2.0
    o = np.full((1, 1, dv), c)
    weight = np.arange(1, dv + 1, dtype=np.float64)
    z = np.zeros((1, 1, dv))
    assert np.array_equal(layer.output_gate(o, z, weight, eps), np.zeros((1, 1, dv)))
    z = np.full((1, 1, dv), 1.0)
    y = layer.output_gate(o, z, weight, eps)
    np.testing.assert_allclose(y[0, 0], c / math.sqrt(c * c + eps) * weight * math.e / (1 + math.e),
                               rtol=1e-14)


def test_output_gate_matches_torch_rms_norm_and_silu():
    rng = _rng(16)
    rows, Hv, dv = 9, 3, 32
    o = rng.standard_normal((rows, Hv, dv)) * 4
    z = rng.standard_normal((rows, Hv, dv)) * 3
    weight = rng.standard_normal(dv)
    y = layer.output_gate(o, z, weight, eps=1e-5)
    ref = F.rms_norm(torch.from_numpy(o), (dv,), torch.from_numpy(weight), eps=1e-5) \
        * F.silu(torch.from_numpy(z))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)
    # with unit weight and a large z, the gated output has unit RMS per head
    big = np.full_like(z, 40.0)
    y1 = layer.output_gate(o, big, np.ones(dv), eps=0.0) / 40.0
    np.testing.assert_allclose(np.sqrt(np.mean(y1 * y1, -1)), 1.0, rtol=1e-12)
