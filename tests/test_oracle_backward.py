"""Pins for the oracle's backward pass (``oracle.backward``).

No GPU is involved.  The gradients are checked against central finite
differences of the forward oracle (``oracle.recurrent``) -- element by element
on a tiny case, and as directional derivatives along random directions on
larger ones -- and against a closed form for the state gradient when the
erase and write gates are zero.  The loss is
L = sum(o * d_o) + sum(S_T * d_state_out), so dL/dx is what the backward
returns for upstream gradients d_o and d_state_out.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, Hk, Hv, dk, dv, channel, with_g=True, s0=True):
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    d = {"q": unit(rng.standard_normal((B, T, Hk, dk))),
         "k": unit(rng.standard_normal((B, T, Hk, dk))),
         "v": rng.standard_normal((B, T, Hv, dv))}
    gs = (B, T, Hv, dk) if channel else (B, T, Hv)
    d["beta_or_b"] = sig(rng.standard_normal(gs))
    d["w"] = sig(rng.standard_normal((B, T, Hv, dv))) if channel else None
    d["g"] = -0.3 * np.log1p(np.exp(rng.standard_normal(gs))) if with_g else None
    d["state_in"] = 0.5 * rng.standard_normal((B, Hv, dk, dv)) if s0 else None
    return d


def _loss(d, d_o, d_sT, scale):
    o, sT = oracle.recurrent(d["q"], d["k"], d["v"], d["beta_or_b"], d["w"], d["g"],
                             scale=scale, state_in=d["state_in"], nthreads=1)
    return float(np.sum(o * d_o) + (0.0 if d_sT is None else np.sum(sT * d_sT)))


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "beta_or_b": "db", "w": "dw", "g": "dg",
           "state_in": "d_state_in"}


def _grads(d, d_o, d_sT, scale):
    return oracle.backward(d["q"], d["k"], d["v"], d["beta_or_b"], d_o, w=d["w"], g=d["g"],
                           scale=scale, state_in=d["state_in"], d_state_out=d_sT, nthreads=1)


@pytest.mark.parametrize("channel", [True, False])
def test_every_gradient_element_matches_finite_differences(channel):
    rng = np.random.default_rng(101)
    B, T, Hk, Hv, dk, dv = 1, 3, 1, 2, 2, 2
    d = _inputs(rng, B, T, Hk, Hv, dk, dv, channel)
    d_o = rng.standard_normal((B, T, Hv, dv))
    d_sT = rng.standard_normal((B, Hv, dk, dv))
    scale = 0.7
    grads = _grads(d, d_o, d_sT, scale)
    h = 1e-6
    for name, gname in GRAD_OF.items():
        x = d[name]
        if x is None:
            continue
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(d, d_o, d_sT, scale)
            x[idx] = old - h
            lm = _loss(d, d_o, d_sT, scale)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[gname], fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("channel,with_g,s0,dsT", [
    (True, True, True, True), (True, False, False, False), (False, True, True, True),
    (False, False, True, False)])
def test_directional_derivatives_match_finite_differences(channel, with_g, s0, dsT):
    """Grouped heads (2 value heads per key head), two sequences, T = 9:
    <dL/dx, delta> equals the central difference along a random delta, for
    every input tensor."""
    rng = np.random.default_rng(202)
    B, T, Hk, Hv, dk, dv = 2, 9, 2, 4, 5, 3
    d = _inputs(rng, B, T, Hk, Hv, dk, dv, channel, with_g=with_g, s0=s0)
    d_o = rng.standard_normal((B, T, Hv, dv))
    d_sT = rng.standard_normal((B, Hv, dk, dv)) if dsT else None
    scale = 1.3
    grads = _grads(d, d_o, d_sT, scale)
    h = 1e-6
    for name, gname in GRAD_OF.items():
        x = d[name]
        if x is None:
            continue
        for _ in range(3):
            delta = rng.standard_normal(x.shape)
            d[name] = x + h * delta
            lp = _loss(d, d_o, d_sT, scale)
            d[name] = x - h * delta
            lm = _loss(d, d_o, d_sT, scale)
            d[name] = x
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grads[gname] * delta))
            assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, an, fd)
    if not s0:
        assert grads["dg"] is None or grads["dg"].shape == d["beta_or_b"].shape


def test_state_gradient_closed_form_under_zero_writes():
    """b = w = 0: P_{t+1} = Diag(alpha_t) P_t, o_t = scale P_{t+1}^T q_t, so
    dL/dP_0 = Diag(prod_t alpha_t) d_state_out
            + sum_t scale Diag(prod_{s<=t} alpha_s) q_t d_o_t^T."""
    rng = np.random.default_rng(303)
    B, T, Hk, Hv, dk, dv = 1, 6, 1, 1, 4, 3
    d = _inputs(rng, B, T, Hk, Hv, dk, dv, channel=True)
    d["beta_or_b"][:] = 0.0
    d["w"][:] = 0.0
    d_o = rng.standard_normal((B, T, Hv, dv))
    d_sT = rng.standard_normal((B, Hv, dk, dv))
    scale = 0.9
    grads = _grads(d, d_o, d_sT, scale)
    alpha = np.exp(d["g"][0, :, 0])                       # [T, dk]
    expect = np.prod(alpha, 0)[:, None] * d_sT[0, 0]
    for t in range(T):
        cum = np.prod(alpha[:t + 1], 0)
        expect += scale * cum[:, None] * np.outer(d["q"][0, t, 0], d_o[0, t, 0])
    np.testing.assert_allclose(grads["d_state_in"][0, 0], expect, rtol=1e-12, atol=1e-13)
    # w = 0: the value gradient vanishes (dv = w * du)
    assert np.array_equal(grads["dv"], np.zeros_like(grads["dv"]))


def test_rejects_bad_arguments():
    rng = np.random.default_rng(1)
    d = _inputs(rng, 1, 2, 1, 1, 2, 2, channel=False, with_g=False)
    with pytest.raises(ValueError):   # dg requested without g is not possible; w in scalar mode
        oracle.backward(d["q"], d["k"], d["v"], d["beta_or_b"], np.zeros((1, 2, 1, 2)),
                        w=np.zeros((1, 2, 1, 3)))
