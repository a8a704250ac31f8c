"""Pins for the CPU oracle, checked against what the pages and mathematics fix.

No GPU is involved.  Each test pins a part of the oracle to something other
than the oracle itself: printed values of a worked example, closed forms,
invariants of the update, and independent formulations of the special cases
the pages name (written here in the page's own orientation, not the oracle's).
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")
rng_global = np.random.default_rng(1234)


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(rng, B, T, Hk, Hv, dk, dv, channel, s0=True, g_scale=1.0):
    q = _unit(rng.standard_normal((B, T, Hk, dk)))
    k = _unit(rng.standard_normal((B, T, Hk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    softplus = lambda x: np.log1p(np.exp(x))
    if channel:
        b = sig(rng.standard_normal((B, T, Hv, dk)))
        w = sig(rng.standard_normal((B, T, Hv, dv)))
        g = -softplus(rng.standard_normal((B, T, Hv, dk))) * g_scale
    else:
        b = sig(rng.standard_normal((B, T, Hv)))
        w = None
        g = -softplus(rng.standard_normal((B, T, Hv))) * g_scale
    S0 = 0.5 * rng.standard_normal((B, Hv, dk, dv)) if s0 else None
    return q, k, v, b, w, g, S0


def _relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------------------
# 1. Worked example with printed outputs ("Gated DeltaNet", §Trois regles).
# ---------------------------------------------------------------------------
def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, b, w, alpha, r1, r2 = line.split()
        rows.append((name, float(b), float(w), float(alpha), float(r1), float(r2)))
    assert len(rows) == 3
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_worked_example_printed_values(row):
    name, bval, wval, alpha, read1, read2 = row
    e = np.eye(3)
    keys = np.stack([e[0], e[1], e[0]])            # k1, k2, k1
    vals = np.array([5.0, 7.0, 9.0])
    T = 3
    k = keys.reshape(1, T, 1, 3)
    v = vals.reshape(1, T, 1, 1)
    b = np.full((1, T, 1, 3), bval)
    w = np.full((1, T, 1, 1), wval)
    g = np.full((1, T, 1, 3), math.log(alpha))
    for qvec, expected in ((e[0], read1), (e[1], read2)):
        q = np.zeros((1, T, 1, 3))
        q[0, T - 1, 0] = qvec                      # read after the third write
        o, S = oracle.recurrent(q, k, v, b, w, g)
        assert o[0, T - 1, 0, 0] == pytest.approx(expected, abs=5e-3)   # printed to 2 decimals
        # the same read through the returned state, S^T q
        assert (S[0, 0].T @ qvec)[0] == pytest.approx(expected, abs=5e-3)
    # The exact values behind the printed ones.
    exact = {"linear": (14.0, 7.0), "global_decay": (10.25, 3.5), "delta": (9.0, 7.0)}[name]
    _, S = oracle.recurrent(np.zeros((1, T, 1, 3)), k, v, b, w, g)
    assert S[0, 0, 0, 0] == pytest.approx(exact[0], rel=1e-15)
    assert S[0, 0, 1, 0] == pytest.approx(exact[1], rel=1e-15)


def test_worked_example_delta_in_scalar_mode():
    """The delta-rule row has b = w = 1, so scalar beta = 1 must give the same."""
    e = np.eye(3)
    k = np.stack([e[0], e[1], e[0]]).reshape(1, 3, 1, 3)
    v = np.array([5.0, 7.0, 9.0]).reshape(1, 3, 1, 1)
    _, S = oracle.recurrent(np.zeros_like(k), k, v, np.ones((1, 3, 1)), None, None)
    assert S[0, 0, :, 0].tolist() == [9.0, 7.0, 0.0]


# ---------------------------------------------------------------------------
# 2. Erase exactness: unit key, b = w = 1 -> reading with k_t returns v_t,
#    whatever the decay ("Gated DeltaNet", §DeltaNet and the parenthetical in
#    §Architecture; holds for any alpha because the read is of the decayed state).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dk,dv", [(5, 7), (16, 16)])
def test_exact_recall_any_decay(dk, dv):
    rng = _rng(7)
    B, T, H = 2, 40, 3
    q, k, v, _, _, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    b = np.ones((B, T, H, dk))
    w = np.ones((B, T, H, dv))
    o, _ = oracle.recurrent(k, k, v, b, w, g, state_in=S0)   # read with q_t = k_t
    assert np.max(np.abs(o - v)) < 1e-12


def test_write_gate_sets_recalled_value():
    """With full erase (b = 1) the read along k_t returns exactly w_t (.) v_t:
    the write gate, not the erase gate, shapes what is stored
    ("Gated DeltaNet-2", Methodologie §1, roles of b_t and w_t)."""
    rng = _rng(8)
    B, T, H, dk, dv = 1, 30, 2, 6, 9
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    b = np.ones_like(b)
    o, _ = oracle.recurrent(k, k, v, b, w, g, state_in=S0)
    assert np.max(np.abs(o - w * v)) < 1e-12


def test_partial_erase_keeps_unerased_part():
    """S_t^T k_t = S_bar^T((1 - b) (.) k_t) + z_t for unit k_t: the erase gate
    removes only the b-weighted part of the old read.  Checked one step at a
    time against the closed form built from the previous state."""
    rng = _rng(9)
    dk, dv = 5, 4
    S = rng.standard_normal((1, 1, dk, dv))
    for _ in range(10):
        k = _unit(rng.standard_normal(dk))
        v = rng.standard_normal(dv)
        b = rng.uniform(0, 1, dk)
        w = rng.uniform(0, 1, dv)
        g = -rng.uniform(0, 2, dk)
        Sbar = np.exp(g)[:, None] * S[0, 0]
        expected = Sbar.T @ ((1 - b) * k) + w * v
        o, S = oracle.decode(k.reshape(1, 1, dk), k.reshape(1, 1, dk), v.reshape(1, 1, dv),
                             b.reshape(1, 1, dk), S, w=w.reshape(1, 1, dv), g=g.reshape(1, 1, dk))
        assert np.max(np.abs(o[0, 0] - expected)) < 1e-12


# ---------------------------------------------------------------------------
# 3. Zero gates keep the state; pure decay has a closed form.
# ---------------------------------------------------------------------------
def test_zero_gates_keep_state():
    rng = _rng(10)
    B, T, H, dk, dv = 2, 33, 2, 8, 6
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    o, S = oracle.recurrent(q, k, v, np.zeros_like(b), np.zeros_like(w), np.zeros_like(g),
                            state_in=S0)
    assert np.array_equal(S, S0)
    expected = np.einsum("bthc,bhcv->bthv", q, S0)
    assert np.max(np.abs(o - expected)) < 1e-13


def test_pure_decay_closed_form():
    """b = w = 0: the state only decays, S_t = Diag(exp(sum_{tau<=t} g)) S_0
    ("Gated DeltaNet", §Mamba-2 with no write; architecture notes page,
    §La recurrence, alpha alone)."""
    rng = _rng(11)
    B, T, H, dk, dv = 1, 20, 3, 7, 5
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    o, S = oracle.recurrent(q, k, v, np.zeros_like(b), np.zeros_like(w), g, state_in=S0)
    G = np.cumsum(g, axis=1)                                    # [B,T,H,dk]
    expected_S = np.exp(G[:, -1])[..., None] * S0
    assert _relerr(S, expected_S) < 1e-13
    expected_o = np.einsum("bthc,bthc,bhcv->bthv", q, np.exp(G), S0)
    assert _relerr(o, expected_o) < 1e-13


def test_alpha_to_zero_leaves_only_current_write():
    """alpha -> 0 wipes the old state: only beta v k^T of this step remains
    ("Gated DeltaNet", §Reunir les deux)."""
    rng = _rng(12)
    B, T, H, dk, dv = 1, 6, 1, 4, 3
    q, k, v, beta, _, _, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=False)
    g = np.full((B, T, H), -200.0)
    _, S = oracle.recurrent(q, k, v, beta, None, g, state_in=S0)
    expected = beta[0, -1, 0] * np.outer(k[0, -1, 0], v[0, -1, 0])
    assert np.max(np.abs(S[0, 0] - expected)) < 1e-15


# ---------------------------------------------------------------------------
# 4. Reductions under gate collapse, against independent formulations written
#    in the orientation the "Gated DeltaNet" notes print (state S' = S^T,
#    d_v x d_k, S' k reads a value, o = S' q).  d_k != d_v catches transposes.
# ---------------------------------------------------------------------------
def _p1_gdn1(q, k, v, beta, alpha, S0T):
    """Gated delta rule as printed in §Reunir les deux:
    S'_t = S'_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T, o_t = S'_t q_t."""
    T, dk = k.shape
    S = S0T.copy()
    I = np.eye(dk)
    out = []
    for t in range(T):
        S = S @ (alpha[t] * (I - beta[t] * np.outer(k[t], k[t]))) + beta[t] * np.outer(v[t], k[t])
        out.append(S @ q[t])
    return np.array(out), S


def _p1_deltanet(q, k, v, beta, S0T):
    """DeltaNet in its read-then-replace form (§DeltaNet): v_old = S' k,
    v_new = beta v + (1 - beta) v_old, S' <- S' - v_old k^T + v_new k^T."""
    S = S0T.copy()
    out = []
    for t in range(k.shape[0]):
        v_old = S @ k[t]
        v_new = beta[t] * v[t] + (1 - beta[t]) * v_old
        S = S - np.outer(v_old, k[t]) + np.outer(v_new, k[t])
        out.append(S @ q[t])
    return np.array(out), S


def _p1_mamba2(q, k, v, alpha, S0T):
    """Decay-only memory of §Mamba-2: S'_t = alpha_t S'_{t-1} + v_t k_t^T."""
    S = S0T.copy()
    out = []
    for t in range(k.shape[0]):
        S = alpha[t] * S + np.outer(v[t], k[t])
        out.append(S @ q[t])
    return np.array(out), S


@pytest.mark.parametrize("mode", ["scalar", "channel_broadcast"])
def test_reduces_to_gated_deltanet(mode):
    rng = _rng(13)
    B, T, H, dk, dv = 1, 25, 1, 6, 4
    q, k, v, beta, _, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=False)
    if mode == "scalar":
        o, S = oracle.recurrent(q, k, v, beta, None, g, state_in=S0)
    else:  # GDN-2 with b = w = beta 1 and alpha = a 1 ("Gated DeltaNet-2", §1)
        bb = np.repeat(beta[..., None], dk, axis=-1)
        ww = np.repeat(beta[..., None], dv, axis=-1)
        gg = np.repeat(g[..., None], dk, axis=-1)
        o, S = oracle.recurrent(q, k, v, bb, ww, gg, state_in=S0)
    o_ref, ST_ref = _p1_gdn1(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0],
                             np.exp(g[0, :, 0]), S0[0, 0].T)
    assert _relerr(o[0, :, 0], o_ref) < 1e-12
    assert _relerr(S[0, 0].T, ST_ref) < 1e-12


def test_reduces_to_deltanet():
    rng = _rng(14)
    B, T, H, dk, dv = 1, 25, 1, 5, 8
    q, k, v, beta, _, _, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=False)
    o, S = oracle.recurrent(q, k, v, beta, None, None, state_in=S0)   # g = NULL: alpha = 1
    o_ref, ST_ref = _p1_deltanet(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0].T)
    assert _relerr(o[0, :, 0], o_ref) < 1e-12
    assert _relerr(S[0, 0].T, ST_ref) < 1e-12


def test_reduces_to_mamba2_and_linear_attention():
    rng = _rng(15)
    B, T, H, dk, dv = 1, 25, 1, 5, 3
    q, k, v, _, _, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=False)
    b0 = np.zeros((B, T, H, dk))
    w1 = np.ones((B, T, H, dv))
    gg = np.repeat(g[..., None], dk, axis=-1)
    o, S = oracle.recurrent(q, k, v, b0, w1, gg, state_in=S0)
    o_ref, ST_ref = _p1_mamba2(q[0, :, 0], k[0, :, 0], v[0, :, 0], np.exp(g[0, :, 0]), S0[0, 0].T)
    assert _relerr(o[0, :, 0], o_ref) < 1e-12
    assert _relerr(S[0, 0].T, ST_ref) < 1e-12
    # linear attention: alpha = 1
    o, S = oracle.recurrent(q, k, v, b0, w1, None, state_in=S0)
    o_ref, ST_ref = _p1_mamba2(q[0, :, 0], k[0, :, 0], v[0, :, 0], np.ones(T), S0[0, 0].T)
    assert _relerr(o[0, :, 0], o_ref) < 1e-12
    assert _relerr(S[0, 0].T, ST_ref) < 1e-12


def test_kda_matrix_form_channel_decay_before_erase():
    """GDN-2 step in the matrix form printed on the "Gated DeltaNet-2" page
    (§1) and the news page: S_t = (I - k (b (.) k)^T) Diag(alpha) S + k (w (.) v)^T.
    Channel-wise alpha makes the order of decay and erase matter; the form puts
    the decay inside, next to S_{t-1}."""
    rng = _rng(16)
    dk, dv, T = 6, 5, 12
    q, k, v, b, w, g, S0 = _rand_inputs(rng, 1, T, 1, 1, dk, dv, channel=True)
    o, S = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    M = S0[0, 0].copy()
    I = np.eye(dk)
    outs = []
    for t in range(T):
        kt, bt, wt, vt = k[0, t, 0], b[0, t, 0], w[0, t, 0], v[0, t, 0]
        M = (I - np.outer(kt, bt * kt)) @ np.diag(np.exp(g[0, t, 0])) @ M + np.outer(kt, wt * vt)
        outs.append(M.T @ q[0, t, 0])
    assert _relerr(S[0, 0], M) < 1e-12
    assert _relerr(o[0, :, 0], np.array(outs)) < 1e-12
    # The other order (erase first, then decay) gives a different state, so the
    # check above does pin the order.
    M2 = S0[0, 0].copy()
    for t in range(T):
        kt, bt, wt, vt = k[0, t, 0], b[0, t, 0], w[0, t, 0], v[0, t, 0]
        M2 = np.diag(np.exp(g[0, t, 0])) @ (I - np.outer(kt, bt * kt)) @ M2 + np.outer(kt, wt * vt)
    assert _relerr(M2, M) > 1e-3


# ---------------------------------------------------------------------------
# 5. The naive chunkwise form reaches the recurrence ("Gated DeltaNet-2", §3;
#    "Gated DeltaNet", §Rendre l'entrainement parallele).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 5, 64, 130])
def test_chunkwise_equals_recurrence(channel, C, T):
    rng = _rng(100 + C + T + int(channel))
    B, Hk, Hv, dk, dv = 1, 1, 2, 5, 7
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, Hk, Hv, dk, dv, channel=channel)
    o_r, S_r = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    o_c, S_c = oracle.chunkwise(q, k, v, b, w, g, state_in=S0, chunk=C)
    assert _relerr(o_c, o_r) < 1e-12
    assert _relerr(S_c, S_r) < 1e-12


def test_chunkwise_strong_decay_no_overflow():
    """Per-token log-decay of -30 (cumulative -1920 over a 64-token chunk): the
    chunkwise form only exponentiates differences G_t - G_s with s <= t."""
    rng = _rng(17)
    q, k, v, b, w, g, S0 = _rand_inputs(rng, 1, 100, 1, 1, 8, 8, channel=True)
    g = np.full_like(g, -30.0)
    o_r, S_r = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    o_c, S_c = oracle.chunkwise(q, k, v, b, w, g, state_in=S0, chunk=64)
    assert np.all(np.isfinite(o_c)) and np.all(np.isfinite(S_c))
    assert _relerr(o_c, o_r) < 1e-12
    assert _relerr(S_c, S_r) < 1e-12


# ---------------------------------------------------------------------------
# 6. Structural identities: chaining, grouping, d_v split, decode.
# ---------------------------------------------------------------------------
def test_chaining_state_in_out():
    rng = _rng(18)
    B, T, H, dk, dv = 2, 50, 2, 6, 5
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    o_full, S_full = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    t1 = 23
    o1, S1 = oracle.recurrent(q[:, :t1], k[:, :t1], v[:, :t1], b[:, :t1], w[:, :t1],
                              g[:, :t1], state_in=S0)
    o2, S2 = oracle.recurrent(q[:, t1:], k[:, t1:], v[:, t1:], b[:, t1:], w[:, t1:],
                              g[:, t1:], state_in=S1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o_full)
    assert np.array_equal(S2, S_full)


def test_grouped_heads_equal_repeated_keys():
    """8 value heads sharing one key head behave as if q, k were copied per
    value head (architecture notes page, §La dissymetrie 16 / 128)."""
    rng = _rng(19)
    B, T, Hk, Hv, dk, dv = 1, 20, 2, 6, 4, 3
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, Hk, Hv, dk, dv, channel=False)
    o_g, S_g = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    rep = Hv // Hk
    qr = np.repeat(q, rep, axis=2)
    kr = np.repeat(k, rep, axis=2)
    o_u, S_u = oracle.recurrent(qr, kr, v, b, w, g, state_in=S0)
    assert np.array_equal(o_g, o_u)
    assert np.array_equal(S_g, S_u)


def test_value_columns_independent():
    rng = _rng(20)
    B, T, H, dk, dv = 1, 30, 2, 5, 8
    q, k, v, b, w, g, S0 = _rand_inputs(rng, B, T, H, H, dk, dv, channel=True)
    o, S = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    cols = slice(2, 6)
    o_s, S_s = oracle.recurrent(q, k, v[..., cols], b, w[..., cols], g,
                                state_in=S0[..., cols].copy())
    assert np.array_equal(o_s, o[..., cols])
    assert np.array_equal(S_s, S[..., cols])


def test_decode_is_one_recurrent_step():
    rng = _rng(21)
    N, Hk, Hv, dk, dv = 3, 2, 4, 6, 5
    q, k, v, b, w, g, S0 = _rand_inputs(rng, N, 1, Hk, Hv, dk, dv, channel=True)
    o_r, S_r = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    o_d, S_d = oracle.decode(q[:, 0], k[:, 0], v[:, 0], b[:, 0], S0, w=w[:, 0], g=g[:, 0])
    assert np.array_equal(o_d, o_r[:, 0])
    assert np.array_equal(S_d, S_r)


def test_scale_argument_scales_output_only():
    rng = _rng(22)
    q, k, v, b, w, g, S0 = _rand_inputs(rng, 1, 10, 1, 1, 4, 4, channel=False)
    o1, S1 = oracle.recurrent(q, k, v, b, w, g, state_in=S0)
    o2, S2 = oracle.recurrent(q, k, v, b, w, g, state_in=S0, scale=0.25)
    assert np.array_equal(S1, S2)
    assert np.max(np.abs(o2 - 0.25 * o1)) < 1e-15


def test_rejects_bad_arguments():
    q = np.zeros((1, 2, 2, 4))
    v = np.zeros((1, 2, 3, 4))   # Hv % Hk != 0
    with pytest.raises(ValueError):
        oracle.recurrent(q, q, v, np.zeros((1, 2, 3)), None, None)
