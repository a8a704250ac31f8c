"""GPU parity of the block operations around the recurrence (gdn_short_conv,
gdn_gates, gdn_output_gate) against the CPU oracle (``oracle.layer``), through
the C ABI, and of the whole block (conv branch -> gates -> chunk forward ->
output gate) against the oracle's composition.

Tolerances are the normwise max-relative errors used for the recurrence:
1e-4 for fp32 inputs and 2e-2 for bf16 inputs.  Conv states are copies of
inputs and are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import announce, relerr, tol_for
from oracle import layer

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402


def _cfg(Hk=2, Hv=4, dk=128, dv=128, channel=True, io=torch.bfloat16, seed=21):
    return synth.BlockConfig("block_case", N=1, T=1, Hk=Hk, Hv=Hv, dk=dk, dv=dv, channel=channel,
                             io_dtype=io, gate_dtype=io, seed=seed)


def _dev(t):
    return None if t is None else t.cuda()


# ----------------------------------------------------------------------------
# short conv branch
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_state", [True, False])
def test_short_conv_equal_length_batch(dk, dv, io, with_state):
    """3 sequences of 300 tokens: several 256-token blocks and a ragged tail;
    x carries the z columns after the branch (row stride > C)."""
    announce(f"short_conv dk={dk} dv={dv} io={io} state={with_state}")
    cfg = _cfg(dk=dk, dv=dv, io=io)
    N, T = 3, 300
    inp = synth.block_inputs(cfg, N=N, T=T, conv_state=with_state)
    C = cfg.conv_channels
    s_out = torch.full((N, 3, C), float("nan"), dtype=io, device="cuda")
    q, k, v, _ = gdn.gdn_short_conv(_dev(inp["x"]), _dev(inp["conv_w"]), cfg.Hk, cfg.Hv, dk, dv,
                                    N=N, conv_state_in=_dev(inp["conv_state"]),
                                    conv_state_out=s_out, eps=1e-6)
    torch.cuda.synchronize()
    rq, rk, rv, rs = layer.short_conv_block(inp["x"], inp["conv_w"], cfg.Hk, cfg.Hv, dk, dv, N=N,
                                            state_in=inp["conv_state"], eps=1e-6)
    tol = tol_for(io)
    assert relerr(q, rq) <= tol and relerr(k, rk) <= tol and relerr(v, rv) <= tol
    assert torch.equal(s_out.cpu().double(), torch.from_numpy(rs))


def test_short_conv_packed_sequences_and_in_place_state():
    """Packed sequences of every length class (empty, shorter than the
    kernel, across block edges) with the conv state updated in place."""
    announce("short_conv varlen in place")
    cfg = _cfg()
    lengths = [0, 1, 2, 3, 5, 255, 256, 257, 100, 0, 4]
    total = sum(lengths)
    inp = synth.block_inputs(cfg, N=1, T=total, conv_state=False)
    C = cfg.conv_channels
    gen = torch.Generator().manual_seed(5)
    s0 = torch.randn((len(lengths), 3, C), generator=gen).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    state = s0.clone().cuda()
    q, k, v, _ = gdn.gdn_short_conv(_dev(inp["x"]), _dev(inp["conv_w"]), cfg.Hk, cfg.Hv, 128, 128,
                                    cu_seqlens=cu.cuda(), conv_state_in=state,
                                    conv_state_out=state)
    torch.cuda.synchronize()
    rq, rk, rv, rs = layer.short_conv_block(inp["x"], inp["conv_w"], cfg.Hk, cfg.Hv, 128, 128,
                                            N=len(lengths), cu_seqlens=cu.numpy(), state_in=s0)
    assert relerr(q, rq) <= 2e-2 and relerr(k, rk) <= 2e-2 and relerr(v, rv) <= 2e-2
    assert torch.equal(state.cpu().double(), torch.from_numpy(rs))


def test_short_conv_decode_steps_match_one_pass():
    """Token-at-a-time steps (one token per sequence, state in place) give
    the one-pass result."""
    announce("short_conv decode steps")
    cfg = _cfg(Hk=1, Hv=2)
    N, T = 5, 7
    inp = synth.block_inputs(cfg, N=N, T=T)
    C = cfg.conv_channels
    x = inp["x"].view(N, T, -1)
    state = inp["conv_state"].clone().cuda()
    w = _dev(inp["conv_w"])
    outs = []
    for t in range(T):
        xt = x[:, t].contiguous().cuda()
        outs.append(gdn.gdn_short_conv(xt, w, 1, 2, 128, 128, N=N, conv_state_in=state,
                                       conv_state_out=state)[:3])
    torch.cuda.synchronize()
    rq, rk, rv, rs = layer.short_conv_block(inp["x"], inp["conv_w"], 1, 2, 128, 128, N=N,
                                            state_in=inp["conv_state"])
    q = torch.stack([o[0] for o in outs], 1).reshape(N * T, 1, 128)
    v = torch.stack([o[2] for o in outs], 1).reshape(N * T, 2, 128)
    assert relerr(q, rq) <= 2e-2 and relerr(v, rv) <= 2e-2
    assert torch.equal(state.cpu().double(), torch.from_numpy(rs))


def test_short_conv_malformed_offsets_stay_in_bounds():
    """Reversed and overshooting offsets: the well-formed sequence is right and
    the kernels touch nothing outside the tensors (outputs are checked to be
    finite; the state of the reversed range passes through)."""
    announce("short_conv malformed offsets")
    cfg = _cfg(Hk=1, Hv=1)
    inp = synth.block_inputs(cfg, N=1, T=120)
    C = cfg.conv_channels
    s0 = torch.randn((3, 3, C), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    cu = torch.tensor([0, 40, 20, 500], dtype=torch.int64)
    s_out = torch.empty_like(s0).cuda()
    q, k, v, _ = gdn.gdn_short_conv(_dev(inp["x"]), _dev(inp["conv_w"]), 1, 1, 128, 128,
                                    cu_seqlens=cu.cuda(), conv_state_in=s0.cuda(),
                                    conv_state_out=s_out)
    torch.cuda.synchronize()
    rq, _, rv, _ = layer.short_conv_block(inp["x"][:40], inp["conv_w"], 1, 1, 128, 128,
                                          state_in=s0[:1])
    assert relerr(q[:40], rq) <= 2e-2 and relerr(v[:40], rv) <= 2e-2
    assert torch.isfinite(q.float()).all() and torch.isfinite(v.float()).all()
    assert torch.equal(s_out[1].cpu(), s0[1])


def test_short_conv_full_size_sampled():
    """The GDN-2 B8 T4096 shape as bench.py launches it (x holds the z columns,
    no carried state): sampled tokens of every sequence, including the first
    three, recomputed by the oracle from their 4-token windows."""
    cfg = synth.BLOCK_CONFIGS["gdn2_block_train"]
    announce(f"short_conv full size {cfg.name}")
    inp = synth.block_inputs(cfg, device="cuda", conv_state=False)
    q, k, v, _ = gdn.gdn_short_conv(inp["x"], inp["conv_w"], cfg.Hk, cfg.Hv, cfg.dk, cfg.dv,
                                    N=cfg.N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    toks = sorted(set([0, 1, 2, 3, 255, 256, cfg.T - 1] + list(rng.integers(0, cfg.T, 24))))
    w = inp["conv_w"].cpu()
    for n in range(cfg.N):
        for t in toks:
            r = n * cfg.T + t
            lo = max(n * cfg.T, r - 3)
            win = inp["x"][lo:r + 1].cpu()
            rq, rk, rv, _ = layer.short_conv_block(win, w, cfg.Hk, cfg.Hv, cfg.dk, cfg.dv)
            assert relerr(q[r], rq[-1]) <= 2e-2, (n, t)
            assert relerr(k[r], rk[-1]) <= 2e-2, (n, t)
            assert relerr(v[r], rv[-1]) <= 2e-2, (n, t)


# ----------------------------------------------------------------------------
# gates
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("io,gdt", [(torch.bfloat16, torch.bfloat16),
                                    (torch.bfloat16, torch.float32),
                                    (torch.float32, torch.float32)])
@pytest.mark.parametrize("params", [True, False])
def test_gates(channel, io, gdt, params):
    announce(f"gates channel={channel} io={io} out={gdt} params={params}")
    cfg = _cfg(Hv=4, dk=64, dv=128, channel=channel, io=io)
    inp = synth.block_inputs(cfg, N=1, T=333)
    # extremes: saturating sigmoid and softplus
    inp["ba"][:4] = torch.tensor([-90.0, -30.0, 30.0, 90.0])[:, None].to(io)
    A = _dev(inp["A_log"]) if params else None
    dt = _dev(inp["dt_bias"]) if params else None
    ba = inp["ba"].cuda()
    n = inp["a_raw"].shape[1]
    g, beta, w = gdn.gdn_gates(ba[:, n:], ba[:, :n], cfg.Hv, w_raw=_dev(inp["w_raw"]), A_log=A,
                               dt_bias=dt, d_k=cfg.dk, d_v=cfg.dv, gate_dtype=gdt)
    torch.cuda.synchronize()
    rg, rb, rw = layer.gates(inp["ba"][:, n:], inp["ba"][:, :n],
                             None if A is None else inp["A_log"],
                             None if dt is None else inp["dt_bias"], inp["w_raw"])
    tol = tol_for(gdt if io == torch.float32 else torch.bfloat16)
    g, beta = g.reshape(rg.shape), beta.reshape(rb.shape)
    # ordinary rows: normwise; the 4 saturating rows: element by element
    assert relerr(g[4:], rg[4:]) <= tol and relerr(beta[4:], rb[4:]) <= tol
    ge = g[:4].double().cpu().numpy()
    assert np.all(np.abs(ge - rg[:4]) <= tol * np.abs(rg[:4]) + 1e-30)
    assert np.all(np.abs(beta[:4].double().cpu().numpy() - rb[:4]) <= tol)
    if channel:
        assert relerr(w.reshape(rw.shape), rw) <= tol
    assert bool((g <= 0).all()) and bool(((beta >= 0) & (beta <= 1)).all())


# ----------------------------------------------------------------------------
# output norm and gate
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("in_place", [False, True])
def test_output_gate(dv, io, in_place):
    announce(f"output_gate dv={dv} io={io} in_place={in_place}")
    cfg = _cfg(Hv=3, dv=dv, io=io)
    inp = synth.block_inputs(cfg, N=1, T=333)           # 999 (token, head) rows: ragged
    o = inp["o"].cuda()
    y = o if in_place else None
    out = gdn.gdn_output_gate(o, inp["z"].cuda(), inp["norm_w"].cuda(), eps=1e-5, y=y)
    torch.cuda.synchronize()
    ref = layer.output_gate(inp["o"], inp["z"].reshape(inp["o"].shape), inp["norm_w"], eps=1e-5)
    assert relerr(out, ref) <= tol_for(io)
    if in_place:
        assert out.data_ptr() == o.data_ptr()


def test_output_gate_full_size_sampled():
    cfg = synth.BLOCK_CONFIGS["gdn2_block_train"]
    announce(f"output_gate full size {cfg.name}")
    inp = synth.block_inputs(cfg, device="cuda", conv_state=False)
    y = gdn.gdn_output_gate(inp["o"], inp["z"], inp["norm_w"])
    torch.cuda.synchronize()
    rows = np.random.default_rng(1).integers(0, cfg.rows, 64)
    rows = np.concatenate([[0, cfg.rows - 1], rows])
    ref = layer.output_gate(inp["o"][rows].cpu(),
                            inp["z"][rows].cpu().reshape(len(rows), cfg.Hv, cfg.dv),
                            inp["norm_w"].cpu())
    assert relerr(y[rows], ref) <= 2e-2


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("channel", [True, False])
def test_block_matches_oracle_composition(channel):
    """x -> short conv branch -> gates -> chunk forward -> output gate, all on
    the GPU, against the oracle's composition of the same steps (the
    recurrence is the token-by-token one)."""
    announce(f"block composition channel={channel}")
    cfg = _cfg(Hk=2, Hv=4, channel=channel)
    N, T = 2, 150
    inp = synth.block_inputs(cfg, N=N, T=T)
    n = inp["a_raw"].shape[1]
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    q, k, v, _ = gdn.gdn_short_conv(d["x"], d["conv_w"], 2, 4, 128, 128, N=N,
                                    conv_state_in=d["conv_state"])
    g, beta, w = gdn.gdn_gates(d["ba"][:, n:], d["ba"][:, :n], 4, w_raw=d["w_raw"],
                               A_log=d["A_log"], dt_bias=d["dt_bias"], d_k=128, d_v=128)
    gs = (N, T, 4, 128) if channel else (N, T, 4)
    o, _ = gdn.gdn_chunk_fwd(q.view(N, T, 2, 128), k.view(N, T, 2, 128), v.view(N, T, 4, 128),
                             beta.view(gs), w=None if w is None else w.view(N, T, 4, 128),
                             g=g.view(gs), scale=128 ** -0.5)
    y = gdn.gdn_output_gate(o.view(N * T, 4, 128), d["z"], d["norm_w"])
    torch.cuda.synchronize()

    rq, rk, rv, _ = layer.short_conv_block(inp["x"], inp["conv_w"], 2, 4, 128, 128, N=N,
                                           state_in=inp["conv_state"])
    rg, rb, rw = layer.gates(inp["ba"][:, n:], inp["ba"][:, :n], inp["A_log"], inp["dt_bias"],
                             inp["w_raw"])
    ro, _ = oracle.recurrent(rq.reshape(N, T, 2, 128), rk.reshape(N, T, 2, 128),
                             rv.reshape(N, T, 4, 128), rb.reshape(gs),
                             None if rw is None else rw.reshape(N, T, 4, 128), rg.reshape(gs),
                             scale=128 ** -0.5)
    ry = layer.output_gate(ro.reshape(N * T, 4, 128), inp["z"].reshape(N * T, 4, 128),
                           inp["norm_w"])
    assert relerr(y, ry) <= 2e-2
