"""GPU parity of the saved-state training path through the C ABI:
gdn_chunk_fwd_save (the chunk forward, leaving the state entering every
16-token block and every u in the backward's workspace) followed by
gdn_backward_saved (the reverse walk alone).

- The forward's own results (o, final state) are bitwise those of
  gdn_chunk_fwd: saving adds stores, no arithmetic.
- The gradients match the oracle's reverse-mode pass at the tolerance of the
  io type, as gdn_backward's do (the bf16 states the backward reads are the
  forward's, rounded to the operand type, instead of its own rebuild's).
- With fp32 io the forward kernel does not save; the backward's own rebuild
  fills the workspace in a launch of its own, so the gradients are bitwise
  those of gdn_backward.
"""
import pytest
import torch

import oracle
import synth
from helpers import TOL_BF16, announce, relerr, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402

NAMES = ["dq", "dk", "dv", "db", "dw", "dg", "d_state_in"]


def _case(B, T, Hk, Hv, dk, dv, channel, io, gate=None, seed=61):
    cfg = synth.ChunkConfig("saved", B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, channel=channel,
                            io_dtype=io, gate_dtype=io if gate is None else gate, seed=seed,
                            state_std=0.3)
    inp = synth.chunk_inputs(cfg, device="cpu")
    gen = torch.Generator().manual_seed(seed + 7)
    d_o = torch.randn((B, T, Hv, dv), generator=gen).to(io)
    d_sT = torch.randn((B, Hv, dk, dv), generator=gen)
    return inp, d_o, d_sT


def _dev(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def _saved(inp, d_o, d_sT, scale):
    """(o, state_out) of gdn_chunk_fwd_save and the gradients of
    gdn_backward_saved on its workspace."""
    d = _dev(inp)
    B, _, _, dk = d["q"].shape
    Hv, dv = d["v"].shape[2], d["v"].shape[3]
    s_out = torch.full((B, Hv, dk, dv), float("nan"), device="cuda")
    o, s, ws = gdn.gdn_chunk_fwd_save(d["q"], d["k"], d["v"], d["beta_or_b"], w=d["w"],
                                      g=d["g"], state_in=d["state_in"], state_out=s_out,
                                      scale=scale)
    grads = gdn.gdn_backward_saved(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), ws,
                                   w=d["w"], g=d["g"], state_in=d["state_in"],
                                   d_state_out=d_sT.cuda(), scale=scale)
    torch.cuda.synchronize()
    return o, s, grads


def _plain(inp, d_o, d_sT, scale):
    d = _dev(inp)
    o, s = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["beta_or_b"], w=d["w"], g=d["g"],
                             state_in=d["state_in"],
                             state_out=torch.empty_like(d["state_in"]), scale=scale)
    grads = gdn.gdn_backward(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), w=d["w"],
                             g=d["g"], state_in=d["state_in"], d_state_out=d_sT.cuda(),
                             scale=scale)
    torch.cuda.synchronize()
    return o, s, grads


def _ref(inp, d_o, d_sT, scale):
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o, w=inp["w"],
                           g=inp["g"], scale=scale, state_in=inp["state_in"], d_state_out=d_sT)


def _check(inp, d_o, d_sT, io, ctx, scale=0.9):
    announce(f"saved {ctx}")
    o, s, got = _saved(inp, d_o, d_sT, scale)
    o_p, s_p, plain = _plain(inp, d_o, d_sT, scale)
    assert torch.equal(o, o_p), ctx
    assert torch.equal(s, s_p), ctx
    ref = _ref(inp, d_o, d_sT, scale)
    for n in NAMES:
        if ref[n] is None:
            assert got[n] is None, (ctx, n)
            continue
        assert torch.isfinite(got[n]).all(), (ctx, n)
        e = relerr(got[n], ref[n])
        assert e <= tol_for(io), (ctx, n, e)
        if io == torch.float32:
            assert torch.equal(got[n], plain[n]), (ctx, n)
    return got


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("Hk,Hv", [(2, 2), (1, 2)])
def test_saved_bf16_matches_oracle(channel, dk, dv, Hk, Hv):
    inp, d_o, d_sT = _case(2, 100, Hk, Hv, dk, dv, channel, torch.bfloat16)
    _check(inp, d_o, d_sT, torch.bfloat16, f"ch={channel} dk={dk} dv={dv} H={Hk}/{Hv}")


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("io,gate", [(torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)])
def test_saved_other_dtypes(channel, io, gate):
    inp, d_o, d_sT = _case(2, 70, 2, 2, 128, 128, channel, io, gate)
    _check(inp, d_o, d_sT, io, f"ch={channel} io={io} gate={gate}")


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130])
def test_saved_ragged_lengths(T):
    """Every kind of last block and chunk: the forward saves only blocks that
    hold tokens, and only their tokens' u."""
    inp, d_o, d_sT = _case(1, T, 1, 1, 128, 128, True, torch.bfloat16, seed=T)
    _check(inp, d_o, d_sT, torch.bfloat16, f"T={T}")


# Sub-block kinds of the chunk kernel with channel gates (16 tokens each;
# F = factored, D = floored decays, S = exact token path): the saved states
# and u must come from every kind.  D is a log-decay of -30 per token, S a
# rising state (g = +1 per token) followed by as much decay.  (Scalar gates
# leave the factored path only for a rise past 2^110 over 16 tokens, where
# the gradients themselves leave fp32.)
_PATTERN = "FSFD" + "DFFS" + "FDSF"


def test_saved_from_every_sub_block_kind():
    T = 16 * len(_PATTERN) - 5
    inp, d_o, d_sT = _case(2, T, 1, 1, 128, 128, True, torch.bfloat16, seed=5)
    g = inp["g"].clone()
    for sb, c in enumerate(_PATTERN):
        lo, hi = 16 * sb, min(16 * sb + 16, T)
        if c == "D":
            g[:, lo:hi] = -30.0
        elif c == "S":
            g[:, lo:hi] = 1.0
            if hi < T:
                g[:, hi:min(hi + 16, T)] = -1.0
    inp["g"] = g.to(inp["g"].dtype)
    _check(inp, d_o, d_sT, torch.bfloat16, f"pattern {_PATTERN}")


def test_saved_full_shape_tokens_per_block():
    """GDN-2 at the training shape's head count and a long sequence (B 1,
    T 2048, H 16): the saved path and gdn_backward agree to the bf16
    tolerance on every gradient, sequence-wide (no oracle at this size)."""
    inp, d_o, d_sT = _case(1, 2048, 16, 16, 128, 128, True, torch.bfloat16, seed=9)
    announce("saved vs backward B1 T2048 H16")
    _, _, got = _saved(inp, d_o, d_sT, 1.0)
    _, _, plain = _plain(inp, d_o, d_sT, 1.0)
    for n in NAMES:
        e = relerr(got[n], plain[n])
        assert e <= TOL_BF16, (n, e)


def test_saved_rejects_a_short_workspace():
    inp, d_o, d_sT = _case(1, 40, 1, 1, 128, 128, True, torch.bfloat16)
    d = _dev(inp)
    need = gdn.gdn_backward_workspace_size(d["q"], d["v"], d["beta_or_b"], d["w"])
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_chunk_fwd_save(d["q"], d["k"], d["v"], d["beta_or_b"], w=d["w"], g=d["g"],
                               workspace=short)
    assert ei.value.status == gdn.GDN_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# Packed sequences: gdn_chunk_fwd_varlen_save + gdn_backward_varlen_saved.
# ---------------------------------------------------------------------------
VL = [0, 1, 17, 64, 100, 5, 130]   # empty, single-token, ragged, whole and multi-chunk


def _packed_case(lengths, channel, io, Hk, Hv, seed=71):
    total = sum(lengths)
    inp, d_o, _ = _case(1, total, Hk, Hv, 128, 128, channel, io, seed=seed)
    packed = {k: (None if v is None else v[0].contiguous()) for k, v in inp.items()
              if k != "state_in"}
    gen = torch.Generator().manual_seed(seed + 3)
    N = len(lengths)
    s0 = 0.3 * torch.randn((N, Hv, 128, 128), generator=gen)
    dsT = torch.randn((N, Hv, 128, 128), generator=gen)
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int64)
    return packed, d_o[0].contiguous(), s0, dsT, cu


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("io,Hk,Hv", [(torch.bfloat16, 2, 2), (torch.bfloat16, 1, 2),
                                      (torch.float32, 2, 2)])
def test_saved_packed_sequences(channel, io, Hk, Hv):
    """Per sequence against the oracle; the forward's o and final states
    bitwise those of gdn_chunk_fwd_varlen (fp32: the gradients bitwise those
    of gdn_backward_varlen)."""
    announce(f"saved packed ch={channel} io={io} H={Hk}/{Hv}")
    packed, d_o, s0, dsT, cu = _packed_case(VL, channel, io, Hk, Hv)
    d = _dev(packed)
    cud, s0d, dsd, dod = cu.cuda(), s0.cuda(), dsT.cuda(), d_o.cuda()
    o_s, s_s, ws = gdn.gdn_chunk_fwd_varlen_save(d["q"], d["k"], d["v"], d["beta_or_b"], cud,
                                                 w=d["w"], g=d["g"], state_in=s0d,
                                                 state_out=torch.empty_like(s0d))
    got = gdn.gdn_backward_varlen_saved(d["q"], d["k"], d["v"], d["beta_or_b"], dod, cud, ws,
                                        w=d["w"], g=d["g"], state_in=s0d, d_state_out=dsd)
    o_p, s_p = gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cud, w=d["w"],
                                        g=d["g"], state_in=s0d, state_out=torch.empty_like(s0d))
    plain = gdn.gdn_backward_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], dod, cud, w=d["w"],
                                    g=d["g"], state_in=s0d, d_state_out=dsd)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_p) and torch.equal(s_s, s_p)
    tol = tol_for(io)
    for n in range(len(VL)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:   # an empty sequence passes its state gradient through
            assert torch.equal(got["d_state_in"][n].cpu(), dsT[n]), n
            continue
        sl = lambda x: None if x is None else x[a:b].unsqueeze(0)
        ref = oracle.backward(sl(packed["q"]), sl(packed["k"]), sl(packed["v"]),
                              sl(packed["beta_or_b"]), sl(d_o), w=sl(packed["w"]),
                              g=sl(packed["g"]), state_in=s0[n:n + 1], d_state_out=dsT[n:n + 1])
        for name in ["dq", "dk", "dv", "db", "dw", "dg"]:
            if ref[name] is None:
                continue
            e = relerr(got[name][a:b].unsqueeze(0), ref[name])
            assert e <= tol, (n, name, e)
        assert relerr(got["d_state_in"][n:n + 1], ref["d_state_in"]) <= tol, n
    if io == torch.float32:
        for name in NAMES:
            if got[name] is not None:
                assert torch.equal(got[name], plain[name]), name
