"""GPU parity of gdn_backward (gradients of the recurrence) against the CPU
oracle's reverse-mode pass, through the C ABI.

Both sides see the same input values (bf16 inputs are widened exactly).  The
GPU's matrix products take bf16 operands for bf16 inputs and fp32 operands
for fp32 inputs (state and accumulation in fp32), so the bar is the fp32
tolerance for fp32 inputs and the bf16 one otherwise, on every gradient
tensor (normwise max-relative error, as for the forward).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_FP32, announce, relerr, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402

NAMES = ["dq", "dk", "dv", "db", "dw", "dg", "d_state_in"]


def _case(B, T, Hk, Hv, dk, dv, channel, io, gate=None, seed=41, state_std=0.3):
    cfg = synth.ChunkConfig("bwd", B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, channel=channel,
                            io_dtype=io, gate_dtype=io if gate is None else gate, seed=seed,
                            state_std=state_std)
    inp = synth.chunk_inputs(cfg, device="cpu")
    gen = torch.Generator().manual_seed(seed + 100)
    d_o = torch.randn((B, T, Hv, dv), generator=gen).to(io)
    d_sT = torch.randn((B, Hv, dk, dv), generator=gen)
    return inp, d_o, d_sT


def _run(inp, d_o, d_sT, with_g=True, scale=1.0, use_dsT=True):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    return gdn.gdn_backward(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), w=d["w"],
                            g=d["g"] if with_g else None, state_in=d["state_in"],
                            d_state_out=d_sT.cuda() if use_dsT else None, scale=scale)


def _ref(inp, d_o, d_sT, with_g=True, scale=1.0, use_dsT=True):
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o, w=inp["w"],
                           g=inp["g"] if with_g else None, scale=scale,
                           state_in=inp["state_in"], d_state_out=d_sT if use_dsT else None)


def _compare(got, ref, tol, ctx):
    for n in NAMES:
        if ref[n] is None:
            assert got[n] is None, (ctx, n)
            continue
        e = relerr(got[n], ref[n])
        assert e <= tol, (ctx, n, e)


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("io,gate", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)])
def test_backward_matches_oracle(channel, dk, dv, io, gate):
    announce(f"backward channel={channel} dk={dk} dv={dv} io={io} gate={gate}")
    inp, d_o, d_sT = _case(2, 37, 1, 2, dk, dv, channel, io, gate)
    got = _run(inp, d_o, d_sT, scale=0.8)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT, scale=0.8), tol_for(io), "main")


@pytest.mark.parametrize("T", [1, 3, 4, 5, 15, 16, 17, 64, 100])
def test_backward_ragged_lengths(T):
    """Every position of the last 16-token block."""
    announce(f"backward T={T}")
    inp, d_o, d_sT = _case(1, T, 1, 1, 128, 128, True, torch.float32)
    got = _run(inp, d_o, d_sT)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT), TOL_FP32, T)


@pytest.mark.parametrize("channel", [True, False])
def test_backward_without_decay_state_or_final_gradient(channel):
    announce(f"backward g=None, S0=0, no d_state_out channel={channel}")
    inp, d_o, d_sT = _case(2, 40, 2, 4, 128, 128, channel, torch.float32, state_std=0.0)
    got = _run(inp, d_o, d_sT, with_g=False, use_dsT=False)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT, with_g=False, use_dsT=False), TOL_FP32, "plain")


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("channel", [True, False])
def test_backward_strong_decay(io, channel):
    """Log-decay of -30 per token: with per-channel gates every block is
    outside the range of the factored operands and takes the term-by-term
    path; with scalar gates the decay mask underflows to zero off the
    diagonal.  Both must stay finite and match."""
    announce(f"backward g=-30 channel={channel} io={io}")
    inp, d_o, d_sT = _case(1, 45, 1, 2, 128, 128, channel, io)
    inp["g"] = torch.full_like(inp["g"], -30.0)
    got = _run(inp, d_o, d_sT, scale=0.9)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT, scale=0.9), tol_for(io), "g=-30")


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_backward_mixed_decay_blocks(io):
    """Per-channel gates with a strong decay in some channels of the second
    block only (that block takes the term-by-term path, the others the
    factored one) and a decay of -5 per token elsewhere (near the edge of the
    factored range)."""
    announce(f"backward mixed decay io={io}")
    inp, d_o, d_sT = _case(2, 70, 1, 2, 128, 128, True, io)
    g = torch.full_like(inp["g"], -5.0)
    g[:, 16:32, :, ::7] = -40.0
    inp["g"] = g.to(inp["g"].dtype)
    got = _run(inp, d_o, d_sT)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT), tol_for(io), "mixed")


def test_backward_grouped_heads_sum_dq_dk():
    """Four value heads per key head: dq and dk collect all four."""
    announce("backward grouped heads")
    inp, d_o, d_sT = _case(1, 50, 2, 8, 128, 128, False, torch.bfloat16)
    got = _run(inp, d_o, d_sT)
    torch.cuda.synchronize()
    _compare(got, _ref(inp, d_o, d_sT), 2e-2, "grouped")


def test_backward_chains_over_a_split_sequence():
    """Backward over [0, T) equals the backward of [T1, T) (from the state the
    forward reaches at T1) followed by the backward of [0, T1) with the first
    call's d_state_in as its d_state_out."""
    announce("backward chaining")
    inp, d_o, d_sT = _case(1, 48, 1, 2, 128, 128, True, torch.float32)
    full = _run(inp, d_o, d_sT)
    T1 = 20
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    s1 = torch.empty_like(d["state_in"])
    cut = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
    gdn.gdn_chunk_fwd(cut(d["q"], 0, T1), cut(d["k"], 0, T1), cut(d["v"], 0, T1),
                      cut(d["beta_or_b"], 0, T1), w=cut(d["w"], 0, T1), g=cut(d["g"], 0, T1),
                      state_in=d["state_in"], state_out=s1)
    second = gdn.gdn_backward(cut(d["q"], T1, 48), cut(d["k"], T1, 48), cut(d["v"], T1, 48),
                              cut(d["beta_or_b"], T1, 48), d_o[:, T1:].contiguous().cuda(),
                              w=cut(d["w"], T1, 48), g=cut(d["g"], T1, 48), state_in=s1,
                              d_state_out=d_sT.cuda())
    first = gdn.gdn_backward(cut(d["q"], 0, T1), cut(d["k"], 0, T1), cut(d["v"], 0, T1),
                             cut(d["beta_or_b"], 0, T1), d_o[:, :T1].contiguous().cuda(),
                             w=cut(d["w"], 0, T1), g=cut(d["g"], 0, T1), state_in=d["state_in"],
                             d_state_out=second["d_state_in"])
    torch.cuda.synchronize()
    for n in ["dq", "dk", "dv", "db", "dw", "dg"]:
        joined = torch.cat([first[n], second[n]], 1)
        assert relerr(joined, full[n]) <= 1e-4, n
    assert relerr(first["d_state_in"], full["d_state_in"]) <= 1e-4


def test_backward_is_deterministic_and_in_place_state_gradient():
    announce("backward determinism, in-place d_state")
    inp, d_o, d_sT = _case(2, 33, 1, 2, 128, 128, True, torch.bfloat16)
    a = _run(inp, d_o, d_sT)
    b = _run(inp, d_o, d_sT)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    ds = d_sT.clone().cuda()
    c = gdn.gdn_backward(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), w=d["w"], g=d["g"],
                         state_in=d["state_in"], d_state_out=ds, grads={"d_state_in": ds})
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
        assert torch.equal(a[n], c[n]), n


def test_backward_direct_row_gradients_are_deterministic():
    """Channel gates with one value head per key head: the two 64-column
    workgroups of a head add their row gradients straight into the outputs
    (exactly two addends onto zero, in whichever order they land).  Repeated
    calls, plain and from saved states, are bitwise equal; plain and saved
    agree to the bf16 tolerance."""
    announce("backward direct row gradients: determinism")
    inp, d_o, d_sT = _case(4, 500, 4, 4, 128, 128, True, torch.bfloat16, seed=12)
    runs = [_run(inp, d_o, d_sT) for _ in range(4)]
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    _, _, ws = gdn.gdn_chunk_fwd_save(d["q"], d["k"], d["v"], d["beta_or_b"], w=d["w"], g=d["g"],
                                      state_in=d["state_in"])
    saved = [gdn.gdn_backward_saved(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), ws,
                                    w=d["w"], g=d["g"], state_in=d["state_in"],
                                    d_state_out=d_sT.cuda()) for _ in range(4)]
    torch.cuda.synchronize()
    for n in NAMES:
        for r in runs[1:]:
            assert torch.equal(runs[0][n], r[n]), n
        for r in saved[1:]:
            assert torch.equal(saved[0][n], r[n]), n
        assert relerr(saved[0][n], runs[0][n]) <= 2e-2, n


def test_backward_full_size_sampled_heads():
    """The GDN-2 B8 T4096 H16 d128 shape as bench.py launches it: two (sequence,
    head) pairs recomputed by the oracle on their own."""
    cfg = synth.CONFIGS["gdn2_bf16_train"]
    announce(f"backward full size {cfg.name}")
    inp = synth.chunk_inputs(cfg, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(77)
    d_o = torch.randn((cfg.B, cfg.T, cfg.Hv, cfg.dv), generator=gen, device="cuda").to(cfg.io_dtype)
    got = gdn.gdn_backward(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o, w=inp["w"],
                           g=inp["g"])
    torch.cuda.synchronize()
    for b, h in [(0, 0), (cfg.B - 1, cfg.Hv - 1)]:
        sl = lambda x: x[b:b + 1, :, h:h + 1].cpu()
        ref = oracle.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta_or_b"]),
                              sl(d_o), w=sl(inp["w"]), g=sl(inp["g"]))
        for n in ["dq", "dk", "dv", "db", "dw", "dg"]:
            assert relerr(got[n][b:b + 1, :, h:h + 1], ref[n]) <= 2e-2, (b, h, n)
        assert relerr(got["d_state_in"][b:b + 1, h:h + 1], ref["d_state_in"]) <= 2e-2


# ----------------------------------------------------------------------------
# packed sequences
# ----------------------------------------------------------------------------
VL = [0, 1, 17, 64, 100, 5]


def _packed_case(lengths, channel, io=torch.bfloat16, Hk=1, Hv=2, seed=61):
    total = sum(lengths)
    inp, d_o, _ = _case(1, total, Hk, Hv, 128, 128, channel, io, seed=seed, state_std=0.0)
    packed = {k: (None if v is None else v[0].contiguous()) for k, v in inp.items() if k != "state_in"}
    gen = torch.Generator().manual_seed(seed + 7)
    N = len(lengths)
    s0 = 0.3 * torch.randn((N, Hv, 128, 128), generator=gen)
    dsT = torch.randn((N, Hv, 128, 128), generator=gen)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    return packed, d_o[0].contiguous(), s0, dsT, cu


def _run_packed(packed, d_o, s0, dsT, cu):
    d = {k: (None if v is None else v.cuda()) for k, v in packed.items()}
    return gdn.gdn_backward_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], d_o.cuda(), cu.cuda(),
                                   w=d["w"], g=d["g"], state_in=s0.cuda(), d_state_out=dsT.cuda())


@pytest.mark.parametrize("channel", [True, False])
def test_backward_varlen_matches_oracle_per_sequence(channel):
    announce(f"backward varlen channel={channel}")
    packed, d_o, s0, dsT, cu = _packed_case(VL, channel)
    got = _run_packed(packed, d_o, s0, dsT, cu)
    torch.cuda.synchronize()
    for n in range(len(VL)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            assert torch.equal(got["d_state_in"][n].cpu(), dsT[n]), n
            continue
        sl = lambda x: None if x is None else x[a:b].unsqueeze(0)
        ref = oracle.backward(sl(packed["q"]), sl(packed["k"]), sl(packed["v"]),
                              sl(packed["beta_or_b"]), sl(d_o), w=sl(packed["w"]),
                              g=sl(packed["g"]), state_in=s0[n:n + 1], d_state_out=dsT[n:n + 1])
        for name in ["dq", "dk", "dv", "db", "dw", "dg"]:
            if ref[name] is None:
                continue
            assert relerr(got[name][a:b].unsqueeze(0), ref[name]) <= 2e-2, (n, name)
        assert relerr(got["d_state_in"][n:n + 1], ref["d_state_in"]) <= 2e-2, n


def test_backward_varlen_equals_separate_calls_bitwise():
    announce("backward varlen vs separate calls")
    packed, d_o, s0, dsT, cu = _packed_case(VL, True)
    got = _run_packed(packed, d_o, s0, dsT, cu)
    for n in range(len(VL)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        sub = {k: (None if v is None else v[a:b].unsqueeze(0).contiguous().cuda())
               for k, v in packed.items()}
        one = gdn.gdn_backward(sub["q"], sub["k"], sub["v"], sub["beta_or_b"],
                               d_o[a:b].unsqueeze(0).contiguous().cuda(), w=sub["w"], g=sub["g"],
                               state_in=s0[n:n + 1].cuda(), d_state_out=dsT[n:n + 1].cuda())
        torch.cuda.synchronize()
        for name in ["dq", "dk", "dv", "db", "dw", "dg"]:
            assert torch.equal(one[name][0], got[name][a:b]), (n, name)
        assert torch.equal(one["d_state_in"], got["d_state_in"][n:n + 1]), n
