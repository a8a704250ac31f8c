"""GPU parity of gdn_chunk_fwd_varlen (packed sequences of different lengths)
against the CPU oracle, and its hand-over to gdn_decode_step.

Each packed sequence must give what the token recurrence gives on that
sequence alone (oracle), and exactly what gdn_chunk_fwd gives on it as a batch
of one (the same kernel arithmetic per sequence and head).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BF16, announce, relerr, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402


def _packed(lengths, channel=True, io=torch.bfloat16, gate=None, Hk=2, Hv=4, dk=128, dv=128,
            seed=31, state_std=0.3):
    """Packed inputs [total_T, H, d] for the given sequence lengths, initial
    states [N, Hv, dk, dv] and the device offsets."""
    total = int(sum(lengths))
    cfg = synth.ChunkConfig("varlen", B=1, T=max(total, 1), Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                            channel=channel, io_dtype=io, gate_dtype=io if gate is None else gate,
                            seed=seed, state_std=state_std)
    inp = synth.chunk_inputs(cfg, device="cpu")
    packed = {}
    for key in ("q", "k", "v", "beta_or_b", "w", "g"):
        t = inp[key]
        packed[key] = None if t is None else t[0, :total].contiguous()
    gen = torch.Generator().manual_seed(seed + 1)
    N = len(lengths)
    s0 = (state_std * torch.randn((N, Hv, dk, dv), generator=gen)).float()
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64)
    return packed, s0, cu


def _dev(d):
    return {k: (None if v is None else v.cuda()) for k, v in d.items()}


def _oracle_seq(packed, s0, a, b, n, with_g=True):
    sub = {k: (None if v is None else v[a:b].unsqueeze(0)) for k, v in packed.items()}
    return oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["beta_or_b"], sub["w"],
                            sub["g"] if with_g else None, state_in=s0[n:n + 1])


LENGTHS = [0, 1, 63, 64, 65, 200, 130, 7]


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("io,gate", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32)])
def test_packed_sequences_match_oracle_per_sequence(channel, io, gate):
    announce(f"varlen channel={channel} io={io}")
    packed, s0, cu = _packed(LENGTHS, channel=channel, io=io, gate=gate)
    d = _dev(packed)
    s_out = torch.full_like(s0, float("nan")).cuda()
    o, _ = gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu.cuda(), w=d["w"],
                                    g=d["g"], state_in=s0.cuda(), state_out=s_out)
    torch.cuda.synchronize()
    tol = tol_for(io)
    for n in range(len(LENGTHS)):
        a, b = int(cu[n]), int(cu[n + 1])
        o_ref, s_ref = _oracle_seq(packed, s0, a, b, n)
        if b > a:
            assert relerr(o[a:b].unsqueeze(0), o_ref) <= tol, (n, "o")
        assert relerr(s_out[n:n + 1], s_ref) <= tol, (n, "state")


def test_more_sequences_than_the_kernel_ranks():
    """300 packed sequences: above the 256 the kernel orders longest first,
    so they run in their given order; every one must still match the oracle."""
    announce("varlen N=300")
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 40, size=300)]
    lengths[123] = 150
    packed, s0, cu = _packed(lengths, channel=True, Hk=1, Hv=2, dk=64, dv=64)
    d = _dev(packed)
    s_out = torch.full_like(s0, float("nan")).cuda()
    o, _ = gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu.cuda(), w=d["w"],
                                    g=d["g"], state_in=s0.cuda(), state_out=s_out)
    torch.cuda.synchronize()
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        o_ref, s_ref = _oracle_seq(packed, s0, a, b, n)
        if b > a:
            assert relerr(o[a:b].unsqueeze(0), o_ref) <= TOL_BF16, (n, "o")
        assert relerr(s_out[n:n + 1], s_ref) <= TOL_BF16, (n, "state")


def test_packed_equals_separate_calls_bitwise():
    announce("varlen vs separate gdn_chunk_fwd calls")
    packed, s0, cu = _packed(LENGTHS, channel=True)
    d = _dev(packed)
    s_out = torch.empty_like(s0).cuda()
    o, _ = gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu.cuda(), w=d["w"],
                                    g=d["g"], state_in=s0.cuda(), state_out=s_out)
    for n in range(len(LENGTHS)):
        a, b = int(cu[n]), int(cu[n + 1])
        s1 = torch.empty_like(s0[n:n + 1]).cuda()
        sub = {k: (None if v is None else v[a:b].unsqueeze(0).contiguous()) for k, v in d.items()}
        o1, _ = gdn.gdn_chunk_fwd(sub["q"], sub["k"], sub["v"], sub["beta_or_b"], w=sub["w"],
                                  g=sub["g"], state_in=s0[n:n + 1].cuda(), state_out=s1)
        torch.cuda.synchronize()
        assert torch.equal(s1, s_out[n:n + 1]), n
        if b > a:
            assert torch.equal(o1[0], o[a:b]), n


def test_empty_sequences_pass_the_state_through():
    announce("varlen empty sequences")
    packed, s0, cu = _packed([0, 5, 0], channel=True)
    d = _dev(packed)
    s_out = torch.full_like(s0, float("nan")).cuda()
    gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu.cuda(), w=d["w"], g=d["g"],
                             state_in=s0.cuda(), state_out=s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_out[0].cpu(), s0[0]) and torch.equal(s_out[2].cpu(), s0[2])


def test_all_sequences_empty_copies_states():
    packed, s0, _ = _packed([3], channel=False)
    d = _dev(packed)
    cu = torch.zeros(4, dtype=torch.int64, device="cuda")
    s_in = torch.randn(3, 4, 128, 128, device="cuda")
    s_out = torch.empty_like(s_in)
    q = d["q"][:0]
    gdn.gdn_chunk_fwd_varlen(q, d["k"][:0], d["v"][:0], d["beta_or_b"][:0], cu, g=d["g"][:0],
                             state_in=s_in, state_out=s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_in, s_out)


def test_malformed_offsets_are_clamped_into_the_tensors():
    """A reversed range is an empty sequence and a range past the end is cut
    at total_T (the kernel clamps; nothing outside the tensors is touched)."""
    announce("varlen malformed offsets")
    packed, s0, _ = _packed([40, 50, 30], channel=True)
    total = 120
    cu = torch.tensor([0, 40, 20, 500], dtype=torch.int64)   # seq 1 reversed, seq 2 overshoots
    d = _dev(packed)
    s_out = torch.full_like(s0, float("nan")).cuda()
    o, _ = gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu.cuda(), w=d["w"],
                                    g=d["g"], state_in=s0.cuda(), state_out=s_out)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle_seq(packed, s0, 0, 40, 0)
    assert relerr(s_out[0:1], s_ref) <= TOL_BF16
    assert torch.equal(s_out[1].cpu(), s0[1])                # reversed: empty
    o_ref, s_ref = _oracle_seq(packed, s0, 20, total, 2)      # [20, 500) cut to [20, 120)
    assert relerr(s_out[2:3], s_ref) <= TOL_BF16
    # rows 20-39 are written by sequences 0 and 2 alike; rows 40+ by 2 only
    assert relerr(o[40:total].unsqueeze(0), o_ref[:, 20:]) <= TOL_BF16


@pytest.mark.parametrize("channel", [True, False])
def test_prefill_hands_over_to_decode(channel):
    """Packed prefill, then one decode step per sequence on the states it left:
    equal to the recurrence over prefill + 1 token."""
    announce(f"varlen prefill -> decode channel={channel}")
    lengths = [17, 64, 100, 1]
    packed, s0, cu = _packed([L + 1 for L in lengths], channel=channel, Hk=2, Hv=8)
    # the prefill is every sequence but its last token; the decode step takes that token
    N = len(lengths)
    last = [int(cu[n + 1]) - 1 for n in range(N)]
    keep = torch.ones(int(cu[-1]), dtype=torch.bool)
    keep[last] = False
    pre = {k: (None if v is None else v[keep].contiguous()) for k, v in packed.items()}
    dec = {k: (None if v is None else v[last].contiguous()) for k, v in packed.items()}
    cu_pre = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64)
    d = _dev(pre)
    state = s0.clone().cuda()
    gdn.gdn_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["beta_or_b"], cu_pre.cuda(), w=d["w"],
                             g=d["g"], state_in=state, state_out=state)
    e = _dev(dec)
    o_dec = gdn.gdn_decode_step(e["q"], e["k"], e["v"], e["beta_or_b"], state, w=e["w"], g=e["g"])
    torch.cuda.synchronize()
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        o_ref, s_ref = _oracle_seq(packed, s0, a, b, n)
        assert relerr(o_dec[n:n + 1].unsqueeze(1), o_ref[:, -1:]) <= TOL_BF16, n
        assert relerr(state[n:n + 1], s_ref) <= TOL_BF16, n
