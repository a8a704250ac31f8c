"""GPU parity of gdn_chunk_fwd against the CPU oracle (via the C ABI).

Small cases are compared element by element over every output; the full-size
workloads are compared on sampled (sequence, value head) pairs, which the
oracle recomputes one by one from the same input bytes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BF16, TOL_FP32, announce, relerr, to_dev, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402


def _cfg(dk=128, dv=128, channel=True, io=torch.bfloat16, gate=None, B=2, T=130, Hk=2, Hv=4,
         seed=21, state_std=0.5):
    return synth.ChunkConfig("t", B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, channel=channel,
                             io_dtype=io, gate_dtype=io if gate is None else gate, seed=seed,
                             state_std=state_std)


def _gpu(inp, with_g=True, scale=1.0, state_out=True):
    s_out = None
    if state_out:
        B, _, _, dk = inp["q"].shape
        Hv, dv = inp["v"].shape[2], inp["v"].shape[3]
        s_out = torch.full((B, Hv, dk, dv), float("nan"), device="cuda")
    o, s = gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], w=inp["w"],
                             g=inp["g"] if with_g else None, state_in=inp["state_in"],
                             state_out=s_out, scale=scale)
    torch.cuda.synchronize()
    return o, s


def _ref(inp, with_g=True, scale=1.0):
    c = {k: (None if v is None else v.cpu()) for k, v in inp.items()}
    return oracle.recurrent(c["q"], c["k"], c["v"], c["beta_or_b"], c["w"],
                            c["g"] if with_g else None, scale=scale, state_in=c["state_in"])


def _check(inp, tol, with_g=True, scale=1.0, label=""):
    announce(label)
    o, s = _gpu(inp, with_g=with_g, scale=scale)
    o_ref, s_ref = _ref(inp, with_g=with_g, scale=scale)
    eo, es = relerr(o, o_ref), relerr(s, s_ref)
    assert eo <= tol and es <= tol, (label, eo, es)
    return eo, es


# ---------------------------------------------------------------------------
# The small fp32 workload, in full.
# ---------------------------------------------------------------------------
def test_fp32_small_workload():
    cfg = synth.CONFIGS["gdn1_fp32_small"]
    inp = to_dev(synth.chunk_inputs(cfg))
    _check(inp, TOL_FP32, label="gdn1_fp32_small")


# ---------------------------------------------------------------------------
# Variants: head sizes, gate modes, dtypes, ragged tails, grouping.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("io,gate", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)])
def test_variants(dk, dv, channel, io, gate):
    cfg = _cfg(dk=dk, dv=dv, channel=channel, io=io, gate=gate, T=130)
    inp = to_dev(synth.chunk_inputs(cfg))
    _check(inp, tol_for(io), label=f"variant dk={dk} dv={dv} ch={channel} io={io} gate={gate}")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 100, 257])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_ragged_lengths(T, io):
    cfg = _cfg(T=T, io=io, B=1, Hk=1, Hv=2)
    inp = to_dev(synth.chunk_inputs(cfg))
    _check(inp, tol_for(io), label=f"ragged T={T} io={io}")


@pytest.mark.parametrize("channel", [True, False])
def test_deltanet_without_decay(channel):
    cfg = _cfg(channel=channel, io=torch.float32, T=200)
    inp = to_dev(synth.chunk_inputs(cfg))
    _check(inp, TOL_FP32, with_g=False, label=f"g=None ch={channel}")


def test_scale_argument():
    cfg = _cfg(io=torch.float32, T=90)
    inp = to_dev(synth.chunk_inputs(cfg))
    _check(inp, TOL_FP32, scale=0.125, label="scale=0.125")


def test_beta_above_one_not_clamped():
    cfg = _cfg(channel=False, io=torch.float32, T=150)
    inp = to_dev(synth.chunk_inputs(cfg))
    inp["beta_or_b"] = torch.full_like(inp["beta_or_b"], 1.5)
    _check(inp, TOL_FP32, label="beta=1.5")


def test_zero_initial_state_null_pointer():
    cfg = _cfg(io=torch.bfloat16, T=160, state_std=0.0)
    inp = to_dev(synth.chunk_inputs(cfg))
    assert inp["state_in"] is None
    _check(inp, TOL_BF16, label="state_in=NULL")


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_strong_decay_takes_exact_path(io):
    """Log-decay of -30 per token: the factored form would leave fp32, so the
    kernel must switch that chunk to the token-by-token recurrence."""
    cfg = _cfg(io=io, T=150)
    inp = to_dev(synth.chunk_inputs(cfg))
    inp["g"] = torch.full_like(inp["g"], -30.0)
    _check(inp, tol_for(io), label=f"g=-30 io={io}")


def test_mixed_chunks_strong_decay_in_one_chunk_only():
    cfg = _cfg(io=torch.float32, T=192)
    inp = to_dev(synth.chunk_inputs(cfg))
    g = inp["g"].clone()
    g[:, 64:128] = -30.0            # the middle chunk only
    inp["g"] = g
    _check(inp, TOL_FP32, label="middle chunk g=-30")


# ---------------------------------------------------------------------------
# Invariants the pages fix.
# ---------------------------------------------------------------------------
def _worked_example_inputs(rule, dk=64, dv=64):
    """The three-write example of the "Gated DeltaNet" notes (§Trois regles),
    zero-padded to d_k = d_v = 64: keys e1, e2, e1 with values 5, 7, 9."""
    b, w, alpha = {"linear": (0.0, 1.0, 1.0), "global_decay": (0.0, 1.0, 0.5),
                   "delta": (1.0, 1.0, 1.0)}[rule]
    T = 3
    k = torch.zeros(1, T, 1, dk)
    k[0, 0, 0, 0] = k[0, 2, 0, 0] = 1.0
    k[0, 1, 0, 1] = 1.0
    v = torch.zeros(1, T, 1, dv)
    v[0, :, 0, 0] = torch.tensor([5.0, 7.0, 9.0])
    q = torch.zeros(1, T, 1, dk)
    q[0, 2, 0, 0] = 1.0  # read k1 after the third write
    return dict(q=q, k=k, v=v, beta_or_b=torch.full((1, T, 1, dk), b),
                w=torch.full((1, T, 1, dv), w), g=torch.full((1, T, 1, dk), math.log(alpha)),
                state_in=None)


@pytest.mark.parametrize("rule,read1,read2", [("linear", 14.0, 7.0), ("global_decay", 10.25, 3.5),
                                              ("delta", 9.0, 7.0)])
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_worked_example_padded(rule, read1, read2, io):
    inp = _worked_example_inputs(rule)
    inp = {k: (None if v is None else v.to(io).cuda()) for k, v in inp.items()}
    announce(f"worked example {rule} io={io}")
    o, s = _gpu(inp)
    # linear and delta are exact; decay carries the rounding of g = log 0.5
    tol = 0.0 if rule != "global_decay" else (1e-5 if io == torch.float32 else 1e-2)
    assert abs(o[0, 2, 0, 0].item() - read1) <= tol * read1
    assert abs(s[0, 0, 0, 0].item() - read1) <= tol * read1
    assert abs(s[0, 0, 1, 0].item() - read2) <= tol * read2


def test_exact_recall_fp32():
    """b = w = 1 and unit keys: reading with q_t = k_t returns v_t, for any decay."""
    cfg = _cfg(io=torch.float32, T=200, Hk=2, Hv=2)
    inp = to_dev(synth.chunk_inputs(cfg))
    inp["q"] = inp["k"].clone()
    inp["beta_or_b"] = torch.ones_like(inp["beta_or_b"])
    inp["w"] = torch.ones_like(inp["w"])
    announce("exact recall")
    o, _ = _gpu(inp)
    assert relerr(o, inp["v"]) <= 1e-4


def test_zero_gates_keep_state():
    cfg = _cfg(io=torch.bfloat16, T=150)
    inp = to_dev(synth.chunk_inputs(cfg))
    inp["beta_or_b"].zero_(); inp["w"].zero_(); inp["g"].zero_()
    announce("zero gates")
    _, s = _gpu(inp)
    assert torch.equal(s, inp["state_in"])


def test_chaining_two_calls_equals_one():
    cfg = _cfg(io=torch.float32, T=256)
    inp = to_dev(synth.chunk_inputs(cfg))
    announce("chaining")
    o_full, s_full = _gpu(inp)
    t1 = 100
    first = {k: (v[:, :t1].contiguous() if k not in ("state_in",) and v is not None else v)
             for k, v in inp.items()}
    second = {k: (v[:, t1:].contiguous() if k not in ("state_in",) and v is not None else v)
              for k, v in inp.items()}
    o1, s1 = _gpu(first)
    second["state_in"] = s1
    o2, s2 = _gpu(second)
    assert relerr(torch.cat([o1, o2], dim=1), o_full) <= TOL_FP32
    assert relerr(s2, s_full) <= TOL_FP32


def test_state_in_place():
    cfg = _cfg(io=torch.bfloat16, T=100)
    inp = to_dev(synth.chunk_inputs(cfg))
    announce("state in place")
    o_ref, s_ref = _gpu(inp)
    st = inp["state_in"].clone()
    gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], w=inp["w"], g=inp["g"],
                      state_in=st, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(st, s_ref)


def test_zero_tokens_copies_state():
    cfg = _cfg(io=torch.bfloat16, T=0)
    inp = to_dev(synth.chunk_inputs(cfg, T=0))
    out = torch.zeros_like(inp["state_in"])
    announce("T=0")
    gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], w=inp["w"], g=inp["g"],
                      state_in=inp["state_in"], state_out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, inp["state_in"])


def test_deterministic():
    cfg = _cfg(io=torch.bfloat16, T=300)
    inp = to_dev(synth.chunk_inputs(cfg))
    announce("determinism")
    a = _gpu(inp)
    b = _gpu(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_steps_equal_chunk_forward():
    """T single-token decode steps reproduce one chunked call (both are also
    checked against the oracle)."""
    cfg = _cfg(io=torch.bfloat16, T=40, B=2, Hk=2, Hv=4)
    inp = to_dev(synth.chunk_inputs(cfg))
    announce("decode x T vs chunk")
    o_c, s_c = _gpu(inp)
    st = inp["state_in"].clone()
    outs = []
    for t in range(cfg.T):
        outs.append(gdn.gdn_decode_step(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(),
                                        inp["v"][:, t].contiguous(),
                                        inp["beta_or_b"][:, t].contiguous(), st,
                                        w=inp["w"][:, t].contiguous(), g=inp["g"][:, t].contiguous()))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    o_ref, s_ref = _ref(inp)
    assert relerr(o_d, o_ref) <= TOL_BF16 and relerr(st, s_ref) <= TOL_BF16
    assert relerr(o_c, o_d.float()) <= TOL_BF16
    assert relerr(s_c, st) <= TOL_BF16


# ---------------------------------------------------------------------------
# Full-size workloads, sampled heads.
# ---------------------------------------------------------------------------
def _sampled_heads_check(name, n_samples, seed=0):
    cfg = synth.CONFIGS[name]
    inp = synth.chunk_inputs(cfg, device="cuda")
    announce(f"full workload {name}")
    o, s = _gpu(inp)
    rng = np.random.default_rng(seed)
    group = cfg.Hv // cfg.Hk
    pairs = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.Hv))) for _ in range(n_samples)]
    o_err = s_err = 0.0
    o_scale = s_scale = 0.0
    for b, h in pairs:
        hk = h // group
        sub = dict(q=inp["q"][b:b + 1, :, hk:hk + 1], k=inp["k"][b:b + 1, :, hk:hk + 1],
                   v=inp["v"][b:b + 1, :, h:h + 1], beta_or_b=inp["beta_or_b"][b:b + 1, :, h:h + 1],
                   w=None if inp["w"] is None else inp["w"][b:b + 1, :, h:h + 1],
                   g=inp["g"][b:b + 1, :, h:h + 1], state_in=None)
        o_ref, s_ref = _ref(sub)
        og = o[b, :, h].double().cpu().numpy()
        sg = s[b, h].double().cpu().numpy()
        o_err = max(o_err, float(np.max(np.abs(og - o_ref[0, :, 0]))))
        s_err = max(s_err, float(np.max(np.abs(sg - s_ref[0, 0]))))
        o_scale = max(o_scale, float(np.max(np.abs(o_ref))))
        s_scale = max(s_scale, float(np.max(np.abs(s_ref))))
    assert o_err / o_scale <= TOL_BF16, (name, o_err / o_scale)
    assert s_err / s_scale <= TOL_BF16, (name, s_err / s_scale)
    return o_err / o_scale, s_err / s_scale


def test_full_gdn1_bf16_train_sampled():
    _sampled_heads_check("gdn1_bf16_train", 6)


def test_full_gdn2_bf16_train_sampled():
    _sampled_heads_check("gdn2_bf16_train", 6)


def test_full_gdn1_grouped_long_sampled():
    _sampled_heads_check("gdn1_grouped_long", 3)
