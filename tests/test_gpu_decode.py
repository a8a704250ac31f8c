"""GPU parity of gdn_decode_step against the CPU oracle (via the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import announce, relerr, to_dev, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402


def _cfg(dk, dv, channel, io, gate, Hk=2, Hv=4, N=3):
    return synth.DecodeConfig("t", N=N, Hk=Hk, Hv=Hv, dk=dk, dv=dv, channel=channel,
                              io_dtype=io, gate_dtype=gate, seed=11)


def _run(inp, with_g=True, scale=1.0):
    st = inp["state"].clone()
    o = gdn.gdn_decode_step(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], st, w=inp["w"],
                            g=inp["g"] if with_g else None, scale=scale)
    torch.cuda.synchronize()
    return o, st


def _ref(inp, with_g=True, scale=1.0):
    c = {k: (None if v is None else v.cpu()) for k, v in inp.items()}
    return oracle.decode(c["q"], c["k"], c["v"], c["beta_or_b"], c["state"], w=c["w"],
                         g=c["g"] if with_g else None, scale=scale)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("io,gate", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)])
def test_decode_small_all_variants(dk, dv, channel, io, gate):
    cfg = _cfg(dk, dv, channel, io, gate)
    inp = to_dev(synth.decode_inputs(cfg))
    announce(f"decode dk={dk} dv={dv} channel={channel} io={io} gate={gate}")
    o, st = _run(inp)
    o_ref, st_ref = _ref(inp)
    tol = tol_for(io)
    assert relerr(o, o_ref) <= tol
    assert relerr(st, st_ref) <= tol


@pytest.mark.parametrize("channel", [True, False])
def test_decode_without_decay_and_with_scale(channel):
    cfg = _cfg(128, 128, channel, torch.float32, torch.float32)
    inp = to_dev(synth.decode_inputs(cfg))
    announce(f"decode g=None scale=0.5 channel={channel}")
    o, st = _run(inp, with_g=False, scale=0.5)
    o_ref, st_ref = _ref(inp, with_g=False, scale=0.5)
    assert relerr(o, o_ref) <= 1e-4
    assert relerr(st, st_ref) <= 1e-4


def test_decode_exact_recall_fp32():
    """b = w = 1 and unit k: reading with q = k returns v (fp32 path)."""
    cfg = _cfg(128, 128, True, torch.float32, torch.float32, Hk=4, Hv=4)
    inp = to_dev(synth.decode_inputs(cfg))
    inp["q"] = inp["k"].clone()
    inp["beta_or_b"] = torch.ones_like(inp["beta_or_b"])
    inp["w"] = torch.ones_like(inp["w"])
    announce("decode exact recall")
    o, _ = _run(inp)
    assert relerr(o, inp["v"]) <= 1e-5


def test_decode_zero_gates_keep_state_bitwise():
    cfg = _cfg(128, 128, True, torch.bfloat16, torch.bfloat16)
    inp = to_dev(synth.decode_inputs(cfg))
    inp["beta_or_b"].zero_(); inp["w"].zero_(); inp["g"].zero_()
    announce("decode zero gates")
    _, st = _run(inp)
    assert torch.equal(st, inp["state"])


def test_decode_full_workload_sampled_heads():
    """256 sequences x 128 value heads (16 key heads), d = 128, channel gates,
    bf16 inputs, 2.1 GB fp32 state updated in place; 48 sampled (n, h) heads
    are checked against the oracle."""
    cfg = synth.CONFIGS["gdn2_decode"]
    inp = synth.decode_inputs(cfg, device="cuda")
    state0 = inp["state"]
    rng = np.random.default_rng(5)
    ns = rng.integers(0, cfg.N, 48)
    hs = rng.integers(0, cfg.Hv, 48)
    sample_state = state0[ns, hs].cpu()
    st = state0  # updated in place
    announce("decode full workload N=256 Hv=128")
    o = gdn.gdn_decode_step(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], st, w=inp["w"],
                            g=inp["g"])
    torch.cuda.synchronize()
    group = cfg.Hv // cfg.Hk
    hk = hs // group
    o_ref, st_ref = oracle.decode(inp["q"][ns, hk].cpu()[:, None], inp["k"][ns, hk].cpu()[:, None],
                                  inp["v"][ns, hs].cpu()[:, None],
                                  inp["beta_or_b"][ns, hs].cpu()[:, None],
                                  sample_state[:, None], w=inp["w"][ns, hs].cpu()[:, None],
                                  g=inp["g"][ns, hs].cpu()[:, None])
    assert relerr(o[ns, hs], o_ref[:, 0]) <= 2e-2
    assert relerr(st[ns, hs], st_ref[:, 0]) <= 2e-2
    # fp32 state arithmetic: far inside the bf16 budget
    assert relerr(st[ns, hs], st_ref[:, 0]) <= 1e-5
