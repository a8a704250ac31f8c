"""GPU parity of gdn_chunk_fwd_gated (the gate activations applied inside the
chunk kernel, reading the raw projections by row stride) against the oracle:
the oracle's gate activations in fp64, then its token recurrence.  Also
against the two-step path (gdn_gates, then gdn_chunk_fwd), which rounds the
activated gates to bf16 in between and so agrees within the bf16 bar."""
import numpy as np
import pytest
import torch

import oracle
from oracle import layer as olayer
from helpers import TOL_BF16, announce, relerr

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402


def _case(channel, B=2, T=130, Hk=2, Hv=4, d=128, seed=3, a_shift=0.0, with_a=True,
          state=True):
    """Inputs with the raw gate projections as column blocks of one wider
    projection output (row stride larger than the columns)."""
    gen = torch.Generator().manual_seed(seed)
    rn = lambda *s: torch.randn(*s, generator=gen)
    q = torch.nn.functional.normalize(rn(B, T, Hk, d), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(rn(B, T, Hk, d), dim=-1).to(torch.bfloat16)
    v = rn(B, T, Hv, d).to(torch.bfloat16)
    n = Hv * d if channel else Hv
    nw = Hv * d if channel else 0
    ld = 2 * n + nw + 8                       # one fused projection row: [a | b | w | pad]
    proj = rn(B * T, ld).to(torch.bfloat16)
    proj[:, :n] += a_shift
    a_raw = proj[:, :n] if with_a else None
    b_raw = proj[:, n:2 * n]
    w_raw = proj[:, 2 * n:2 * n + nw] if channel else None
    A_log = torch.log(torch.empty(n).uniform_(1, 16, generator=gen)).float()
    dt_bias = (-2.0 + 0.5 * rn(n)).float()
    s0 = (0.3 * rn(B, Hv, d, d)).float() if state else None
    return dict(q=q, k=k, v=v, a_raw=a_raw, b_raw=b_raw, w_raw=w_raw, A_log=A_log,
                dt_bias=dt_bias, state_in=s0, B=B, T=T, Hv=Hv, d=d, channel=channel)


def _gpu(c):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    s_out = torch.full((c["B"], c["Hv"], c["d"], c["d"]), float("nan"), device="cuda")
    o, s = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["b_raw"], a_raw=d["a_raw"],
                                   w_raw=d["w_raw"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                                   state_in=d["state_in"], state_out=s_out)
    torch.cuda.synchronize()
    return o, s


def _oracle_gates(c):
    """fp64 gates in the layouts of gdn_chunk_fwd."""
    B, T, Hv, d = c["B"], c["T"], c["Hv"], c["d"]
    a = c["a_raw"] if c["a_raw"] is not None else torch.zeros_like(c["b_raw"])
    g, beta, w = olayer.gates(a.float(), c["b_raw"].float(), c["A_log"], c["dt_bias"],
                              None if c["w_raw"] is None else c["w_raw"].float())
    shape = (B, T, Hv, d) if c["channel"] else (B, T, Hv)
    g = g.reshape(shape) if c["a_raw"] is not None else None
    beta = beta.reshape(shape)
    w = None if w is None else w.reshape(B, T, Hv, d)
    return g, beta, w


def _ref(c):
    g, beta, w = _oracle_gates(c)
    return oracle.recurrent(c["q"], c["k"], c["v"], beta, w=w, g=g, state_in=c["state_in"])


@pytest.mark.parametrize("channel", [True, False])
@pytest.mark.parametrize("with_a", [True, False])
def test_gated_fwd_matches_oracle(channel, with_a):
    announce(f"gated fwd channel={channel} with_a={with_a}")
    c = _case(channel, with_a=with_a)
    o, s = _gpu(c)
    o_ref, s_ref = _ref(c)
    assert relerr(o, o_ref) <= TOL_BF16
    assert relerr(s, s_ref) <= TOL_BF16


@pytest.mark.parametrize("channel", [True, False])
def test_gated_fwd_matches_two_step_path(channel):
    """gdn_gates then gdn_chunk_fwd: the same computation with the activated
    gates rounded to bf16 in between."""
    announce(f"gated fwd vs gdn_gates + gdn_chunk_fwd channel={channel}")
    c = _case(channel, T=257, state=False)
    o, s = _gpu(c)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    B, T, Hv, dd = c["B"], c["T"], c["Hv"], c["d"]
    g, beta, w = gdn.gdn_gates(d["a_raw"], d["b_raw"], Hv, w_raw=d["w_raw"], A_log=d["A_log"],
                               dt_bias=d["dt_bias"], d_k=dd, d_v=dd)
    shape = (B, T, Hv, dd) if channel else (B, T, Hv)
    o2, s2 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], beta.reshape(shape),
                               w=None if w is None else w.reshape(B, T, Hv, dd),
                               g=g.reshape(shape), state_out=torch.empty_like(s))
    torch.cuda.synchronize()
    assert relerr(o, o2) <= TOL_BF16
    assert relerr(s, s2) <= TOL_BF16


@pytest.mark.parametrize("channel", [True, False])
def test_gated_fwd_strong_decay(channel):
    """Decay projections shifted by +6: -exp(A_log) softplus(a + dt_bias)
    reaches about -60 per token, so channel sub-blocks take the floored scan."""
    announce(f"gated fwd strong decay channel={channel}")
    c = _case(channel, a_shift=6.0, T=100)
    o, s = _gpu(c)
    o_ref, s_ref = _ref(c)
    assert relerr(o, o_ref) <= TOL_BF16
    assert relerr(s, s_ref) <= TOL_BF16


@pytest.mark.parametrize("channel", [True, False])
def test_gated_fwd_exact_path(channel):
    """Tokens 16-31 share one key of norm 3: |A| = b |k|^2 there exceeds the
    diagonal inverse's guard, so that sub-block runs the exact token
    recurrence, which applies the activations itself (channel gates: staged
    per wave in LDS)."""
    announce(f"gated fwd exact path channel={channel}")
    c = _case(channel, T=70, Hk=1, Hv=2, B=1)
    k = c["k"].float()
    k[:, 16:32] = 3.0 * k[:, 16:17]
    c["k"] = k.to(torch.bfloat16)
    o, s = _gpu(c)
    o_ref, s_ref = _ref(c)
    assert relerr(o, o_ref) <= TOL_BF16
    assert relerr(s, s_ref) <= TOL_BF16
