"""gdn_backward_noalloc (the backward on the library's static workspace) against
gdn_backward (caller workspace), through the C ABI: the same gradients on two
calls in a row, the second on a smaller input, so that the second call runs
on a workspace the first one left filled.  Bar: the tolerance of the inputs'
precision on every gradient (the two entry points run the same kernels).
"""
import pytest
import torch

import synth
from helpers import announce, relerr, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd as gdn  # noqa: E402

NAMES = ["dq", "dk", "dv", "db", "dw", "dg", "d_state_in"]


def _inputs(B, T, H, d, channel, io, seed):
    cfg = synth.ChunkConfig("noalloc", B=B, T=T, Hk=H, Hv=H, dk=d, dv=d, channel=channel,
                            io_dtype=io, gate_dtype=io, seed=seed, state_std=0.3)
    inp = {k: (None if v is None else v.cuda()) for k, v in synth.chunk_inputs(cfg, device="cpu").items()}
    gen = torch.Generator().manual_seed(seed + 7)
    d_o = torch.randn((B, T, H, d), generator=gen).to(io).cuda()
    d_sT = torch.randn((B, H, d, d), generator=gen).cuda()
    return inp, d_o, d_sT


def _both(inp, d_o, d_sT):
    args = (inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o)
    kw = dict(w=inp["w"], g=inp["g"], state_in=inp["state_in"], d_state_out=d_sT, scale=0.9)
    ref = gdn.gdn_backward(*args, **kw)
    got = gdn.gdn_backward_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("channel,io", [(True, torch.bfloat16), (False, torch.float32)])
def test_noalloc_matches_backward_on_two_calls(channel, io):
    for call, (B, T, H, d) in enumerate([(2, 150, 2, 128), (1, 37, 1, 64)]):
        announce(f"noalloc call={call} B={B} T={T} H={H} d={d} channel={channel} io={io}")
        inp, d_o, d_sT = _inputs(B, T, H, d, channel, io, seed=90 + call)
        got, ref = _both(inp, d_o, d_sT)
        for n in NAMES:
            if ref[n] is None:
                assert got[n] is None, (call, n)
                continue
            assert torch.isfinite(got[n]).all(), (call, n)
            e = relerr(got[n].cpu(), ref[n].cpu())
            assert e <= tol_for(io), (call, n, e)


def test_noalloc_rejects_a_workspace_beyond_its_array():
    cap = gdn.gdn_backward_noalloc_max_bytes()
    B, T, H, d = 1, 2048, 16, 128
    assert gdn.gdn_backward_workspace_size(torch.empty(B, T, H, d), torch.empty(B, T, H, d),
                                           torch.empty(B, T, H, d), w=torch.empty(B, T, H, d)) > cap
    inp, d_o, d_sT = _inputs(B, T, H, d, True, torch.bfloat16, seed=5)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_backward_noalloc(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o, w=inp["w"],
                                 g=inp["g"], state_in=inp["state_in"], d_state_out=d_sT)
    assert ei.value.status == gdn.GDN_ERR_UNSUPPORTED
