"""Seeded synthetic inputs for the gated-delta-rule workloads.

This module only draws random tensors and shapes them; it holds none of the
method's arithmetic, so both the CPU oracle and the GPU library can consume
its output.  Every tensor is drawn in fp32 as N(0, 1) from a seeded
``torch.Generator``, transformed, then cast once to its storage dtype.  Draw
order is fixed: q, k, v, beta (or erase gate b), write gate w, log-decay g,
initial state.

Transforms (the workload descriptions):
  q, k  : x / ||x||_2 over the key dimension (per head, per token)
  v     : x
  beta, b, w : sigmoid(x)            (values in (0, 1))
  g     : -softplus(x) = log(alpha)  (alpha = exp(-softplus(x)) in (0, 1))
  state : 0.02 * x                   (decode workload; zeros otherwise)

The decay is handed over in log space (g = log alpha), as the library's C
ABI takes it.

Packed variable-length batches (``varlen_inputs``) draw the sequence lengths
first, from a generator of their own (log-normal around a mean length,
rounded, at least 1), then the packed tensors with the same transforms.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    channel: bool          # GDN-2 channel gates (b, w, g per channel) vs scalar beta/g
    io_dtype: torch.dtype  # q, k, v, o
    gate_dtype: torch.dtype
    seed: int
    state_std: float = 0.0  # 0 -> S0 = 0

    @property
    def tokens(self) -> int:
        return self.B * self.T


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    channel: bool
    io_dtype: torch.dtype
    gate_dtype: torch.dtype
    seed: int
    state_std: float = 0.02


# The five workloads.  Index = seed.
CONFIGS = {
    "gdn1_fp32_small": ChunkConfig("gdn1_fp32_small", B=1, T=256, Hk=2, Hv=2, dk=64, dv=64,
                                   channel=False, io_dtype=torch.float32,
                                   gate_dtype=torch.float32, seed=1),
    "gdn1_bf16_train": ChunkConfig("gdn1_bf16_train", B=8, T=4096, Hk=16, Hv=16, dk=128, dv=128,
                                   channel=False, io_dtype=torch.bfloat16,
                                   gate_dtype=torch.bfloat16, seed=2),
    "gdn2_bf16_train": ChunkConfig("gdn2_bf16_train", B=8, T=4096, Hk=16, Hv=16, dk=128, dv=128,
                                   channel=True, io_dtype=torch.bfloat16,
                                   gate_dtype=torch.bfloat16, seed=3),
    "gdn1_grouped_long": ChunkConfig("gdn1_grouped_long", B=1, T=32768, Hk=16, Hv=128, dk=128,
                                     dv=128, channel=False, io_dtype=torch.bfloat16,
                                     gate_dtype=torch.bfloat16, seed=4),
    "gdn2_decode": DecodeConfig("gdn2_decode", N=256, Hk=16, Hv=128, dk=128, dv=128,
                                channel=True, io_dtype=torch.bfloat16,
                                gate_dtype=torch.bfloat16, seed=5),
}


@dataclasses.dataclass(frozen=True)
class VarlenConfig:
    name: str
    N: int                 # sequences
    total_T: int           # packed tokens (the lengths sum to this)
    Hk: int
    Hv: int
    dk: int
    dv: int
    channel: bool
    io_dtype: torch.dtype
    gate_dtype: torch.dtype
    seed: int
    sigma: float = 0.8     # log-normal spread of the lengths


# A serving-style prefill: 16 sequences of mixed lengths, as many tokens as the
# B8 T4096 training shape, GDN-2 gates.
VARLEN_CONFIGS = {
    "gdn2_varlen_mix": VarlenConfig("gdn2_varlen_mix", N=16, total_T=32768, Hk=16, Hv=16, dk=128,
                                    dv=128, channel=True, io_dtype=torch.bfloat16,
                                    gate_dtype=torch.bfloat16, seed=6),
}


def varlen_lengths(cfg: VarlenConfig) -> list:
    """Seeded sequence lengths (each >= 1) summing to cfg.total_T."""
    gen = torch.Generator().manual_seed(int(cfg.seed) * 1000 + 7)
    w = torch.exp(cfg.sigma * torch.randn(cfg.N, generator=gen, dtype=torch.float64))
    raw = torch.clamp(torch.floor(w / w.sum() * cfg.total_T), min=1).to(torch.int64)
    raw[-1] += cfg.total_T - int(raw.sum())
    assert int(raw.min()) >= 1 and int(raw.sum()) == cfg.total_T
    return [int(x) for x in raw]


def varlen_inputs(cfg: VarlenConfig, *, device="cpu"):
    """Packed inputs of a variable-length batch: q, k [total_T, Hk, dk],
    v [total_T, Hv, dv], gates [total_T, Hv(, d)], cu_seqlens int64 [N + 1]
    (on ``device``) and the lengths."""
    lengths = varlen_lengths(cfg)
    one = ChunkConfig(cfg.name, B=1, T=cfg.total_T, Hk=cfg.Hk, Hv=cfg.Hv, dk=cfg.dk, dv=cfg.dv,
                      channel=cfg.channel, io_dtype=cfg.io_dtype, gate_dtype=cfg.gate_dtype,
                      seed=cfg.seed)
    inp = chunk_inputs(one, device=device)
    out = {k: (None if v is None else v[0].contiguous())
           for k, v in inp.items() if k != "state_in"}
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int64, device=device)
    out["lengths"] = lengths
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _unit(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def chunk_inputs(cfg: ChunkConfig, *, device="cpu", seed=None, T=None, B=None,
                 state_std=None):
    """Inputs of a chunk-forward workload as a dict of tensors on ``device``.

    Keys: q, k, v, beta_or_b, w (None in scalar mode), g, state_in (None when
    the initial state is zero).  ``T``, ``B``, ``seed`` and ``state_std``
    override the configuration (used for parity cases at reduced size).
    """
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    state_std = cfg.state_std if state_std is None else state_std
    gen = _gen(seed, device)
    q = _unit(_randn((B, T, cfg.Hk, cfg.dk), gen, device)).to(cfg.io_dtype)
    k = _unit(_randn((B, T, cfg.Hk, cfg.dk), gen, device)).to(cfg.io_dtype)
    v = _randn((B, T, cfg.Hv, cfg.dv), gen, device).to(cfg.io_dtype)
    if cfg.channel:
        b = torch.sigmoid(_randn((B, T, cfg.Hv, cfg.dk), gen, device)).to(cfg.gate_dtype)
        w = torch.sigmoid(_randn((B, T, cfg.Hv, cfg.dv), gen, device)).to(cfg.gate_dtype)
        g = (-torch.nn.functional.softplus(_randn((B, T, cfg.Hv, cfg.dk), gen, device))
             ).to(cfg.gate_dtype)
    else:
        b = torch.sigmoid(_randn((B, T, cfg.Hv), gen, device)).to(cfg.gate_dtype)
        w = None
        g = (-torch.nn.functional.softplus(_randn((B, T, cfg.Hv), gen, device))
             ).to(cfg.gate_dtype)
    s0 = None
    if state_std:
        s0 = (state_std * _randn((B, cfg.Hv, cfg.dk, cfg.dv), gen, device)).contiguous()
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), beta_or_b=b.contiguous(),
                w=None if w is None else w.contiguous(), g=g.contiguous(), state_in=s0)


def decode_inputs(cfg: DecodeConfig, *, device="cpu", seed=None, N=None, Hv=None, Hk=None):
    """Inputs of a decode step as a dict: q, k, v, beta_or_b, w, g, state."""
    N = cfg.N if N is None else N
    Hv = cfg.Hv if Hv is None else Hv
    Hk = cfg.Hk if Hk is None else Hk
    seed = cfg.seed if seed is None else seed
    gen = _gen(seed, device)
    q = _unit(_randn((N, Hk, cfg.dk), gen, device)).to(cfg.io_dtype)
    k = _unit(_randn((N, Hk, cfg.dk), gen, device)).to(cfg.io_dtype)
    v = _randn((N, Hv, cfg.dv), gen, device).to(cfg.io_dtype)
    if cfg.channel:
        b = torch.sigmoid(_randn((N, Hv, cfg.dk), gen, device)).to(cfg.gate_dtype)
        w = torch.sigmoid(_randn((N, Hv, cfg.dv), gen, device)).to(cfg.gate_dtype)
        g = (-torch.nn.functional.softplus(_randn((N, Hv, cfg.dk), gen, device))
             ).to(cfg.gate_dtype)
    else:
        b = torch.sigmoid(_randn((N, Hv), gen, device)).to(cfg.gate_dtype)
        w = None
        g = (-torch.nn.functional.softplus(_randn((N, Hv), gen, device))).to(cfg.gate_dtype)
    state = (cfg.state_std * _randn((N, Hv, cfg.dk, cfg.dv), gen, device)).contiguous()
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), beta_or_b=b.contiguous(),
                w=None if w is None else w.contiguous(), g=g.contiguous(), state=state)


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """The operations around the recurrence (short conv branch, gates, output
    gate) at one layer shape: `rows` packed tokens in N equal sequences."""
    name: str
    N: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    channel: bool
    io_dtype: torch.dtype
    gate_dtype: torch.dtype
    seed: int

    @property
    def rows(self) -> int:
        return self.N * self.T

    @property
    def conv_channels(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


# The GDN-2 B8 T4096 training shape.
BLOCK_CONFIGS = {
    "gdn2_block_train": BlockConfig("gdn2_block_train", N=8, T=4096, Hk=16, Hv=16, dk=128,
                                    dv=128, channel=True, io_dtype=torch.bfloat16,
                                    gate_dtype=torch.bfloat16, seed=7),
}


def block_inputs(cfg: BlockConfig, *, device="cpu", seed=None, N=None, T=None, conv_state=True):
    """Raw inputs of the block operations as a dict of tensors on ``device``.

    x       [rows, C + Hv dv]: the q|k|v|z projection output, N(0, 1); the
            first C = 2 Hk dk + Hv dv columns feed the short conv, the last
            Hv dv are the output-gate branch z
    conv_w  [C, 4] fp32, 0.5 N(0, 1); conv_state [N, 3, C], N(0, 1) (or None)
    a_raw, b_raw  [rows, n] with n = Hv (scalar gates) or Hv dk (channel),
            N(0, 1), in one [rows, 2n] buffer (b columns first, then a)
    w_raw   [rows, Hv dv] (channel gates) or None, N(0, 1)
    A_log   [n] fp32, log of U(1, 16); dt_bias [n] fp32, N(-2, 0.5^2)
    norm_w  [dv] fp32, 1 + 0.1 N(0, 1)
    o       [rows, Hv, dv], N(0, 1): a stand-in recurrence output for the
            output gate on its own
    Draw order is the key order above.
    """
    N = cfg.N if N is None else N
    T = cfg.T if T is None else T
    rows = N * T
    seed = cfg.seed if seed is None else seed
    gen = _gen(seed, device)
    C = cfg.conv_channels
    n = cfg.Hv * cfg.dk if cfg.channel else cfg.Hv
    x = _randn((rows, C + cfg.Hv * cfg.dv), gen, device).to(cfg.io_dtype)
    conv_w = 0.5 * _randn((C, 4), gen, device)
    cs = _randn((N, 3, C), gen, device).to(cfg.io_dtype) if conv_state else None
    ba = _randn((rows, 2 * n), gen, device).to(cfg.io_dtype)
    w_raw = _randn((rows, cfg.Hv * cfg.dv), gen, device).to(cfg.io_dtype) if cfg.channel else None
    u = torch.rand(n, generator=gen, device=device, dtype=torch.float32)
    A_log = torch.log(1.0 + 15.0 * u)
    dt_bias = -2.0 + 0.5 * _randn((n,), gen, device)
    norm_w = 1.0 + 0.1 * _randn((cfg.dv,), gen, device)
    o = _randn((rows, cfg.Hv, cfg.dv), gen, device).to(cfg.io_dtype)
    return dict(x=x.contiguous(), conv_w=conv_w.contiguous(), conv_state=cs, ba=ba.contiguous(),
                b_raw=ba[:, :n], a_raw=ba[:, n:], w_raw=w_raw, A_log=A_log, dt_bias=dt_bias,
                norm_w=norm_w, o=o.contiguous(), z=x[:, C:])
