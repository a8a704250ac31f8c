#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  1. gdn_chunk_fwd on the GDN-2 prefill workload
     (B=8, H_k=H_v=16, T=4096, d_k=d_v=128, channel gates, bf16 inputs,
      fp32 state, chunk 64), and
  2. gdn_decode_step on the GDN-2 decode workload
     (256 sequences x 128 value heads / 16 key heads, d=128, channel gates,
      bf16 inputs, 2.1 GB fp32 state updated in place).

Prints ONE JSON line.  `value` is the chunk forward's tokens/s (B*T per
launch / mean launch time); the decode step's state bandwidth is reported in
`decode_state_GBps`.  Inputs are resident in HBM before timing starts.  Kernel
durations come from HIP events recorded on the stream the kernels run on.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3        # MI355X dense fp32 MFMA, published
CHUNK = 64


def chunk_algorithmic(cfg, gate_bytes, io_bytes=2, state_in=False):
    """Bytes each input is read once, o and the final state written once; and
    the flops the chunkwise method must do, triangular work counted as half:
    2*[C/2*(3 d_k + 2 d_v) + 3 d_k d_v] per (token, value head)."""
    B, T, Hk, Hv, dk, dv = cfg.B, cfg.T, cfg.Hk, cfg.Hv, cfg.dk, cfg.dv
    qk = 2 * B * T * Hk * dk * io_bytes
    v = B * T * Hv * dv * io_bytes
    o = B * T * Hv * dv * io_bytes
    if cfg.channel:
        gates = B * T * Hv * (2 * dk + dv) * gate_bytes
    else:
        gates = 2 * B * T * Hv * gate_bytes
    state = B * Hv * dk * dv * 4 * (2 if state_in else 1)
    flops = 2.0 * (CHUNK / 2 * (3 * dk + 2 * dv) + 3 * dk * dv) * B * T * Hv
    return qk + v + o + gates + state, flops


def decode_algorithmic(cfg, io_bytes=2, gate_bytes=2):
    N, Hk, Hv, dk, dv = cfg.N, cfg.Hk, cfg.Hv, cfg.dk, cfg.dv
    state = 2 * N * Hv * dk * dv * 4
    qk = 2 * N * Hk * dk * io_bytes
    vo = 2 * N * Hv * dv * io_bytes
    gates = N * Hv * (2 * dk + dv) * gate_bytes if cfg.channel else 2 * N * Hv * gate_bytes
    flops = 6.0 * N * Hv * dk * dv
    return state + qk + vo + gates, flops


# Sources each profiled kernel is built from; its counter figures stay valid
# while these files are unchanged.
KERNEL_SOURCES = {
    "chunk_fwd": ("chunk_fwd_sb.hip", "chunk_fwd.hip", "chunk_common.hpp", "gdn_device.hpp"),
    "chunk_fwd_save": ("chunk_fwd_sb.hip", "chunk_common.hpp", "gdn_device.hpp"),
    "decode_step": ("decode.hip", "gdn_device.hpp"),
    "short_conv": ("layer_ops.hip", "gdn_device.hpp"),
    "gates": ("layer_ops.hip", "gdn_device.hpp"),
    "output_gate": ("layer_ops.hip", "gdn_device.hpp"),
    "backward": ("backward.hip", "chunk_common.hpp", "gdn_device.hpp"),
    "backward_saved": ("backward.hip", "chunk_common.hpp", "gdn_device.hpp"),
    "backward_fill": ("backward.hip",),
    "backward_reduce": ("backward.hip", "chunk_common.hpp", "gdn_device.hpp"),
}


def source_digest(names=None):
    """sha256 prefix over the named files of the kernel sources (all of them
    when names is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_gdn_amd", "csrc")
    for name in sorted(os.listdir(csrc) if names is None else names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, per_launch_bytes_alg):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic.json), or None when it is absent or was taken on other
    sources of that kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel_key)
    if not ent or kernel_key not in KERNEL_SOURCES:
        return None
    if ent.get("source_digest") != source_digest(KERNEL_SOURCES[kernel_key]):
        return None
    return ent.get("hbm_bytes_per_launch")


def time_cold(fn, torch, flush, steps, warmup):
    """Per-repetition launch times (ms) with HIP events on the launch stream,
    each repetition after a 512 MB write that evicts L2 and the Infinity
    Cache; returns (median, min) over the repetitions and the warm mean of as
    many back-to-back launches."""
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        flush.zero_()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        fn()
        ev[1].record()
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    warm = ev[0].elapsed_time(ev[1]) / steps
    times.sort()
    return times[len(times) // 2], times[0], warm


def sub_block_paths(g, channel, torch, sub=16, limit=110.0, floor=13.0):
    """Fractions of (sequence, value head, 16-token sub-block) units that the
    chunk kernel scans a second time with floored decays, and that it runs on
    its exact token path, from the log-decay tensor g ([B, T, H_v, d_k] or
    [B, T, H_v]) and the kernel's own criterion.  With G the cumulative
    log2-decay from the sub-block start, channel gates need |G - m| <= limit
    (m = G at token 7) and the rising-state bounds (m, G_15 - m and G_15 at
    most 10); a sub-block that fails is scanned again with every per-token
    log2-decay raised to -floor, and takes the token path only if it still
    fails.  Scalar gates: no rise G_t - min_{s<=t} G_s, G_t or G_15 - G_t
    above the limit (no floor)."""
    B, T = g.shape[0], g.shape[1]
    Tb = (T // sub) * sub
    x = g[:, :Tb].float() * 1.4426950408889634
    if not channel:
        x = x.unsqueeze(-1)
    x = x.reshape(B, Tb // sub, sub, x.shape[2], x.shape[3])

    def fails(lx):
        G = torch.cumsum(lx, dim=2)
        g15 = G[:, :, 15:16]
        if channel:
            m = G[:, :, 7:8]
            worst = torch.maximum((G - m).abs(),
                                  torch.maximum(torch.maximum(m, g15 - m), g15) + (limit - 10.0))
        else:
            rise = G - torch.cummin(G, dim=2).values
            worst = torch.maximum(torch.maximum(G, g15 - G), rise)
        return worst.amax(dim=(2, 4)) > limit

    first = fails(x)
    if not channel:
        return 0.0, float(first.float().mean())
    second = first & fails(torch.clamp(x, min=-floor))
    return float(first.float().mean()), float(second.float().mean())


def realistic_gates(gdn, synth, torch, cfg):
    """g, beta or b, w for the shape of cfg from gdn_gates over the Mamba-2
    recipe of the block inputs (A_log = log U(1, 16), dt_bias ~ N(-2, 0.5^2),
    raw projections N(0, 1); seed 7)."""
    bcfg = synth.BlockConfig("gates", N=cfg.B, T=cfg.T, Hk=cfg.Hk, Hv=cfg.Hv, dk=cfg.dk,
                             dv=cfg.dv, channel=cfg.channel, io_dtype=torch.bfloat16,
                             gate_dtype=torch.bfloat16, seed=7)
    blk = synth.block_inputs(bcfg, device="cuda", conv_state=False)
    g, beta, w = gdn.gdn_gates(blk["a_raw"], blk["b_raw"], cfg.Hv, w_raw=blk["w_raw"],
                               A_log=blk["A_log"], dt_bias=blk["dt_bias"], d_k=cfg.dk, d_v=cfg.dv)
    torch.cuda.synchronize()
    del blk
    return g, beta, w


def secondary_chunk_workloads(gdn, synth, torch, dev, steps=10, warmup=2):
    """Chunk-forward timings of the other prefill workloads (not part of the
    step): HIP events on the launch stream, cold caches per repetition
    (median and min) and warm, against the same algorithmic bytes and flops
    as the headline workload.  The rows "*_mamba2_gates" run the B8 T4096
    shapes on gates from gdn_gates over the Mamba-2 recipe and report the
    fractions of sub-blocks scanned with floored decays and on the exact
    path."""
    res = {}
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)   # 512 MB
    rows = [("gdn1_fp32_small", None, None), ("gdn1_bf16_train", None, None),
            ("gdn2_bf16_train", "fp32_gates", None), ("gdn1_grouped_long", None, None),
            ("gdn2_bf16_train", "mamba2_gates", None), ("gdn1_bf16_train", "mamba2_gates", None)]
    for name, variant, _ in rows:
        cfg = synth.CONFIGS[name]
        if variant == "fp32_gates":
            cfg = synth.ChunkConfig(name, B=cfg.B, T=cfg.T, Hk=cfg.Hk, Hv=cfg.Hv, dk=cfg.dk,
                                    dv=cfg.dv, channel=cfg.channel, io_dtype=cfg.io_dtype,
                                    gate_dtype=torch.float32, seed=cfg.seed)
        inp = synth.chunk_inputs(cfg, device="cuda")
        frac = None
        if variant == "mamba2_gates":
            g, beta, w = realistic_gates(gdn, synth, torch, cfg)
            inp["g"], inp["beta_or_b"] = g.reshape(inp["g"].shape), beta.reshape(inp["g"].shape)
            if cfg.channel:
                inp["w"] = w.reshape(inp["v"].shape)
            floored, frac = sub_block_paths(inp["g"], cfg.channel, torch)
        o = torch.empty((cfg.B, cfg.T, cfg.Hv, cfg.dv), dtype=cfg.io_dtype, device=dev)
        s = torch.empty((cfg.B, cfg.Hv, cfg.dk, cfg.dv), dtype=torch.float32, device=dev)

        def run():
            gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], w=inp["w"], g=inp["g"],
                              state_in=inp["state_in"], state_out=s, o=o)
        ms, ms_min, ms_warm = time_cold(run, torch, flush, steps, warmup)
        io_bytes = 4 if cfg.io_dtype == torch.float32 else 2
        gate_bytes = 4 if cfg.gate_dtype == torch.float32 else 2
        nbytes, flops = chunk_algorithmic(cfg, gate_bytes, io_bytes=io_bytes,
                                          state_in=inp["state_in"] is not None)
        if cfg.Hv != cfg.Hk:  # q k^T and k k^T are shared by the value heads of a key head
            G = cfg.Hv // cfg.Hk
            flops = 2.0 * (CHUNK / 2 * (cfg.dk + 2 * cfg.dv) + 3 * cfg.dk * cfg.dv
                           + CHUNK * cfg.dk / G) * cfg.B * cfg.T * cfg.Hv
        key = name if variant is None else f"{name}_{variant}"
        res[key] = {"ms": round(ms, 4), "ms_min": round(ms_min, 4), "ms_warm": round(ms_warm, 4),
                    "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
                    "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                    "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                    "mfma_frac": round(flops / (ms * 1e-3) / 1e12 /
                                       (PEAK_FP32_TFLOPS if io_bytes == 4 else PEAK_BF16_TFLOPS), 4)}
        if frac is not None:
            res[key]["floored_fraction"] = round(floored, 6)
            res[key]["exact_path_fraction"] = round(frac, 6)
        del inp, o, s
        torch.cuda.empty_cache()
    # packed variable-length prefill (serving): the final states are the
    # layout the decode step consumes
    for name, vcfg in synth.VARLEN_CONFIGS.items():
        inp = synth.varlen_inputs(vcfg, device="cuda")
        o = torch.empty((vcfg.total_T, vcfg.Hv, vcfg.dv), dtype=vcfg.io_dtype, device=dev)
        s = torch.empty((vcfg.N, vcfg.Hv, vcfg.dk, vcfg.dv), dtype=torch.float32, device=dev)

        def run():
            gdn.gdn_chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["beta_or_b"],
                                     inp["cu_seqlens"], w=inp["w"], g=inp["g"], state_out=s, o=o)
        ms, ms_min, ms_warm = time_cold(run, torch, flush, steps, warmup)
        one = synth.ChunkConfig(name, B=1, T=vcfg.total_T, Hk=vcfg.Hk, Hv=vcfg.Hv, dk=vcfg.dk,
                                dv=vcfg.dv, channel=vcfg.channel, io_dtype=vcfg.io_dtype,
                                gate_dtype=vcfg.gate_dtype, seed=vcfg.seed)
        nbytes, flops = chunk_algorithmic(one, 2)
        nbytes += (vcfg.N - 1) * vcfg.Hv * vcfg.dk * vcfg.dv * 4   # one final state per sequence
        res[name] = {"ms": round(ms, 4), "ms_min": round(ms_min, 4), "ms_warm": round(ms_warm, 4),
                     "tokens_per_s": round(vcfg.total_T / (ms * 1e-3), 1),
                     "sequences": vcfg.N, "lengths": inp["lengths"],
                     "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del inp, o, s
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return res


def single_workload(gdn, synth, torch, dev, name, steps, warmup):
    """gdn_chunk_fwd (or gdn_chunk_fwd_varlen for a packed mix) alone on one
    workload, warm back-to-back launches."""
    if name in synth.VARLEN_CONFIGS:
        vcfg = synth.VARLEN_CONFIGS[name]
        inp = synth.varlen_inputs(vcfg, device="cuda")
        o = torch.empty((vcfg.total_T, vcfg.Hv, vcfg.dv), dtype=vcfg.io_dtype, device=dev)
        s = torch.empty((vcfg.N, vcfg.Hv, vcfg.dk, vcfg.dv), dtype=torch.float32, device=dev)

        def run_v():
            gdn.gdn_chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["beta_or_b"],
                                     inp["cu_seqlens"], w=inp["w"], g=inp["g"], state_out=s, o=o)
        for _ in range(warmup):
            run_v()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            run_v()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        return {"workload": name, "ms": round(ms, 4),
                "tokens_per_s": round(vcfg.total_T / (ms * 1e-3), 1)}
    mamba2 = name.endswith("_mamba2_gates")
    fp32g = name.endswith("_fp32_gates")
    base = name[:-len("_mamba2_gates")] if mamba2 else (name[:-len("_fp32_gates")] if fp32g else name)
    cfg = synth.CONFIGS[base]
    if fp32g:
        cfg = synth.ChunkConfig(base, B=cfg.B, T=cfg.T, Hk=cfg.Hk, Hv=cfg.Hv, dk=cfg.dk, dv=cfg.dv,
                                channel=cfg.channel, io_dtype=cfg.io_dtype,
                                gate_dtype=torch.float32, seed=cfg.seed)
    inp = synth.chunk_inputs(cfg, device="cuda")
    if mamba2:
        g, beta, w = realistic_gates(gdn, synth, torch, cfg)
        inp["g"], inp["beta_or_b"] = g.reshape(inp["g"].shape), beta.reshape(inp["g"].shape)
        if cfg.channel:
            inp["w"] = w.reshape(inp["v"].shape)
    o = torch.empty((cfg.B, cfg.T, cfg.Hv, cfg.dv), dtype=cfg.io_dtype, device=dev)
    s = torch.empty((cfg.B, cfg.Hv, cfg.dk, cfg.dv), dtype=torch.float32, device=dev)

    def run():
        gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], w=inp["w"], g=inp["g"],
                          state_in=inp["state_in"], state_out=s, o=o)
    for _ in range(warmup):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    return {"workload": name, "ms": round(ms, 4),
            "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1)}


def copy_bandwidth(torch, dev):
    """A plain 2 GiB device-to-device copy through torch: read + write bytes
    per second, the practical streaming rate beside the 8 TB/s nominal peak."""
    a = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(5):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    del a, b
    torch.cuda.empty_cache()
    return round(2 * (1 << 31) / (ms * 1e-3) / 1e9, 1)


def block_op_workloads(gdn, synth, torch, dev, steps=20, warmup=3):
    """The operations around the recurrence at the GDN-2 B8 T4096 layer shape
    (not part of the step): the short conv branch, the gate activations and
    the output norm x swish(z), each timed with HIP events on the launch
    stream against the bytes it must move (each operand read once, each
    output written once)."""
    cfg = synth.BLOCK_CONFIGS["gdn2_block_train"]
    inp = synth.block_inputs(cfg, device="cuda", conv_state=False)
    rows, C, Hv, dk, dv = cfg.rows, cfg.conv_channels, cfg.Hv, cfg.dk, cfg.dv
    n = Hv * dk if cfg.channel else Hv
    eb = 2 if cfg.io_dtype == torch.bfloat16 else 4
    gb = 2 if cfg.gate_dtype == torch.bfloat16 else 4
    q = torch.empty((rows, cfg.Hk, dk), dtype=cfg.io_dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((rows, Hv, dv), dtype=cfg.io_dtype, device=dev)
    gshape = (rows, Hv, dk) if cfg.channel else (rows, Hv)
    g = torch.empty(gshape, dtype=cfg.gate_dtype, device=dev)
    beta = torch.empty_like(g)
    w = torch.empty((rows, Hv, dv), dtype=cfg.gate_dtype, device=dev) if cfg.channel else None
    y = torch.empty_like(inp["o"])
    ops = {
        "short_conv": (lambda: gdn.gdn_short_conv(inp["x"], inp["conv_w"], cfg.Hk, Hv, dk, dv,
                                                  N=cfg.N, q=q, k=k, v=v),
                       2 * rows * C * eb + C * 16),
        "gates": (lambda: gdn.gdn_gates(inp["a_raw"], inp["b_raw"], Hv, w_raw=inp["w_raw"],
                                        A_log=inp["A_log"], dt_bias=inp["dt_bias"], d_k=dk,
                                        d_v=dv, gate_dtype=cfg.gate_dtype, g=g, beta_or_b=beta,
                                        w=w),
                  rows * (2 * n + (Hv * dv if cfg.channel else 0)) * (eb + gb) + 8 * n),
        "output_gate": (lambda: gdn.gdn_output_gate(inp["o"], inp["z"], inp["norm_w"], y=y),
                        3 * rows * Hv * dv * eb + 4 * dv),
    }
    res = {"workload": f"{cfg.name}: {cfg.N} x {cfg.T} tokens, H_k={cfg.Hk}, H_v={Hv}, "
                       f"d_k={dk}, d_v={dv}, {'channel' if cfg.channel else 'scalar'} gates, bf16"}
    for name, (fn, nbytes) in ops.items():
        for _ in range(warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "GBps": round(gbps, 1),
                     "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(name, nbytes)}
    del inp, q, k, v, g, beta, w, y
    torch.cuda.empty_cache()
    return res


def fused_gate_workloads(gdn, synth, torch, dev, steps=20, warmup=3):
    """Gate activations inside the chunk kernel (gdn_chunk_fwd_gated) against
    gdn_gates followed by gdn_chunk_fwd, at the GDN-2 and GDN-1 B8 T4096
    shapes on the block recipe's raw projections (warm, back-to-back
    launches, HIP events on the launch stream)."""
    res = {}
    for name in ("gdn2_bf16_train", "gdn1_bf16_train"):
        cfg = synth.CONFIGS[name]
        inp = synth.chunk_inputs(cfg, device="cuda")
        bcfg = synth.BlockConfig("gates", N=cfg.B, T=cfg.T, Hk=cfg.Hk, Hv=cfg.Hv, dk=cfg.dk,
                                 dv=cfg.dv, channel=cfg.channel, io_dtype=torch.bfloat16,
                                 gate_dtype=torch.bfloat16, seed=7)
        blk = synth.block_inputs(bcfg, device="cuda", conv_state=False)
        B, T, Hv, d = cfg.B, cfg.T, cfg.Hv, cfg.dk
        shape = (B, T, Hv, d) if cfg.channel else (B, T, Hv)
        o = torch.empty((B, T, Hv, d), dtype=torch.bfloat16, device=dev)
        s = torch.empty((B, Hv, d, d), dtype=torch.float32, device=dev)
        g, beta, w = gdn.gdn_gates(blk["a_raw"], blk["b_raw"], Hv, w_raw=blk["w_raw"],
                                   A_log=blk["A_log"], dt_bias=blk["dt_bias"], d_k=d, d_v=d)

        def two_step():
            gdn.gdn_gates(blk["a_raw"], blk["b_raw"], Hv, w_raw=blk["w_raw"], A_log=blk["A_log"],
                          dt_bias=blk["dt_bias"], d_k=d, d_v=d, g=g, beta_or_b=beta, w=w)
            gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], beta.view(shape),
                              w=None if w is None else w.view(B, T, Hv, d), g=g.view(shape),
                              state_out=s, o=o)

        def fused():
            gdn.gdn_chunk_fwd_gated(inp["q"], inp["k"], inp["v"], blk["b_raw"], a_raw=blk["a_raw"],
                                    w_raw=blk["w_raw"], A_log=blk["A_log"], dt_bias=blk["dt_bias"],
                                    state_out=s, o=o)
        row = {}
        for key, fn in (("gates_then_chunk_ms", two_step), ("fused_ms", fused)):
            for _ in range(warmup):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(steps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            row[key] = round(ev[0].elapsed_time(ev[1]) / steps, 4)
        res[name] = row
        del inp, blk, o, s, g, beta, w
        torch.cuda.empty_cache()
    return res


def backward_exact_fraction(g, torch, block=16, limit=96.0):
    """Fraction of (sequence, 16-token block, value head, channel) units the
    backward computes term by term, from channel log-decays g [B, T, H_v,
    d_k] and the kernel's criterion: with G the inclusive cumulative
    log2-decay from the block start, half the channel's range of G over the
    block above the limit (the other channels of the block stay on the
    factored MFMA products)."""
    B, T = g.shape[0], g.shape[1]
    Tb = (T // block) * block
    x = g[:, :Tb].float() * 1.4426950408889634
    G = torch.cumsum(x.reshape(B, Tb // block, block, g.shape[2], g.shape[3]), dim=2)
    half = 0.5 * (G.amax(dim=2) - G.amin(dim=2))
    return float((half > limit).float().mean())


def backward_workload(gdn, synth, torch, dev, steps=5, warmup=2):
    """gdn_backward on the GDN-2 B8 T4096 shape (not part of the step): the
    gradients of every input for a random upstream gradient of o.  The
    kernel works in 16-token blocks whose dense products run on the bf16
    MFMA, so it is judged against the bf16 dense peak, counting the products
    with the state per block of C tokens and value head: 2 C d_k d_v
    multiply-adds to rebuild the forward ((gs e) S and (ge k)^T U) and
    6 C d_k d_v for the reverse ((k ge) D, dO S^T, DU S^T, U D^T and the two
    products of the state-gradient update), i.e. 16 d_k d_v flops per (token,
    value head).  The C x C products (Gram matrices, triangular solve,
    intra-block terms) add about 8 % and are not counted."""
    cfg = synth.CONFIGS["gdn2_bf16_train"]
    inp = synth.chunk_inputs(cfg, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(77)
    d_o = torch.randn((cfg.B, cfg.T, cfg.Hv, cfg.dv), generator=gen, device="cuda").to(cfg.io_dtype)
    nws = gdn.gdn_backward_workspace_size(inp["q"], inp["v"], inp["beta_or_b"], inp["w"])
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    grads = None

    def run(grads):
        return gdn.gdn_backward(inp["q"], inp["k"], inp["v"], inp["beta_or_b"], d_o, w=inp["w"],
                                g=inp["g"], workspace=ws, grads=grads)
    for _ in range(warmup):
        grads = run(grads)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        run(grads)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    flops = 16.0 * cfg.dk * cfg.dv * cfg.B * cfg.T * cfg.Hv
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": f"{cfg.name} backward: B={cfg.B}, T={cfg.T}, H={cfg.Hv}, d=128, "
                       "channel gates, bf16 inputs, fp32 gradients",
           "ms": round(ms, 3), "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
           "workspace_bytes": nws, "mfma_tflops": round(tf, 2),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "flops_per_launch": flops,
                        "traffic": measured_traffic("backward", None)}}
    # The training pair on the same inputs: gdn_chunk_fwd then gdn_backward
    # (which rebuilds the forward's states first), against gdn_chunk_fwd_save
    # (which leaves them in the workspace) then gdn_backward_saved.
    o = torch.empty_like(inp["v"])
    s_out = torch.empty((cfg.B, cfg.Hv, cfg.dk, cfg.dv), device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    fwd_ms = timed(lambda: gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta_or_b"],
                                             w=inp["w"], g=inp["g"], state_out=s_out, o=o))
    save_ms = timed(lambda: gdn.gdn_chunk_fwd_save(inp["q"], inp["k"], inp["v"], inp["beta_or_b"],
                                                   w=inp["w"], g=inp["g"], state_out=s_out, o=o,
                                                   workspace=ws))
    saved_ms = timed(lambda: gdn.gdn_backward_saved(inp["q"], inp["k"], inp["v"], inp["beta_or_b"],
                                                    d_o, ws, w=inp["w"], g=inp["g"], grads=grads))
    res["saved_states"] = {
        "forward_ms": round(fwd_ms, 3), "forward_save_ms": round(save_ms, 3),
        "backward_saved_ms": round(saved_ms, 3),
        "forward_plus_backward_ms": round(fwd_ms + ms, 3),
        "forward_save_plus_backward_saved_ms": round(save_ms + saved_ms, 3)}
    del o, s_out
    # the same shape on gates from gdn_gates over the Mamba-2 recipe: the
    # channels whose decay range in a block exceeds the factored form's are
    # taken term by term
    g, beta, w = realistic_gates(gdn, synth, torch, cfg)
    inp["g"], inp["beta_or_b"], inp["w"] = (g.reshape(inp["g"].shape), beta.reshape(inp["g"].shape),
                                           w.reshape(inp["v"].shape))
    del g, beta, w
    for _ in range(warmup):
        run(grads)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        run(grads)
    ev[1].record()
    torch.cuda.synchronize()
    ms2 = ev[0].elapsed_time(ev[1]) / steps
    res["mamba2_gates"] = {"ms": round(ms2, 3),
                           "term_by_term_fraction": round(backward_exact_fraction(inp["g"], torch), 4)}
    del inp, ws, grads, d_o
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args):
    """The oracle, untuned, on the machine's host cores over the whole prefill
    workload (8 sequences x 16 heads x T=4096; under a second of wall time on
    16 cores, about 12 s of CPU time); the decode leg is not part of the
    sample."""
    import torch

    import oracle
    import synth
    cfg = synth.CONFIGS["gdn2_bf16_train"]
    B = cfg.B
    inp = synth.chunk_inputs(cfg, B=B)
    args64 = {k: (None if v is None else v.to(torch.float64).numpy()) for k, v in inp.items()}
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = min(cores, args.cpu_threads) if args.cpu_threads else cores
    t0 = time.perf_counter()
    oracle.recurrent(args64["q"], args64["k"], args64["v"], args64["beta_or_b"], args64["w"],
                     args64["g"], nthreads=cores)
    dt = time.perf_counter() - t0
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": B * cfg.T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"GDN-2 prefill chunk forward only, all {B} sequences x {cfg.Hv} heads x "
                      f"T={cfg.T} (fp64 token recurrence, OpenMP over heads); {dt:.2f} s wall",
            "cpu_model": model, "seconds": dt}


KERNEL_KEYS = {"chunk_fwd": ("chunk_fwd_sb_kernel", "chunk_fwd_kernel"),
               "chunk_fwd_save": (),
               "decode_step": ("decode_kernel",),
               "short_conv": ("short_conv_kernel",),
               "gates": ("gates_kernel", "gates_vec_kernel"),
               "output_gate": ("output_gate_kernel",),
               "backward": ("bwd_kernel",),
               "backward_saved": (),
               "backward_fill": ("zero4_kernel",),
               "backward_reduce": ("bwd_reduce_kernel",)}


def _last_template_arg_true(name, params):
    """Whether a kernel's last template argument (a bool) is true, in the
    mangled (...Lb1EEEv<params>) or the demangled (..., true>(<params>)) name."""
    return ("Lb1EEEv" + params[0]) in name or name.endswith("true>(" + params[1] + ")")


def _kernel_key(name):
    for key, pats in KERNEL_KEYS.items():
        if any(p in name for p in pats):
            # the variants that store (forward) or read (backward) the saved
            # states carry a last template argument of true
            if key == "chunk_fwd" and "chunk_fwd_sb_kernel" in name and _last_template_arg_true(
                    name, ("NS0_6ParamsE", "gdn::(anonymous namespace)::Params")):
                return "chunk_fwd_save"
            if key == "backward" and _last_template_arg_true(name, ("NS_7BwdArgsE", "gdn::BwdArgs")):
                return "backward_saved"
            return key
    return None


def summarize_profiles(kt_csv, fetch_csv, write_csv, commands):
    """Turn rocprofv3 output into profiles/traffic.json: kernel-trace stats
    (average launch duration per kernel) and HBM traffic per launch from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the same
    counter reads for the plain 1 GiB device copy that `--copy-calibration`
    runs last in the same process.  Profile with `--no-secondary`, so that the
    only chunk-forward dispatches are those of the headline workload."""
    import csv

    def rows(path):
        with open(path, newline="") as f:
            return list(csv.DictReader(f))

    stats = {}
    for r in rows(kt_csv):
        key = _kernel_key(r["Name"])
        if key:
            stats[key] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                          "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}

    def counter(path, name):
        per = {}
        copy = []
        for r in rows(path):
            if r["Counter_Name"] != name:
                continue
            v = float(r["Counter_Value"])
            key = _kernel_key(r["Kernel_Name"])
            if key:
                per.setdefault(key, []).append(v)
            elif "copy" in r["Kernel_Name"].lower():
                copy.append((int(r["Dispatch_Id"]), v))
        # the calibration copies are the last dispatches of the process
        copy = [v for _, v in sorted(copy)[-1:]]
        return per, copy

    fetch, copy_f = counter(fetch_csv, "FETCH_SIZE")
    write, copy_w = counter(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    # the calibration copy is the largest copy dispatch in the run
    f_scale = gib_kib / max(copy_f) if copy_f else None
    w_scale = gib_kib / max(copy_w) if copy_w else None
    out = {"source_digest": source_digest(), "commands": commands,
           "calibration": {"copy_bytes": 1 << 30, "fetch_kib": max(copy_f) if copy_f else None,
                           "write_kib": max(copy_w) if copy_w else None,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": {}}
    for key in KERNEL_KEYS:
        if key not in fetch or key not in write or not f_scale or not w_scale:
            continue
        fk = sum(fetch[key]) / len(fetch[key])
        wk = sum(write[key]) / len(write[key])
        out["kernels"][key] = {
            "source_digest": source_digest(KERNEL_SOURCES[key]),
            "fetch_kib_raw": fk, "write_kib_raw": wk,
            "hbm_bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024)),
            "dispatches": len(fetch[key]),
            "trace": stats.get(key)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out, stats


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the chunk-forward timings of the other prefill workloads")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the backward pass")
    ap.add_argument("--no-block-ops", action="store_true",
                    help="skip the timings of the block operations around the recurrence")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="cap on oracle threads (the box's CPU share)")
    ap.add_argument("--workload", default=None,
                    help="time only gdn_chunk_fwd on this workload (a key of synth.CONFIGS, "
                         "optionally with the suffix _mamba2_gates or _fp32_gates) and print "
                         "its timing; "
                         "for profiling one kernel in isolation")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward row (gdn_backward and the saved-state pair) "
                         "and print it; for profiling the backward kernels in isolation")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KERNEL_STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 output and exit (no GPU)")
    ap.add_argument("--profile-commands", nargs="*", default=[],
                    help="the rocprofv3 commands that made the CSVs (recorded in the summary)")
    args = ap.parse_args()

    if args.summarize_profiles:
        out, _ = summarize_profiles(*args.summarize_profiles, commands=args.profile_commands)
        print(json.dumps(out, indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_gdn_amd as gdn
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.workload:
        print(json.dumps(single_workload(gdn, synth, torch, dev, args.workload, args.steps,
                                         args.warmup)), flush=True)
        return
    if args.backward_only:
        print(json.dumps(backward_workload(gdn, synth, torch, dev, steps=args.steps,
                                           warmup=args.warmup)), flush=True)
        return
    cfg_c = synth.CONFIGS["gdn2_bf16_train"]
    cfg_d = synth.CONFIGS["gdn2_decode"]
    inp_c = synth.chunk_inputs(cfg_c, device="cuda")
    inp_d = synth.decode_inputs(cfg_d, device="cuda")
    o_c = torch.empty((cfg_c.B, cfg_c.T, cfg_c.Hv, cfg_c.dv), dtype=cfg_c.io_dtype, device=dev)
    s_c = torch.empty((cfg_c.B, cfg_c.Hv, cfg_c.dk, cfg_c.dv), dtype=torch.float32, device=dev)
    o_d = torch.empty((cfg_d.N, cfg_d.Hv, cfg_d.dv), dtype=cfg_d.io_dtype, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gdn.gdn_chunk_fwd(inp_c["q"], inp_c["k"], inp_c["v"], inp_c["beta_or_b"], w=inp_c["w"],
                          g=inp_c["g"], state_in=inp_c["state_in"], state_out=s_c, o=o_c)
        if ev is not None:
            ev[1].record()
        gdn.gdn_decode_step(inp_d["q"], inp_d["k"], inp_d["v"], inp_d["beta_or_b"],
                            inp_d["state"], w=inp_d["w"], g=inp_d["g"], o=o_d)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    chunk_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    chunk_avg = sum(chunk_ms) / len(chunk_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    gate_bytes = 2 if cfg_c.gate_dtype == torch.bfloat16 else 4
    c_bytes, c_flops = chunk_algorithmic(cfg_c, gate_bytes, state_in=inp_c["state_in"] is not None)
    d_bytes, d_flops = decode_algorithmic(cfg_d)
    tokens = cfg_c.B * cfg_c.T
    chunk_tps = tokens / (chunk_avg * 1e-3)
    c_gbps = c_bytes / (chunk_avg * 1e-3) / 1e9
    d_gbps = d_bytes / (dec_avg * 1e-3) / 1e9
    c_tflops = c_flops / (chunk_avg * 1e-3) / 1e12

    def roof(bytes_alg, avg_ms, key, flops=None):
        r = {"bound": "hbm", "achieved": round(bytes_alg / (avg_ms * 1e-3) / 1e9, 1),
             "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(bytes_alg / (avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
             "traffic": measured_traffic(key, bytes_alg),
             "algorithmic_bytes_per_launch": bytes_alg, "avg_launch_ms": round(avg_ms, 4)}
        if flops is not None:
            r["mfma_tflops"] = round(flops / (avg_ms * 1e-3) / 1e12, 1)
            r["mfma_frac"] = round(flops / (avg_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        return r

    roof_c = roof(c_bytes, chunk_avg, "chunk_fwd", c_flops)
    roof_d = roof(d_bytes, dec_avg, "decode_step")
    dominant = "chunk_fwd" if chunk_avg >= dec_avg else "decode_step"
    out = {
        "metric": "tokens/s gated-delta chunk fwd (GDN-2, T=4K) + decode state HBM GB/s",
        "value": round(chunk_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), gates sigmoid/-softplus of N(0,1))",
        "config": {
            "workload": "gdn2_bf16_train chunk fwd + gdn2_decode step",
            "chunk_fwd": {"B": cfg_c.B, "T": cfg_c.T, "H_k": cfg_c.Hk, "H_v": cfg_c.Hv,
                          "d_k": cfg_c.dk, "d_v": cfg_c.dv, "gates": "channel (b, w, g) bf16",
                          "chunk": CHUNK, "state": "fp32, S0=0"},
            "decode": {"N": cfg_d.N, "H_k": cfg_d.Hk, "H_v": cfg_d.Hv, "d_k": cfg_d.dk,
                       "d_v": cfg_d.dv, "gates": "channel bf16", "state": "fp32 in place, 2.15 GB"},
            "global_batch": tokens,
            "seq_len": cfg_c.T,
            "parallelism": "single GPU",
            "operands": "bf16 MFMA operands, fp32 accumulation and state",
        },
        "chunk_fwd_ms": round(chunk_avg, 4),
        "chunk_fwd_GBps": round(c_gbps, 1),
        "chunk_fwd_TFLOPs": round(c_tflops, 1),
        "decode_step_ms": round(dec_avg, 4),
        "decode_state_GBps": round(d_gbps, 1),
        "decode_tokens_per_s": round(cfg_d.N / (dec_avg * 1e-3), 1),
        "roofline": roof_c if dominant == "chunk_fwd" else roof_d,
        "roofline_kernel": dominant,
        "rooflines": {"chunk_fwd": roof_c, "decode_step": roof_d},
        "source_digest": source_digest(),
    }
    out["device_copy_GBps"] = copy_bandwidth(torch, dev)
    if not args.no_secondary:
        out["secondary"] = secondary_chunk_workloads(gdn, synth, torch, dev)
        out["secondary"]["fused_gates"] = fused_gate_workloads(gdn, synth, torch, dev)
    if not args.no_block_ops:
        out["block_ops"] = block_op_workloads(gdn, synth, torch, dev)
    if not args.no_backward:
        out["backward"] = backward_workload(gdn, synth, torch, dev)
    if args.copy_calibration:  # the last GPU work of the process
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                  "cpu_model")}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
