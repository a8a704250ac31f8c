"""The C-ABI library loads, exports what include/gdn.h declares, and rejects bad
arguments on the host before any launch.  No GPU is needed: every call here
fails validation, which returns before the HIP runtime is touched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

gdn = pytest.importorskip("gated_delta_rule_gdn_amd")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(gdn_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(
        ["gdn_chunk_fwd", "gdn_chunk_fwd_varlen", "gdn_decode_step", "gdn_status_string",
         "gdn_abi_version", "gdn_short_conv", "gdn_gates", "gdn_output_gate", "gdn_backward",
         "gdn_backward_workspace_size", "gdn_backward_varlen",
         "gdn_backward_varlen_workspace_size", "gdn_backward_noalloc",
         "gdn_backward_noalloc_max_bytes", "gdn_chunk_fwd_gated", "gdn_chunk_fwd_save",
         "gdn_backward_saved", "gdn_chunk_fwd_varlen_save", "gdn_backward_varlen_saved",
         "gdn_check_selftest"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.gdn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(gdn_\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(gdn.lib, name)


def test_check_library_exports_every_declared_symbol():
    """The debug twin (-DGDN_CHECK) has the same ABI; loaded here without any
    GPU call."""
    path = os.path.join(os.path.dirname(gdn.gdn.LIB_PATH), "libgdn_check.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(gdn_\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported
    lib = ctypes.CDLL(path)
    lib.gdn_abi_version.restype = ctypes.c_int
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    assert lib.gdn_abi_version() == gdn.abi_version()
    assert lib.gdn_status_string(4).startswith(b"GDN_ERR_CHECK")


def test_version_and_status_strings():
    assert gdn.abi_version() == 9
    for st in range(5):
        s = gdn.status_string(st)
        assert s.startswith("GDN_")
    assert "UNKNOWN" in gdn.status_string(99)


# ---------------------------------------------------------------------------
# Validation: fake, never-dereferenced device addresses.
# ---------------------------------------------------------------------------
BASE = 0x7f0000000000   # 16-byte aligned fake addresses, far apart
STEP = 1 << 36


def _addr(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def _fwd_desc(**kw):
    d = dict(B=2, T=100, H_k=2, H_v=4, d_k=128, d_v=128, io_dtype=gdn.GDN_BF16,
             gate_dtype=gdn.GDN_BF16, gate_mode=gdn.GDN_GATES_CHANNEL, chunk=64, scale=1.0)
    d.update(kw)
    return gdn.GdnFwdDesc(**d)


def _fwd(desc, **ptrs):
    names = ["q", "k", "v", "b", "w", "g", "s_in", "s_out", "o"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w"] = None
    p.update(ptrs)
    return gdn.lib.gdn_chunk_fwd(ctypes.byref(desc) if desc is not None else None,
                                 *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("H_v", 3, 1),            # H_v % H_k != 0
    ("H_k", 0, 1),
    ("d_k", 96, 2),           # unsupported head size
    ("d_v", 256, 2),
    ("chunk", 32, 2),         # only C = 64 is built
    ("io_dtype", 7, 1),
    ("gate_mode", 5, 1),
    ("B", -1, 1),
    ("T", -5, 1),
    ("scale", float("nan"), 1),
    ("scale", float("inf"), 1),
    ("B", 2 ** 30, 2),        # more workgroups than a grid holds
    ("T", 3 * 10 ** 9, 2),    # token index beyond 32 bits of chunk arithmetic
    ("H_v", 2 ** 16, 2),      # a token row of v beyond 2^22 elements
])
def test_fwd_rejects_bad_descriptor(field, value, expected):
    assert _fwd(_fwd_desc(**{field: value})) == expected


def test_fwd_rejects_fp32_io_with_bf16_gates():
    assert _fwd(_fwd_desc(io_dtype=gdn.GDN_F32, gate_dtype=gdn.GDN_BF16)) == gdn.GDN_ERR_UNSUPPORTED


def test_fwd_rejects_null_descriptor():
    assert gdn.lib.gdn_chunk_fwd(None, *([None] * 10)) == gdn.GDN_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["q", "k", "v", "b", "o"])
def test_fwd_rejects_null_required_pointer(name):
    assert _fwd(_fwd_desc(), **{name: None}) == gdn.GDN_ERR_INVALID_ARG


def test_fwd_gate_pointer_rules():
    # channel mode needs w; scalar mode forbids it
    assert _fwd(_fwd_desc(), w=None) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd(_fwd_desc(gate_mode=gdn.GDN_GATES_SCALAR), w=_addr(4)) == gdn.GDN_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["q", "k", "v", "b", "w", "g", "s_in", "s_out", "o"])
def test_fwd_rejects_misaligned_pointer(name):
    idx = ["q", "k", "v", "b", "w", "g", "s_in", "s_out", "o"].index(name)
    assert _fwd(_fwd_desc(), **{name: _addr(idx, 2)}) == gdn.GDN_ERR_INVALID_ARG


def test_fwd_rejects_output_overlapping_input():
    assert _fwd(_fwd_desc(), o=_addr(0, 4096)) == gdn.GDN_ERR_INVALID_ARG      # o inside q
    assert _fwd(_fwd_desc(), s_out=_addr(2, 4096)) == gdn.GDN_ERR_INVALID_ARG  # state_out inside v
    assert _fwd(_fwd_desc(), s_out=_addr(6, 16)) == gdn.GDN_ERR_INVALID_ARG    # partial overlap w/ state_in


def test_fwd_empty_batch_is_a_noop():
    assert _fwd(_fwd_desc(B=0)) == gdn.GDN_OK


def _gated(desc, gates=None, **ptrs):
    """gdn_chunk_fwd_gated with fake pointers; gates defaults to channel raw
    projections with row strides of a fused projection output."""
    names = ["q", "k", "v", "s_in", "s_out", "o"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    p.update(ptrs)
    ch = desc is not None and desc.gate_mode == gdn.GDN_GATES_CHANNEL
    g = dict(a=_addr(10), b=_addr(11), w=_addr(12) if ch else None, A_log=_addr(13),
             dt_bias=_addr(14), ld_a=4096 if ch else 64, ld_b=4096 if ch else 64, ld_w=4096)
    if gates:
        g.update(gates)
    raw = gdn.GdnRawGates(**g)
    return gdn.lib.gdn_chunk_fwd_gated(ctypes.byref(desc) if desc is not None else None,
                                       p["q"], p["k"], p["v"], ctypes.byref(raw),
                                       p["s_in"], p["s_out"], p["o"], None)


@pytest.mark.parametrize("desc_kw,gates,expected", [
    (dict(d_k=64), None, 2),                          # built for d_k = d_v = 128 only
    (dict(d_v=64), None, 2),
    (dict(io_dtype=gdn.GDN_F32, gate_dtype=gdn.GDN_F32), None, 2),
    (dict(gate_dtype=gdn.GDN_F32), None, 2),
    (dict(chunk=32), None, 2),
    (dict(B=-1), None, 1),
    (dict(), dict(b=None), 1),                        # b projection required
    (dict(), dict(w=None), 1),                        # channel gates need w
    (dict(gate_mode=gdn.GDN_GATES_SCALAR), dict(w=_addr(12)), 1),   # scalar gates forbid it
    (dict(), dict(ld_b=100), 1),                      # fewer columns than H_v d_k = 512
    (dict(), dict(ld_a=500), 1),
    (dict(), dict(ld_w=511), 1),
    (dict(), dict(ld_b=1028), 1),                     # channel rows read in 16-byte pieces
    (dict(), dict(b=_addr(11, 8)), 1),
    (dict(), dict(ld_b=2 ** 25), 2),                  # a chunk beyond 32-bit offsets
    (dict(), dict(A_log=_addr(13, 2)), 1),
])
def test_gated_fwd_rejects_bad_arguments(desc_kw, gates, expected):
    assert _gated(_fwd_desc(**desc_kw), gates) == expected


def test_gated_fwd_pointer_rules():
    assert _gated(None) == gdn.GDN_ERR_INVALID_ARG
    assert _gated(_fwd_desc(), q=None) == gdn.GDN_ERR_INVALID_ARG
    assert _gated(_fwd_desc(), o=_addr(5, 2)) == gdn.GDN_ERR_INVALID_ARG       # misaligned o
    assert _gated(_fwd_desc(), o=_addr(11, 64)) == gdn.GDN_ERR_INVALID_ARG     # o inside b
    assert _gated(_fwd_desc(), s_out=_addr(12, 64)) == gdn.GDN_ERR_INVALID_ARG  # state inside w
    # scalar gates: 2-byte projections at any even offset and row stride
    assert _gated(_fwd_desc(gate_mode=gdn.GDN_GATES_SCALAR, B=0),
                  dict(b=_addr(11, 2), ld_b=13, ld_a=13)) == gdn.GDN_OK
    assert _gated(_fwd_desc(B=0)) == gdn.GDN_OK
    assert _gated(_fwd_desc(T=0), s_out=_addr(3)) == gdn.GDN_OK               # in place, nothing to do


def test_fwd_zero_tokens_in_place_state_is_a_noop():
    # T = 0 with state_out == state_in (or no state_out) enqueues nothing.
    assert _fwd(_fwd_desc(T=0), s_out=_addr(6)) == gdn.GDN_OK
    assert _fwd(_fwd_desc(T=0), s_out=None) == gdn.GDN_OK


def _dec_desc(**kw):
    d = dict(N=4, H_k=2, H_v=4, d_k=128, d_v=128, io_dtype=gdn.GDN_BF16, gate_dtype=gdn.GDN_BF16,
             gate_mode=gdn.GDN_GATES_CHANNEL, scale=1.0)
    d.update(kw)
    return gdn.GdnDecodeDesc(**d)


def _dec(desc, **ptrs):
    names = ["q", "k", "v", "b", "w", "g", "s", "o"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w"] = None
    p.update(ptrs)
    return gdn.lib.gdn_decode_step(ctypes.byref(desc), *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("H_v", 5, 1), ("d_k", 32, 2), ("N", -1, 1), ("io_dtype", 3, 1), ("scale", float("nan"), 1),
    ("N", 2 ** 31, 2),        # more workgroups than a grid holds
])
def test_decode_rejects_bad_descriptor(field, value, expected):
    assert _dec(_dec_desc(**{field: value})) == expected


def test_decode_pointer_rules():
    assert _dec(_dec_desc(), s=None) == gdn.GDN_ERR_INVALID_ARG
    assert _dec(_dec_desc(), w=None) == gdn.GDN_ERR_INVALID_ARG
    assert _dec(_dec_desc(), o=_addr(6, 64)) == gdn.GDN_ERR_INVALID_ARG   # o inside state
    assert _dec(_dec_desc(), s=_addr(0, 32)) == gdn.GDN_ERR_INVALID_ARG   # state inside q
    assert _dec(_dec_desc(), q=_addr(0, 8)) == gdn.GDN_ERR_INVALID_ARG    # misaligned
    assert _dec(_dec_desc(N=0)) == gdn.GDN_OK


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 128)
    with pytest.raises(ValueError):
        gdn.gdn_chunk_fwd(q, q, q, torch.zeros(1, 64, 1))


# ---------------------------------------------------------------------------
# Packed sequences (gdn_chunk_fwd_varlen): validation only.
# ---------------------------------------------------------------------------
def _varlen_desc(**kw):
    d = dict(N=3, total_T=300, H_k=2, H_v=4, d_k=128, d_v=128, io_dtype=gdn.GDN_BF16,
             gate_dtype=gdn.GDN_BF16, gate_mode=gdn.GDN_GATES_CHANNEL, chunk=64, scale=1.0)
    d.update(kw)
    return gdn.GdnVarlenDesc(**d)


def _varlen(desc, **ptrs):
    names = ["cu", "q", "k", "v", "b", "w", "g", "s_in", "s_out", "o"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc is not None and desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w"] = None
    p.update(ptrs)
    return gdn.lib.gdn_chunk_fwd_varlen(ctypes.byref(desc) if desc is not None else None,
                                        *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("N", -1, 1),
    ("total_T", -5, 1),
    ("H_v", 3, 1),
    ("d_k", 96, 2),
    ("chunk", 32, 2),
    ("gate_mode", 9, 1),
    ("scale", float("inf"), 1),
])
def test_varlen_rejects_bad_descriptor(field, value, expected):
    assert _varlen(_varlen_desc(**{field: value})) == expected


def test_varlen_null_descriptor_and_offsets():
    assert _varlen(None) == gdn.GDN_ERR_INVALID_ARG
    assert _varlen(_varlen_desc(), cu=None) == gdn.GDN_ERR_INVALID_ARG


def test_varlen_offsets_must_be_8_byte_aligned():
    assert _varlen(_varlen_desc(), cu=_addr(0, 4)) == gdn.GDN_ERR_INVALID_ARG


def test_varlen_offsets_must_not_alias_outputs():
    assert _varlen(_varlen_desc(), cu=_addr(9)) == gdn.GDN_ERR_INVALID_ARG      # == o
    assert _varlen(_varlen_desc(), cu=_addr(8)) == gdn.GDN_ERR_INVALID_ARG      # == state_out


def test_varlen_pointer_checks_of_the_batched_entry_apply():
    assert _varlen(_varlen_desc(), q=None) == gdn.GDN_ERR_INVALID_ARG
    assert _varlen(_varlen_desc(), w=None) == gdn.GDN_ERR_INVALID_ARG          # channel needs w
    assert _varlen(_varlen_desc(), o=_addr(1)) == gdn.GDN_ERR_INVALID_ARG      # o aliases q
    assert _varlen(_varlen_desc(gate_mode=gdn.GDN_GATES_SCALAR), w=_addr(5)) == \
        gdn.GDN_ERR_INVALID_ARG


def test_varlen_nothing_to_do_returns_ok_without_launch():
    assert _varlen(_varlen_desc(N=0), cu=None) == gdn.GDN_OK
    # no token at all and no state to move
    assert _varlen(_varlen_desc(total_T=0), s_out=None) == gdn.GDN_OK
    assert _varlen(_varlen_desc(total_T=0), s_out=_addr(7)) == gdn.GDN_OK    # in place


# ---------------------------------------------------------------------------
# Block operations around the recurrence: short conv, gates, output gate.
# ---------------------------------------------------------------------------
def _conv_desc(**kw):
    d = dict(N=2, total_T=100, ld_x=2 * 2 * 128 + 4 * 128, H_k=2, H_v=4, d_k=128, d_v=128,
             io_dtype=gdn.GDN_BF16, eps=1e-6)
    d.update(kw)
    return gdn.GdnConvDesc(**d)


def _conv(desc, cu=None, **ptrs):
    names = ["x", "w", "s_in", "s_out", "q", "k", "v"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return gdn.lib.gdn_short_conv(ctypes.byref(desc) if desc is not None else None, cu,
                                  *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("N", -1, 1), ("total_T", -1, 1), ("H_k", 0, 1), ("d_k", 96, 2), ("d_v", 32, 2),
    ("io_dtype", 4, 1), ("eps", float("nan"), 1), ("eps", -1.0, 1),
    ("ld_x", 100, 1),          # narrower than the branch
    ("ld_x", 1028, 1),         # rows not 16-byte aligned
    ("total_T", 101, 1),       # equal-length batch needs total_T % N == 0
])
def test_short_conv_rejects_bad_descriptor(field, value, expected):
    assert _conv(_conv_desc(**{field: value})) == expected


@pytest.mark.parametrize("name", ["x", "w", "q", "k", "v"])
def test_short_conv_rejects_null_and_misaligned(name):
    assert _conv(_conv_desc(), **{name: None}) == gdn.GDN_ERR_INVALID_ARG
    assert _conv(_conv_desc(), **{name: _addr(9, 8)}) == gdn.GDN_ERR_INVALID_ARG


def test_short_conv_overlap_rules():
    # an output inside x
    assert _conv(_conv_desc(), q=_addr(0, 256)) == gdn.GDN_ERR_INVALID_ARG
    # k on top of q
    assert _conv(_conv_desc(), k=_addr(4, 16)) == gdn.GDN_ERR_INVALID_ARG
    # state_out partly over state_in
    assert _conv(_conv_desc(), s_out=_addr(2, 32)) == gdn.GDN_ERR_INVALID_ARG
    # offsets must be 8-byte aligned
    assert _conv(_conv_desc(), cu=_addr(8, 4)) == gdn.GDN_ERR_INVALID_ARG


def test_short_conv_nothing_to_do_returns_ok_without_launch():
    assert _conv(_conv_desc(N=0)) == gdn.GDN_OK
    assert _conv(_conv_desc(total_T=0), s_out=None) == gdn.GDN_OK
    assert _conv(_conv_desc(total_T=0), s_out=_addr(2)) == gdn.GDN_OK   # in place, no tokens


def _gate_desc(**kw):
    d = dict(rows=64, ld_a=8, ld_b=8, ld_w=0, H_v=4, d_k=0, d_v=0,
             gate_mode=gdn.GDN_GATES_SCALAR, in_dtype=gdn.GDN_BF16, gate_dtype=gdn.GDN_F32)
    d.update(kw)
    return gdn.GdnGateDesc(**d)


def _gates(desc, **ptrs):
    names = ["a", "b", "w_raw", "A_log", "dt_bias", "g", "beta", "w"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc is not None and desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w_raw"] = p["w"] = None
    p.update(ptrs)
    return gdn.lib.gdn_gates(ctypes.byref(desc) if desc is not None else None,
                             *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("rows", -1, 1), ("H_v", 0, 1), ("gate_mode", 3, 1), ("in_dtype", 9, 1),
    ("gate_dtype", 9, 1), ("ld_a", 3, 1), ("ld_b", 2, 1),
    ("rows", 1 << 31, 2),      # rows * columns must fit 32-bit indices
])
def test_gates_rejects_bad_descriptor(field, value, expected):
    assert _gates(_gate_desc(**{field: value})) == expected


def test_gates_pointer_rules():
    assert _gates(None) == gdn.GDN_ERR_INVALID_ARG
    assert _gates(_gate_desc(), a=None) == gdn.GDN_ERR_INVALID_ARG
    assert _gates(_gate_desc(), w=_addr(7)) == gdn.GDN_ERR_INVALID_ARG     # w in scalar mode
    ch = dict(gate_mode=gdn.GDN_GATES_CHANNEL, d_k=64, d_v=64, ld_a=256, ld_b=256, ld_w=256)
    assert _gates(_gate_desc(**ch), w_raw=None) == gdn.GDN_ERR_INVALID_ARG
    assert _gates(_gate_desc(**{**ch, "ld_w": 100})) == gdn.GDN_ERR_INVALID_ARG
    assert _gates(_gate_desc(**{**ch, "d_k": 0})) == gdn.GDN_ERR_INVALID_ARG
    assert _gates(_gate_desc(), a=_addr(0, 1)) == gdn.GDN_ERR_INVALID_ARG  # bf16 needs 2 bytes
    assert _gates(_gate_desc(), g=_addr(5, 2)) == gdn.GDN_ERR_INVALID_ARG  # fp32 needs 4 bytes
    assert _gates(_gate_desc(), g=_addr(0, 4)) == gdn.GDN_ERR_INVALID_ARG  # g over a_raw
    assert _gates(_gate_desc(), beta=_addr(5, 64)) == gdn.GDN_ERR_INVALID_ARG  # beta over g
    assert _gates(_gate_desc(rows=0)) == gdn.GDN_OK


def _norm_desc(**kw):
    d = dict(rows=64, ld_z=4 * 128, H_v=4, d_v=128, io_dtype=gdn.GDN_BF16, eps=1e-6)
    d.update(kw)
    return gdn.GdnNormDesc(**d)


def _outgate(desc, **ptrs):
    names = ["o", "z", "w", "y"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return gdn.lib.gdn_output_gate(ctypes.byref(desc) if desc is not None else None,
                                   *[p[n] for n in names], None)


@pytest.mark.parametrize("field,value,expected", [
    ("rows", -1, 1), ("H_v", 0, 1), ("d_v", 96, 2), ("io_dtype", 3, 1),
    ("eps", float("inf"), 1), ("ld_z", 100, 1), ("ld_z", 4 * 128 + 4, 1),
])
def test_output_gate_rejects_bad_descriptor(field, value, expected):
    assert _outgate(_norm_desc(**{field: value})) == expected


def test_output_gate_pointer_rules():
    assert _outgate(None) == gdn.GDN_ERR_INVALID_ARG
    for name in ["o", "z", "w", "y"]:
        assert _outgate(_norm_desc(), **{name: None}) == gdn.GDN_ERR_INVALID_ARG
        assert _outgate(_norm_desc(), **{name: _addr(6, 8)}) == gdn.GDN_ERR_INVALID_ARG
    assert _outgate(_norm_desc(), y=_addr(1, 64)) == gdn.GDN_ERR_INVALID_ARG   # y over z
    assert _outgate(_norm_desc(), y=_addr(0, 64)) == gdn.GDN_ERR_INVALID_ARG   # y partly over o
    assert _outgate(_norm_desc(rows=0)) == gdn.GDN_OK


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def _bwd_desc(**kw):
    d = dict(B=2, T=100, H_k=2, H_v=4, d_k=128, d_v=128, io_dtype=gdn.GDN_BF16,
             gate_dtype=gdn.GDN_BF16, gate_mode=gdn.GDN_GATES_CHANNEL, scale=1.0)
    d.update(kw)
    return gdn.GdnBwdDesc(**d)


def _bwd(desc, ws_bytes=None, **ptrs):
    names = ["q", "k", "v", "b", "w", "g", "s_in", "d_o", "d_sT", "ws", "dq", "dk", "dv", "db",
             "dw", "dg", "d_s0"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc is not None and desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w"] = p["dw"] = None
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = gdn.lib.gdn_backward_workspace_size(ctypes.byref(desc)) if desc else 0
    args = [p[n] for n in names]
    return gdn.lib.gdn_backward(ctypes.byref(desc) if desc is not None else None,
                                *args[:10], ctypes.c_size_t(ws_bytes), *args[10:], None)


def test_backward_workspace_size_formula():
    r = lambda x: (x + 255) // 256 * 256
    # channel gates, one value head per key head: bf16 checkpoints and u, no partials
    d = _bwd_desc(B=8, T=4096, H_k=16, H_v=16)
    got = gdn.lib.gdn_backward_workspace_size(ctypes.byref(d))
    ck = 8 * 16 * 257 * 128 * 128 * 2
    u = 8 * 4096 * 16 * 128 * 2
    assert got == r(ck) + r(u)
    assert got < 1.5e9
    # grouped heads (or scalar gates, or fp32): partial row gradients too
    part = (2 * 4 * 8 * 4096 * 32 * 128 + 2 * 8 * 4096 * 32) * 4
    d = _bwd_desc(B=8, T=4096, H_k=16, H_v=32)
    ck2, u2 = 2 * ck, 2 * u
    assert gdn.lib.gdn_backward_workspace_size(ctypes.byref(d)) == r(ck2) + r(u2) + r(part)
    d = _bwd_desc(B=8, T=4096, H_k=16, H_v=16, io_dtype=gdn.GDN_F32, gate_dtype=gdn.GDN_F32,
                  gate_mode=gdn.GDN_GATES_SCALAR)
    part = (2 * 4 * 8 * 4096 * 16 * 128 + 2 * 8 * 4096 * 16) * 4
    assert gdn.lib.gdn_backward_workspace_size(ctypes.byref(d)) == r(2 * ck) + r(2 * u) + r(part)
    assert gdn.lib.gdn_backward_workspace_size(ctypes.byref(_bwd_desc(T=0))) == 0
    assert gdn.lib.gdn_backward_workspace_size(ctypes.byref(_bwd_desc(H_v=3))) == 0
    assert gdn.lib.gdn_backward_workspace_size(None) == 0


@pytest.mark.parametrize("field,value,expected", [
    ("H_v", 3, 1), ("d_k", 96, 2), ("io_dtype", 7, 1), ("gate_mode", 5, 1),
    ("scale", float("nan"), 1), ("B", -1, 1), ("T", -3, 1), ("T", 3 * 10 ** 9, 2)])
def test_backward_rejects_bad_descriptor(field, value, expected):
    assert _bwd(_bwd_desc(**{field: value}), ws_bytes=1 << 40) == expected


def test_backward_rejects_overflowing_token_count():
    """B T beyond int64 is rejected before any arithmetic on it."""
    d = _bwd_desc(B=2 ** 62, T=2 ** 62)
    assert gdn.lib.gdn_backward_workspace_size(ctypes.byref(d)) == 0
    assert _bwd(d, ws_bytes=1 << 40) == gdn.GDN_ERR_INVALID_ARG


def test_backward_pointer_rules():
    assert _bwd(None) == gdn.GDN_ERR_INVALID_ARG
    for name in ["q", "k", "v", "b", "w", "d_o", "ws", "dq", "dk", "dv", "db", "dw"]:
        assert _bwd(_bwd_desc(), **{name: None}) == gdn.GDN_ERR_INVALID_ARG, name
    assert _bwd(_bwd_desc(), ws_bytes=1000) == gdn.GDN_ERR_INVALID_ARG        # too small
    assert _bwd(_bwd_desc(), dg=_addr(15), g=None) == gdn.GDN_ERR_INVALID_ARG  # dg without g
    assert _bwd(_bwd_desc(), dq=_addr(10, 8)) == gdn.GDN_ERR_INVALID_ARG      # misaligned
    assert _bwd(_bwd_desc(), dk=_addr(10, 16)) == gdn.GDN_ERR_INVALID_ARG     # dk over dq
    assert _bwd(_bwd_desc(), dv=_addr(9, 64)) == gdn.GDN_ERR_INVALID_ARG      # dv in workspace
    assert _bwd(_bwd_desc(), db=_addr(0, 64)) == gdn.GDN_ERR_INVALID_ARG      # db over q
    sc = _bwd_desc(gate_mode=gdn.GDN_GATES_SCALAR)
    assert _bwd(sc, dw=_addr(14)) == gdn.GDN_ERR_INVALID_ARG                  # dw in scalar mode
    assert _bwd(_bwd_desc(B=0)) == gdn.GDN_OK
    assert _bwd(_bwd_desc(T=0), d_s0=None) == gdn.GDN_OK


def _fwd_save(desc, ws_bytes=None, **ptrs):
    names = ["q", "k", "v", "b", "w", "g", "s_in", "s_out", "o", "ws"]
    p = {n: _addr(i) for i, n in enumerate(names)}
    if desc.gate_mode == gdn.GDN_GATES_SCALAR:
        p["w"] = None
    p.update(ptrs)
    if ws_bytes is None:
        bd = _bwd_desc(B=desc.B, T=desc.T, H_k=desc.H_k, H_v=desc.H_v, d_k=desc.d_k,
                       d_v=desc.d_v, io_dtype=desc.io_dtype, gate_dtype=desc.gate_dtype,
                       gate_mode=desc.gate_mode, scale=desc.scale)
        ws_bytes = gdn.lib.gdn_backward_workspace_size(ctypes.byref(bd))
    args = [p[n] for n in names]
    return gdn.lib.gdn_chunk_fwd_save(ctypes.byref(desc), *args, ctypes.c_size_t(ws_bytes), None)


def test_forward_save_validation():
    """The forward's checks, then the workspace's: present, aligned, large
    enough, overlapping nothing (no launch happens on a rejected call)."""
    assert _fwd_save(_fwd_desc(chunk=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert _fwd_save(_fwd_desc(H_v=3)) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd_save(_fwd_desc(), ws=None) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd_save(_fwd_desc(), ws=_addr(9, 8)) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd_save(_fwd_desc(), ws_bytes=1000) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd_save(_fwd_desc(), ws=_addr(8, 64)) == gdn.GDN_ERR_INVALID_ARG   # over o
    assert _fwd_save(_fwd_desc(), q=None) == gdn.GDN_ERR_INVALID_ARG
    assert _fwd_save(_fwd_desc(B=0)) == gdn.GDN_OK


def test_forward_varlen_save_validation():
    d = gdn.GdnVarlenDesc(N=3, total_T=100, H_k=2, H_v=4, d_k=128, d_v=128,
                          io_dtype=gdn.GDN_BF16, gate_dtype=gdn.GDN_BF16,
                          gate_mode=gdn.GDN_GATES_CHANNEL, chunk=64, scale=1.0)
    bd = gdn.GdnBwdVarlenDesc(N=3, total_T=100, H_k=2, H_v=4, d_k=128, d_v=128,
                              io_dtype=gdn.GDN_BF16, gate_dtype=gdn.GDN_BF16,
                              gate_mode=gdn.GDN_GATES_CHANNEL, scale=1.0)
    need = gdn.lib.gdn_backward_varlen_workspace_size(ctypes.byref(bd))
    names = ["q", "k", "v", "b", "w", "g", "s_in", "s_out", "o", "ws"]

    def call(cu=_addr(11), ws_bytes=need, **ptrs):
        p = {n: _addr(i) for i, n in enumerate(names)}
        p.update(ptrs)
        args = [p[n] for n in names]
        return gdn.lib.gdn_chunk_fwd_varlen_save(ctypes.byref(d), cu, *args,
                                                 ctypes.c_size_t(ws_bytes), None)

    assert call(ws=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == gdn.GDN_ERR_INVALID_ARG
    assert call(ws=_addr(11)) == gdn.GDN_ERR_INVALID_ARG      # over cu_seqlens
    assert call(ws=_addr(2, 32)) == gdn.GDN_ERR_INVALID_ARG   # over v
    assert call(cu=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(cu=_addr(11, 4)) == gdn.GDN_ERR_INVALID_ARG   # misaligned offsets
    assert gdn.lib.gdn_chunk_fwd_varlen_save(None, None, *([None] * 10), ctypes.c_size_t(0),
                                             None) == gdn.GDN_ERR_INVALID_ARG


def test_backward_saved_validation():
    """gdn_backward_saved takes gdn_backward's arguments and checks."""
    names = ["q", "k", "v", "b", "w", "g", "s_in", "d_o", "d_sT", "ws", "dq", "dk", "dv", "db",
             "dw", "dg", "d_s0"]

    def call(desc, ws_bytes=None, **ptrs):
        p = {n: _addr(i) for i, n in enumerate(names)}
        p.update(ptrs)
        if ws_bytes is None:
            ws_bytes = gdn.lib.gdn_backward_workspace_size(ctypes.byref(desc))
        args = [p[n] for n in names]
        return gdn.lib.gdn_backward_saved(ctypes.byref(desc), *args[:10],
                                          ctypes.c_size_t(ws_bytes), *args[10:], None)

    assert call(_bwd_desc(), ws_bytes=1000) == gdn.GDN_ERR_INVALID_ARG
    assert call(_bwd_desc(), dq=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(_bwd_desc(), dk=_addr(10, 16)) == gdn.GDN_ERR_INVALID_ARG
    assert call(_bwd_desc(H_v=3), ws_bytes=1 << 40) == gdn.GDN_ERR_INVALID_ARG
    assert call(_bwd_desc(B=0)) == gdn.GDN_OK
    assert gdn.lib.gdn_backward_saved(None, *([None] * 10), ctypes.c_size_t(0),
                                      *([None] * 7), None) == gdn.GDN_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# The product path has no fallback and no dependency on the oracle.
# ---------------------------------------------------------------------------
def test_binding_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libgdn.so cannot be imported."""
    import shutil
    import sys
    pkg = os.path.join(ROOT, "gated_delta_rule_gdn_amd")
    dst = tmp_path / "gated_delta_rule_gdn_amd"
    dst.mkdir()
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            shutil.copy(os.path.join(pkg, name), dst / name)
    r = subprocess.run([sys.executable, "-c", "import gated_delta_rule_gdn_amd"],
                       cwd=tmp_path, capture_output=True, text=True,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libgdn.so" in r.stderr


def test_product_sources_never_reference_the_oracle():
    pkg = os.path.join(ROOT, "gated_delta_rule_gdn_amd")
    for base, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".cpp", ".hpp")):
                text = open(os.path.join(base, name)).read()
                assert not re.search(r"\boracle\b", text), os.path.join(base, name)


def test_backward_varlen_validation():
    d = gdn.GdnBwdVarlenDesc(N=3, total_T=100, H_k=2, H_v=4, d_k=128, d_v=128,
                             io_dtype=gdn.GDN_BF16, gate_dtype=gdn.GDN_BF16,
                             gate_mode=gdn.GDN_GATES_CHANNEL, scale=1.0)
    n = gdn.lib.gdn_backward_varlen_workspace_size(ctypes.byref(d))
    r = lambda x: (x + 255) // 256 * 256
    ck = 4 * (100 // 16 + 2 * 3 + 2) * 128 * 128 * 2
    u = 100 * 4 * 128 * 2
    part = (2 * 4 * 100 * 4 * 128 + 2 * 100 * 4) * 4
    assert n == r(ck) + r(u) + r(part)
    names = ["q", "k", "v", "b", "w", "g", "s_in", "d_o", "d_sT", "ws", "dq", "dk", "dv", "db",
             "dw", "dg", "d_s0"]

    def call(cu, **ptrs):
        p = {nm: _addr(i) for i, nm in enumerate(names)}
        p.update(ptrs)
        args = [p[nm] for nm in names]
        return gdn.lib.gdn_backward_varlen(ctypes.byref(d), cu, *args[:10], ctypes.c_size_t(n),
                                           *args[10:], None)
    assert call(None) == gdn.GDN_ERR_INVALID_ARG                    # offsets required
    assert call(_addr(20, 4)) == gdn.GDN_ERR_INVALID_ARG            # misaligned offsets
    assert call(_addr(10, 0)) == gdn.GDN_ERR_INVALID_ARG            # offsets inside dq
    assert call(_addr(9, 64)) == gdn.GDN_ERR_INVALID_ARG            # offsets inside the workspace
