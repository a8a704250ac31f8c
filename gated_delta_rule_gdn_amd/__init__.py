"""Gated delta rule (GDN-2 / Gated DeltaNet / DeltaNet) on AMD MI355X (gfx950).

The computation lives in libgdn.so (C ABI, include/gdn.h), built from the HIP
sources under csrc/.  This package holds the thin ctypes binding only.
"""
from .gdn import (  # noqa: F401
    GDN_BF16, GDN_ERR_CHECK, GDN_ERR_HIP, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_F32,
    GDN_GATES_CHANNEL, GDN_GATES_SCALAR, GDN_OK, GdnBwdDesc, GdnBwdVarlenDesc, GdnConvDesc, GdnDecodeDesc, GdnError,
    GdnFwdDesc, GdnGateDesc, GdnNormDesc, GdnRawGates, GdnVarlenDesc, abi_version, check_selftest, gdn_backward,
    gdn_backward_noalloc, gdn_backward_noalloc_max_bytes, gdn_backward_saved,
    gdn_backward_varlen, gdn_backward_varlen_saved, gdn_backward_workspace_size, gdn_chunk_fwd,
    gdn_chunk_fwd_gated, gdn_chunk_fwd_save, gdn_chunk_fwd_varlen, gdn_chunk_fwd_varlen_save, gdn_decode_step, gdn_gates, gdn_output_gate, gdn_short_conv, lib,
    status_string,
)
