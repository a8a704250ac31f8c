"""GPU parity under the debug library libgdn_check.so (built with -DGDN_CHECK).

That build fills each kernel's LDS with NaN before the kernel uses it, checks
every LDS access made through the kernels' fragment, store and
transposing-read helpers against the kernel's LDS size, checks the chunk
kernel's block indices against its layout, and makes every call wait for its
kernels and return GDN_ERR_CHECK (raised by the binding) on a violation.

Each case below is an existing parity test (same inputs, same oracle, same
tolerance) run with that library in place of libgdn.so: passing means no
kernel on the path read LDS that nothing had written (a NaN would reach the
outputs) and no checked access left the layout.  The cases cover every
sub-block kind of the bf16 chunk kernel (factored, floored, exact) in both
gate modes, both head sizes, the fp32 chunk kernel, ragged tails, packed
sequences (the in-kernel ranking uses LDS too), raw gates on the exact path,
the decode step and the backward (plain, saved states, packed).
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_gdn_amd.gdn as binding  # noqa: E402
import test_gpu_backward as tb  # noqa: E402
import test_gpu_chunk as tc  # noqa: E402
import test_gpu_decode as td  # noqa: E402
import test_gpu_gated as tg  # noqa: E402
import test_gpu_saved as ts  # noqa: E402
import test_gpu_varlen as tv  # noqa: E402

CHECK_LIB = os.path.join(os.path.dirname(binding.LIB_PATH), "libgdn_check.so")

BF, F32 = torch.bfloat16, torch.float32
CASES = {
    "chunk sub-block transitions, channel gates": lambda: tc.test_sub_block_transitions_bf16(True),
    "chunk sub-block transitions, scalar gates": lambda: tc.test_sub_block_transitions_bf16(False),
    "chunk strong decays around an undecayed pair": tc.test_reference_ratio_underflow_channel,
    "chunk d_k 64, channel, bf16": lambda: tc.test_variants(64, 64, True, BF, BF),
    "chunk d_k 64 d_v 128, scalar, bf16": lambda: tc.test_variants(64, 128, False, BF, BF),
    "chunk d 128, channel, bf16 io fp32 gates": lambda: tc.test_variants(128, 128, True, BF, F32),
    "chunk fp32 kernel, channel": lambda: tc.test_variants(128, 64, True, F32, F32),
    "chunk fp32 small workload": tc.test_fp32_small_workload,
    "chunk ragged T=1 bf16": lambda: tc.test_ragged_lengths(1, BF),
    "chunk ragged T=65 bf16": lambda: tc.test_ragged_lengths(65, BF),
    "chunk ragged T=100 fp32": lambda: tc.test_ragged_lengths(100, F32),
    "chunk growing state": lambda: tc.test_growing_state_within_range(True),
    "packed sequences, channel, bf16": lambda: tv.test_packed_sequences_match_oracle_per_sequence(True, BF, BF),
    "packed sequences, scalar, bf16": lambda: tv.test_packed_sequences_match_oracle_per_sequence(False, BF, BF),
    "packed, empty sequences": tv.test_empty_sequences_pass_the_state_through,
    "raw gates on the exact path, channel": lambda: tg.test_gated_fwd_exact_path(True),
    "raw gates on the exact path, scalar": lambda: tg.test_gated_fwd_exact_path(False),
    "decode, channel, bf16": lambda: td.test_decode_small_all_variants(128, 128, True, BF, BF),
    "decode, scalar, d 64": lambda: td.test_decode_small_all_variants(64, 64, False, BF, BF),
    "backward, channel, bf16": lambda: tb.test_backward_matches_oracle(True, 128, 128, BF, BF),
    "backward, scalar, fp32": lambda: tb.test_backward_matches_oracle(False, 64, 128, F32, F32),
    "backward, mixed decay blocks (term by term)": lambda: tb.test_backward_mixed_decay_blocks(BF),
    "backward, ragged T=17": lambda: tb.test_backward_ragged_lengths(17),
    "backward, packed sequences": lambda: tb.test_backward_varlen_matches_oracle_per_sequence(True),
    "saved states, channel": lambda: ts.test_saved_bf16_matches_oracle(True, 128, 128, 2, 2),
    "saved states, scalar, grouped": lambda: ts.test_saved_bf16_matches_oracle(False, 64, 128, 1, 2),
}


@pytest.fixture(scope="module")
def check_library():
    """The debug library in place of libgdn.so for the duration of the module."""
    assert os.path.exists(CHECK_LIB), f"{CHECK_LIB} is missing: run the build"
    saved_path, saved_lib = binding.LIB_PATH, binding.lib
    binding.LIB_PATH = CHECK_LIB
    try:
        lib = binding._load()
    finally:
        binding.LIB_PATH = saved_path
    binding.lib = lib
    yield lib
    binding.lib = saved_lib


def test_check_status_is_named(check_library):
    assert check_library.gdn_status_string(4).startswith(b"GDN_ERR_CHECK")


def test_selftest_counts_a_planted_unmade_access(check_library):
    """The checks fire: the self-test kernel computes one address past its LDS
    per lane (counted, never dereferenced) and reads LDS it never wrote (in
    bounds), which the debug build's fill leaves at NaN."""
    out = torch.zeros(64, device="cuda")
    assert binding.check_selftest(out) == binding.GDN_OK
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # the counter was reset: an ordinary call afterwards still succeeds
    tc.test_ragged_lengths(1, BF)


def test_selftest_is_unsupported_in_the_normal_library():
    normal = ctypes.CDLL(binding.LIB_PATH)   # libgdn.so (already loaded by the binding)
    normal.gdn_check_selftest.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    normal.gdn_check_selftest.restype = ctypes.c_int
    out = torch.zeros(64, device="cuda")
    assert normal.gdn_check_selftest(binding._ptr(out), binding._stream(None)) == \
        binding.GDN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out == 0).all()


@pytest.mark.parametrize("case", list(CASES))
def test_parity_under_lds_checks(check_library, case):
    CASES[case]()
