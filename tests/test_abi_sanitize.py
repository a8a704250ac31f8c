"""The C ABI layer (gdn_api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, host code only: g++ builds it with stub kernel
launchers (tests/abi_check/launch_stubs.cpp) and a driver
(tests/abi_check/abi_check.cpp) that calls every entry point over a grid of
valid and absurd descriptors (negative, huge and overflowing sizes, unknown
dtypes and modes, non-finite scales) with fake device addresses and with
exact-size host buffers.  Any out-of-bounds access or signed overflow in the
validation aborts the run; a call that returns an error must have launched
nothing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_check")
    src = [os.path.join(ROOT, "gated_delta_rule_gdn_amd", "csrc", "gdn_api.cpp"),
           os.path.join(ROOT, "tests", "abi_check", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "abi_check", "abi_check.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "gated_delta_rule_gdn_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *src, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
