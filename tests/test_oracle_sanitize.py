"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
entry point on small odd shapes in exact-size heap buffers, with the
recurrent/chunkwise and decode/recurrent agreements checked in the same run
(oracle/sanitize_check.c).  Host code only."""
import os
import shutil
import subprocess

import pytest

import oracle.build as obuild


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    obuild.build_sanitize_check(exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
