"""Build libgdn.so (and its debug twin libgdn_check.so) in-tree with hipcc for gfx950.

    python gated_delta_rule_gdn_amd/build.py [-v]

(Run as a script: importing the package first would load the library.)

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
LIB_CHECK = os.path.join(PKG, "libgdn_check.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["gdn_api.cpp", "decode.hip", "chunk_fwd.hip", "chunk_fwd_sb.hip", "layer_ops.hip",
           "backward.hip", "noalloc.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


# The product library and its debug twin (-DGDN_CHECK: LDS filled with NaN
# at kernel start, LDS accesses and block indices checked, every call waits
# for its kernels and reports GDN_ERR_CHECK on a violation).
VARIANTS = [(LIB, BUILD_DIR, []),
            (LIB_CHECK, os.path.join(BUILD_DIR, "check"), ["-DGDN_CHECK"])]
MAX_JOBS = 8


def build(verbose: bool = False) -> str:
    jobs = []
    for lib, bdir, flags in VARIANTS:
        os.makedirs(bdir, exist_ok=True)
        for src in SOURCES:
            obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = ["hipcc", *COMMON, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append((lib, src, obj, cmd))
    failed = []
    running = []

    def reap(entry):
        lib, src, obj, p = entry
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        noise = "is not a recognized feature for this target"
        lines = [ln for ln in text.splitlines() if noise not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append((os.path.basename(lib), src))

    for lib, src, obj, cmd in jobs:
        if len(running) >= MAX_JOBS:
            reap(running.pop(0))
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((lib, src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                        stderr=subprocess.STDOUT)))
    for entry in running:
        reap(entry)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for lib, bdir, _ in VARIANTS:
        objs = [os.path.join(bdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        tmp = lib + ".tmp"
        cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
