"""Compile the CPU oracle (plain C, gcc, OpenMP) into ``oracle/liboracle.so``.

Test infrastructure: building the checker is not using it.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    src = os.path.join(_HERE, "gdn_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sanitize_check(out, verbose=False):
    """Compile sanitize_check.c with the oracle into the executable `out`,
    with AddressSanitizer and UndefinedBehaviorSanitizer (host code; gcc)."""
    srcs = [os.path.join(_HERE, "sanitize_check.c"), os.path.join(_HERE, "gdn_oracle.c")]
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Wextra", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", out, *srcs, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
