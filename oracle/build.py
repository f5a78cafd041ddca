"""Build the CPU oracle (test infrastructure) into oracle/librmsn_ref.so.

gcc, -O2 with contraction off and no fast-math, so binary32 arithmetic is
the IEEE operations the source spells out. fmaf resolves to glibc's correctly
rounded fused multiply-add.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "librmsn_ref.so")
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-D_POSIX_C_SOURCE=200809L"]


def build(verbose=True):
    src = os.path.join(HERE, "rmsn_ref.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print("[oracle] " + " ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
