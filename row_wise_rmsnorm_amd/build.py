"""Build the gfx950 HIP libraries in place:
  row_wise_rmsnorm_amd/librmsnorm_amd.so       the library (256 lane chains)
  row_wise_rmsnorm_amd/librmsnorm_amd_l128.so  the 128-lane build (the sum of
                                               squares on 128 threads, as the
                                               lecture's kernel; same C ABI)

hipcc cross-compiles for gfx950 without a GPU present. Floating point:
contraction off (-ffp-contract=off), no fast-math, HIP's default correctly
rounded binary32 division and square root; packed-FP32 instructions are
disabled for the device code. Kernel arguments are preloaded into SGPRs by
the dispatcher (the first 16 arguments), so a kernel's first loads do not wait
for a scalar load of its argument segment.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "librmsnorm_amd.so")
LIB128 = os.path.join(HERE, "librmsnorm_amd_l128.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in
           ("rmsn_kernels.hip", "rmsn_persistent.hip", "rmsn_wide.hip", "rmsn_aux.hip",
            "rmsn_api.hip", "rmsn_plan.cpp")]
SOURCES128 = [os.path.join(HERE, "csrc", f) for f in
              ("rmsn_kernels_l128.hip", "rmsn_aux.hip", "rmsn_api.hip", "rmsn_plan.cpp")]
ARCH = os.environ.get("RMSN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(HERE, "csrc"),
]


def _compile(out, sources, extra, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *extra, "-o", tmp, *sources]
    if verbose:
        print("[hip] " + " ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose=True):
    _compile(LIB, SOURCES, [], verbose)
    _compile(LIB128, SOURCES128, ["-DRMSN_LANES=128"], verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
