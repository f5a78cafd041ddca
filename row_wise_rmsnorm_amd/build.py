"""Build the gfx950 HIP libraries in place:
  row_wise_rmsnorm_amd/librmsnorm_amd.so       the library (256 lane chains)
  row_wise_rmsnorm_amd/librmsnorm_amd_l128.so  the 128-lane build (the sum of
                                               squares on 128 threads, as the
                                               lecture's kernel; same C ABI)

hipcc cross-compiles for gfx950 without a GPU present. Each source is compiled
to an object of its own (side by side), then the objects are linked. Floating
point: contraction off (-ffp-contract=off), no fast-math, HIP's default
correctly rounded binary32 division and square root; packed-FP32 instructions
are disabled for the device code.

Kernel arguments: the kernels are built with their first 16 arguments
preloaded into SGPRs by the dispatcher (PRELOAD), so a kernel's first loads do
not wait for a scalar load of its argument segment. The descriptor kernels
(rmsn_desc.hip) are built both ways: preloaded for the launches a sequence
graph records, and loading their own arguments for launches enqueued one by
one, where preloading measured slower.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsnorm_amd.so")
LIB128 = os.path.join(HERE, "librmsnorm_amd_l128.so")
ARCH = os.environ.get("RMSN_OFFLOAD_ARCH", "gfx950")

PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]

# (source, extra flags) per object
UNITS = [
    ("rmsn_kernels.hip", PRELOAD),
    ("rmsn_desc.hip", PRELOAD + ["-DRMSN_DESC_PRELOADED=1"]),
    ("rmsn_desc.hip", ["-DRMSN_DESC_PRELOADED=0"]),
    ("rmsn_persistent.hip", PRELOAD),
    ("rmsn_wide.hip", PRELOAD),
    ("rmsn_aux.hip", PRELOAD),
    ("rmsn_api.hip", PRELOAD),
    ("rmsn_plan.cpp", []),
]
UNITS128 = [(src, extra + ["-DRMSN_LANES=128"]) for src, extra in [
    ("rmsn_kernels_l128.hip", PRELOAD),
    ("rmsn_aux.hip", PRELOAD),
    ("rmsn_api.hip", PRELOAD),
    ("rmsn_plan.cpp", []),
]]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print("[hip] " + " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _link(out, units, verbose, jobs):
    with tempfile.TemporaryDirectory(prefix="rmsn_build_") as tmpdir:
        objs, cmds = [], []
        for i, (src, extra) in enumerate(units):
            obj = os.path.join(tmpdir, f"{i}_{os.path.splitext(src)[0]}.o")
            objs.append(obj)
            cmds.append([_hipcc(), *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)])
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, out)


def build(verbose=True, jobs=None):
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    _link(LIB, UNITS, verbose, jobs)
    _link(LIB128, UNITS128, verbose, jobs)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
