"""Host code under the sanitizers (CPU only).

* The oracle, rebuilt with gcc's UndefinedBehaviorSanitizer (aborting on the
  first report), runs the whole pin suite.
* The library's host code (validation, planning, options, the C ABI), rebuilt
  with clang's AddressSanitizer and, separately, its UndefinedBehaviorSanitizer
  on the host side only (the device code is built as usual), runs the CPU ABI
  tests with the sanitizer runtime preloaded. This one builds the library twice
  with hipcc (about a minute each), so it runs only when RMSN_SANITIZE=1.

Everything happens in a scratch copy; the repository's builds are not touched.
"""
import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy(dst, names):
    for name in names:
        src = os.path.join(ROOT, name)
        if os.path.isdir(src):
            shutil.copytree(src, dst / name, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
        else:
            shutil.copy(src, dst / name)


def _pytest(cwd, test_file, env_extra=None):
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, "-m", "pytest", test_file, "-x", "-q",
                           "-p", "no:cacheprovider"], cwd=cwd, env=env, capture_output=True,
                          text=True, timeout=900)


def test_oracle_pins_under_ubsan(tmp_path):
    dst = tmp_path / "copy"
    dst.mkdir()
    _copy(dst, ["oracle", "tests", "workloads", "pytest.ini"])
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-D_POSIX_C_SOURCE=200809L",
                           "-fsanitize=undefined", "-fno-sanitize-recover=all",
                           "-o", str(dst / "oracle" / "librmsn_ref.so"),
                           str(dst / "oracle" / "rmsn_ref.c"), "-lm", "-lpthread"])
    r = _pytest(dst, "tests/test_oracle_pins.py")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def _clang_runtime(name):
    hits = glob.glob(f"/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.{name}-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.skipif(os.environ.get("RMSN_SANITIZE") != "1",
                    reason="builds the library twice with hipcc; set RMSN_SANITIZE=1")
@pytest.mark.parametrize("sanitizer,runtime,options", [
    ("address", "asan", {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"}),
    ("undefined", "ubsan_standalone", {"UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
])
def test_library_host_code_under_sanitizer(tmp_path, sanitizer, runtime, options):
    rt = _clang_runtime(runtime)
    if rt is None:
        pytest.skip(f"no clang {runtime} runtime found")
    dst = tmp_path / "copy"
    dst.mkdir()
    _copy(dst, ["row_wise_rmsnorm_amd", "include", "oracle", "tests", "workloads", "pytest.ini",
                "bench.py", "__graft_entry__.py"])
    pkg = dst / "row_wise_rmsnorm_amd"
    csrc = pkg / "csrc"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-ffp-contract=off", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             "-I", str(dst / "include"), "-I", str(csrc),
             "-Xarch_host", f"-fsanitize={sanitizer}"]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    # the library's own list of objects and their per-object flags
    spec = importlib.util.spec_from_file_location("rmsn_build_copy", str(pkg / "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)

    def link(out, units):
        objs = []
        for i, (src, extra) in enumerate(units):
            obj = str(tmp_path / f"{out}.{i}.o")
            subprocess.check_call([hipcc, *flags, *extra, "-c", "-o", obj, str(csrc / src)])
            objs.append(obj)
        subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
                               "-Xarch_host", f"-fsanitize={sanitizer}", "-o", str(pkg / out),
                               *objs])

    link("librmsnorm_amd.so", build.UNITS)
    link("librmsnorm_amd_l128.so", build.UNITS128)
    r = _pytest(dst, "tests/test_abi_cpu.py", {"LD_PRELOAD": rt, **options})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
