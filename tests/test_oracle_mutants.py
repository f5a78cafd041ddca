"""The pins catch plausible mistakes in the oracle (CPU only).

Each case copies the oracle, the tests and the input generators to a scratch
directory, plants one mistake in the copy of `oracle/rmsn_ref.c` -- the kind
a transcription of the association could plausibly contain -- rebuilds it, and
runs the pin suite (`test_oracle_pins.py`) against it: the suite must fail. A
control copy with no mistake must pass, so a failure is the mistake's doing.
The repository's own oracle is never touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (text in oracle/rmsn_ref.c, replacement)
MUTANTS = {
    "group totals combined in order (W0+W1)+(W2+W3)": (
        "float a = W[0] + W[2];\n    float b = W[1] + W[3];",
        "float a = W[0] + W[1];\n    float b = W[2] + W[3];"),
    "adjacent-pair halving inside a group": (
        "for (int j = 0; j < s; ++j) q[j] = q[j] + q[j + s];",
        "for (int j = 0; j < s; ++j) q[j] = q[2 * j] + q[2 * j + 1];"),
    "square rounded before the add (no fused multiply-add)": (
        "acc = fmaf(xd, xd, acc);",
        "acc = acc + xd * xd;"),
    "128 lane chains": (
        "#define LANES 256",
        "#define LANES 128"),
    "mean by multiplying with 1/n": (
        "float m = ss / (float)n;",
        "float m = ss * (1.0f / (float)n);"),
    "inverse as one rounding of 1/sqrt in double": (
        "float inv = 1.0f / r;",
        "float inv = (float)(1.0 / sqrt((double)t)); (void)r;"),
    "weight applied first, x * (inv * w)": (
        "float a = x[d] * inv;  /* step 8, left to right */\n        y[d] = a * w[d];",
        "float a = inv * w[d];\n        y[d] = x[d] * a;"),
    "bf16 narrowing by truncation": (
        "u += 0x7FFFu + lsb;",
        "(void)lsb;"),
}


def _scratch(tmp_path, mutation):
    dst = tmp_path / "copy"
    for name in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, name), dst / name,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst / "pytest.ini")
    if mutation is not None:
        src = dst / "oracle" / "rmsn_ref.c"
        text = src.read_text()
        old, new = mutation
        assert text.count(old) == 1, f"mutation site not found once: {old!r}"
        src.write_text(text.replace(old, new))
    subprocess.check_call([sys.executable, "oracle/build.py"], cwd=dst,
                          stdout=subprocess.DEVNULL)
    return dst


def _pins(dst):
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                           "-p", "no:cacheprovider"], cwd=dst, env=env, capture_output=True,
                          text=True, timeout=600)


def test_control_copy_passes(tmp_path):
    r = _pins(_scratch(tmp_path, None))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_the_mistake(tmp_path, name):
    r = _pins(_scratch(tmp_path, MUTANTS[name]))
    assert r.returncode != 0, f"no pin caught: {name}\n{r.stdout[-2000:]}"
