"""The eager decode-step arm when the HIP runtime keeps kernel arguments in
host memory (HIP_FORCE_DEV_KERNARG=0).

The library holds two builds of its descriptor kernels, one with the kernel
arguments preloaded into SGPRs by the dispatcher and one whose kernels load
them; eager launches take the preloaded build only under that setting, which
the library reads once per process. So the check runs in a child process with
the variable set: the eager sequence, plain and positioned, is compared bit for
bit with the CPU oracle, as the default process's tests do for the other build.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import oracle
import row_wise_rmsnorm_amd as rn
import workloads as wl

dev = torch.device("cuda", 0)
rows = wl.decode()[:40]
xs = [torch.from_numpy(x).to(dev) for x, _ in rows]
ws = [torch.from_numpy(w).to(dev) for _, w in rows]
ys = [torch.full_like(t, float("nan")) for t in xs]
table, widths = rn.make_table(list(zip(xs, ws, ys)))
rn.rmsnorm_sequence_eager(table, widths, wl.EPS, rn.F32)
torch.cuda.synchronize()
for i, ((x, w), y) in enumerate(zip(rows, ys)):
    want = oracle.row_f32(x, w, wl.EPS).view(np.uint32)
    got = y.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want), f"eager norm {i} differs from the oracle"

# positioned: two positions of each row, x and y at base + pos * pitch
n = 512
period = 2
xb = [torch.from_numpy(np.concatenate([wl.misc_f32(7000 + 10 * j + p, n)[0]
                                       for p in range(period)])).to(dev) for j in range(6)]
wb = [torch.from_numpy(wl.misc_f32(7500 + j, n)[1]).to(dev) for j in range(6)]
yb = [torch.full((period * n,), float("nan"), dtype=torch.float32, device=dev) for _ in range(6)]
ptable, pwidths = rn.make_table([(x[:n], w, y[:n]) for x, w, y in zip(xb, wb, yb)])
pos = torch.zeros(1, dtype=torch.int64, device=dev)
for step in range(period):
    rn.rmsnorm_sequence_eager(ptable, pwidths, wl.EPS, rn.F32, position=(pos, 4 * n, 4 * n, period))
torch.cuda.synchronize()
assert int(pos.item()) == 0, "the position did not wrap"
for j in range(6):
    for p in range(period):
        x = xb[j][p * n:(p + 1) * n].cpu().numpy()
        want = oracle.row_f32(x, wb[j].cpu().numpy(), wl.EPS).view(np.uint32)
        got = yb[j][p * n:(p + 1) * n].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, want), f"positioned norm {j} position {p} differs"
print("OK", flush=True)
"""


def test_eager_sequence_with_host_memory_kernel_arguments():
    env = dict(os.environ)
    env["HIP_FORCE_DEV_KERNARG"] = "0"
    print("[gpu] eager sequence in a child process, HIP_FORCE_DEV_KERNARG=0", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "OK" in r.stdout
