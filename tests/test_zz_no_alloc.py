"""rmsnorm_batched_rows_noalloc, the entry point for callers that cannot
allocate: the same launches as rmsnorm_batched_rows_ws with the WIDE path's
group totals in the library's own per-GPU device array. Called through the C
ABI (ctypes, device pointers from torch tensors) and compared bit for bit with
rmsnorm_batched_rows_ws on the same inputs; two calls in a row, the second
with fewer, narrower rows, so the second runs on what the first left in the
library's array. A few rows are also checked against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import (assert_bits_bf16, assert_bits_f32, bf16_host, dev, f32_host, say,
                      to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    yield m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)


def _inputs(kind, rows, n, item):
    xs, w = [], None
    for r in range(rows):
        x, wr = wl.misc_f32(item * 1000 + r, n)
        xs.append(x)
        w = wr if w is None else w
    x = np.stack(xs)
    if kind == "bf16":
        return wl.to_bf16_bits(x), wl.to_bf16_bits(w)
    return x, w


def _dev(kind, a):
    return to_dev_bf16(a) if kind == "bf16" else to_dev_f32(a)


def _host(kind, t):
    return bf16_host(t) if kind == "bf16" else f32_host(t)


def _check(kind, got, want, what):
    (assert_bits_bf16 if kind == "bf16" else assert_bits_f32)(got, want, what)


def _call_ws(rn, code, xd, wd, yd, ws):
    rows, n = xd.shape
    st = rn.lib().rmsnorm_batched_rows_ws(code, xd.data_ptr(), n, wd.data_ptr(), yd.data_ptr(),
                                          n, rows, n, ctypes.c_float(wl.EPS), ws.data_ptr(),
                                          ws.numel(), None)
    assert st == rn.RMSN_OK, rn.last_error()


def _call_noalloc(rn, code, xd, wd, yd):
    rows, n = xd.shape
    st = rn.lib().rmsnorm_batched_rows_noalloc(code, xd.data_ptr(), n, wd.data_ptr(),
                                               yd.data_ptr(), n, rows, n,
                                               ctypes.c_float(wl.EPS), None)
    assert st == rn.RMSN_OK, rn.last_error()


# (rows, n) of the first call, then of the second (fewer rows, narrower):
# every shape takes the WIDE path, the one that uses the workspace.
CASES = [("f32", (6, 1 << 16), (2, 1 << 14)),
         ("bf16", (5, 1 << 17), (3, 40000))]


@pytest.mark.parametrize("kind,first,second", CASES)
def test_noalloc_equals_workspace_entry_point(rn, kind, first, second):
    code = rn.BF16 if kind == "bf16" else rn.F32
    torch.cuda.set_device(dev())
    for call, (rows, n) in enumerate((first, second)):
        plan, need = rn.workspace_query(code, rows, n)
        assert plan["path"] == rn.PATH_WIDE and need == 16 * rows, (plan, need)
        say(f"noalloc {kind} call {call}: {rows} x {n} (WIDE)")
        x, w = _inputs(kind, rows, n, 900 + call)
        xd, wd = _dev(kind, x), _dev(kind, w)
        y_ws = torch.full_like(xd, float("nan"))
        y_na = torch.full_like(xd, float("nan"))
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev())
        _call_ws(rn, code, xd, wd, y_ws, ws)
        _call_noalloc(rn, code, xd, wd, y_na)
        torch.cuda.synchronize()
        got, want = _host(kind, y_na), _host(kind, y_ws)
        _check(kind, got, want, f"{kind} call {call}: noalloc vs workspace entry point")
        for r in (0, rows - 1):
            ref, _ = oracle.rows(x[r:r + 1], w, wl.EPS)
            _check(kind, got[r:r + 1], ref, f"{kind} call {call} row {r}: noalloc vs oracle")


def test_noalloc_without_wide_plan_equals_plain_entry_point(rn):
    """A batch the plan does not take WIDE for (the 64-row bf16 batch) runs
    exactly as rmsnorm_batched_rows."""
    xb, wb = wl.batch64()
    xd, wd = to_dev_bf16(xb), to_dev_bf16(wb)
    y1 = torch.full_like(xd, float("nan"))
    y2 = torch.full_like(xd, float("nan"))
    rn.rmsnorm_batched_rows(xd, wd, wl.EPS, out=y1)
    _call_noalloc(rn, rn.BF16, xd, wd, y2)
    torch.cuda.synchronize()
    assert_bits_bf16(bf16_host(y2), bf16_host(y1), "batch64: noalloc vs plain entry point")
