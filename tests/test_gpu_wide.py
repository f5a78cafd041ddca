"""Rows too wide for the register-resident layouts: STREAM (one workgroup per
row, the row streamed twice) and WIDE (the sum split over four one-wavefront
workgroups per row, one per association group, the group totals through a
caller's workspace, then the apply over many workgroups), bit for bit against
the oracle.

Covers widths around every block and batch boundary of the streamed sum (1024
elements per quad load, 16 blocks or 24 chunks per batch) up to 2^24, binary32
and bf16, x quad-aligned (quad loads) or not (element loads), w and y
misaligned (element apply), n not a multiple of 4, several rows, in-place rows,
strided rows, special values, the association probes, the workspace left
untouched when the launch needs none, and the automatic plan.
"""
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


def _inputs(kind, rows, n, item, sigma=1.0):
    xs, w = [], None
    for r in range(rows):
        x, wr = wl.misc_f32(item * 1000 + r, n, sigma=sigma)
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


def _placed(kind, a, offset):
    """A device copy of the 2-D array `a` whose rows start `offset` elements
    past a 256-byte boundary (row stride n + 8, so every row keeps the offset's
    alignment class)."""
    rows, n = a.shape
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    buf = torch.zeros(rows, n + 8, dtype=dt, device=dev())
    view = buf[:, offset:offset + n]
    view.copy_(_dev(kind, a))
    return buf, view


def _run(rn, kind, x, w, eps, path, offsets=(0, 0, 0)):
    """x (rows, n) and w on the device at the given element offsets of x, w, y;
    path PATH_WIDE runs rmsnorm_batched_rows_ws, PATH_STREAM the plain entry."""
    rows, n = x.shape
    _, xd = _placed(kind, x, offsets[0])
    _, wd = _placed(kind, w[None, :], offsets[1])
    wd = wd[0]
    ybuf, yd = _placed(kind, np.zeros_like(x), offsets[2])
    ybuf.fill_(float("nan"))
    try:
        rn.set_option(rn.OPT_PATH, path)
        if path == rn.PATH_WIDE:
            rn.rmsnorm_batched_rows_ws(xd, wd, eps, out=yd)
        else:
            rn.rmsnorm_batched_rows(xd, wd, eps, out=yd)
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    torch.cuda.synchronize()
    full = _host(kind, ybuf)
    off = offsets[2]
    # nothing written outside the rows
    pad = np.concatenate([full[:, :off], full[:, off + n:]], axis=1)
    if kind == "bf16":
        assert (pad == 0x7FC0).all() or np.isnan(oracle.bf16_to_f32(pad)).all()
    else:
        assert np.isnan(pad).all()
    return full[:, off:off + n]


WIDTHS = [1, 3, 4, 255, 256, 257, 1000, 1023, 1024, 1025, 4095, 4096, 4097, 6144, 8192, 9000,
          16388, 16389, 24 * 256 + 5, 32 * 1024, 32 * 1024 + 3, 49 * 1024 + 4, 100003]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["wide", "stream"])
def test_widths_aligned(rn, kind, path):
    p = rn.PATH_WIDE if path == "wide" else rn.PATH_STREAM
    say(f"{path} {kind}: {len(WIDTHS)} widths, aligned")
    for i, n in enumerate(WIDTHS):
        rows = 3 if n < 50000 else 1
        x, w = _inputs(kind, rows, n, 7000 + i)
        want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
        got = _run(rn, kind, x, w, wl.EPS, p)
        _check(kind, got, want, f"{path} {kind} n={n}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["wide", "stream"])
@pytest.mark.parametrize("offsets", [(1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 2, 3), (2, 2, 2)])
def test_widths_misaligned(rn, kind, path, offsets):
    """x not quad-aligned: the sum takes element loads; w or y not: the apply
    does."""
    p = rn.PATH_WIDE if path == "wide" else rn.PATH_STREAM
    say(f"{path} {kind}: offsets {offsets}")
    for i, n in enumerate([5, 1024, 1029, 6200, 6 * 1024 * 4 + 17, 70001]):
        x, w = _inputs(kind, 2, n, 8000 + i)
        want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
        got = _run(rn, kind, x, w, wl.EPS, p, offsets)
        _check(kind, got, want, f"{path} {kind} n={n} offsets {offsets}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_largest_width_wide_and_stream(rn, kind):
    """One row of 2^24 elements: the automatic plan with a workspace (WIDE) and
    without one (STREAM)."""
    n = 1 << 24
    say(f"n = 2^24 {kind}, wide and stream")
    x, w = _inputs(kind, 1, n, 9001)
    want = (oracle.row_bf16 if kind == "bf16" else oracle.row_f32)(x[0], w, wl.EPS)
    code = rn.BF16 if kind == "bf16" else rn.F32
    assert rn.workspace_query(code, 1, n)[0]["path"] == rn.PATH_WIDE
    assert rn.plan_query(code, 1, n)["path"] == rn.PATH_STREAM
    xd, wd = _dev(kind, x), _dev(kind, w)
    y = rn.rmsnorm_batched_rows_ws(xd, wd, wl.EPS)
    torch.cuda.synchronize()
    _check(kind, _host(kind, y)[0], want, f"wide 2^24 {kind}")
    y = rn.rmsnorm_batched_rows(xd, wd, wl.EPS)
    torch.cuda.synchronize()
    _check(kind, _host(kind, y)[0], want, f"stream 2^24 {kind}")


def test_association_probes_wide(rn):
    """The association probes of the parity suite, made wide (each probe row
    repeated past 16 blocks of 1024 so that it spans a batch boundary), through
    WIDE and STREAM, aligned and misaligned, binary32 and bf16."""
    say("association probes, wide")
    from test_gpu_parity import _probe_rows
    for i, base in enumerate(_probe_rows()):
        x = np.tile(base, (40000 // base.size) + 1)[: 40000 + i]
        w = np.ones_like(x)
        for kind in ("f32", "bf16"):
            xa = wl.to_bf16_bits(x) if kind == "bf16" else x
            wa = wl.to_bf16_bits(w) if kind == "bf16" else w
            want = (oracle.row_bf16 if kind == "bf16" else oracle.row_f32)(xa, wa, np.float32(0))
            for p in (rn.PATH_WIDE, rn.PATH_STREAM):
                for offsets in ((0, 0, 0), (1, 1, 1)):
                    got = _run(rn, kind, xa[None, :], wa, np.float32(0), p, offsets)
                    _check(kind, got[0], want, f"probe {i} {kind} path {p} offsets {offsets}")


def test_special_values_wide(rn):
    say("special values, wide")
    g = np.random.Generator(np.random.PCG64(321))
    n = 20000
    cases = [(np.zeros(n, np.float32), np.float32(0)), (np.zeros(n, np.float32), wl.EPS)]
    sub = (g.standard_normal(n) * 1e-40).astype(np.float32)
    cases += [(sub, np.float32(0)), (sub, wl.EPS)]
    cases.append(((g.standard_normal(n) * 3e19).astype(np.float32), wl.EPS))
    inf = g.standard_normal(n).astype(np.float32); inf[17000] = np.inf; cases.append((inf, wl.EPS))
    nan = g.standard_normal(n).astype(np.float32); nan[3] = np.nan; cases.append((nan, wl.EPS))
    w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
    for i, (x, eps) in enumerate(cases):
        for kind in ("f32", "bf16"):
            xa = wl.to_bf16_bits(x) if kind == "bf16" else x
            wa = wl.to_bf16_bits(w) if kind == "bf16" else w
            want = (oracle.row_bf16 if kind == "bf16" else oracle.row_f32)(xa, wa, eps)
            for p in (rn.PATH_WIDE, rn.PATH_STREAM):
                got = _run(rn, kind, xa[None, :], wa, eps, p)
                _check(kind, got[0], want, f"special case {i} {kind} path {p}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_in_place_and_strided_wide(rn, kind):
    say(f"in place and strided, wide {kind}")
    rows, n = 5, 70000
    x, w = _inputs(kind, rows, n, 9100)
    want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
    for p in (rn.PATH_WIDE, rn.PATH_STREAM):
        t = _dev(kind, x)
        try:
            rn.set_option(rn.OPT_PATH, p)
            if p == rn.PATH_WIDE:
                rn.rmsnorm_batched_rows_ws(t, _dev(kind, w), wl.EPS, out=t)
            else:
                rn.rmsnorm_batched_rows(t, _dev(kind, w), wl.EPS, out=t)
        finally:
            rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        torch.cuda.synchronize()
        _check(kind, _host(kind, t), want, f"in place path {p}")
        dt = torch.bfloat16 if kind == "bf16" else torch.float32
        bx = torch.zeros(rows, n + 40, dtype=dt, device=dev())
        by = torch.zeros(rows, n + 72, dtype=dt, device=dev())
        bx[:, :n].copy_(_dev(kind, x))
        try:
            rn.set_option(rn.OPT_PATH, p)
            if p == rn.PATH_WIDE:
                rn.rmsnorm_batched_rows_ws(bx[:, :n], _dev(kind, w), wl.EPS, out=by[:, :n])
            else:
                rn.rmsnorm_batched_rows(bx[:, :n], _dev(kind, w), wl.EPS, out=by[:, :n])
        finally:
            rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        torch.cuda.synchronize()
        _check(kind, _host(kind, by[:, :n]), want, f"strided path {p}")
        assert (_host(kind, by[:, n:]) == 0).all()


def test_automatic_wide_batch(rn):
    """64 rows of 65536 bf16 take WIDE automatically with a workspace (and the
    caller's workspace is used), STREAM without one; both match the oracle."""
    say("automatic wide batch 64 x 65536 bf16")
    rows, n = 64, 65536
    x, w = _inputs("bf16", rows, n, 9200)
    want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
    plan, need = rn.workspace_query(rn.BF16, rows, n)
    assert plan["path"] == rn.PATH_WIDE and need == 16 * rows
    ws = torch.full((need + 64,), 0xA5, dtype=torch.uint8, device=dev())
    xd, wd = _dev("bf16", x), _dev("bf16", w)
    y = rn.rmsnorm_batched_rows_ws(xd, wd, wl.EPS, workspace=ws)
    torch.cuda.synchronize()
    _check("bf16", _host("bf16", y), want, "auto wide")
    assert (ws[:need].cpu().numpy() != 0xA5).any(), "the group totals went elsewhere"
    assert (ws[need:].cpu().numpy() == 0xA5).all(), "wrote past the workspace it needs"
    y = rn.rmsnorm_batched_rows(xd, wd, wl.EPS)
    torch.cuda.synchronize()
    _check("bf16", _host("bf16", y), want, "auto stream")


def test_workspace_untouched_when_not_needed(rn):
    """A batch the plan does not send to WIDE runs the ordinary kernels and
    leaves the workspace as it was."""
    say("workspace untouched")
    x, w = _inputs("f32", 64, 7168, 9300)
    want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
    plan, need = rn.workspace_query(rn.F32, 64, 7168)
    assert plan["path"] != rn.PATH_WIDE and need == 0
    ws = torch.full((256,), 0x5A, dtype=torch.uint8, device=dev())
    y = rn.rmsnorm_batched_rows_ws(to_dev_f32(x), to_dev_f32(w), wl.EPS, workspace=ws)
    torch.cuda.synchronize()
    assert_bits_f32(f32_host(y), want, "not wide")
    assert (ws.cpu().numpy() == 0x5A).all()
