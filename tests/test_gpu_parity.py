"""Bitwise parity of the HIP kernels with the CPU oracle, through the C ABI.

Covers the single row (binary32 1 x 7168), the tail/alignment sweep (widths
1..7168 at byte offsets 0/4/8/12), the bf16 batches (64 x 7168 and the full
8192 x 7168 prefill batch in the benchmark's launch configuration), every code
path and rows-per-workgroup setting, ragged tails, association probes, special
values, in-place and strided rows, the largest width (2^24), and the device
square root / division against the CPU over every positive finite binary32.
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
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    m.set_option(m.OPT_ROWS_PER_BLOCK, 0)
    m.set_option(m.OPT_STREAMING, -1)
    m.set_option(m.OPT_SPLIT_LOADS, 0)
    return m


def sync():
    import torch
    torch.cuda.synchronize()


def gpu_rows(rn, x, w, eps, dtype):
    """Run rmsnorm_batched_rows on host arrays; returns host result."""
    if dtype == rn.F32:
        y = rn.rmsnorm_batched_rows(to_dev_f32(x), to_dev_f32(w), eps)
        sync()
        return f32_host(y)
    y = rn.rmsnorm_batched_rows(to_dev_bf16(x), to_dev_bf16(w), eps)
    sync()
    return bf16_host(y)


def oracle_rows(x, w, eps):
    y, _ = oracle.rows(x, w, eps, nthreads=8)
    return y


def assert_rows(rn, got, want, dtype, what):
    if dtype == rn.F32:
        assert_bits_f32(got, want, what)
    else:
        assert_bits_bf16(got, want, what)


# ---- the workloads ----------------------------------------------------------------

def test_single_row_f32(rn):
    say("single binary32 row 1 x 7168")
    x, w = wl.single()
    y = rn.rmsnorm_f32(to_dev_f32(x), to_dev_f32(w), wl.EPS)
    sync()
    assert_bits_f32(f32_host(y), oracle.row_f32(x, w, wl.EPS), "single")


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_sweep_widths_and_offsets(rn, offset):
    """Widths 1..7168 with x, w and y all starting `offset` elements (4*offset
    bytes) past a 256-byte boundary."""
    import torch
    say(f"sweep, byte offset {4 * offset}")
    for i, (x, w) in enumerate(wl.sweep()):
        n = len(x)
        bx = torch.zeros(n + 8, dtype=torch.float32, device=dev())
        bw = torch.zeros(n + 8, dtype=torch.float32, device=dev())
        by = torch.full((n + 8,), float("nan"), dtype=torch.float32, device=dev())
        xs, ws, ys = bx[offset:offset + n], bw[offset:offset + n], by[offset:offset + n]
        xs.copy_(to_dev_f32(x))
        ws.copy_(to_dev_f32(w))
        rn.rmsnorm_f32(xs, ws, wl.EPS, out=ys)
        sync()
        assert_bits_f32(f32_host(ys), oracle.row_f32(x, w, wl.EPS), f"sweep n={n} off={offset}")
        # nothing outside the row was written
        rest = f32_host(by)
        assert np.isnan(rest[:offset]).all() and np.isnan(rest[offset + n:]).all()


def test_sweep_independent_offsets(rn):
    import torch
    say("sweep, independent offsets of x, w, y")
    g = np.random.Generator(np.random.PCG64(42))
    for i, (x, w) in enumerate(wl.sweep()):
        n = len(x)
        want = oracle.row_f32(x, w, wl.EPS)
        for _ in range(4):
            ox, ow, oy = (int(v) for v in g.integers(0, 4, size=3))
            bx = torch.zeros(n + 8, dtype=torch.float32, device=dev())
            bw = torch.zeros(n + 8, dtype=torch.float32, device=dev())
            by = torch.zeros(n + 8, dtype=torch.float32, device=dev())
            bx[ox:ox + n].copy_(to_dev_f32(x))
            bw[ow:ow + n].copy_(to_dev_f32(w))
            rn.rmsnorm_f32(bx[ox:ox + n], bw[ow:ow + n], wl.EPS, out=by[oy:oy + n])
            sync()
            assert_bits_f32(f32_host(by[oy:oy + n]), want, f"n={n} offsets {ox},{ow},{oy}")


@pytest.mark.parametrize("n", [1, 2, 3, 64, 129, 255, 256, 1000, 4097, 7167, 7168, 9000])
def test_bf16_independent_offsets(rn, n):
    """bf16 rows whose x, w, y start 0..3 elements (0/2/4/6 bytes) past a
    256-byte boundary, independently: exercises the dword loads of
    2-byte-misaligned rows and both the paired and the 16-bit stores."""
    import torch
    say(f"bf16 offsets n={n}")
    x, w = wl.misc_f32(70000 + n, n, sigma=3.0)
    xb, wb = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
    want = oracle.row_bf16(xb, wb, wl.EPS)
    for ox, ow, oy in ((0, 0, 0), (1, 1, 1), (1, 0, 3), (2, 3, 1), (3, 2, 0), (0, 1, 2)):
        bx = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev())
        bw = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev())
        by = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev())
        bx[ox:ox + n].copy_(to_dev_bf16(xb))
        bw[ow:ow + n].copy_(to_dev_bf16(wb))
        rn.rmsnorm_bf16(bx[ox:ox + n], bw[ow:ow + n], wl.EPS, out=by[oy:oy + n])
        sync()
        got = bf16_host(by)
        assert_bits_bf16(got[oy:oy + n], want, f"n={n} offsets {ox},{ow},{oy}")
        # the neighbours of the row are untouched (paired stores stay inside it)
        assert (got[:oy] == 0).all() and (got[oy + n:] == 0).all(), f"n={n} wrote outside"


def test_batch64_bf16(rn):
    say("bf16 64 x 7168")
    xb, wb = wl.batch64()
    assert_bits_bf16(gpu_rows(rn, xb, wb, wl.EPS, rn.BF16), oracle_rows(xb, wb, wl.EPS), "batch64")


def test_prefill_bf16_full(rn):
    """The full 8192 x 7168 batch, automatic plan (the benchmark's launch)."""
    say("bf16 8192 x 7168 (generating inputs)")
    xb, wb = wl.prefill()
    plan = rn.plan_query(rn.BF16, 8192, 7168)
    assert plan["path"] == rn.PATH_SPLIT
    say(f"bf16 8192 x 7168 plan {plan}")
    got = gpu_rows(rn, xb, wb, wl.EPS, rn.BF16)
    say("bf16 8192 x 7168 oracle")
    want = oracle_rows(xb, wb, wl.EPS)
    assert_bits_bf16(got, want, "prefill")
    try:
        rn.set_option(rn.OPT_STREAMING, 0)
        assert_bits_bf16(gpu_rows(rn, xb, wb, wl.EPS, rn.BF16), want, "prefill, cached loads")
        rn.set_option(rn.OPT_STREAMING, -1)
        rn.set_option(rn.OPT_PATH, rn.PATH_WAVE)
        assert_bits_bf16(gpu_rows(rn, xb, wb, wl.EPS, rn.BF16), want, "prefill, WAVE path")
    finally:
        rn.set_option(rn.OPT_STREAMING, -1)
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)


# ---- every code path gives the same bits ---------------------------------------------

PATH_CASES = [
    (8, 7168, "f32"), (33, 1000, "bf16"), (40, 257, "bf16"), (5, 8192, "f32"),
    (6, 8192, "bf16"), (3, 9000, "f32"), (17, 1536, "f32"), (9, 512, "bf16"), (4, 1, "f32"),
    (12, 255, "f32"), (7, 7167, "bf16"), (19, 7168, "bf16"), (21, 2048, "bf16"),
    (13, 3072, "f32"),
    # SPLIT shapes: rows of one partial slice, a last slice of one vector,
    # partial last wavefronts, and rows of 64 and 128 KB (8 and 16 wavefronts)
    (5, 24, "f32"), (4, 8, "bf16"), (6, 2056, "bf16"), (3, 12000, "f32"),
    (3, 16384, "f32"), (2, 20000, "bf16"), (2, 32768, "bf16"), (2, 65536, "bf16"),
    # GROUP shapes: one quad, a last block of one quad, exact blocks
    (3, 4, "bf16"), (3, 1028, "f32"), (2, 4096, "f32"), (5, 5124, "bf16"),
]

# (path, rows per block, streaming, split loads) settings every case runs under
PATH_SETTINGS = (
    [(-1, 0, -1, 0)]
    + [(0, rpb, st, 0) for rpb in (0, 4, 8) for st in (-1, 0, 1)]
    + [(1, 0, -1, 0), (2, 0, -1, 0), (4, 0, -1, 0)]
    + [(3, 0, st, u) for u in (0, 1, 2, 4, 8) for st in (-1, 0, 1)]
)


def _rows_input(rows, n, kind, item):
    x = np.empty((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r], w = wl.misc_f32(50000 + item * 97 + r, n, sigma=float(10.0 ** ((r % 5) - 2)))
    if kind == "bf16":
        return wl.to_bf16_bits(x), wl.to_bf16_bits(w)
    return x, w


def _reset_options(rn):
    rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    rn.set_option(rn.OPT_ROWS_PER_BLOCK, 0)
    rn.set_option(rn.OPT_STREAMING, -1)
    rn.set_option(rn.OPT_SPLIT_LOADS, 0)


@pytest.mark.parametrize("rows,n,kind", PATH_CASES)
def test_paths_and_rows_per_block_identical(rn, rows, n, kind):
    say(f"paths: {rows} x {n} {kind}")
    dtype = rn.F32 if kind == "f32" else rn.BF16
    x, w = _rows_input(rows, n, kind, n)
    want = oracle_rows(x, w, wl.EPS)
    try:
        for path, rpb, st, u in PATH_SETTINGS:
            rn.set_option(rn.OPT_PATH, path)
            rn.set_option(rn.OPT_ROWS_PER_BLOCK, rpb)
            rn.set_option(rn.OPT_STREAMING, st)
            rn.set_option(rn.OPT_SPLIT_LOADS, u)
            got = gpu_rows(rn, x, w, wl.EPS, dtype)
            assert_rows(rn, got, want, dtype,
                        f"path {path} rpb {rpb} streaming {st} split loads {u}")
    finally:
        _reset_options(rn)


def test_split_plans_cover_their_shapes(rn):
    """The SPLIT cases above really take the SPLIT path, with the geometry the
    kernel assumes (a check of the test itself, host only)."""
    for rows, n, kind in PATH_CASES:
        dtype = rn.F32 if kind == "f32" else rn.BF16
        es = 4 if kind == "f32" else 2
        if (n * es) % 16:
            continue
        p = rn.plan_query(dtype, rows, n, align=16)
        slices = -(-n * es // 1024)
        if p["path"] != rn.PATH_SPLIT:
            assert p["path"] in (rn.PATH_BLOCK, rn.PATH_GROUP) and n <= 8192, (rows, n, kind, p)
            try:
                rn.set_option(rn.OPT_PATH, rn.PATH_SPLIT)
                p = rn.plan_query(dtype, rows, n, align=16)
            finally:
                _reset_options(rn)
        assert p["path"] == rn.PATH_SPLIT, (rows, n, kind, p)
        assert p["block"] == 64 * -(-slices // p["loads"]) and p["block"] <= 1024


def test_single_row_entry_equals_batched(rn):
    say("single-row entry points vs batched rows")
    x, w = _rows_input(6, 3000, "f32", 1)
    yb = gpu_rows(rn, x, w, wl.EPS, rn.F32)
    for r in range(6):
        y = rn.rmsnorm_f32(to_dev_f32(x[r]), to_dev_f32(w), wl.EPS)
        sync()
        assert_bits_f32(f32_host(y), yb[r], f"row {r}")
    xb, wb = _rows_input(6, 3000, "bf16", 2)
    yb = gpu_rows(rn, xb, wb, wl.EPS, rn.BF16)
    for r in range(6):
        y = rn.rmsnorm_bf16(to_dev_bf16(xb[r]), to_dev_bf16(wb), wl.EPS)
        sync()
        assert_bits_bf16(bf16_host(y), yb[r], f"bf16 row {r}")


# ---- ragged tails, probes, special values ----------------------------------------------

def test_ragged_widths(rn):
    say("ragged widths")
    g = np.random.Generator(np.random.PCG64(9))
    widths = list(range(1, 21)) + [int(v) for v in g.integers(21, 8300, size=24)]
    for n in widths:
        for kind in ("f32", "bf16"):
            dtype = rn.F32 if kind == "f32" else rn.BF16
            x, w = _rows_input(3, n, kind, 7 + n)
            want = oracle_rows(x, w, wl.EPS)
            assert_rows(rn, gpu_rows(rn, x, w, wl.EPS, dtype), want, dtype, f"n={n} {kind}")
            # many rows: the WAVE path for widths it can hold
            xr = np.repeat(x, 400, axis=0)
            wantr = np.repeat(want, 400, axis=0)
            assert_rows(rn, gpu_rows(rn, xr, w, wl.EPS, dtype), wantr, dtype, f"n={n} {kind} x1200")


def _probe_rows():
    probes = []
    x = np.ones(1024, dtype=np.float32); x[0] = 4096.0; probes.append(x)
    x = np.ones(768, dtype=np.float32); x[100] = 4096.0; probes.append(x)
    x = np.zeros(34, dtype=np.float32); x[0], x[1], x[33] = 4096.0, 1.0, 1.0; probes.append(x)
    x = np.ones(512, dtype=np.float32); x[64:128] = 512.0; probes.append(x)
    # a huge square in every lane position of one group, one at a time
    for lane in (0, 1, 3, 4, 15, 16, 31, 32, 63, 64, 100, 128, 200, 255):
        x = np.ones(2048, dtype=np.float32)
        x[lane] = 4096.0
        x[lane + 256] = 3.0
        probes.append(x)
    return probes


def test_association_probes(rn):
    say("association probes")
    for i, x in enumerate(_probe_rows()):
        w = np.ones_like(x)
        want = oracle.row_f32(x, w, np.float32(0))
        for path in (rn.PATH_WAVE, rn.PATH_BLOCK, rn.PATH_STREAM, rn.PATH_SPLIT, rn.PATH_GROUP):
            try:
                rn.set_option(rn.OPT_PATH, path)
                xr = np.repeat(x[None, :], 2, axis=0)
                got = gpu_rows(rn, xr, w, np.float32(0), rn.F32)
            finally:
                rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
            assert_bits_f32(got[0], want, f"probe {i} path {path}")
            assert_bits_f32(got[1], want, f"probe {i} path {path}")


def test_association_probes_bf16(rn):
    """The same probes in bf16 (every probe value is a bf16 number): the bf16
    layouts place association lanes differently from the binary32 ones."""
    say("association probes, bf16")
    for i, x in enumerate(_probe_rows()):
        xb = wl.to_bf16_bits(x)
        wb = wl.to_bf16_bits(np.ones_like(x))
        assert np.array_equal(oracle.bf16_to_f32(xb), x)
        want = oracle.row_bf16(xb, wb, np.float32(0))
        for path in (rn.PATH_WAVE, rn.PATH_BLOCK, rn.PATH_STREAM, rn.PATH_SPLIT, rn.PATH_GROUP):
            for u in ((0, 1, 2, 4) if path == rn.PATH_SPLIT else (0,)):
                try:
                    rn.set_option(rn.OPT_PATH, path)
                    rn.set_option(rn.OPT_SPLIT_LOADS, u)
                    got = gpu_rows(rn, np.repeat(xb[None, :], 2, axis=0), wb, np.float32(0),
                                   rn.BF16)
                finally:
                    _reset_options(rn)
                assert_bits_bf16(got[0], want, f"bf16 probe {i} path {path} loads {u}")
                assert_bits_bf16(got[1], want, f"bf16 probe {i} path {path} loads {u}")


@pytest.mark.parametrize("n", [777, 1000])
def test_special_values(rn, n):
    say(f"special values n={n}")
    g = np.random.Generator(np.random.PCG64(123))
    cases = []
    cases.append((np.zeros(n, np.float32), np.float32(0)))               # 0 * inf = NaN
    cases.append((np.zeros(n, np.float32), wl.EPS))                      # signed zeros kept
    z = np.zeros(n, np.float32); z[::2] = -0.0; cases.append((z, wl.EPS))
    sub = (g.standard_normal(n) * 1e-40).astype(np.float32); cases.append((sub, np.float32(0)))
    cases.append((sub, wl.EPS))
    big = (g.standard_normal(n) * 3e19).astype(np.float32); cases.append((big, wl.EPS))   # ss overflows
    mid = (g.standard_normal(n) * 1e18).astype(np.float32); cases.append((mid, wl.EPS))
    inf = g.standard_normal(n).astype(np.float32); inf[5] = np.inf; cases.append((inf, wl.EPS))
    nan = g.standard_normal(n).astype(np.float32); nan[9] = np.nan; cases.append((nan, wl.EPS))
    tiny = np.full(n, 1e-30, np.float32); cases.append((tiny, np.float32(1e-30)))
    w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
    for i, (x, eps) in enumerate(cases):
        want = oracle.row_f32(x, w, eps)
        for path in (rn.PATH_WAVE, rn.PATH_BLOCK, rn.PATH_STREAM, rn.PATH_SPLIT, rn.PATH_GROUP):
            try:
                rn.set_option(rn.OPT_PATH, path)
                got = gpu_rows(rn, np.repeat(x[None, :], 2, axis=0), w, eps, rn.F32)
            finally:
                rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
            assert_bits_f32(got[1], want, f"case {i} path {path}")
        # bf16 with the same values rounded to bf16
        xb, wb = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
        want_b = oracle.row_bf16(xb, wb, eps)
        for path in (rn.PATH_WAVE, rn.PATH_BLOCK, rn.PATH_STREAM, rn.PATH_SPLIT, rn.PATH_GROUP):
            try:
                rn.set_option(rn.OPT_PATH, path)
                got = gpu_rows(rn, np.repeat(xb[None, :], 2, axis=0), wb, eps, rn.BF16)
            finally:
                rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
            assert_bits_bf16(got[1], want_b, f"bf16 case {i} path {path}")


def test_in_place(rn):
    say("in place")
    import torch
    for kind in ("f32", "bf16"):
        for rows, n in ((1, 7168), (5000, 7168), (3, 9000), (64, 100)):
            x, w = _rows_input(rows, n, kind, rows + n)
            want = oracle_rows(x, w, wl.EPS)
            if kind == "f32":
                t = to_dev_f32(x)
                rn.rmsnorm_batched_rows(t, to_dev_f32(w), wl.EPS, out=t)
                sync()
                assert_bits_f32(f32_host(t), want, f"in-place {rows}x{n}")
            else:
                t = to_dev_bf16(x)
                rn.rmsnorm_batched_rows(t, to_dev_bf16(w), wl.EPS, out=t)
                sync()
                assert_bits_bf16(bf16_host(t), want, f"in-place bf16 {rows}x{n}")


def test_strided_rows(rn):
    say("strided rows")
    import torch
    for kind, rows, n, sx, sy in (("f32", 2000, 1000, 1030, 1001), ("bf16", 50, 7168, 7200, 7296),
                                  ("bf16", 3000, 512, 520, 516), ("bf16", 100, 1000, 1001, 1003),
                                  ("bf16", 33, 7168, 7169, 7171)):
        x, w = _rows_input(rows, n, kind, sx)
        want = oracle_rows(x, w, wl.EPS)
        if kind == "f32":
            bx = torch.zeros(rows, sx, dtype=torch.float32, device=dev())
            by = torch.zeros(rows, sy, dtype=torch.float32, device=dev())
            bx[:, :n].copy_(to_dev_f32(x))
            rn.rmsnorm_batched_rows(bx[:, :n], to_dev_f32(w), wl.EPS, out=by[:, :n])
            sync()
            assert_bits_f32(f32_host(by[:, :n]), want, f"strided {rows}x{n}")
        else:
            bx = torch.zeros(rows, sx, dtype=torch.bfloat16, device=dev())
            by = torch.zeros(rows, sy, dtype=torch.bfloat16, device=dev())
            bx[:, :n].copy_(to_dev_bf16(x))
            rn.rmsnorm_batched_rows(bx[:, :n], to_dev_bf16(w), wl.EPS, out=by[:, :n])
            sync()
            assert_bits_bf16(bf16_host(by[:, :n]), want, f"strided bf16 {rows}x{n}")
            assert (bf16_host(by[:, n:]) == 0).all()


def test_largest_width(rn):
    say("n = 2^24")
    n = 1 << 24
    g = np.random.Generator(np.random.PCG64(2))
    x = g.standard_normal(n).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
    y = rn.rmsnorm_f32(to_dev_f32(x), to_dev_f32(w), wl.EPS)
    sync()
    assert_bits_f32(f32_host(y), oracle.row_f32(x, w, wl.EPS), "n=2^24")
    xb, wb = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
    yb = rn.rmsnorm_bf16(to_dev_bf16(xb), to_dev_bf16(wb), wl.EPS)
    sync()
    assert_bits_bf16(bf16_host(yb), oracle.row_bf16(xb, wb, wl.EPS), "bf16 n=2^24")


def test_unit_rows_full_scale(rn):
    """x in {+1, -1}, eps = 0: y = x * w exactly, at the prefill shape."""
    say("unit rows 8192 x 7168 bf16")
    import torch
    g = np.random.Generator(np.random.PCG64(8))
    rows, n = wl.PREFILL_SHAPE
    sign = np.where(g.random((rows, n)) < 0.5, -1.0, 1.0).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
    xb, wb = wl.to_bf16_bits(sign), wl.to_bf16_bits(w)
    got = gpu_rows(rn, xb, wb, np.float32(0), rn.BF16)
    want = wl.to_bf16_bits(sign * oracle.bf16_to_f32(wb)[None, :])
    assert np.array_equal(got, want)


# ---- device square root and division (steps 4-7) ------------------------------------------

@pytest.mark.timeout(600)
def test_sqrt_and_reciprocal_exhaustive(rn):
    """r = sqrtf(t) and 1/r on the device equal the CPU's correctly rounded
    results for every positive finite binary32 t (n = 1, eps = 0: t = ss)."""
    import torch
    chunk = 1 << 26
    first, last = 1, 0x7F800000          # [smallest subnormal, +inf)
    r_d = torch.empty(chunk, dtype=torch.float32, device=dev())
    i_d = torch.empty(chunk, dtype=torch.float32, device=dev())
    r_h = torch.empty(chunk, dtype=torch.float32).pin_memory()
    i_h = torch.empty(chunk, dtype=torch.float32).pin_memory()
    bits = np.empty(chunk, dtype=np.uint32)
    r_ref = np.empty(chunk, dtype=np.float32)
    i_ref = np.empty(chunk, dtype=np.float32)
    start = first
    k = 0
    while start < last:
        cnt = min(chunk, last - start)
        rn.diag_inverse(start, cnt, 1, 0.0, r_d, i_d)
        r_h[:cnt].copy_(r_d[:cnt], non_blocking=True)
        i_h[:cnt].copy_(i_d[:cnt], non_blocking=True)
        np.add(np.arange(cnt, dtype=np.uint32), np.uint32(start), out=bits[:cnt])
        t = bits[:cnt].view(np.float32)
        np.sqrt(t, out=r_ref[:cnt])
        np.divide(np.float32(1.0), r_ref[:cnt], out=i_ref[:cnt])
        sync()
        gr = r_h[:cnt].numpy().view(np.uint32)
        gi = i_h[:cnt].numpy().view(np.uint32)
        assert np.array_equal(gr, r_ref[:cnt].view(np.uint32)), f"sqrt differs in chunk at {start:#x}"
        assert np.array_equal(gi, i_ref[:cnt].view(np.uint32)), f"1/r differs in chunk at {start:#x}"
        if k % 8 == 0:
            say(f"sqrt/recip exhaustive: {start:#010x}")
        start += cnt
        k += 1


@pytest.mark.timeout(600)
def test_bf16_narrowing_exhaustive(rn):
    """The kernels' binary32 -> bf16 narrowing (the hardware conversion every
    bf16 store uses) equals the oracle's round-to-nearest-even for every one
    of the 2^32 binary32 patterns; NaN stays NaN with its sign."""
    import torch
    chunk = 1 << 28
    out_d = torch.empty(chunk, dtype=torch.int16, device=dev())
    out_h = torch.empty(chunk, dtype=torch.int16).pin_memory()
    want = np.empty(chunk, dtype=np.uint16)
    for k, start in enumerate(range(0, 1 << 32, chunk)):
        rn.diag_bf16(start, chunk, out_d)
        out_h.copy_(out_d, non_blocking=True)
        oracle.f32_to_bf16_range(start, chunk, out=want)
        sync()
        got = out_h.numpy().view(np.uint16)
        bits = (np.arange(chunk, dtype=np.uint64) + start).astype(np.uint32)
        nan = (bits & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal(got[~nan], want[~nan]), f"bf16 narrowing differs in chunk at {start:#x}"
        gn = got[nan]
        assert np.all((gn & 0x7FFF) > 0x7F80), f"NaN not kept in chunk at {start:#x}"
        assert np.array_equal(gn & 0x8000, (bits[nan] >> 16).astype(np.uint16) & 0x8000)
        if k % 4 == 0:
            say(f"bf16 narrowing exhaustive: {start:#010x}")


def test_mean_division_sampled(rn):
    """m = ss/(float)n and t = m + eps on the device, for n in [1, 2^24]."""
    import torch
    g = np.random.Generator(np.random.PCG64(31))
    cnt = 1 << 20
    r_d = torch.empty(cnt, dtype=torch.float32, device=dev())
    i_d = torch.empty(cnt, dtype=torch.float32, device=dev())
    for trial in range(24):
        n = int(g.integers(1, 8193)) if trial < 16 else int(g.integers(1, 1 << 24))
        eps = np.float32([0.0, 1e-6, 1e-12, 3.0][trial % 4])
        start = int(g.integers(1, 0x7F800000 - cnt))
        rn.diag_inverse(start, cnt, n, float(eps), r_d, i_d)
        sync()
        t = (np.arange(cnt, dtype=np.uint32) + np.uint32(start)).view(np.float32)
        r_ref = np.sqrt((t / np.float32(n)) + eps)
        i_ref = np.float32(1.0) / r_ref
        assert np.array_equal(f32_host(r_d).view(np.uint32), r_ref.view(np.uint32)), (n, eps)
        assert np.array_equal(f32_host(i_d).view(np.uint32), i_ref.view(np.uint32)), (n, eps)


@pytest.mark.parametrize("vectors,block", [(1, 64), (2, 448), (4, 256), (1, 1024)])
def test_diag_copy(rn, vectors, block):
    """The diagnostic streaming copy moves exactly the requested bytes: sizes
    that are and are not a whole number of workgroups, nothing written past
    the end."""
    for nbytes in (16, 16 * 64 * vectors * 3, 16 * (64 * vectors * 7 + 5), 1 << 20):
        say(f"diag copy {vectors} x 16 B, {block} threads, {nbytes} bytes")
        src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev())
        dst = torch.full((nbytes // 4 + 64,), 0x5A5A5A5A, dtype=torch.int32, device=dev())
        rn.diag_copy(src, dst[:nbytes // 4], vectors, block)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes // 4], src)
        assert (dst[nbytes // 4:] == 0x5A5A5A5A).all()
