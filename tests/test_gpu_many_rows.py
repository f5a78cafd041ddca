"""Batches with more rows than one launch can hold.

A dispatch counts its grid in work-items as a 32-bit number, so one launch of a
256-thread layout holds at most 2^24 - 1 rows, and rmsnorm_batched_rows issues
a larger batch as consecutive launches of the same layout. Each case here
normalises two launches' worth of rows and a few more in one call, on the
one-workgroup-per-row layouts (binary32 rows of one element on BLOCK, of four on
GROUP) and on the wavefront-per-row layout (bf16 rows of four, eight rows per
workgroup).

Every row is +-c, ..., +-c with c a power of two and eps = 0, so the mean of
squares is c^2 exactly, the root c and its inverse 1/c exactly, and
y = sign(x) * w with no rounding (the textbook special case of a row of equal
magnitudes). That closed form is checked on the GPU for every element of the
batch (a skipped, repeated or misplaced row breaks it: the signs differ from
row to row, and y starts as NaN), and sampled rows -- the first ones, both
sides of every launch boundary, the last ones and random ones -- are compared
bit for bit with the oracle.

Inputs are made on the device by a counter-based formula (integer hashes of
the row and element index) that the test evaluates again on the CPU for the
sampled rows; none comes from the library.
"""
import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24           # elements generated or checked per device step


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    m.set_option(m.OPT_ROWS_PER_BLOCK, 0)
    m.set_option(m.OPT_STREAMING, -1)
    yield m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)


def _row_exponent(r):
    """Row r's magnitude 2^k, k in [-20, 20] (int64 array or tensor in, same out)."""
    return (r * 40503) % 41 - 20


def _element_sign(i):
    """+1 or -1 for element index i, from a bit of an integer hash."""
    return 1 - 2 * (((i * 40503) >> 9) & 1)          # i < 2^40: no int64 overflow


def _host_rows(rows_idx, n):
    """The sampled rows on the CPU: float32 array (len(rows_idx), n)."""
    r = np.asarray(rows_idx, dtype=np.int64)[:, None]
    i = r * n + np.arange(n, dtype=np.int64)[None, :]
    return (_element_sign(i).astype(np.float64) *
            np.exp2(_row_exponent(r).astype(np.float64))).astype(np.float32)


def _fill(x, n):
    """x (rows, n) on the device from the same formula, CHUNK elements at a time."""
    flat = x.view(-1)
    total = flat.numel()
    for start in range(0, total, CHUNK):
        stop = min(total, start + CHUNK)
        i = torch.arange(start, stop, dtype=torch.int64, device=x.device)
        v = _element_sign(i).to(torch.float64) * torch.exp2(_row_exponent(i // n).to(torch.float64))
        flat[start:stop] = v.to(x.dtype)


def _check_closed_form(x, w, y):
    """y == sign(x) * w for every element, in chunks (exact, no tolerance)."""
    n = x.shape[1]
    rows_per = max(1, CHUNK // n)
    for r0 in range(0, x.shape[0], rows_per):
        xs, ys = x[r0:r0 + rows_per], y[r0:r0 + rows_per]
        bad = ys != torch.sign(xs) * w[None, :]
        if bool(bad.any()):
            k = int(bad.view(-1).nonzero()[0])
            pytest.fail(f"row {r0 + k // n} element {k % n}: got {float(ys.reshape(-1)[k])}")


# name: (torch dtype, n, byte alignment of the rows, forced path or None,
#        expected path, expected rows per workgroup)
CASES = {
    "block-f32-n1": (torch.float32, 1, 4, None, "PATH_BLOCK", 1),
    "group-f32-n4": (torch.float32, 4, 16, "PATH_GROUP", "PATH_GROUP", 1),
    "wave-bf16-n4": (torch.bfloat16, 4, 8, None, "PATH_WAVE", 8),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_batch_beyond_one_launch(rn, name):
    dtype, n, align, force, want_path, want_rpb = CASES[name]
    code = rn.BF16 if dtype == torch.bfloat16 else rn.F32
    rn.set_option(rn.OPT_PATH, getattr(rn, force) if force else rn.PATH_AUTO)
    try:
        probe = rn.plan_query(code, 1 << 26, n, align=align)
        assert probe["path"] == getattr(rn, want_path) and probe["rows_per_block"] == want_rpb
        per_launch = (0xFFFFFFFF // probe["block"]) * probe["rows_per_block"]
        rows = 2 * per_launch + 5                                  # three launches
        plan = rn.plan_query(code, rows, n, align=align)
        assert (plan["path"], plan["block"], plan["rows_per_block"]) == \
            (probe["path"], probe["block"], probe["rows_per_block"])
        say(f"{name}: {rows} rows x {n}, {per_launch} rows per launch")

        torch.cuda.empty_cache()
        x = torch.empty(rows, n, dtype=dtype, device=dev())
        _fill(x, n)
        y = torch.full((rows, n), float("nan"), dtype=dtype, device=dev())
        w_f32 = np.array([1.25, 0.75, -1.5, 2.0][:n], dtype=np.float32)   # exact in bf16
        w = torch.from_numpy(w_f32).to(dev()).to(dtype)
        rn.rmsnorm_batched_rows(x, w, 0.0, out=y)
        torch.cuda.synchronize()
        _check_closed_form(x, w, y)

        g = np.random.Generator(np.random.PCG64(17))
        edges = [per_launch, 2 * per_launch]
        picks = [np.arange(0, 64), np.arange(rows - 64, rows), g.integers(0, rows, 1024)]
        picks += [np.arange(e - 64, e + 64) for e in edges]
        rows_idx = np.unique(np.concatenate(picks))
        rows_idx = rows_idx[(rows_idx >= 0) & (rows_idx < rows)]
        # a device gather with an index out of range faults instead of raising
        assert rows_idx.min() >= 0 and rows_idx.max() < rows
        xh = _host_rows(rows_idx, n)
        idx = torch.from_numpy(rows_idx).to(dev())
        if dtype == torch.bfloat16:
            xb = (xh.view(np.uint32) >> 16).astype(np.uint16)         # exact: powers of two
            wb = (w_f32.view(np.uint32) >> 16).astype(np.uint16)
            assert np.array_equal(x[idx].view(torch.int16).cpu().numpy().view(np.uint16), xb)
            got = y[idx].view(torch.int16).cpu().numpy().view(np.uint16)
            for j, r in enumerate(rows_idx):
                want = oracle.row_bf16(xb[j], wb, np.float32(0))
                assert got[j].tolist() == want.tolist(), f"row {r}"
        else:
            assert np.array_equal(x[idx].cpu().numpy(), xh)
            got = y[idx].cpu().numpy()
            for j, r in enumerate(rows_idx):
                want = oracle.row_f32(xh[j], w_f32, np.float32(0))
                assert got[j].view(np.uint32).tolist() == want.view(np.uint32).tolist(), f"row {r}"
        del x, y
        torch.cuda.empty_cache()
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
