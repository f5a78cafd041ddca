"""REPLICA: one launch of `parts` workgroups per row, each computing the whole
row's sum (the same R256 bits in every workgroup) and applying only its share
of the row's 1024-element blocks. Bit for bit against the oracle: the single
binary32 norm (1 x 7168), the 64-row bf16 batch (64 x 7168), ragged widths
around every block boundary, every parts value (1..8, capped at the row's
blocks), in-place and strided rows, and the association probes.
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
    yield m
    _reset(m)


def _reset(rn):
    rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    rn.set_option(rn.OPT_REPLICA_PARTS, 0)


def _run(rn, kind, x, w, parts, xs=None, ys=None, in_place=False):
    """x (rows, n) through REPLICA with `parts` workgroups per row; row
    strides xs / ys (elements) >= n. Returns the output rows on the host."""
    rows, n = x.shape
    xs = n if xs is None else xs
    ys = xs if in_place else (n if ys is None else ys)
    tdt = torch.bfloat16 if kind == "bf16" else torch.float32
    todev = to_dev_bf16 if kind == "bf16" else to_dev_f32
    host = bf16_host if kind == "bf16" else f32_host
    bx = torch.zeros(rows, xs, dtype=tdt, device=dev())
    bx[:, :n].copy_(todev(x))
    by = bx if in_place else torch.full((rows, ys), float("nan"), dtype=tdt, device=dev())
    wd = todev(w)
    rn.set_option(rn.OPT_PATH, rn.PATH_REPLICA)
    rn.set_option(rn.OPT_REPLICA_PARTS, parts)
    try:
        plan = rn.plan_query(rn.BF16 if kind == "bf16" else rn.F32, rows, n)
        assert plan["path"] == rn.PATH_REPLICA, plan
        assert plan["parts"] == min(parts if parts else 4, -(-n // 1024)), plan
        rn.rmsnorm_batched_rows(bx[:, :n], wd, wl.EPS, out=by[:, :n])
        torch.cuda.synchronize()
    finally:
        _reset(rn)
    full = host(by)
    if not in_place and ys > n:
        pad = full[:, n:]
        assert (np.isnan(pad) if kind == "f32" else pad == 0x7FC0).all(), "wrote past the rows"
    return full[:, :n]


def _check(kind, got, want, what):
    (assert_bits_bf16 if kind == "bf16" else assert_bits_f32)(got, want, what)


@pytest.mark.parametrize("parts", [0, 1, 2, 3, 4, 5, 6, 7, 8])
def test_single_norm(rn, parts):
    x, w = wl.single()
    say(f"replica single norm, parts {parts}")
    got = _run(rn, "f32", x[None, :], w, parts)
    _check("f32", got[0], oracle.row_f32(x, w, wl.EPS), f"single norm, parts {parts}")


@pytest.mark.parametrize("parts", [0, 2, 4, 7])
def test_batch64(rn, parts):
    xb, wb = wl.batch64()
    say(f"replica batch64, parts {parts}")
    got = _run(rn, "bf16", xb, wb, parts)
    want, _ = oracle.rows(xb, wb, wl.EPS, nthreads=8)
    _check("bf16", got, want, f"batch64, parts {parts}")


RAGGED = [4, 8, 252, 1020, 1024, 1028, 2044, 2048, 2052, 3072, 4092, 4100, 5120, 6140,
          7164, 7168, 7172, 8188, 8192]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_ragged_widths(rn, kind):
    g = np.random.Generator(np.random.PCG64(0x5E71CA))
    for n in RAGGED:
        for parts in (2, 3, 8):
            rows = int(g.integers(1, 6))
            x = np.stack([wl.misc_f32(7_000_000 + 16 * n + r, n, sigma=10.0 ** g.uniform(-3, 3))[0]
                          for r in range(rows)])
            w = wl.misc_f32(7_000_000 + n, n)[1]
            if kind == "bf16":
                x, w = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
            say(f"replica ragged {kind} {rows} x {n} parts {parts}")
            got = _run(rn, kind, x, w, parts, xs=n + 8, ys=n + 12)
            want, _ = oracle.rows(x, w, wl.EPS)
            _check(kind, got, want, f"{kind} {rows} x {n}, parts {parts}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_in_place_takes_group(rn, kind):
    """An in-place launch with REPLICA forced runs GROUP instead (a REPLICA
    workgroup still reading the row would see its siblings' stores): the
    output is exact."""
    x, w = wl.batch64()
    if kind == "f32":
        x = x.view(np.uint16).astype(np.uint32) << 16
        x, w = x.view(np.float32), (w.astype(np.uint32) << 16).view(np.float32)
    x = x[:7]
    for parts in (2, 4, 7):
        say(f"replica forced, in place {kind}, parts {parts}")
        got = _run(rn, kind, x, w, parts, in_place=True)
        want, _ = oracle.rows(x, w, wl.EPS)
        _check(kind, got, want, f"in place {kind}, parts {parts}")


def test_association_probes(rn):
    """Rows built so that other lane counts or tree orders give other sum
    bits (one large square among many small ones at chosen lanes)."""
    n = 7168
    for lane in (0, 63, 64, 130, 255):
        for big in (2.0 ** 12, 2.0 ** 11 + 2.0 ** -1):
            x = np.full(n, 1.0, np.float32)
            x[lane::256] = 0.5
            x[lane] = big
            w = np.ones(n, np.float32)
            for parts in (2, 7):
                got = _run(rn, "f32", x[None, :], w, parts)
                _check("f32", got[0], oracle.row_f32(x, w, wl.EPS),
                       f"probe lane {lane} big {big} parts {parts}")
