"""Seeded random shapes through every code path, bit for bit against the oracle.

Each case draws a dtype, a row count, a width (biased towards the widths the
layouts care about: multiples of 4, 8, 256 and 1024, one more or one less,
and arbitrary values), independent element offsets of x, w and y, row
strides with padding, sometimes in-place rows, a path setting (automatic, or
one path forced, with random rows-per-workgroup, streaming,
slices-per-wavefront and workgroups-per-row options), and whether the launch goes through the
workspace entry point (always when WIDE is forced). Every output element is
compared with the CPU oracle, and the padding around the rows must stay
untouched.
"""
import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import assert_bits_bf16, assert_bits_f32, bf16_host, dev, f32_host, say

pytestmark = pytest.mark.gpu

CASES = 72


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    return m


def _reset(rn):
    rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    rn.set_option(rn.OPT_ROWS_PER_BLOCK, 0)
    rn.set_option(rn.OPT_STREAMING, -1)
    rn.set_option(rn.OPT_SPLIT_LOADS, 0)
    rn.set_option(rn.OPT_REPLICA_PARTS, 0)


def _width(g):
    kind = int(g.integers(0, 6))
    base = int(g.choice([4, 8, 256, 512, 1024, 1536, 4096, 7168, 8192]))
    if kind == 0:
        return int(g.integers(1, 64))
    if kind == 1:
        return base * int(g.integers(1, 4))
    if kind == 2:
        return max(1, base + int(g.integers(-3, 4)))
    if kind == 3:
        return 4 * int(g.integers(1, 4097))
    if kind == 4:
        return 8 * int(g.integers(1, 2049))
    return int(g.integers(1, 20000))


def _case(g, i):
    kind = "f32" if g.random() < 0.5 else "bf16"
    n = _width(g)
    budget = max(1, 1_500_000 // n)
    rows = int(min(budget, g.choice([1, 2, 3, 7, 64, 300, 1024, 1500, 4096])))
    ox, ow, oy = (int(v) for v in g.integers(0, 4, size=3))
    if g.random() < 0.5:
        ox = ow = oy = 0
    xs = n + int(g.choice([0, 0, 1, 4, 8, 37]))
    ys = n + int(g.choice([0, 0, 2, 8, 21]))
    in_place = g.random() < 0.15
    if in_place:
        oy, ys = ox, xs
    path = int(g.choice([-1, -1, 0, 1, 2, 3, 4, 5, 6]))
    parts = int(g.integers(0, 9))
    rpb = int(g.choice([0, 4, 8]))
    streaming = int(g.choice([-1, 0, 1]))
    loads = int(g.choice([0, 1, 2, 4, 8]))
    sigma = float(10.0 ** g.uniform(-3, 3))
    ws = path == 5 or g.random() < 0.3
    return dict(i=i, kind=kind, n=n, rows=rows, ox=ox, ow=ow, oy=oy, xs=xs, ys=ys,
                in_place=in_place, path=path, rpb=rpb, streaming=streaming, loads=loads,
                parts=parts, sigma=sigma, ws=ws)


@pytest.mark.parametrize("block", range(6))
def test_fuzz(rn, block):
    g = np.random.Generator(np.random.PCG64(0xF022 + block))
    try:
        for i in range(CASES // 6):
            c = _case(g, block * 100 + i)
            say(f"fuzz {c}")
            n, rows = c["n"], c["rows"]
            x = np.empty((rows, n), np.float32)
            for r in range(rows):
                x[r], w = wl.misc_f32(1_000_000 + 1000 * c["i"] + r, n, sigma=c["sigma"])
            if c["kind"] == "bf16":
                x, w = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
                tdt, dtype = torch.bfloat16, rn.BF16
                todev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
                host, check = bf16_host, assert_bits_bf16
            else:
                tdt, dtype = torch.float32, rn.F32
                todev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
                host, check = f32_host, assert_bits_f32
            want, _ = oracle.rows(x, w, wl.EPS, nthreads=8)
            fill = float("nan") if c["kind"] == "f32" else 0.0
            bx = torch.full((rows * c["xs"] + 8,), fill, dtype=tdt, device=dev())
            bw = torch.full((n + 8,), fill, dtype=tdt, device=dev())
            bx_rows = bx[c["ox"]:c["ox"] + rows * c["xs"]].view(rows, c["xs"])[:, :n]
            bx_rows.copy_(todev(x))
            bw[c["ow"]:c["ow"] + n].copy_(todev(w))
            if c["in_place"]:
                by, by_rows = bx, bx_rows
            else:
                by = torch.full((rows * c["ys"] + 8,), fill, dtype=tdt, device=dev())
                by_rows = by[c["oy"]:c["oy"] + rows * c["ys"]].view(rows, c["ys"])[:, :n]
            rn.set_option(rn.OPT_PATH, c["path"])
            rn.set_option(rn.OPT_ROWS_PER_BLOCK, c["rpb"])
            rn.set_option(rn.OPT_STREAMING, c["streaming"])
            rn.set_option(rn.OPT_SPLIT_LOADS, c["loads"])
            rn.set_option(rn.OPT_REPLICA_PARTS, c["parts"])
            if c["ws"]:
                rn.rmsnorm_batched_rows_ws(bx_rows, bw[c["ow"]:c["ow"] + n], wl.EPS, out=by_rows)
            else:
                rn.rmsnorm_batched_rows(bx_rows, bw[c["ow"]:c["ow"] + n], wl.EPS, out=by_rows)
            torch.cuda.synchronize()
            check(host(by_rows), want, f"case {c}")
            # nothing outside the output rows was written
            full = host(by)
            mask = np.ones(full.size, dtype=bool)
            start, stride = c["oy"], c["ys"]
            for r in range(rows):
                mask[start + r * stride:start + r * stride + n] = False
            rest = full[mask]
            if c["in_place"]:
                continue  # the padding of an in-place buffer is the input's padding
            if c["kind"] == "f32":
                assert np.isnan(rest).all(), f"case {c}: wrote outside the rows"
            else:
                assert (rest == 0).all(), f"case {c}: wrote outside the rows"
    finally:
        _reset(rn)
