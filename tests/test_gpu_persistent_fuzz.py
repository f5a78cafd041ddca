"""Seeded random descriptor tables through the persistent launch and the eager
sequence, bit for bit against the rows applied in order on the CPU.

Each table draws a dtype, a row count, a width class (multiples of 8, 4 mod
8, arbitrary with a few beyond 8192) and per row a width of that class,
element offsets, and where its x, w and y live: fresh buffers, or x reading
what an earlier row wrote (at distances of 4-20, 16-40, 1 and more, or every
row the one before), x
reading a buffer a later row overwrites, y rewriting the row before's
output. The CPU model keeps every buffer's contents and applies the
oracle row by row in table order -- the semantics of the launch sequence --
and the whole of every buffer, padding included, must match after the
persistent launch (free rows spread over workgroups, and the whole table in
one workgroup) and after the eager sequence. Which of the persistent kernel's
walks a table takes, and how many of its rows are free, depends on what it
draws; all must agree.
"""
import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

TABLES = 48


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    return m


def _width(g, cls):
    """A row width of class `cls`: "vec" (a multiple of 8, whole 16-byte
    vectors for both dtypes), "quad" (4 mod 8), or "any" (arbitrary, a few
    beyond 8192)."""
    if cls == "vec":
        return 8 * int(g.integers(1, 1025))
    if cls == "quad":
        return 8 * int(g.integers(0, 1024)) + 4
    if g.random() < 0.2:
        return int(g.integers(8193, 9500))
    return int(g.integers(1, 8193))


def _table(g):
    """A list of rows (x, w, y), each a (buffer, offset, n) slice, and the
    buffer sizes. The table's kind decides its dependencies: none, only at
    distances of 4 to 20 rows, of 16 to 40 rows, anywhere (from 1), or a
    chain (every row reads the output of the row before)."""
    count = int(g.choice([1, 2, 3, 5, 9, 16, 17, 33, 64, 300, 700, 1024]))
    aligned = g.random() < 0.7
    deps = str(g.choice(["none", "none", "far", "far", "farther", "any", "chain"]))
    cls = str(g.choice(["vec", "vec", "quad", "any"]))
    rate = float(g.choice([0.05, 0.15, 0.3]))
    sizes, rows = [], []

    def new_buffer(n):
        off = 0 if aligned else int(g.integers(0, 4))
        sizes.append(off + n + int(g.integers(0, 9)))
        return (len(sizes) - 1, off, n)

    shared_n = _width(g, cls) if g.random() < 0.5 else None
    lo, hi = {"far": (4, 20), "farther": (16, 40)}.get(deps, (1, 20))
    for j in range(count):
        r = g.random()
        if deps == "chain" and j > 0:                     # every row reads the row before's output
            x = rows[j - 1][2]
            n = x[2]
        elif deps not in ("none", "chain") and j >= lo and r < rate:
            d = int(g.integers(lo, min(j, hi) + 1))        # read an earlier row's output
            x = rows[j - d][2]
            n = x[2]
        elif deps == "any" and j > 0 and r < rate + 0.05:
            n = rows[j - 1][2][2]                         # rewrite the previous row's output
            x = new_buffer(n)
            rows.append((x, new_buffer(n), rows[j - 1][2]))
            continue
        else:
            n = shared_n if shared_n is not None else _width(g, cls)
            x = new_buffer(n)
        w = new_buffer(n)
        y = x if g.random() < 0.1 else new_buffer(n)
        rows.append((x, w, y))
    # a row reading a buffer that a later row overwrites
    if deps == "any" and count >= 3 and g.random() < 0.5:
        j = int(g.integers(0, count - 1))
        k = int(g.integers(j + 1, count))
        xj, wj, yj = rows[j]
        if rows[k][2][2] == xj[2] and rows[k][2] != xj:
            rows[j] = (rows[k][2], wj, yj)
    return rows, sizes


def _walk(rows, es):
    """The walk the kernel's rules pick for a table (round16, round4,
    pipelined, row-after-row), from the rows' byte ranges with every buffer
    256-byte aligned (as torch allocates them) -- used to show coverage."""
    base = {}
    rng = []
    for x, w, y in rows:
        r = []
        for b, o, n in (x, w, y):
            start = base.setdefault(b, len(base) << 32) + o * es
            r.append((start, n * es))
        rng.append(r)

    def meet(a, b):
        return a[0] < b[0] + b[1] and b[0] < a[0] + a[1]

    fits = all(x[2] % 4 == 0 and 1 <= x[2] <= 8192 and all((o * es) % (4 * es) == 0 for _, o, _ in (x, w, y))
               for x, w, y in rows)
    vec = fits and all((x[2] * es) % 16 == 0 and all((o * es) % 16 == 0 for _, o, _ in (x, w, y))
                       for x, w, y in rows)

    def clash(j, k):        # row j reads or writes what row k writes (k != j)
        return meet(rng[j][0], rng[k][2]) or meet(rng[j][1], rng[k][2])

    def group_ok(size):
        for j in range(len(rows)):
            g0 = j - j % size
            for k in range(g0, min(len(rows), g0 + size)):
                if k != j and (clash(j, k) or (k < j and meet(rng[j][2], rng[k][2]))):
                    return False
        return True

    def pipe_ok():
        for j in range(len(rows)):
            for k in range(max(0, j - 3), j):
                if clash(j, k) or (k == j - 1 and meet(rng[j][2], rng[k][2])):
                    return False
        return True

    if vec and group_ok(16):
        return "round16"
    if vec and group_ok(4):
        return "round4"
    if fits and pipe_ok():
        return "pipelined"
    return "row-after-row"


def _free_kinds(rows, es):
    """'all free', 'mixed' or 'all bound': rows whose reads and output meet no
    other row's output and whose output meets no other row's reads are free
    (the persistent launch spreads them over workgroups)."""
    base = {}
    rng = []
    for x, w, y in rows:
        rng.append([(base.setdefault(b, len(base) << 32) + o * es, n * es) for b, o, n in (x, w, y)])

    def meet(a, b):
        return a[1] > 0 and b[1] > 0 and a[0] < b[0] + b[1] and b[0] < a[0] + a[1]

    def meets_output(j, k):
        return any(meet(rng[j][i], rng[k][2]) for i in range(3))

    free = [not any(k != j and (meets_output(j, k) or meets_output(k, j)) for k in range(len(rows)))
            for j in range(len(rows))]
    return "all free" if all(free) else ("all bound" if not any(free) else "mixed")


WALKS_SEEN = set()
SPREAD_SEEN = set()


@pytest.mark.parametrize("block", range(4))
def test_persistent_fuzz(rn, block):
    g = np.random.Generator(np.random.PCG64(0x9E75 + block))
    for t in range(TABLES // 4):
        kind = "f32" if g.random() < 0.5 else "bf16"
        rows, sizes = _table(g)
        walk = _walk(rows, 2 if kind == "bf16" else 4)
        WALKS_SEEN.add(walk)
        if len(rows) > 1:
            SPREAD_SEEN.add(_free_kinds(rows, 2 if kind == "bf16" else 4))
        say(f"persistent fuzz block {block} table {t}: {kind}, {len(rows)} rows, {walk}, "
            f"widths {[r[0][2] for r in rows][:12]}...")
        seed = 3_000_000 + 10_000 * block + 100 * t
        host = []
        for b, size in enumerate(sizes):
            v, _ = wl.misc_f32(seed + b, size, sigma=float(10.0 ** g.uniform(-2, 2)))
            host.append(wl.to_bf16_bits(v) if kind == "bf16" else v)
        # the launch sequence, on the CPU
        want = [h.copy() for h in host]
        row_fn = oracle.row_bf16 if kind == "bf16" else oracle.row_f32
        for (xb, xo, n), (wb, wo, _), (yb, yo, _) in rows:
            out = row_fn(want[xb][xo:xo + n].copy(), want[wb][wo:wo + n].copy(), wl.EPS)
            want[yb][yo:yo + n] = out
        if kind == "bf16":
            tdt, dtype = torch.bfloat16, rn.BF16
            todev = lambda a: torch.from_numpy(a.view(np.int16).copy()).to(dev()).view(torch.bfloat16)
            tohost = lambda t_: t_.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            tdt, dtype = torch.float32, rn.F32
            todev = lambda a: torch.from_numpy(a.copy()).to(dev())
            tohost = lambda t_: t_.cpu().numpy()
        for arm in ("persistent", "persistent one workgroup", "eager"):
            bufs = [todev(h) for h in host]
            table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n],
                                            bufs[yb][yo:yo + n])
                                           for (xb, xo, n), (wb, wo, _), (yb, yo, _) in rows])
            if arm.startswith("persistent"):
                rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1 if arm.endswith("workgroup") else 0)
                try:
                    rn.rmsnorm_sequence_persistent(table, len(rows), wl.EPS, dtype)
                finally:
                    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
            else:
                rn.rmsnorm_sequence_eager(table, widths, wl.EPS, dtype)
            torch.cuda.synchronize()
            for b, buf in enumerate(bufs):
                got = tohost(buf)
                same = got.view(np.uint32 if kind == "f32" else np.uint16) == \
                    want[b].view(np.uint32 if kind == "f32" else np.uint16)
                if kind == "f32":   # NaN-ness, not payload (none expected here)
                    same |= np.isnan(got) & np.isnan(want[b])
                assert same.all(), (f"{arm}: table {t} buffer {b}: first difference at "
                                    f"{int(np.argmin(same))} of {len(same)}")


def test_persistent_fuzz_reached_every_walk():
    """The tables above drew conditions for each of the four walks of one
    workgroup, and tables whose rows are all free, partly free and all bound."""
    if len(WALKS_SEEN) == 0:
        pytest.skip("the fuzz tables did not run in this session")
    assert WALKS_SEEN == {"round16", "round4", "pipelined", "row-after-row"}, WALKS_SEEN
    assert SPREAD_SEEN == {"all free", "mixed", "all bound"}, SPREAD_SEEN
