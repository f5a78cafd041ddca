"""The persistent launch on long tables with dependent rows far into the table,
and on a table whose rows span more than 4 GB, bit for bit against the rows
applied in table order on the CPU.

Each thread of the persistent launch's first workgroup holds the ranges of up
to four rows (rows j, j + 256, j + 512, j + 768), and the check that marks
the rows bound to table order runs per slot; the decode step's 327 rows reach
the second slot only with every row independent. The tables here put chains,
rows sharing an output, rows whose reads meet another row's output in exactly
one element, a row reading what a later row overwrites, and in-place rows in
every slot (rows 0-255, 256-511, 512-767, 768 and on), among free rows, in
tables of 327 and 1000 rows, binary32 and bf16. A last table takes its rows at
both ends of one allocation of more than 4 GB, so the ranges are compared as
64-bit addresses instead of 32-bit offsets.

Every buffer is compared whole after the persistent launch (free rows spread
over workgroups, then the whole table in one workgroup) and after the eager
launch sequence. The decode step's widths chained (each norm reading the
previous same-width norm's output, every row bound) run through the first
workgroup's run walk (rows meeting only at the same addresses); the same
chains read 8 elements past each output take its dependency walk instead.
Both are replayed three times. A table of every kind of dependency at
addresses a multiple of 1024 elements apart, with quad-only widths, takes the
run walk too. Forcing the dependency walk's ordered waits to time out (a spin
cap of one poll) must end the launch and be counted.
"""
import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

ARMS = ("persistent", "persistent one workgroup", "eager")


class Table:
    """Rows (x, w, y) as (buffer, offset, n) slices of host buffers."""

    def __init__(self):
        self.sizes, self.rows = [], []

    def buf(self, size):
        self.sizes.append(size)
        return len(self.sizes) - 1

    def fresh(self, n):
        return (self.buf(n + 3), 0, n)

    def add(self, x, w, y):
        assert x[2] == w[2] == y[2]
        self.rows.append((x, w, y))

    def free_row(self, n):
        self.add(self.fresh(n), self.fresh(n), self.fresh(n))


def _dependent_block(t, start, width):
    """Rows `start`.. of table t (which must already hold `start` rows) with
    every kind of dependency, all of width `width`."""
    n = width
    assert len(t.rows) == start
    # a chain of 6: each row reads the row before's output
    t.free_row(n)
    for _ in range(5):
        t.add(t.rows[-1][2], t.fresh(n), t.fresh(n))
    # two free rows, then two rows writing the same output, eleven rows apart
    t.free_row(n)
    t.free_row(n)
    shared = t.fresh(n)
    t.add(t.fresh(n), t.fresh(n), shared)
    for _ in range(10):
        t.free_row(n)
    t.add(t.fresh(n), t.fresh(n), shared)
    # one-element overlaps: a row's x starts on the last element of an earlier
    # row's output; a later row's output ends on the first element of an
    # earlier row's w
    b = t.buf(2 * n + 2)
    t.add(t.fresh(n), t.fresh(n), (b, 1, n))
    t.free_row(n)
    t.add((b, n, n), t.fresh(n), t.fresh(n))
    b2 = t.buf(2 * n + 2)
    t.add(t.fresh(n), (b2, n, n), t.fresh(n))
    t.free_row(n)
    t.add(t.fresh(n), t.fresh(n), (b2, 1, n))
    # a row reading what a later row overwrites (write after read)
    war = t.fresh(n)
    t.add(war, t.fresh(n), t.fresh(n))
    t.free_row(n)
    t.add(t.fresh(n), t.fresh(n), war)
    # an in-place row on the chain's last output, and a plain in-place row
    last = t.rows[start + 5][2]
    t.add(last, t.fresh(n), last)
    ip = t.fresh(n)
    t.add(ip, t.fresh(n), ip)


def _fill_to(t, count, widths):
    while len(t.rows) < count:
        t.free_row(widths[len(t.rows) % len(widths)])


def _table_327():
    widths = wl.decode_widths()
    t = Table()
    _fill_to(t, 40, widths)
    _dependent_block(t, 40, 512)
    _fill_to(t, 262, widths)
    _dependent_block(t, 262, 1536)
    _fill_to(t, 327, widths)
    assert len(t.rows) == 327
    return t


def _table_1000():
    widths = [256, 512, 1024, 1536, 2048, 4096, 7168, 8, 4]
    t = Table()
    for start, n in ((100, 2048), (300, 512), (600, 1024), (800, 7168), (950, 256)):
        _fill_to(t, start, widths)
        _dependent_block(t, start, n)
    _fill_to(t, 1000, widths)
    assert len(t.rows) == 1000
    return t


def _bound_rows(t, es):
    """Indices of rows bound to table order (same rule as the kernel, on the
    host buffers laid 4 GB apart): a row whose reads or output meet another
    row's output, or whose output meets another row's reads."""
    rng = [[(b << 32) + o * es for b, o, n in r] + [r[0][2] * es] for r in t.rows]

    def meet(a, la, b, lb):
        return a < b + lb and b < a + la

    out = []
    for j, (xj, wj, yj, lj) in enumerate(rng):
        for k, (xk, wk, yk, lk) in enumerate(rng):
            if k != j and (meet(xj, lj, yk, lk) or meet(wj, lj, yk, lk) or meet(yj, lj, yk, lk) or
                           meet(xk, lk, yj, lj) or meet(wk, lk, yj, lj)):
                out.append(j)
                break
    return out


def _host_buffers(t, kind, seed):
    host = []
    for b, size in enumerate(t.sizes):
        v, _ = wl.misc_f32(seed + b, size)
        host.append(wl.to_bf16_bits(v) if kind == "bf16" else v)
    return host


def _in_order(t, host, kind):
    want = [h.copy() for h in host]
    row_fn = oracle.row_bf16 if kind == "bf16" else oracle.row_f32
    for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows:
        want[yb][yo:yo + n] = row_fn(want[xb][xo:xo + n].copy(), want[wb][wo:wo + n].copy(), wl.EPS)
    return want


def _codec(kind):
    if kind == "bf16":
        return (lambda a: torch.from_numpy(a.view(np.int16).copy()).to(dev()).view(torch.bfloat16),
                lambda t_: t_.view(torch.int16).cpu().numpy().view(np.uint16), np.uint16)
    return (lambda a: torch.from_numpy(a.copy()).to(dev()),
            lambda t_: t_.cpu().numpy(), np.uint32)


def _launch(rn, arm, table, widths, count, dtype):
    if arm.startswith("persistent"):
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1 if arm.endswith("workgroup") else 0)
        try:
            rn.rmsnorm_sequence_persistent(table, count, wl.EPS, dtype)
        finally:
            rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
    else:
        rn.rmsnorm_sequence_eager(table, widths, wl.EPS, dtype)
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    m.set_option(m.OPT_PERSISTENT_WORKGROUPS, 0)
    return m


@pytest.mark.parametrize("which", ["327", "1000"])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_long_tables_with_dependencies(rn, which, kind):
    t = _table_327() if which == "327" else _table_1000()
    es = 2 if kind == "bf16" else 4
    bound = _bound_rows(t, es)
    slots = {j // 256 for j in bound}
    assert slots == ({0, 1} if which == "327" else {0, 1, 2, 3}), slots
    say(f"persistent long table {which} {kind}: {len(t.rows)} rows, {len(bound)} bound, "
        f"bound rows in slots {sorted(slots)}")
    host = _host_buffers(t, kind, 5_000_000 + 1000 * len(t.rows))
    want = _in_order(t, host, kind)
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    for arm in ARMS:
        bufs = [todev(h) for h in host]
        table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n],
                                        bufs[yb][yo:yo + n])
                                       for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
        _launch(rn, arm, table, widths, len(t.rows), dtype)
        for b, buf in enumerate(bufs):
            same = tohost(buf).view(bits) == want[b].view(bits)
            assert same.all(), (f"{arm}: {which} {kind} buffer {b}: first difference at "
                                f"{int(np.argmin(same))} of {len(same)}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_rows_more_than_4gb_apart(rn, kind):
    """Rows at both ends of one device allocation of 4.1 GB: free rows at each
    end, a chain and a pair sharing an output at the far end, a row reading
    near the start and writing near the end. The row ranges span more than
    4 GB, so the persistent launch compares them as 64-bit addresses."""
    es = 2 if kind == "bf16" else 4
    total = (41 << 30) // 10 // es                        # elements in 4.1 GB
    region = 1 << 16                                       # elements per end region
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    big = torch.empty(total, dtype=dt, device=dev())
    lo0, hi0 = 0, total - region
    n = 1024
    # slots of n + 8 elements in each region
    slot = lambda base, i: base + 8 + i * (n + 8)
    rows = []
    for i in range(6):                                     # free rows near the start
        rows.append((slot(lo0, 3 * i), slot(lo0, 3 * i + 1), slot(lo0, 3 * i + 2)))
    for i in range(6):                                     # free rows near the end
        rows.append((slot(hi0, 3 * i), slot(hi0, 3 * i + 1), slot(hi0, 3 * i + 2)))
    c0 = 30                                                # a chain of 4 near the end
    rows.append((slot(hi0, c0), slot(hi0, c0 + 1), slot(hi0, c0 + 2)))
    for k in range(3):
        rows.append((rows[-1][2], slot(hi0, c0 + 3 + 2 * k), slot(hi0, c0 + 4 + 2 * k)))
    shared = slot(hi0, 45)                                 # two rows writing one output
    rows.append((slot(hi0, 46), slot(hi0, 47), shared))
    rows.append((slot(lo0, 40), slot(lo0, 41), slot(hi0, 48)))   # reads the start, writes the end
    rows.append((slot(hi0, 49), slot(hi0, 50), shared))
    rows.append((slot(hi0, 48), slot(lo0, 42), slot(lo0, 43)))   # reads that far-end output
    regions = [(lo0, region), (hi0, region)]
    g = np.random.Generator(np.random.PCG64(0x4B16))
    host = []
    for base, size in regions:
        v = (g.standard_normal(size) * 2.0).astype(np.float32)
        host.append(wl.to_bf16_bits(v) if kind == "bf16" else v)

    def where(e):
        for r, (base, size) in enumerate(regions):
            if base <= e < base + size:
                return r, e - base
        raise AssertionError(e)

    want = [h.copy() for h in host]
    row_fn = oracle.row_bf16 if kind == "bf16" else oracle.row_f32
    for xe, we, ye in rows:
        (xr, xo), (wr, wo), (yr, yo) = where(xe), where(we), where(ye)
        want[yr][yo:yo + n] = row_fn(want[xr][xo:xo + n].copy(), want[wr][wo:wo + n].copy(),
                                     wl.EPS)
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    say(f"persistent rows 4.1 GB apart {kind}: {len(rows)} rows")
    for arm in ARMS:
        for (base, size), h in zip(regions, host):
            big[base:base + size].copy_(todev(h))
        table, widths = rn.make_table([(big[xe:xe + n], big[we:we + n], big[ye:ye + n])
                                       for xe, we, ye in rows])
        _launch(rn, arm, table, widths, len(rows), dtype)
        for r, (base, size) in enumerate(regions):
            same = tohost(big[base:base + size]).view(bits) == want[r].view(bits)
            assert same.all(), (f"{arm}: {kind} region {r}: first difference at "
                                f"{int(np.argmin(same))} of {len(same)}")
    del big
    torch.cuda.empty_cache()


def _chained_decode(kind, shift=0):
    """The decode step's widths, each norm reading the previous norm of its
    width's output (every row bound to table order): three chains, of 7168,
    1536 and 512 wide rows, interleaved as in the step. With `shift` each x
    starts that many elements past the output it reads (into the output
    buffer's padding)."""
    widths = wl.decode_widths()
    t = Table()
    last = {}
    for n in widths:
        if n in last:
            yb, yo, _ = t.rows[last[n]][2]
            x = (yb, yo + shift, n)
        else:
            x = t.fresh(n)
        t.add(x, t.fresh(n), (t.buf(n + shift + 3), 0, n))
        last[n] = len(t.rows) - 1
    return t


@pytest.mark.parametrize("shift", [0, 8])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_chained_decode_table(rn, kind, shift):
    """Every row bound, chains at distances 1 to 8, against the rows applied
    in order. Unshifted, every row meets others only at the same addresses
    (the run walk, 7168-wide rows forwarded in registers); shifted by 8
    elements (whole 16-byte vectors, other addresses) the dependency walk
    takes them. No ordered wait may time out."""
    t = _chained_decode(kind, shift)
    say(f"persistent chained decode table {kind} shift {shift}: {len(t.rows)} rows")
    host = _host_buffers(t, kind, 6_000_000)
    want = _in_order(t, host, kind)
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    rn.diag_walk_timeouts(reset=True)
    for arm in ARMS[:2]:
        bufs = [todev(h) for h in host]
        table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n],
                                        bufs[yb][yo:yo + n])
                                       for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
        for rep in range(3):                       # replays on the same buffers: results move on
            _launch(rn, arm, table, widths, len(t.rows), dtype)
            exp = want if rep == 0 else _in_order(t, [tohost(b) for b in prev], kind)
            for b, buf in enumerate(bufs):
                same = tohost(buf).view(bits) == exp[b].view(bits)
                assert same.all(), (f"{arm} replay {rep}: chained {kind} buffer {b}: first "
                                    f"difference at {int(np.argmin(same))} of {len(same)}")
            prev = [b.clone() for b in bufs]
    assert rn.diag_walk_timeouts() == 0


def test_walk_timeout_is_counted(rn):
    """A spin cap of one poll makes the ordered waits of a chained table (the
    dependency walk: chains 8 elements off) time out: the launch still ends,
    and the device counter reports it (the rows' outputs are then not ordered
    and are not checked). With the default cap the same table is exact again
    and nothing is counted."""
    t = _chained_decode("f32", shift=8)
    host = _host_buffers(t, "f32", 6_100_000)
    todev, tohost, bits = _codec("f32")
    bufs = [todev(h) for h in host]
    table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n], bufs[yb][yo:yo + n])
                                   for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
    rn.diag_walk_timeouts(reset=True)
    rn.set_option(rn.OPT_WALK_SPIN_CAP, 1)
    try:
        assert rn.get_option(rn.OPT_WALK_SPIN_CAP) == 1
        for _ in range(3):
            _launch(rn, "persistent", table, widths, len(t.rows), rn.F32)
    finally:
        rn.set_option(rn.OPT_WALK_SPIN_CAP, 0)
    assert rn.diag_walk_timeouts(reset=True) > 0
    assert rn.diag_walk_timeouts() == 0
    bufs = [todev(h) for h in host]
    table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n], bufs[yb][yo:yo + n])
                                   for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
    _launch(rn, "persistent", table, widths, len(t.rows), rn.F32)
    want = _in_order(t, host, "f32")
    for b, buf in enumerate(bufs):
        assert (tohost(buf).view(bits) == want[b].view(bits)).all(), b
    assert rn.diag_walk_timeouts() == 0


def _aligned_block(t, n, period):
    """Rows of width n with every kind of dependency, every pair of them
    meeting at addresses a multiple of `period` elements apart: a chain read
    at the same addresses, a row reading the second period of a two-period
    output, the same output written twice, a row overwriting an earlier read,
    an in-place row, a row whose w is its output, a row whose output is one
    period into an earlier output."""
    big = lambda: (t.buf(n + 2 * period + 3), 0, n)
    a = big()
    t.add(t.fresh(n), t.fresh(n), a)
    t.add(a, t.fresh(n), big())                              # forwarded: x is the output before
    t.add(t.rows[-1][2], t.fresh(n), t.fresh(n))             # forwarded again
    t.free_row(n)
    t.add((a[0], period, n), t.fresh(n), t.fresh(n))         # a period into an earlier output
    shared = big()
    t.add(t.fresh(n), t.fresh(n), shared)
    t.add(t.fresh(n), t.fresh(n), shared)                    # the same output, twice in a row
    war = t.fresh(n)
    t.add(war, t.fresh(n), t.fresh(n))
    t.add(t.fresh(n), t.fresh(n), war)                       # overwrites the read before
    ip = t.fresh(n)
    t.add(ip, t.fresh(n), ip)                                # in place
    wy = t.fresh(n)
    t.add(t.fresh(n), wy, wy)                                # w is the output
    t.add(t.fresh(n), t.fresh(n), (shared[0], period, n))    # output a period into another


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_run_walk_aligned_dependencies(rn, kind):
    """Blocks of aligned dependencies (every meeting a multiple of 1024
    elements apart) at widths 4, 12, 1028, 4100 (quads, not whole 16-byte
    vectors in bf16) and 8192, among free rows: the run walk, against the
    rows applied in order, replayed three times."""
    t = Table()
    for n in (4, 12, 1028, 4100, 8192, 7168):
        t.free_row(n)
        _aligned_block(t, n, 1024)
    say(f"persistent aligned dependencies {kind}: {len(t.rows)} rows")
    host = _host_buffers(t, kind, 6_200_000)
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    rn.diag_walk_timeouts(reset=True)
    bufs = [todev(h) for h in host]
    table, widths = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n], bufs[yb][yo:yo + n])
                                   for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
    prev = [h.copy() for h in host]
    for rep in range(3):
        _launch(rn, "persistent", table, widths, len(t.rows), dtype)
        exp = _in_order(t, prev, kind)
        for b, buf in enumerate(bufs):
            same = tohost(buf).view(bits) == exp[b].view(bits)
            assert same.all(), (f"replay {rep}: aligned {kind} buffer {b}: first difference at "
                                f"{int(np.argmin(same))} of {len(same)}")
        prev = [tohost(b) for b in bufs]
    assert rn.diag_walk_timeouts() == 0


@pytest.mark.parametrize("shift", [0, 8, "mixed"])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_many_components(rn, kind, shift):
    """Forty chains of six rows (each row reading the one before's output,
    `shift` elements on; "mixed": 8 on every other chain, so a walker's rows
    mix components of both kinds), interleaved in the table with free rows:
    forty components, more than the launch's walkers, each walker taking
    every fourth of them in order of their first row; widths 8 to 7168.
    Against the rows applied in order, replayed twice."""
    g = np.random.Generator(np.random.PCG64(0x40C))
    t = Table()
    chains = 40
    widths = [int(g.choice([8, 64, 512, 1536, 4096, 7168])) for _ in range(chains)]
    last = [None] * chains
    order = [c for c in range(chains) for _ in range(6)]
    g.shuffle(order)
    for c in order:
        n = widths[c]
        sh = (8 if c % 2 else 0) if shift == "mixed" else shift
        if last[c] is None:
            x = t.fresh(n)
        else:
            yb, yo, _ = t.rows[last[c]][2]
            x = (yb, yo + sh, n)
        t.add(x, t.fresh(n), (t.buf(n + sh + 3), 0, n))
        last[c] = len(t.rows) - 1
        if g.random() < 0.3:
            t.free_row(int(g.choice([256, 1024, 7168])))
    say(f"persistent many components {kind} shift {shift}: {len(t.rows)} rows, {chains} chains")
    host = _host_buffers(t, kind, 6_300_000 + (9 if shift == "mixed" else shift))
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    bufs = [todev(h) for h in host]
    table, widths_t = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n], bufs[yb][yo:yo + n])
                                     for (xb, xo, n), (wb, wo, _), (yb, yo, _) in t.rows])
    prev = [h.copy() for h in host]
    for rep in range(2):
        _launch(rn, "persistent", table, widths_t, len(t.rows), dtype)
        exp = _in_order(t, prev, kind)
        for b, buf in enumerate(bufs):
            same = tohost(buf).view(bits) == exp[b].view(bits)
            assert same.all(), (f"replay {rep}: {kind} shift {shift} buffer {b}: first "
                                f"difference at {int(np.argmin(same))} of {len(same)}")
        prev = [tohost(b) for b in bufs]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_more_meeting_pairs_than_the_edge_list_holds(rn, kind):
    """Eighty rows writing the same output (every pair meets: 3160 pairs,
    more than the walkers' list of 2048), among free rows and a separate
    chain: the walkers cannot tell the components apart and keep every bound
    row in the first walker, in table order. The last writer's row must win,
    and the chain must be exact."""
    t = Table()
    n = 1024
    shared = t.fresh(n)
    for i in range(80):
        t.add(t.fresh(n), t.fresh(n), shared)
        if i % 7 == 0:
            t.free_row(512)
    t.free_row(n)
    for _ in range(5):
        t.add(t.rows[-1][2], t.fresh(n), t.fresh(n))
    say(f"persistent edge-list overflow {kind}: {len(t.rows)} rows")
    host = _host_buffers(t, kind, 6_400_000)
    want = _in_order(t, host, kind)
    todev, tohost, bits = _codec(kind)
    dtype = rn.BF16 if kind == "bf16" else rn.F32
    for arm in ARMS:
        bufs = [todev(h) for h in host]
        table, widths = rn.make_table([(bufs[xb][xo:xo + n_], bufs[wb][wo:wo + n_],
                                        bufs[yb][yo:yo + n_])
                                       for (xb, xo, n_), (wb, wo, _), (yb, yo, _) in t.rows])
        _launch(rn, arm, table, widths, len(t.rows), dtype)
        for b, buf in enumerate(bufs):
            same = tohost(buf).view(bits) == want[b].view(bits)
            assert same.all(), (f"{arm}: {kind} buffer {b}: first difference at "
                                f"{int(np.argmin(same))} of {len(same)}")
