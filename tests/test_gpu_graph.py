"""The decode step's 327 norms, eager and as one captured HIP graph.

Follows the testing discipline of Lecture 08 "Graph-resident decode":
* section 4: one replay proves nothing -- several replays, each after the
  descriptor table has been rewritten to point at different rows, each
  compared byte for byte with the eager arm and the CPU oracle;
* a negative control: the same check applied to a graph whose pointers were
  frozen at capture (a plain by-value launch captured with torch) must fail
  from the second replay, so the check can tell the difference;
* section 5: A/A controls (eager vs eager, graph vs graph) before A/B;
* section 2: widths are read from device memory, so a replay whose widths
  differ from the capture-time widths is still exact;
* section 3: a capture broken on purpose degrades to eager replay with the
  same bits and reports it.
"""
import os

import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import assert_bits_f32, dev, f32_host, say, to_dev_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    m.set_option(m.OPT_ROWS_PER_BLOCK, 0)
    return m


def sync():
    import torch
    torch.cuda.synchronize()


class Step:
    """Device buffers for one decode step: `sets` alternative input sets per
    norm, one output per norm, and a descriptor table pointing at set 0."""

    def __init__(self, rn, rows, sets=3):
        import torch
        self.rn = rn
        self.widths = [len(x) for x, _ in rows]
        self.inputs = []  # inputs[s][i] = (x_host, w_host, x_dev, w_dev)
        for s in range(sets):
            cur = []
            for i, (x, w) in enumerate(rows):
                if s > 0:   # other sets: differently seeded rows of the same widths
                    x, w = wl.misc_f32(900000 + 1000 * s + i, len(x))
                cur.append((x, w, to_dev_f32(x), to_dev_f32(w)))
            self.inputs.append(cur)
        self.ys = [torch.empty(n, dtype=torch.float32, device=dev()) for n in self.widths]
        self.table, _ = rn.make_table([(c[2], c[3], y) for c, y in zip(self.inputs[0], self.ys)])

    def point_at(self, s, widths=None):
        """Rewrite the table in place (same device buffer) to input set s,
        optionally with other widths (prefixes of the same rows)."""
        rows = []
        for i, (c, y) in enumerate(zip(self.inputs[s], self.ys)):
            n = self.widths[i] if widths is None else widths[i]
            rows.append((c[2][:n], c[3][:n], y[:n]))
        new, _ = self.rn.make_table(rows)
        self.table.copy_(new)
        sync()

    def clear_outputs(self):
        for y in self.ys:
            y.fill_(float("nan"))
        sync()

    def outputs(self):
        return [f32_host(y) for y in self.ys]

    def expected(self, s, widths=None):
        out = []
        for i, (x, w, _, _) in enumerate(self.inputs[s]):
            n = len(x) if widths is None else widths[i]
            out.append(oracle.row_f32(x[:n], w[:n], wl.EPS))
        return out


def compare(got, want, what):
    for i, (g, w) in enumerate(zip(got, want)):
        n = len(w)
        assert_bits_f32(g[:n], w, f"{what}: norm {i}")


@pytest.fixture(scope="module")
def step(rn):
    say("building the 327-norm decode step")
    return Step(rn, wl.decode())


@pytest.fixture(params=[0, 1], ids=["spread", "one-workgroup"])
def pwg(rn, request):
    """The persistent launch with free rows spread over many workgroups (the
    default) or the whole table walked by one workgroup."""
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, request.param)
    yield request.param
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)


@pytest.fixture(params=["auto", "block", "group"])
def desc_path(rn, request):
    """Plan the captured nodes (and the eager arm) with the automatic choice,
    or force the BLOCK or GROUP descriptor kernels."""
    path = {"auto": rn.PATH_AUTO, "block": rn.PATH_BLOCK, "group": rn.PATH_GROUP}[request.param]
    rn.set_option(rn.OPT_PATH, path)
    yield request.param
    rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)


def test_eager_sequence_matches_oracle(rn, step, desc_path):
    say(f"eager sequence ({desc_path})")
    step.point_at(0)
    step.clear_outputs()
    rn.rmsnorm_sequence_eager(step.table, step.widths, wl.EPS, rn.F32)
    sync()
    compare(step.outputs(), step.expected(0), "eager")


def test_aa_eager_vs_eager(rn, step):
    say("A/A eager")
    step.point_at(1)
    runs = []
    for _ in range(2):
        step.clear_outputs()
        rn.rmsnorm_sequence_eager(step.table, step.widths, wl.EPS, rn.F32)
        sync()
        runs.append(step.outputs())
    compare(runs[0], runs[1], "A/A eager")


def test_graph_replays_follow_the_table(rn, step, desc_path):
    say(f"graph capture ({desc_path})")
    step.point_at(0)
    g = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    assert g.status == rn.RMSN_OK, g.capture_error
    assert not g.is_fallback()
    assert g.node_count() == len(step.widths) == 327
    previous = None
    for rep, s in enumerate([0, 1, 2, 0, 2, 1, 1]):
        step.point_at(s)
        step.clear_outputs()
        g.launch()
        sync()
        got = step.outputs()
        compare(got, step.expected(s), f"replay {rep} (set {s})")
        # eager on the same table gives the same bytes
        step.clear_outputs()
        rn.rmsnorm_sequence_eager(step.table, step.widths, wl.EPS, rn.F32)
        sync()
        compare(got, step.outputs(), f"replay {rep} vs eager")
        if previous is not None and previous[0] == s:
            compare(got, previous[1], f"A/A graph replay {rep}")
        previous = (s, got)
    g.destroy()


def test_graph_replay_with_changed_widths(rn, step, desc_path):
    """Widths are loop bounds read from the table: replays with other
    (smaller) widths than the capture-time ones are exact and write nothing
    past the new width; crossing below a register bucket streams the row."""
    say(f"graph replay with changed widths ({desc_path})")
    step.point_at(0)
    g = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    assert g.status == rn.RMSN_OK
    gen = np.random.Generator(np.random.PCG64(4))
    for rep in range(3):
        widths = [int(gen.integers(1, n + 1)) for n in step.widths]
        step.point_at(rep % 3, widths=widths)
        step.clear_outputs()
        g.launch()
        sync()
        got = step.outputs()
        want = step.expected(rep % 3, widths=widths)
        compare(got, want, f"changed widths replay {rep}")
        for i, (y, n) in enumerate(zip(got, widths)):
            assert np.isnan(y[n:]).all(), f"norm {i} wrote past its width"
    step.point_at(0)
    g.destroy()


def test_graph_rows_can_be_wider_than_capture(rn, desc_path):
    """A node captured at width 512 replays a row of width 9000 exactly."""
    import torch
    say("replay wider than capture")
    x, w = wl.misc_f32(77, 9000)
    xd, wd = to_dev_f32(x), to_dev_f32(w)
    y = torch.empty(9000, dtype=torch.float32, device=dev())
    table, _ = rn.make_table([(xd[:512], wd[:512], y[:512])])
    g = rn.SequenceGraph(table, [512], wl.EPS, rn.F32)
    assert g.status == rn.RMSN_OK
    new, _ = rn.make_table([(xd, wd, y)])
    table.copy_(new)
    y.fill_(float("nan"))
    g.launch()
    sync()
    assert_bits_f32(f32_host(y), oracle.row_f32(x, w, wl.EPS), "wider than capture")
    g.destroy()


def test_negative_control_frozen_pointers(rn, step):
    """A graph that froze its row pointers at capture (by-value launches
    captured with torch) passes replay 1 and fails the same check once the
    rows change -- the check has discriminating power."""
    import torch
    say("negative control: frozen pointers")
    k = 6
    step.point_at(0)
    ys = step.ys[:k]
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        # warm up outside capture, then capture by-value launches of set 0
        for i in range(k):
            c = step.inputs[0][i]
            rn.rmsnorm_f32(c[2], c[3], wl.EPS, out=ys[i])
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(graph, stream=s_cap):
            for i in range(k):
                c = step.inputs[0][i]
                rn.rmsnorm_f32(c[2], c[3], wl.EPS, out=ys[i])
    torch.cuda.current_stream().wait_stream(s_cap)
    sync()
    failures = []
    for rep, s in enumerate([0, 1, 2]):
        for y in ys:
            y.fill_(float("nan"))
        sync()
        graph.replay()
        sync()
        want = step.expected(s)[:k]
        ok = all(np.array_equal(f32_host(y).view(np.uint32), w.view(np.uint32))
                 for y, w in zip(ys, want))
        failures.append(not ok)
    assert failures == [False, True, True], failures


def test_forced_capture_failure_falls_back_to_eager(rn, step):
    say("forced capture failure")
    step.point_at(2)
    os.environ["RMSN_TEST_BREAK_CAPTURE"] = "1"
    try:
        g = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    finally:
        del os.environ["RMSN_TEST_BREAK_CAPTURE"]
    assert g.status == rn.RMSN_ECAPTURE
    assert "capture" in g.capture_error.lower()
    assert g.is_fallback()
    assert g.node_count() == 0
    for rep in range(3):
        step.point_at((2 + rep) % 3)
        step.clear_outputs()
        g.launch()
        sync()
        compare(step.outputs(), step.expected((2 + rep) % 3), f"fallback replay {rep}")
    g.destroy()
    # the library still captures normally afterwards
    g2 = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    assert g2.status == rn.RMSN_OK
    g2.destroy()
    step.point_at(0)


def test_graph_of_bf16_rows(rn, desc_path):
    import torch
    from gpu_util import assert_bits_bf16, bf16_host, to_dev_bf16
    say(f"bf16 sequence graph ({desc_path})")
    rows = []
    for i, n in enumerate([7168, 1536, 512, 100, 7168]):
        x, w = wl.misc_f32(300 + i, n)
        rows.append((wl.to_bf16_bits(x), wl.to_bf16_bits(w)))
    xs = [to_dev_bf16(x) for x, _ in rows]
    ws = [to_dev_bf16(w) for _, w in rows]
    ys = [torch.empty_like(t) for t in xs]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    g = rn.SequenceGraph(table, widths, wl.EPS, rn.BF16)
    assert g.status == rn.RMSN_OK
    for rep in range(3):
        for y in ys:
            y.zero_()
        g.launch()
        sync()
        for (x, w), y in zip(rows, ys):
            assert_bits_bf16(bf16_host(y), oracle.row_bf16(x, w, wl.EPS), f"bf16 replay {rep}")
    g.destroy()


def test_graph_rows_rewritten_to_misaligned_pointers(rn, step, desc_path):
    """Descriptor rows may move to any element alignment between replays: a
    node captured for aligned rows streams a misaligned one with the same bits."""
    import torch
    say(f"replay on misaligned rows ({desc_path})")
    step.point_at(0)
    g = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    assert g.status == rn.RMSN_OK
    k = 12
    bufs = []
    rows = []
    for i in range(k):
        x, w, _, _ = step.inputs[1][i]
        n = len(x)
        o = 1 + i % 3                                     # 4, 8 or 12 bytes past 16-byte alignment
        bx = torch.zeros(n + 4, dtype=torch.float32, device=dev())
        bw = torch.zeros(n + 4, dtype=torch.float32, device=dev())
        by = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev())
        bx[o:o + n].copy_(to_dev_f32(x))
        bw[o:o + n].copy_(to_dev_f32(w))
        bufs.append((bx, bw, by, o, n))
        rows.append((bx[o:o + n], bw[o:o + n], by[o:o + n]))
    for i in range(k, len(step.widths)):
        c = step.inputs[1][i]
        rows.append((c[2], c[3], step.ys[i]))
    new, _ = rn.make_table(rows)
    step.table.copy_(new)
    sync()
    g.launch()
    sync()
    for i, (bx, bw, by, o, n) in enumerate(bufs):
        x, w, _, _ = step.inputs[1][i]
        got = f32_host(by)
        assert_bits_f32(got[o:o + n], oracle.row_f32(x, w, wl.EPS), f"misaligned norm {i}")
        assert np.isnan(got[:o]).all() and np.isnan(got[o + n:]).all()
    g.destroy()
    step.point_at(0)


# ---- positioned sequences: the state update inside the graph ----------------------

class Ring:
    """`period` positions of every norm's x and y rows, packed per norm with a
    pitch of the row's width (rows of one norm are consecutive), one w per
    norm, and the descriptor table pointing at position 0."""

    def __init__(self, rn, widths, period, kind="f32"):
        import torch
        self.rn, self.widths, self.period = rn, widths, period
        self.kind = kind
        self.x, self.w, self.xd, self.wd, self.yd = [], [], [], [], []
        for i, n in enumerate(widths):
            xs = np.empty((period, n), np.float32)
            for p in range(period):
                xs[p], w = wl.misc_f32(700000 + 97 * i + p, n, sigma=float(10.0 ** ((p % 5) - 2)))
            _, w = wl.misc_f32(800000 + i, n)
            if kind == "bf16":
                xs, w = wl.to_bf16_bits(xs), wl.to_bf16_bits(w)
                from gpu_util import to_dev_bf16
                xd, wd = to_dev_bf16(xs), to_dev_bf16(w)
            else:
                xd, wd = to_dev_f32(xs), to_dev_f32(w)
            self.x.append(xs)
            self.w.append(w)
            self.xd.append(xd)
            self.wd.append(wd)
            self.yd.append(torch.full_like(xd, float("nan")))
        self.table, _ = rn.make_table([(self.xd[i][0], self.wd[i], self.yd[i][0])
                                       for i in range(len(widths))])
        self.d_pos = torch.zeros(1, dtype=torch.int64, device=dev())

    def position(self, n):
        # the rings used here give every norm the same width n, so one pitch
        # (one row of n elements) serves every entry of the table
        es = 4 if self.kind == "f32" else 2
        return (self.d_pos, n * es, n * es, self.period)

    def expected(self, i, p):
        if self.kind == "f32":
            return oracle.row_f32(self.x[i][p], self.w[i], wl.EPS)
        return oracle.row_bf16(self.x[i][p], self.w[i], wl.EPS)

    def got(self, i, p):
        if self.kind == "f32":
            return f32_host(self.yd[i][p])
        from gpu_util import bf16_host
        return bf16_host(self.yd[i][p])


def _check_ring(ring, positions_done):
    from gpu_util import assert_bits_bf16
    for i in range(len(ring.widths)):
        for p in range(ring.period):
            got = ring.got(i, p)
            if p in positions_done:
                if ring.kind == "f32":
                    assert_bits_f32(got, ring.expected(i, p), f"norm {i} position {p}")
                else:
                    assert_bits_bf16(got, ring.expected(i, p), f"norm {i} position {p}")
            elif ring.kind == "f32":
                assert np.isnan(got).all(), f"norm {i} position {p} written too early"


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_positioned_graph_walks_the_ring(rn, kind):
    """A graph replayed with no host work between replays: each replay
    normalises the next position's rows, the position lives in device memory
    and is advanced by the graph's last node; 7 replays over a ring of 5."""
    say(f"positioned graph ({kind})")
    n = 1536
    ring = Ring(rn, [n] * 24, period=5, kind=kind)
    dt = rn.F32 if kind == "f32" else rn.BF16
    g = rn.SequenceGraph(ring.table, ring.widths, wl.EPS, dt, position=ring.position(n))
    assert g.status == rn.RMSN_OK, g.capture_error
    assert g.node_count() == 24 + 1
    assert int(ring.d_pos.item()) == 0, "pre-warm or capture moved the caller's position"
    for rep in range(7):
        g.launch()
        sync()
        assert int(ring.d_pos.item()) == (rep + 1) % 5   # the update wraps the position
        if rep < 5:
            _check_ring(ring, set(range(rep + 1)))
    # replays 5 and 6 wrapped to positions 0 and 1 and rewrote them identically
    _check_ring(ring, set(range(5)))
    g.destroy()


def test_positioned_eager_equals_graph(rn):
    """Eager and graph arms of a positioned sequence: the same rows, the same
    bits, the same position updates (A/B after an A/A of the eager arm)."""
    say("positioned eager vs graph")
    n = 7168
    ring = Ring(rn, [n] * 6, period=3)
    pos = ring.position(n)
    runs = {}
    for arm in ("eager", "eager2", "graph"):
        for y in ring.yd:
            y.fill_(float("nan"))
        ring.d_pos.fill_(1)
        if arm.startswith("eager"):
            for _ in range(3):
                rn.rmsnorm_sequence_eager(ring.table, ring.widths, wl.EPS, rn.F32, position=pos)
        else:
            g = rn.SequenceGraph(ring.table, ring.widths, wl.EPS, rn.F32, position=pos)
            assert g.status == rn.RMSN_OK
            for _ in range(3):
                g.launch()
            sync()
            g.destroy()
        sync()
        assert int(ring.d_pos.item()) == (1 + 3) % 3
        runs[arm] = [f32_host(y) for y in ring.yd]
        _check_ring(ring, {0, 1, 2})
    for a in ("eager2", "graph"):
        for i, (u, v) in enumerate(zip(runs["eager"], runs[a])):
            assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), f"{a} norm {i}"


def test_positioned_capture_failure_keeps_position(rn):
    """A capture broken on purpose leaves the caller's position untouched and
    replays eagerly, position update included."""
    say("positioned capture failure")
    n = 512
    ring = Ring(rn, [n] * 5, period=4)
    ring.d_pos.fill_(2)
    os.environ["RMSN_TEST_BREAK_CAPTURE"] = "1"
    try:
        g = rn.SequenceGraph(ring.table, ring.widths, wl.EPS, rn.F32, position=ring.position(n))
    finally:
        del os.environ["RMSN_TEST_BREAK_CAPTURE"]
    assert g.status == rn.RMSN_ECAPTURE and g.is_fallback()
    sync()
    assert int(ring.d_pos.item()) == 2
    for rep in range(4):
        g.launch()
        sync()
        assert int(ring.d_pos.item()) == (3 + rep) % 4
    _check_ring(ring, {0, 1, 2, 3})
    g.destroy()


def test_positioned_caller_position_beyond_period(rn):
    """A position the caller sets at or beyond the period counts modulo the
    period (positions 12 and 2 of a ring of 5 are the same rows); the update
    brings it back into [0, period)."""
    say("positioned: caller position beyond the period")
    n = 1024
    ring = Ring(rn, [n] * 3, period=5)
    g = rn.SequenceGraph(ring.table, ring.widths, wl.EPS, rn.F32, position=ring.position(n))
    assert g.status == rn.RMSN_OK
    ring.d_pos.fill_(12)
    g.launch()
    sync()
    assert int(ring.d_pos.item()) == 3
    _check_ring(ring, {2})
    ring.d_pos.fill_((1 << 62) + 4)          # (2^62 + 4) mod 5 = 3
    rn.rmsnorm_sequence_eager(ring.table, ring.widths, wl.EPS, rn.F32, position=ring.position(n))
    sync()
    assert int(ring.d_pos.item()) == 4
    _check_ring(ring, {2, 3})
    g.destroy()


def test_update_recaptures_only_when_the_plan_moves(rn, step):
    """Widths are a capture key only through the launch plan: widths inside
    the same register buckets keep the graph; widths that move a node to
    another kernel instance re-capture it; every replay stays exact."""
    say("plan-keyed re-capture")
    step.point_at(0)
    g = rn.SequenceGraph(step.table, step.widths, wl.EPS, rn.F32)
    assert g.status == rn.RMSN_OK
    same = [n - 3 if n > 7000 else n for n in step.widths]          # 7165: still 28 chunks
    st, rec = g.update(same)
    assert st == rn.RMSN_OK and not rec
    step.point_at(1, widths=same)
    step.clear_outputs()
    g.launch()
    sync()
    compare(step.outputs(), step.expected(1, widths=same), "same-plan widths")
    moved = [4000 if n == 7168 else n for n in step.widths]          # 28 -> 16 chunks
    st, rec = g.update(moved)
    assert st == rn.RMSN_OK and rec
    assert not g.is_fallback() and g.node_count() == len(step.widths)
    for rep, s in enumerate([2, 0, 1]):
        step.point_at(s, widths=moved)
        step.clear_outputs()
        g.launch()
        sync()
        compare(step.outputs(), step.expected(s, widths=moved), f"re-captured replay {rep}")
    # back to the original plans: re-captured again
    st, rec = g.update(step.widths)
    assert st == rn.RMSN_OK and rec
    step.point_at(0)
    step.clear_outputs()
    g.launch()
    sync()
    compare(step.outputs(), step.expected(0), "original plans again")
    g.destroy()


# ---- the whole step in one launch -------------------------------------------------

def test_persistent_step_matches_oracle_and_eager(rn, step, pwg):
    """One launch walks the 327 descriptors in order: the bits of the eager
    sequence and of the oracle, on two tables."""
    say("persistent decode step")
    for s in (0, 2):
        step.point_at(s)
        step.clear_outputs()
        rn.rmsnorm_sequence_persistent(step.table, len(step.widths), wl.EPS, rn.F32)
        sync()
        got = step.outputs()
        compare(got, step.expected(s), f"persistent set {s}")
        step.clear_outputs()
        rn.rmsnorm_sequence_eager(step.table, step.widths, wl.EPS, rn.F32)
        sync()
        compare(got, step.outputs(), f"persistent vs eager set {s}")
    step.point_at(0)


@pytest.mark.parametrize("kind,n,offset", [("f32", 7168, 0), ("f32", 1000, 1), ("bf16", 1536, 0),
                                           ("bf16", 9000, 3), ("f32", 8193, 0)])
def test_persistent_dependent_chain(rn, kind, n, offset, pwg):
    """Rows that depend on earlier outputs: norm i reads buffer i and writes
    buffer i+1 (and the last norm works in place), so each row must see the
    previous row's stores -- the order the launch sequence gives."""
    import torch
    from gpu_util import assert_bits_bf16, bf16_host, to_dev_bf16
    say(f"persistent dependent chain {kind} n={n} offset {offset}")
    k = 6
    x0, _ = wl.misc_f32(500 + n, n, sigma=3.0)
    ws = [wl.misc_f32(600 + n + i, n)[1] for i in range(k)]
    if kind == "bf16":
        x0 = wl.to_bf16_bits(x0)
        ws = [wl.to_bf16_bits(w) for w in ws]
        tdt, todev, host, check = torch.bfloat16, to_dev_bf16, bf16_host, assert_bits_bf16
        row = oracle.row_bf16
    else:
        tdt, todev, host, check = torch.float32, to_dev_f32, f32_host, assert_bits_f32
        row = oracle.row_f32
    bufs = [torch.zeros(n + 4, dtype=tdt, device=dev()) for _ in range(k + 1)]
    bufs[0][offset:offset + n].copy_(todev(x0))
    wd = [todev(w) for w in ws]
    rows = [(bufs[i][offset:offset + n], wd[i], bufs[i + 1][offset:offset + n]) for i in range(k - 1)]
    rows.append((bufs[k - 1][offset:offset + n], wd[k - 1], bufs[k - 1][offset:offset + n]))
    table, widths = rn.make_table(rows)
    dtype = rn.F32 if kind == "f32" else rn.BF16
    want = []
    cur = x0
    for i in range(k):
        cur = row(cur, ws[i], wl.EPS)
        want.append(cur)
    rn.rmsnorm_sequence_persistent(table, k, wl.EPS, dtype)
    sync()
    for i in range(k - 2):     # bufs[k - 1] holds step k - 2 only until the in-place step
        check(host(bufs[i + 1][offset:offset + n]), want[i], f"chain step {i}")
    check(host(bufs[k - 1][offset:offset + n]), want[k - 1], "in place last step")


@pytest.mark.parametrize("kind,n,norms", [("f32", 7168, 9), ("bf16", 1536, 40), ("bf16", 1532, 9),
                                           ("f32", 1000, 37)])
def test_persistent_positioned_ring(rn, kind, n, norms, pwg):
    """The persistent launch on a positioned table: its rows spread over
    workgroups (the position then advanced by a launch of its own), or every
    walk one workgroup can take (binary32 and bf16 1536: the round walk, over
    several groups of 16 rows for 40 and 37 norms; bf16 1532: the pipelined
    walk)."""
    say(f"persistent positioned ring {kind} n={n} norms={norms} workgroups option {pwg}")
    ring = Ring(rn, [n] * norms, period=4, kind=kind)
    dt = rn.F32 if kind == "f32" else rn.BF16
    ring.d_pos.fill_(3)
    for rep in range(5):
        rn.rmsnorm_sequence_persistent(ring.table, norms, wl.EPS, dt, position=ring.position(n))
        sync()
        assert int(ring.d_pos.item()) == (4 + rep) % 4
    _check_ring(ring, {0, 1, 2, 3})


def test_persistent_call_captured_in_a_graph(rn, step, pwg):
    """The single launch captured by the caller: replays follow table
    rewrites (three replays, the oracle each time)."""
    import torch
    say("persistent call captured")
    step.point_at(0)
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        rn.rmsnorm_sequence_persistent(step.table, len(step.widths), wl.EPS, rn.F32)
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(graph, stream=s_cap):
            rn.rmsnorm_sequence_persistent(step.table, len(step.widths), wl.EPS, rn.F32)
    torch.cuda.current_stream().wait_stream(s_cap)
    sync()
    for rep, s in enumerate([1, 2, 0]):
        step.point_at(s)
        step.clear_outputs()
        graph.replay()
        sync()
        compare(step.outputs(), step.expected(s), f"captured persistent replay {rep}")
    step.point_at(0)



def test_persistent_positioned_call_captured_in_a_graph(rn, pwg):
    """The positioned persistent call captured by the caller (rows spread over
    workgroups: the rows' launch and the position's own update launch): each
    replay takes the rows at the next position and advances it."""
    import torch
    n, norms = 1536, 12
    say(f"persistent positioned call captured, workgroups option {pwg}")
    ring = Ring(rn, [n] * norms, period=4, kind="f32")
    ring.d_pos.fill_(1)
    sync()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        rn.rmsnorm_sequence_persistent(ring.table, norms, wl.EPS, rn.F32, position=ring.position(n))
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(graph, stream=s_cap):
            rn.rmsnorm_sequence_persistent(ring.table, norms, wl.EPS, rn.F32,
                                           position=ring.position(n))
    torch.cuda.current_stream().wait_stream(s_cap)
    sync()
    assert int(ring.d_pos.item()) == 2   # the call before the capture ran at position 1
    for rep in range(5):
        graph.replay()
        sync()
        assert int(ring.d_pos.item()) == (3 + rep) % 4, f"replay {rep}"
    _check_ring(ring, {0, 1, 2, 3})

# ---- the persistent launch's three walks -----------------------------------------
# Round walk: every row a whole number of 16-byte vectors (at most 8192
# elements, 16-byte aligned) and no row of a round of four consecutive rows
# reading or writing what another row of the round writes: one wavefront per
# row, four rows at a time. Pipelined walk: rows fit the GROUP mapping (width a
# multiple of 4, quad-aligned) and never read what one of the three rows
# before writes (nor write what the row before writes). Anything else: row
# after row. All three must give the launch sequence's bits. binary32 rows
# that fit GROUP are whole vectors, so binary32 tables without in-round
# dependencies take the round walk; bf16 rows of width 4 mod 8 take the
# pipelined walk.

def _rows_of(kind, widths, seed):
    """Seeded host rows (x, w) of the given widths, float32 or bf16 bits."""
    out = []
    for i, n in enumerate(widths):
        x, w = wl.misc_f32(seed + i, n, sigma=2.0)
        if kind == "bf16":
            x, w = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
        out.append((x, w))
    return out


def _dev_kind(kind):
    import torch
    from gpu_util import assert_bits_bf16, bf16_host, to_dev_bf16
    if kind == "bf16":
        return torch.bfloat16, to_dev_bf16, bf16_host, assert_bits_bf16, oracle.row_bf16, rn_dtype("bf16")
    return torch.float32, to_dev_f32, f32_host, assert_bits_f32, oracle.row_f32, rn_dtype("f32")


def rn_dtype(kind):
    import row_wise_rmsnorm_amd as m
    return m.BF16 if kind == "bf16" else m.F32


PIPE_WIDTHS = [4, 8, 12, 100, 1000, 1020, 1024, 1028, 3000, 5000, 8188, 8192, 512, 1536, 7168, 4]
ROUND_WIDTHS = [8, 16, 64, 256, 264, 512, 1000, 1024, 1032, 3000, 4104, 8184, 8192, 7168, 1536,
                8, 24]


@pytest.mark.parametrize("kind,widths", [("f32", PIPE_WIDTHS), ("bf16", PIPE_WIDTHS),
                                         ("f32", ROUND_WIDTHS), ("bf16", ROUND_WIDTHS)],
                         ids=["f32-mult4", "bf16-mult4", "f32-mult8", "bf16-mult8"])
def test_persistent_walk_widths(rn, kind, widths, pwg):
    """Independent rows of every kind of width the fast walks take: multiples
    of 4 (bf16: the pipelined walk; binary32: the round walk) and of 8 (the
    round walk), from 4 to 8192, partial and exact slices and blocks."""
    import torch
    say(f"persistent walk widths {kind} {len(widths)} rows")
    tdt, todev, host, check, row, dtype = _dev_kind(kind)
    rows = _rows_of(kind, widths, 7000)
    xs = [todev(x) for x, _ in rows]
    ws = [todev(w) for _, w in rows]
    ys = [torch.full((len(x),), float("nan"), dtype=tdt, device=dev()) for x, _ in rows]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    for rep in range(2):
        rn.rmsnorm_sequence_persistent(table, len(widths), wl.EPS, dtype)
        sync()
        for i, (x, w) in enumerate(rows):
            check(host(ys[i]), row(x, w, wl.EPS), f"rep {rep} row {i} n={len(x)}")


@pytest.mark.parametrize("kind,odd", [("f32", "width 4097"), ("f32", "width 9000"),
                                      ("f32", "misaligned"), ("bf16", "width 1001"),
                                      ("bf16", "misaligned")])
def test_persistent_table_with_a_row_the_pipeline_cannot_take(rn, kind, odd, pwg):
    """One row the GROUP mapping cannot take sends the whole table down the
    row-after-row walk; every row still matches the oracle."""
    import torch
    say(f"persistent serial fallback {kind} {odd}")
    tdt, todev, host, check, row, dtype = _dev_kind(kind)
    widths = [7168, 1536, 512, 7168, 1536]
    special = 2
    if odd.startswith("width"):
        widths[special] = int(odd.split()[1])
    rows = _rows_of(kind, widths, 7100)
    xs, ws, ys, views = [], [], [], []
    for i, (x, w) in enumerate(rows):
        off = 1 if (odd == "misaligned" and i == special) else 0
        n = len(x)
        xb = torch.zeros(n + 8, dtype=tdt, device=dev())
        xb[off:off + n].copy_(todev(x))
        yb = torch.full((n + 8,), float("nan"), dtype=tdt, device=dev())
        xs.append(xb[off:off + n]); ws.append(todev(w)); ys.append(yb[off:off + n])
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    rn.rmsnorm_sequence_persistent(table, len(widths), wl.EPS, dtype)
    sync()
    for i, (x, w) in enumerate(rows):
        check(host(ys[i]), row(x, w, wl.EPS), f"row {i} n={len(x)}")


@pytest.mark.parametrize("kind,n", [("f32", 2048), ("bf16", 2048), ("bf16", 2044)])
@pytest.mark.parametrize("dist", [1, 2, 3, 4, 5, 8, 16, 17, 64, 65])
def test_persistent_dependency_at_distance(rn, kind, n, dist, pwg):
    """Row j reads the output of row j - dist (rows 0 .. dist-1 read fresh
    inputs). Distances 1 to 3 must take the row-after-row walk; 4 to 15 the
    round walk with a barrier every 4 rows (width 2048) or the pipelined walk
    (bf16 width 2044); 16 and more the round walk with a barrier every 16
    rows: all give the sequence's bits."""
    import torch
    say(f"persistent dependency at distance {dist} {kind} n={n}")
    tdt, todev, host, check, row, dtype = _dev_kind(kind)
    k = max(12, dist + 8)
    rows = _rows_of(kind, [n] * k, 7200 + 10 * dist)
    xs = [todev(x) for x, _ in rows[:dist]]
    ws = [todev(w) for _, w in rows]
    ys = [torch.full((n,), float("nan"), dtype=tdt, device=dev()) for _ in range(k)]
    for j in range(dist, k):
        xs.append(ys[j - dist])
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    want = []
    for j in range(k):
        x = rows[j][0] if j < dist else want[j - dist]
        want.append(row(x, rows[j][1], wl.EPS))
    rn.rmsnorm_sequence_persistent(table, k, wl.EPS, dtype)
    sync()
    for j in range(k):
        check(host(ys[j]), want[j], f"row {j}")


@pytest.mark.parametrize("shift", [0, 4, 1000])
def test_persistent_adjacent_rows_writing_the_same_memory(rn, shift, pwg):
    """Row j writes memory row j - 1 also writes (the same buffer, or shifted
    by `shift` elements): the later row's values must win, as in the sequence."""
    import torch
    say(f"persistent overlapping outputs shift {shift}")
    n = 2048
    rows = _rows_of("f32", [n] * 6, 7300 + shift)
    xs = [to_dev_f32(x) for x, _ in rows]
    ws = [to_dev_f32(w) for _, w in rows]
    buf = torch.full((n + shift + 8,), float("nan"), dtype=torch.float32, device=dev())
    others = [torch.full((n,), float("nan"), dtype=torch.float32, device=dev()) for _ in range(6)]
    ys = list(others)
    ys[2] = buf[:n]                    # rows 2 and 3 write overlapping memory
    ys[3] = buf[shift:shift + n]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    rn.rmsnorm_sequence_persistent(table, 6, wl.EPS, rn.F32)
    sync()
    outs = [oracle.row_f32(x, w, wl.EPS) for x, w in rows]
    want = np.full(n + shift + 8, np.nan, dtype=np.float32)
    want[:n] = outs[2]
    want[shift:shift + n] = outs[3]
    assert_bits_f32(f32_host(buf)[:n + shift], want[:n + shift], "overlapping outputs")
    for j in (0, 1, 4, 5):
        assert_bits_f32(f32_host(ys[j]), outs[j], f"row {j}")


@pytest.mark.parametrize("kind,n", [("f32", 2048), ("bf16", 2044)])
def test_persistent_row_reads_what_a_later_row_overwrites(rn, kind, n, pwg):
    """Row j reads buffer B that row j + 1 then overwrites: row j must see B's
    old contents, as in the sequence (no round walk for such a round; the
    pipelined walk, where it applies, issues row j's loads before row j + 1's
    stores)."""
    import torch
    say(f"persistent write-after-read {kind} n={n}")
    tdt, todev, host, check, row, dtype = _dev_kind(kind)
    k = 8
    rows = _rows_of(kind, [n] * (k + 1), 7400)
    shared = todev(rows[k][0])           # B: old contents = an extra input row
    xs = [todev(x) for x, _ in rows[:k]]
    ws = [todev(w) for _, w in rows[:k]]
    ys = [torch.full((n,), float("nan"), dtype=tdt, device=dev()) for _ in range(k)]
    xs[2] = shared                       # row 2 reads B ...
    ys[3] = shared                       # ... which row 3 overwrites
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    want = [row(x, w, wl.EPS) for x, w in rows[:k]]
    want[2] = row(rows[k][0], rows[2][1], wl.EPS)
    rn.rmsnorm_sequence_persistent(table, k, wl.EPS, dtype)
    sync()
    for j in range(k):
        check(host(ys[j]), want[j], f"row {j}")


@pytest.mark.parametrize("dist", [0, 2, 5])
def test_persistent_table_beyond_the_lds_check(rn, dist):
    """More than 1024 rows: the launch-time check reads the descriptors from
    memory instead of LDS. 1100 independent rows (dist 0: the round walk) or
    with row j reading row j - dist's output (2: row after row; 5: the round
    walk with a barrier every 4 rows)."""
    import torch
    say(f"persistent 1100-row table, dependency distance {dist}")
    k, n = 1100, 64
    rows = _rows_of("f32", [n] * k, 7600 + dist)
    xs = [to_dev_f32(x) for x, _ in rows]
    ws = [to_dev_f32(w) for _, w in rows]
    ys = [torch.full((n,), float("nan"), dtype=torch.float32, device=dev()) for _ in range(k)]
    want = []
    for j in range(k):
        if dist and j >= dist:
            xs[j] = ys[j - dist]
            want.append(oracle.row_f32(want[j - dist], rows[j][1], wl.EPS))
        else:
            want.append(oracle.row_f32(rows[j][0], rows[j][1], wl.EPS))
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    rn.rmsnorm_sequence_persistent(table, k, wl.EPS, rn.F32)
    sync()
    for j in range(k):
        assert_bits_f32(f32_host(ys[j]), want[j], f"row {j}")


@pytest.mark.parametrize("arm", ["graph", "eager", "persistent"])
def test_rows_with_out_of_range_widths_write_nothing(rn, desc_path, arm, pwg):
    """A descriptor whose width, rewritten in the device table, is outside
    [1, 2^24] (0, negative, 2^24 + 1) makes its row write nothing; the rows
    around it are still exact. The host widths stay the valid capture-time
    ones, as a caller's would."""
    import struct
    import torch
    say(f"out-of-range widths ({arm}, {desc_path})")
    widths = [512, 1536, 7168, 512, 64, 7168, 1024]
    bad = {1: 0, 3: -3, 4: (1 << 24) + 1}
    rows = _rows_of("f32", widths, 8100)
    xs = [to_dev_f32(x) for x, _ in rows]
    ws = [to_dev_f32(w) for _, w in rows]
    ys = [torch.full((n,), float("nan"), dtype=torch.float32, device=dev()) for n in widths]
    table, host_widths = rn.make_table(list(zip(xs, ws, ys)))
    g = rn.SequenceGraph(table, host_widths, wl.EPS, rn.F32) if arm == "graph" else None
    for i, n in bad.items():        # the n field of record i: bytes 24..31
        table[32 * i + 24:32 * i + 32].copy_(torch.frombuffer(bytearray(struct.pack("<q", n)),
                                                                dtype=torch.uint8))
    sync()
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        if arm == "graph":
            g.launch()
        elif arm == "eager":
            rn.rmsnorm_sequence_eager(table, host_widths, wl.EPS, rn.F32)
        else:
            rn.rmsnorm_sequence_persistent(table, len(widths), wl.EPS, rn.F32)
        sync()
        for i, (x, w) in enumerate(rows):
            got = f32_host(ys[i])
            if i in bad:
                assert np.isnan(got).all(), f"rep {rep}: row {i} (n={bad[i]}) wrote"
            else:
                assert_bits_f32(got, oracle.row_f32(x, w, wl.EPS), f"rep {rep} row {i}")
    if g is not None:
        g.destroy()


def _apply_in_order(rows, host, kind):
    """The launch sequence on the CPU: every row, in table order, on copies of
    the buffers (rows are ((buffer, offset, n), w, y) slices)."""
    want = [h.copy() for h in host]
    row_fn = oracle.row_bf16 if kind == "bf16" else oracle.row_f32
    for (xb, xo, n), (wb, wo, _), (yb, yo, _) in rows:
        want[yb][yo:yo + n] = row_fn(want[xb][xo:xo + n].copy(), want[wb][wo:wo + n].copy(), wl.EPS)
    return want


def test_persistent_spread_mixed_table(rn, pwg):
    """Free rows (their own buffers, an in-place one, several reading one x and
    one w), a chain of rows each reading the previous one's output, and two
    rows writing the same output, interleaved in one table: every buffer ends
    as the rows applied in table order on the CPU leave it."""
    import torch
    say(f"persistent mixed table, workgroups option {pwg}")
    g = np.random.Generator(np.random.PCG64(77))
    sizes, rows = [], []

    def buf(n):
        sizes.append(n + 8)
        return len(sizes) - 1

    shared_x, shared_w = buf(1536), buf(1536)
    chain = [buf(2048) for _ in range(6)]
    twice = buf(512)
    chain_w = buf(2048)
    plan = []
    for i in range(40):
        kind_of = i % 5
        if kind_of == 0 and i // 5 < 5:                 # chain step i//5: reads chain[k], writes chain[k+1]
            k = i // 5
            plan.append(((chain[k], 0, 2048), (chain_w, 0, 2048), (chain[k + 1], 0, 2048)))
        elif kind_of == 1:                              # free row reading the shared x and w
            plan.append(((shared_x, 0, 1536), (shared_w, 0, 1536), (buf(1536), 0, 1536)))
        elif kind_of == 2 and i in (7, 27):             # two rows writing the same output
            plan.append(((buf(512), 0, 512), (buf(512), 0, 512), (twice, 0, 512)))
        elif kind_of == 3:                              # free row in place
            b = buf(7168)
            plan.append(((b, 4, 7164), (buf(7164), 0, 7164), (b, 4, 7164)))
        else:                                           # free row on its own buffers
            n = int(g.choice([64, 512, 1000, 7168, 9000]))
            plan.append(((buf(n), 0, n), (buf(n), 0, n), (buf(n), 0, n)))
    host = [wl.misc_f32(88_000 + b, size)[0] for b, size in enumerate(sizes)]
    want = _apply_in_order(plan, host, "f32")
    bufs = [to_dev_f32(h) for h in host]
    table, _ = rn.make_table([(bufs[xb][xo:xo + n], bufs[wb][wo:wo + n], bufs[yb][yo:yo + n])
                              for (xb, xo, n), (wb, wo, _), (yb, yo, _) in plan])
    rn.rmsnorm_sequence_persistent(table, len(plan), wl.EPS, rn.F32)
    sync()
    for b, t in enumerate(bufs):
        assert_bits_f32(f32_host(t), want[b], f"buffer {b}")


@pytest.mark.gpu
@pytest.mark.parametrize("what", ["x", "w", "y", "touch"])
@pytest.mark.parametrize("writer_first", [True, False], ids=["writer_first", "reader_first"])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_persistent_spread_one_element_overlap(rn, pwg, what, writer_first, kind):
    """Among 60 free rows, one row's x (or w, or output) shares exactly one
    element with another row's output: the writer's last element is the
    other range's first. Those two rows must keep table order. With 'touch'
    the other x starts just past the writer's output, so nothing is shared
    and every row is free. Every buffer ends as the rows applied in table
    order on the CPU leave it. In bf16 the shared element is 2 bytes."""
    from gpu_util import assert_bits_bf16, bf16_host, to_dev_bf16
    say(f"persistent one-element overlap {what} {kind}, writer first {writer_first}, "
        f"workgroups option {pwg}")
    n = 512
    sizes, plan = [], []

    def buf(m):
        sizes.append(m)
        return len(sizes) - 1

    big = buf(2 * n)                       # the writer's output is big[0:n]
    start = n if what == "touch" else n - 1
    writer = ((buf(n), 0, n), (buf(n), 0, n), (big, 0, n))
    if what == "y":
        other = ((buf(n), 0, n), (buf(n), 0, n), (big, start, n))
    elif what == "w":
        other = ((buf(n), 0, n), (big, start, n), (buf(n), 0, n))
    else:
        other = ((big, start, n), (buf(n), 0, n), (buf(n), 0, n))
    first, second = (writer, other) if writer_first else (other, writer)
    for i in range(62):
        if i == 20:
            plan.append(first)
        elif i == 41:
            plan.append(second)
        else:
            plan.append(((buf(n), 0, n), (buf(n), 0, n), (buf(n), 0, n)))
    host = [wl.misc_f32(91_000 + b, size)[0] for b, size in enumerate(sizes)]
    if kind == "bf16":
        host = [wl.to_bf16_bits(h) for h in host]
    want = _apply_in_order(plan, host, kind)
    bufs = [to_dev_bf16(h) if kind == "bf16" else to_dev_f32(h) for h in host]
    table, _ = rn.make_table([(bufs[xb][xo:xo + m], bufs[wb][wo:wo + m], bufs[yb][yo:yo + m])
                              for (xb, xo, m), (wb, wo, _), (yb, yo, _) in plan])
    rn.rmsnorm_sequence_persistent(table, len(plan), wl.EPS, rn.BF16 if kind == "bf16" else rn.F32)
    sync()
    for b, t in enumerate(bufs):
        if kind == "bf16":
            assert_bits_bf16(bf16_host(t), want[b], f"buffer {b}")
        else:
            assert_bits_f32(f32_host(t), want[b], f"buffer {b}")


def test_persistent_positioned_mixed_table(rn, pwg):
    """A positioned table (rings of 4 positions, one pitch) whose rows at
    every position include a chain (row 1 reads row 0's output, row 10 works
    in place on row 1's output) among free rows: one launch per position
    through a whole cycle leaves every buffer as the rows applied in table
    order, position after position, on the CPU."""
    import torch
    say(f"persistent positioned mixed table, workgroups option {pwg}")
    n, period = 1536, 4
    sizes, plan = [], []

    def buf(m):
        sizes.append(m)
        return len(sizes) - 1

    ring = lambda: buf(period * n)
    x0, y0, y1 = ring(), ring(), ring()
    plan.append(((x0, 0, n), (buf(n), 0, n), (y0, 0, n)))        # row 0
    plan.append(((y0, 0, n), (buf(n), 0, n), (y1, 0, n)))        # row 1 reads row 0's output
    for _ in range(8):                                           # rows 2..9: free
        plan.append(((ring(), 0, n), (buf(n), 0, n), (ring(), 0, n)))
    plan.append(((y1, 0, n), (buf(n), 0, n), (y1, 0, n)))        # row 10: in place on row 1's output
    for _ in range(5):                                           # rows 11..15: free
        plan.append(((ring(), 0, n), (buf(n), 0, n), (ring(), 0, n)))
    rings = {b for (xb, _, _), _, (yb, _, _) in plan for b in (xb, yb)}
    host = [wl.misc_f32(93_000 + b, size)[0] for b, size in enumerate(sizes)]
    want = host
    for p in range(period):
        want = _apply_in_order([((xb, xo + p * n, m), w, (yb, yo + p * n, m))
                                for (xb, xo, m), w, (yb, yo, _) in plan], want, "f32")
    bufs = [to_dev_f32(h) for h in host]
    assert all(sizes[b] == period * n for b in rings)
    table, _ = rn.make_table([(bufs[xb][xo:xo + m], bufs[wb][wo:wo + m], bufs[yb][yo:yo + m])
                              for (xb, xo, m), (wb, wo, _), (yb, yo, _) in plan])
    d_pos = torch.zeros(1, dtype=torch.int64, device="cuda")
    for p in range(period):
        rn.rmsnorm_sequence_persistent(table, len(plan), wl.EPS, rn.F32,
                                       position=(d_pos, n * 4, n * 4, period))
        sync()
        assert int(d_pos.item()) == (p + 1) % period
    for b, t in enumerate(bufs):
        assert_bits_f32(f32_host(t), want[b], f"buffer {b}")
