"""CPU model of the persistent launch's dependency walk: its ordering rules,
checked against in-order application on random tables before any GPU runs it.

The model restates, in Python, what the first workgroup of the spread
persistent launch decides and does with the rows bound to table order:

* a row is bound when its x, w or output range meets another row's output,
  or its output meets another row's x or w (every pair tested here);
* the walk list is the bound rows in table order; for entry i, dep is the
  latest earlier entry it meets within the 64 entries before it, else every
  entry before that window (the entry just before it); dep_w the same for the
  earlier outputs that meet its w alone;
* four wavefronts: wavefront v takes entries v, v + 4, ... in order and
  publishes next[v] (the entry it is on); a row waits until every other
  wavefront's next is past dep_w, reads w, waits until every other next is
  past dep, reads x, computes, writes its output, and only then moves
  next[v] on.

A discrete-event simulation runs that protocol with random durations: reads
take the memory's contents at the moment they happen and writes land at
theirs, rows of the same wavefront run in order, and free rows run at random
moments in parallel. Every simulated run must end (no wavefront waits
forever) and leave memory exactly as applying the rows one after another in
table order does. The row function is y = 2x + w + 1 elementwise: any
reordering of dependent rows shows in the result.
"""
import heapq

import numpy as np
import pytest

WINDOW = 64
WAVES = 4


def meet(a0, alen, b0, blen):
    return alen > 0 and blen > 0 and a0 < b0 + blen and b0 < a0 + alen


def rows_meet(a, b):
    """a = (x, w, y, n) element offsets: a reads b's output, b reads a's, or
    their outputs overlap."""
    ax, aw, ay, an = a
    bx, bw, by, bn = b
    return (meet(ax, an, by, bn) or meet(aw, an, by, bn) or meet(ay, an, by, bn) or
            meet(bx, bn, ay, an) or meet(bw, bn, ay, an))


def w_meets_output(a, b):
    return meet(a[1], a[3], b[2], b[3])


def bound_rows(rows):
    return [j for j in range(len(rows))
            if any(k != j and rows_meet(rows[j], rows[k]) for k in range(len(rows)))]


def deps(rows, lst):
    dep, dep_w = [], []
    for i in range(len(lst)):
        a = rows[lst[i]]
        lo = max(0, i - WINDOW)
        da = dw = -1
        for k in range(i - 1, lo - 1, -1):
            b = rows[lst[k]]
            if da < 0 and rows_meet(a, b):
                da = k
            if w_meets_output(a, b):
                dw = k
                break
        dep.append(da if da >= 0 else lo - 1)
        dep_w.append(dw if dw >= 0 else lo - 1)
    return dep, dep_w


def apply_row(mem, x, w, y, n, xv=None, wv=None):
    xv = mem[x:x + n].copy() if xv is None else xv
    wv = mem[w:w + n].copy() if wv is None else wv
    mem[y:y + n] = 2.0 * xv + wv + 1.0


def in_order(mem0, rows):
    mem = mem0.copy()
    for x, w, y, n in rows:
        apply_row(mem, x, w, y, n)
    return mem


def simulate(mem0, rows, rng):
    """The walk's protocol on the bound rows, free rows at random moments."""
    mem = mem0.copy()
    b = bound_rows(rows)
    bset = set(b)
    dep, dep_w = deps(rows, b)
    nb = len(b)
    nxt = list(range(WAVES))
    # event queue of (time, seq, kind, payload)
    q, seq = [], [0]

    def push(t, kind, payload):
        seq[0] += 1
        heapq.heappush(q, (t, seq[0], kind, payload))

    for j in range(len(rows)):
        if j not in bset:
            push(float(rng.uniform(0, 40)), "free", j)
    state = {}
    for v in range(WAVES):
        if v < nb:
            state[v] = {"i": v, "phase": "wait_w"}
            push(float(rng.uniform(0, 2)), "wave", v)
        else:
            nxt[v] = 1 << 30
    steps = 0
    while q:
        steps += 1
        assert steps < 200_000, "the walk did not finish"
        t, _, kind, payload = heapq.heappop(q)
        if kind == "free":
            x, w, y, n = rows[payload]
            apply_row(mem, x, w, y, n)
            continue
        v = payload
        st = state[v]
        i = st["i"]
        x, w, y, n = rows[b[i]]
        ph = st["phase"]
        if ph in ("wait_w", "wait_x"):
            d = dep_w[i] if ph == "wait_w" else dep[i]
            ok = d < 0 or all(nxt[u] > d for u in range(WAVES) if u != v)
            if not ok:
                push(t + float(rng.uniform(0.1, 1.0)), "wave", v)      # poll again later
                continue
            if ph == "wait_w":
                st["wv"] = mem[w:w + n].copy()                           # w read now
                st["phase"] = "wait_x"
            else:
                st["xv"] = mem[x:x + n].copy()                           # x read now
                st["phase"] = "store"
            push(t + float(rng.uniform(0.1, 3.0)), "wave", v)
        elif ph == "store":
            apply_row(mem, x, w, y, n, st["xv"], st["wv"])               # output lands
            st["phase"] = "mark"
            push(t + float(rng.uniform(0.1, 2.0)), "wave", v)
        else:  # mark: stores complete, next entry
            i += WAVES
            nxt[v] = i if i < nb else 1 << 30
            if i < nb:
                state[v] = {"i": i, "phase": "wait_w"}
                push(t + float(rng.uniform(0.0, 1.0)), "wave", v)
    assert all(v == 1 << 30 for v in nxt)
    return mem


def random_table(rng, count):
    """Rows over one memory of elements: fresh slices, chains at random
    distances (some beyond the window), shared outputs, one-element overlaps,
    reads of what a later row overwrites, in-place rows."""
    top = [0]

    def fresh(n):
        o = top[0] + int(rng.integers(0, 3))
        top[0] = o + n + int(rng.integers(0, 3))
        return o

    rows = []
    for j in range(count):
        n = int(rng.choice([1, 2, 3, 5, 8]))
        r = rng.random()
        if j > 0 and r < 0.25:
            k = j - 1 - int(min(j - 1, rng.choice([0, 0, 1, 2, 3, 7, 70, 200])))
            kx, kw, ky, kn = rows[k]
            n = kn
            y = ky if rng.random() < 0.2 else fresh(n)          # sometimes the same output
            rows.append((ky, fresh(n), y, n))                  # read that row's output
        elif j > 0 and r < 0.35:
            k = int(rng.integers(0, j))
            kx, kw, ky, kn = rows[k]
            shift = int(rng.choice([-1, 1])) * (kn - 1)        # one element in common
            o = max(0, ky + shift)
            which = rng.random()
            if which < 0.4:
                rows.append((o, fresh(kn), fresh(kn), kn))       # x on its output
            elif which < 0.7:
                rows.append((fresh(kn), o, fresh(kn), kn))       # w on its output
            else:
                rows.append((fresh(kn), fresh(kn), o, kn))       # output on its output
        elif j > 0 and r < 0.42:
            k = int(rng.integers(0, j))
            kx, kw, ky, kn = rows[k]
            rows.append((fresh(kn), fresh(kn), kx, kn))         # overwrite an earlier read
        elif r < 0.47:
            o = fresh(n)
            rows.append((o, fresh(n), o, n))                    # in place
        else:
            rows.append((fresh(n), fresh(n), fresh(n), n))
    return rows, top[0] + 16


def test_deps_cover_every_conflict():
    """The conservative window: every earlier entry that meets entry i is at
    or before dep[i], and every earlier output meeting its w at or before
    dep_w[i] (so waiting for all entries up to dep covers every conflict)."""
    rng = np.random.Generator(np.random.PCG64(0xDA6))
    for t in range(300):
        rows, _ = random_table(rng, int(rng.choice([5, 30, 150, 400])))
        b = bound_rows(rows)
        dep, dep_w = deps(rows, b)
        for i in range(len(b)):
            for k in range(i):
                if rows_meet(rows[b[i]], rows[b[k]]):
                    assert dep[i] >= k, (t, i, k, dep[i])
                if w_meets_output(rows[b[i]], rows[b[k]]):
                    assert dep_w[i] >= k, (t, i, k, dep_w[i])
            assert dep_w[i] <= dep[i] and dep[i] < i


@pytest.mark.parametrize("block", range(4))
def test_walk_equals_in_order_application(block):
    rng = np.random.Generator(np.random.PCG64(0x5A1 + block))
    for t in range(150):
        count = int(rng.choice([1, 2, 4, 9, 33, 80, 300]))
        rows, size = random_table(rng, count)
        mem0 = rng.standard_normal(size)
        want = in_order(mem0, rows)
        for rep in range(3):
            got = simulate(mem0, rows, rng)
            assert np.array_equal(got, want), (block, t, rep, count)


def test_a_plain_wavefront_order_without_waits_would_be_caught():
    """Control: the same simulation with the waits removed (every dep -1)
    produces a different result on chained tables, so the check has teeth."""
    global deps
    saved = deps
    rng = np.random.Generator(np.random.PCG64(0xC0))
    try:
        deps = lambda rows, lst: ([-1] * len(lst), [-1] * len(lst))
        caught = 0
        for t in range(40):
            rows = []
            for j in range(12):                       # a chain: row j reads row j-1's output
                rows.append((8 * (j - 1) if j else 200, 300 + 8 * j, 8 * j, 4))
            mem0 = rng.standard_normal(400)
            caught += not np.array_equal(simulate(mem0, rows, rng), in_order(mem0, rows))
        assert caught > 0
    finally:
        deps = saved
