"""CPU model of the persistent launch's run walk: its ordering rules, checked
against in-order application on random tables before any GPU runs it.

The model restates, in Python, what the first workgroup of the spread
persistent launch does with the rows bound to table order when it takes the
run walk:

* every row is shared by the workgroup's threads in one fixed mapping: the
  element at index e of any row belongs to thread (e mod P) // Q (P elements
  per period, Q per quad; the kernel has P = 1024, Q = 4, 256 threads);
* the walk is taken only when every pair of rows that meet, meets at ranges
  whose starts are a multiple of P apart, and a row's own w meets its output
  only at the same addresses;
* each row's stored values stay in each thread's registers until the next
  row is done; entry j is "forwarded" when its x is exactly entry j - 1's
  output: x is then taken from those registers, not loaded (the model keeps
  the last R rows, R = 1 as in the kernel);
* entry j is "ahead" when its w, and its x unless forwarded, meet none of the
  outputs of the D entries before it; a run is a stretch of entries each
  ahead but the first: at its start the loads of its first D entries are
  issued (after every store before it), and while entry i is reduced the
  loads of entry i + D are in flight (issued before entry i + 1 stores);
  an entry that is not ahead starts a new run, and so does the first and
  the entry after the last of a stretch of at least FWD_RUN entries each
  forwarded from the one just before (a forward run: the kernel then loads
  w only, and only the entries of one kind of run are issued early);
* a row sums its x over all threads (a barrier between each thread's
  partial and the total), then applies and stores.

The hardware facts the model allows and nothing more: each thread's memory
operations take effect at any moment after they are issued, in any order
among themselves, except that two operations of one thread on the same
address take effect in program order; a load has taken effect before its
value is used; a barrier waits for every thread to arrive, and for nothing
else. A random scheduler interleaves the threads and the operations. Every
run must end and leave memory exactly as applying the rows one after
another in table order does. Controls show that the model catches a
misaligned table, a forbidden prefetch and a forwarded row whose x is not
the previous output.
"""
import random

import numpy as np
import pytest

P = 8          # elements per period
Q = 2          # elements per quad (one thread's share of a period)
THREADS = P // Q
MOD = 1_000_003


def owner(e):
    return (e % P) // Q


def meet(a0, alen, b0, blen):
    return alen > 0 and blen > 0 and a0 < b0 + blen and b0 < a0 + alen


def range_pairs(a, b):
    """The five (reader-or-writer range of one row, output of the other)
    pairs that make rows a and b meet, as (start_1, start_2, length_1, length_2)."""
    ax, aw, ay, an = a
    bx, bw, by, bn = b
    return [(ax, by, an, bn), (aw, by, an, bn), (ay, by, an, bn), (bx, ay, bn, an), (bw, ay, bn, an)]


def rows_meet(a, b):
    return any(meet(s1, l1, s2, l2) for s1, s2, l1, l2 in range_pairs(a, b))


def eligible(rows):
    """The kernel's rule: every meeting pair of ranges starts a multiple of P
    apart; a row's own w meets its output only at the same addresses."""
    for j in range(len(rows)):
        x, w, y, n = rows[j]
        if meet(w, n, y, n) and (w - y) % P:
            return False
        for k in range(j):
            for s1, s2, l1, l2 in range_pairs(rows[j], rows[k]):
                if meet(s1, l1, s2, l2) and (s1 - s2) % P:
                    return False
    return True


def one_owner(rows):
    """What the rule stands for: every address that two rows both touch, one
    of them writing it, is taken by the same thread in both; and in a row
    whose w meets its output, each such address by one thread."""
    def touches(r):
        x, w, y, n = r
        return ([(x + e, owner(e), "r") for e in range(n)] + [(w + e, owner(e), "r") for e in range(n)] +
                [(y + e, owner(e), "w") for e in range(n)])
    for j in range(len(rows)):
        x, w, y, n = rows[j]
        for e in range(n):
            for f in range(n):
                if w + e == y + f and owner(e) != owner(f):
                    return False
        tj = touches(rows[j])
        for k in range(j):
            tk = touches(rows[k])
            for a, oa, ka in tj:
                for b, ob, kb in tk:
                    if a == b and "w" in (ka, kb) and oa != ob:
                        return False
    return True


D = 2          # entries whose loads are in flight beyond the one reduced
R = 1          # earlier outputs kept in registers (the row just before)
FWD_RUN = 4    # shortest forward run


def flags(rows):
    """Per entry: (ahead, forwarding distance or 0)."""
    out = []
    for j in range(len(rows)):
        x, w, y, n = rows[j]
        fwd, found, xnear, wnear = 0, False, False, False
        for k in range(1, max(R, D) + 1):
            if j - k < 0:
                break
            px, pw, py, pn = rows[j - k]
            xm = meet(x, n, py, pn)
            if k <= D:
                xnear |= xm
                wnear |= meet(w, n, py, pn)
            if not found and xm and k <= R:
                fwd = k if (x == py and n == pn) else 0
            found |= xm
        ahead = j > 0 and not wnear and (fwd > 0 or not xnear)
        out.append((ahead, fwd))
    return out


def run_marks(fl):
    """Per entry: (forward run, continues the run before, deep), from the
    (ahead, forwarding distance) flags: a forward run is a stretch of at
    least FWD_RUN entries each ahead and forwarded from the entry just
    before; an entry continues the run before when it is ahead and of the
    same kind; it is deep when it and the D - 1 entries before it all
    continue (its loads may go out D entries early)."""
    nb = len(fl)
    chained = [0 < j and fl[j][0] and fl[j][1] == 1 for j in range(nb)]
    fr = []
    for j in range(nb):
        if not chained[j]:
            fr.append(False)
            continue
        a = j
        while a - 1 >= 0 and chained[a - 1]:
            a -= 1
        b = j
        while b + 1 < nb and chained[b + 1]:
            b += 1
        fr.append(b - a + 1 >= FWD_RUN)
    cont = [j > 0 and fl[j][0] and fr[j] == fr[j - 1] for j in range(nb)]
    deep = [j >= D and all(cont[j - k] for k in range(D)) for j in range(nb)]
    return fr, cont, deep


def row_values(xs, ws, total):
    return [(2 * xv + wv + total) % MOD for xv, wv in zip(xs, ws)]


def in_order(mem0, rows):
    mem = mem0.copy()
    for x, w, y, n in rows:
        xs = [int(v) for v in mem[x:x + n]]
        ws = [int(v) for v in mem[w:w + n]]
        total = sum(xs) % MOD
        mem[y:y + n] = row_values(xs, ws, total)
    return mem


class Thread:
    """One thread's program, run as a generator of steps: ('issue', op),
    ('use', op), ('barrier', key)."""

    def __init__(self, t, rows, fl):
        self.t, self.rows, self.fl = t, rows, fl

    def mine(self, n):
        return [e for e in range(n) if owner(e) == self.t]

    def loads(self, i, x_too):
        x, w, y, n = self.rows[i]
        ops = {}
        if x_too:
            ops["x"] = {"kind": "load", "addr": [x + e for e in self.mine(n)]}
        ops["w"] = {"kind": "load", "addr": [w + e for e in self.mine(n)]}
        return ops

    def program(self, partials):
        rows, fl, nb = self.rows, self.fl, len(self.rows)
        fwd = lambda j: fl[j][1]
        fr, cont, deep = run_marks(fl)
        ring = [None] * R            # ring[k - 1]: this thread's stored values k entries back
        i = 0
        while i < nb:
            bufs = {}
            chain = True
            for m in range(D):          # a run starts: its first D entries load
                chain = chain and (m == 0 or (i + m < nb and cont[i + m]))
                if chain and i + m < nb:
                    bufs[i + m] = self.loads(i + m, fwd(i + m) == 0)
                    for op in bufs[i + m].values():
                        yield ("issue", op)
            while True:
                j = i + D
                if j < nb and deep[j]:
                    bufs[j] = self.loads(j, fwd(j) == 0)
                    for op in bufs[j].values():
                        yield ("issue", op)
                x, w, y, n = rows[i]
                cur = bufs.pop(i)
                if fwd(i):
                    xs = ring[fwd(i) - 1]
                else:
                    yield ("use", cur["x"])
                    xs = cur["x"]["value"]
                partials[i][self.t] = sum(xs) % MOD
                yield ("barrier", i)
                total = sum(partials[i]) % MOD
                yield ("use", cur["w"])
                vals = row_values(xs, cur["w"]["value"], total)
                yield ("issue", {"kind": "store", "addr": [y + e for e in self.mine(n)],
                                 "value": vals})
                ring = [vals] + ring[:-1]
                i += 1
                if i >= nb or not cont[i]:
                    break


def simulate(mem0, rows, fl, rng, perform_bias):
    mem = mem0.copy()
    nb = len(rows)
    partials = [[0] * THREADS for _ in range(nb)]
    progs = [Thread(t, rows, fl).program(partials) for t in range(THREADS)]
    state = [None] * THREADS           # the step a thread is blocked on
    pending = [[] for _ in range(THREADS)]
    done = [False] * THREADS
    at_barrier = {}

    def perform(t, k):
        op = pending[t].pop(k)
        if op["kind"] == "load":
            op["value"] = [int(mem[a]) for a in op["addr"]]
            op["done"] = True
        else:
            for a, v in zip(op["addr"], op["value"]):
                mem[a] = v

    def performable(t):
        """Pending operations of thread t that no earlier pending operation
        on a common address holds back."""
        out = []
        for k, op in enumerate(pending[t]):
            if not any(set(op["addr"]) & set(pending[t][m]["addr"]) for m in range(k)):
                out.append(k)
        return out

    def advance(t):
        while True:
            if state[t] is not None:
                kind, arg = state[t]
                if kind == "use" and not arg.get("done"):
                    return False
                if kind == "barrier":
                    if at_barrier.get(arg, 0) < THREADS:
                        return False
                state[t] = None
            try:
                step = next(progs[t])
            except StopIteration:
                done[t] = True
                return True
            kind, arg = step
            if kind == "issue":
                pending[t].append(arg)
                return True
            if kind == "barrier":
                at_barrier[arg] = at_barrier.get(arg, 0) + 1
            state[t] = step

    steps = 0
    while not all(done) or any(pending):
        steps += 1
        assert steps < 400_000, "the walk did not finish"
        choices = []
        for t in range(THREADS):
            ks = performable(t)
            if ks:
                choices.append(("perform", t, ks))
        runnable = [t for t in range(THREADS) if not done[t]]
        if choices and (not runnable or rng.random() < perform_bias):
            _, t, ks = rng.choice(choices)
            perform(t, rng.choice(ks))
            continue
        moved = False
        for t in rng.sample(runnable, len(runnable)):
            if advance(t):
                moved = True
                break
        if not moved:
            assert choices, "every thread is blocked with nothing in flight: deadlock"
            _, t, ks = rng.choice(choices)
            perform(t, rng.choice(ks))
    return mem


def random_table(rng, count, aligned=True):
    """Rows over one memory: chains at random distances, the same output
    written twice, reads of what a later row overwrites, partial overlaps,
    in-place rows. With `aligned`, every overlap is a multiple of P apart;
    otherwise some are shifted by a quad."""
    top = [0]

    def fresh(n):
        o = top[0] + P * rng.randint(0, 2)
        top[0] = o + n + P * rng.randint(0, 2)
        top[0] += (-top[0]) % P
        return o

    shift = lambda: (P * rng.choice([-1, 1])) if aligned else Q * rng.choice([-1, 1])
    rows = []
    while len(rows) < count:
        j = len(rows)
        n = Q * rng.choice([1, 2, 3, 4, 6, 8])
        r = rng.random()
        if j > 0 and r < 0.06:
            for _ in range(min(rng.randint(4, 7), count - j)):   # a chain: each reads the one before
                kx, kw, ky, kn = rows[-1]
                rows.append((ky, fresh(kn), fresh(kn), kn))
        elif j > 0 and r < 0.35:
            k = j - 1 - min(j - 1, rng.choice([0, 0, 0, 1, 1, 2, 3, 5, 9]))
            kx, kw, ky, kn = rows[k]
            n = kn
            y = ky if rng.random() < 0.15 else fresh(n)
            rows.append((ky, fresh(n), y, n))                     # reads that row's output
        elif j > 0 and r < 0.45:
            k = rng.randrange(j)
            kx, kw, ky, kn = rows[k]
            o = max(0, ky + shift())                              # part of an earlier output
            which = rng.random()
            if which < 0.4:
                rows.append((o, fresh(kn), fresh(kn), kn))
            elif which < 0.7:
                rows.append((fresh(kn), o, fresh(kn), kn))
            else:
                rows.append((fresh(kn), fresh(kn), o, kn))
        elif j > 0 and r < 0.52:
            k = rng.randrange(j)
            kx, kw, ky, kn = rows[k]
            rows.append((fresh(kn), fresh(kn), kx, kn))           # overwrites an earlier read
        elif r < 0.58:
            o = fresh(n)
            rows.append((o, fresh(n), o, n))                      # in place
        elif r < 0.61:
            o = fresh(n)
            rows.append((fresh(n), o, o, n))                      # w is the output
        else:
            rows.append((fresh(n), fresh(n), fresh(n), n))
    return rows, top[0] + 2 * P + 16


def test_rule_means_one_owner():
    """The alignment rule (starts a multiple of P apart) holds exactly when
    every address two rows share, one of them writing it, has one owner
    thread; checked both ways on random tables, aligned and not."""
    rng = random.Random(0x0A11)
    agree = {True: 0, False: 0}
    for t in range(400):
        rows, _ = random_table(rng, rng.choice([2, 3, 5, 8, 12]), aligned=rng.random() < 0.25)
        e = eligible(rows)
        assert e == one_owner(rows), (t, rows)
        agree[e] += 1
    assert agree[True] > 40 and agree[False] > 40, agree


def test_flags_on_the_decode_chains():
    """The decode step's three chains (each norm reads the previous norm of
    its width), as one list: a 7168-wide norm right after a 7168-wide one
    takes its x from registers; a norm whose source is D entries back (the
    second 7168-wide norm of a layer without the 512-wide one) starts a run;
    every other entry but the first is ahead."""
    import workloads as wl
    widths = wl.decode_widths()
    top, rows, last = 0, [], {}
    for n in widths:
        def fresh():
            nonlocal top
            top += n
            return top - n
        x = rows[last[n]][2] if n in last else fresh()
        rows.append((x, fresh(), fresh(), n))
        last[n] = len(rows) - 1
    fl = flags(rows)
    assert fl[0][0] is False
    src = {}
    for i, n in enumerate(widths):
        back = i - src[n] if n in src else None
        want = back if back is not None and back <= R else 0
        assert fl[i][1] == want, (i, n, fl[i], back)
        if i > 0:
            assert fl[i][0] == (back is None or back == 1 or back > D), (i, n, fl[i], back)
        src[n] = i
    assert sum(1 for _, f in fl if f) == 93             # 92 layer boundaries and the last norm


@pytest.mark.parametrize("block", range(4))
def test_run_walk_equals_in_order_application(block):
    rng = random.Random(0x7A1 + block)
    kinds = {"ahead": 0, "forward": 0, "run": 0, "deep": 0, "forward run": 0}
    checked = 0
    for t in range(120):
        count = rng.choice([1, 2, 3, 5, 9, 17, 40])
        rows, size = random_table(rng, count, aligned=True)
        assert eligible(rows)
        fl = flags(rows)
        for j, (ahead, fwd) in enumerate(fl):
            kinds["run" if not ahead else "ahead"] += 1
            kinds["forward"] += fwd > 0
        fr, cont, deep = run_marks(fl)
        kinds["deep"] += sum(deep)
        kinds["forward run"] += sum(fr)
        mem0 = np.array([rng.randrange(MOD) for _ in range(size)], dtype=np.int64)
        want = in_order(mem0, rows)
        for rep in range(3):
            got = simulate(mem0, rows, fl, rng, perform_bias=rng.choice([0.2, 0.5, 0.8]))
            assert np.array_equal(got, want), (block, t, rep, rows, fl)
            checked += 1
    assert min(kinds.values()) > 20, kinds
    assert checked == 360


def _caught(make_rows, make_flags, seed, tries=60):
    rng = random.Random(seed)
    caught = 0
    for _ in range(tries):
        rows, size = make_rows(rng)
        mem0 = np.array([rng.randrange(MOD) for _ in range(size)], dtype=np.int64)
        got = simulate(mem0, rows, make_flags(rows), rng, perform_bias=rng.choice([0.1, 0.3, 0.6]))
        caught += not np.array_equal(got, in_order(mem0, rows))
    return caught


def test_control_misaligned_tables_are_caught():
    """The same walk on tables whose rows meet a quad apart (the rule would
    refuse them) gives wrong results in some schedules: the simulation sees
    threads racing."""
    def rows_(rng):
        rows = []
        for j in range(10):                     # a chain, each x a quad past the output before
            rows.append((200 + 16 * (j - 1) + Q if j else 900, 400 + 16 * j, 200 + 16 * j, 2 * P))
        return rows, 3000
    assert not eligible(rows_(random.Random(0))[0])
    assert _caught(rows_, flags, 0xC1) > 0


def test_control_forbidden_prefetch_is_caught():
    """Aligned chains at distance 1 (x is the previous output, same range)
    loaded ahead instead of forwarded: the load may run before the previous
    row's store."""
    def rows_(rng):
        rows = []
        for j in range(10):
            rows.append((8 * P * (j - 1) if j else 900, 2000 + 8 * P * j, 8 * P * j, 2 * P))
        return rows, 3000
    assert eligible(rows_(random.Random(0))[0])
    assert flags(rows_(random.Random(0))[0])[1:] == [(True, 1)] * 9
    assert _caught(rows_, lambda rows: [(False, 0)] + [(True, 0)] * (len(rows) - 1), 0xC2) > 0


def test_control_forward_of_a_different_range_is_caught():
    """A row whose x is a period past the previous output (meets it, not the
    same range) treated as forwarded takes the wrong values."""
    def rows_(rng):
        rows = []
        for j in range(8):
            rows.append(((8 * P * (j - 1) + P) if j else 900, 2000 + 8 * P * j, 8 * P * j, 2 * P))
        return rows, 3000
    assert flags(rows_(random.Random(0))[0])[1:] == [(False, 0)] * 7
    assert _caught(rows_, lambda rows: [(False, 0)] + [(True, 1)] * (len(rows) - 1), 0xC3) > 0


# --- Components: the bound rows split into groups that share no memory, each
# walked in table order by a workgroup of its own.

MAX_ROUNDS = 24


def meeting_pairs(rows):
    return [(j, k) for j in range(len(rows)) for k in range(j) if rows_meet(rows[j], rows[k])]


def components(count, edges, rng, max_rounds=MAX_ROUNDS):
    """The kernel's rounds restated: every pair whose labels differ hooks the
    greater label to the lesser (a minimum, in any order of the pairs), then
    every row follows its labels to the root (rows in any order, each seeing
    the others' writes); the rounds end when no pair has two labels. None
    when they do not settle within max_rounds."""
    label = list(range(count))
    for _ in range(max_rounds):
        hooked = False
        for a, b in rng.sample(edges, len(edges)):
            la, lb = label[a], label[b]
            if la != lb:
                hi, lo = max(la, lb), min(la, lb)
                label[hi] = min(label[hi], lo)
                hooked = True
        if not hooked:
            return label
        for j in rng.sample(range(count), count):
            r = label[j]
            while label[r] != r:
                r = label[r]
            label[j] = r
    return None


def bfs_components(count, edges):
    adj = [[] for _ in range(count)]
    for a, b in edges:
        adj[a].append(b)
        adj[b].append(a)
    comp = [-1] * count
    for s in range(count):
        if comp[s] < 0:
            comp[s] = s
            todo = [s]
            while todo:
                u = todo.pop()
                for v in adj[u]:
                    if comp[v] < 0:
                        comp[v] = s
                        todo.append(v)
    return comp


def walkers_of(rows, label, walkers):
    """Components in order of their least row, round-robin over the walkers."""
    bound = [j for j in range(len(rows)) if any(k != j and rows_meet(rows[j], rows[k])
                                               for k in range(len(rows)))]
    roots = sorted({label[j] for j in bound})
    rank = {r: i for i, r in enumerate(roots)}
    return {j: rank[label[j]] % walkers for j in bound}


@pytest.mark.parametrize("block", range(3))
def test_components_equal_connected_components(block):
    """On random tables (chains, shared outputs, overlaps, in-place rows) the
    labels are the least row of each connected component of the meeting
    pairs, whatever the order the threads take; rows given to different
    walkers never meet."""
    rng = random.Random(0xC0C0 + block)
    sizes = []
    for t in range(150):
        rows, _ = random_table(rng, rng.choice([2, 5, 12, 40, 90]), aligned=rng.random() < 0.5)
        edges = meeting_pairs(rows)
        label = components(len(rows), edges, rng)
        assert label is not None, (t, len(edges))
        assert label == bfs_components(len(rows), edges), t
        sizes.append(len(set(label[a] for a, _ in edges)))
        w = walkers_of(rows, label, 4)
        for a, b in edges:
            assert w[a] == w[b]
    assert max(sizes) >= 4


def test_components_of_the_decode_chains():
    """The chained decode table falls into three components: the 7168, 1536
    and 512-wide chains, on walkers 0, 1 and 2."""
    import workloads as wl
    widths = wl.decode_widths()
    top, rows, last = 0, [], {}
    for n in widths:
        x = rows[last[n]][2] if n in last else top
        top += n if n not in last else 0
        rows.append((x, top, top + n, n))
        top += 2 * n
        last[n] = len(rows) - 1
    edges = meeting_pairs(rows)
    label = components(len(rows), edges, random.Random(1))
    w = walkers_of(rows, label, 4)
    for j, n in enumerate(widths):
        assert w[j] == {7168: 0, 1536: 1, 512: 2}[n], (j, n)


def test_components_settle_in_few_rounds():
    """Long chains in either direction and a star settle well within the
    round cap; a cap of one round leaves a chain unsettled (the kernel then
    keeps every bound row in one walk)."""
    rng = random.Random(7)
    n = 400
    for edges in ([(j, j - 1) for j in range(1, n)],
                  [(n - 1 - j, n - j) for j in range(1, n)],
                  [(j, 0) for j in range(1, n)],
                  [(j, j // 2) for j in range(1, n)]):
        rounds = [0]
        for cap in range(1, MAX_ROUNDS + 1):
            if components(n, edges, random.Random(cap), max_rounds=cap) is not None:
                rounds[0] = cap
                break
        assert 0 < rounds[0] <= 6, rounds
    assert components(n, [(j, j - 1) for j in range(1, n)], rng, max_rounds=1) is None
