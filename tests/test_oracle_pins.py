"""Pins for the CPU oracle: checks against things other than the oracle itself.

* hand-derived worked examples (tests/golden/worked_examples.json)
* brute force on widths 1..8 with numpy's binary32 scalar operations
* an independent exact-rational second transcription of the association
* association probes that tell R256 apart from neighbouring orders
* zero padding, power-of-two scaling, constant rows, unit rows (closed forms)
* the float64 formula (max relative error <= 1e-6) on every workload
* the bf16 rounding against torch's round-to-nearest-even cast

Definition: Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per
Token", section 2.1; the pairwise-tree-after-chains shape follows Lecture 08
"Graph-resident decode", section 8.
"""
import json
import os

import numpy as np
import pytest

import exact_f32 as ex
import r256_second
import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def same_bits(a, b):
    """Bitwise equality, except that any two NaNs compare equal."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    nan = np.isnan(a)
    if not np.array_equal(nan, np.isnan(b)):
        return False
    return np.array_equal(bits32(a)[~nan], bits32(b)[~nan])


def f32_from_hex(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


# ---- golden worked examples -------------------------------------------------

def _golden():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_worked_examples(oracle_mod, case):
    eps = f32_from_hex(case["eps"])
    if case["dtype"] == "f32":
        x = np.array([int(h, 16) for h in case["x"]], dtype=np.uint32).view(np.float32)
        w = np.array([int(h, 16) for h in case["w"]], dtype=np.uint32).view(np.float32)
        y = oracle_mod.row_f32(x, w, eps)
        for got, want in zip(y, case["y"]):
            if want == "nan":
                assert np.isnan(got)
            else:
                assert int(got.view(np.uint32)) == int(want, 16), case["name"]
    else:
        x = np.array([int(h, 16) for h in case["x"]], dtype=np.uint16)
        w = np.array([int(h, 16) for h in case["w"]], dtype=np.uint16)
        y = oracle_mod.row_bf16(x, w, eps)
        assert [int(v) for v in y] == [int(h, 16) for h in case["y"]], case["name"]


# ---- brute force, widths 1..8 (R5) ------------------------------------------

def closed_form_small(x, w, eps):
    """R256 for n <= 8 written out: lanes 0..n-1 hold x_l^2 (one rounding;
    +0 for missing lanes), the first group's halving gives
    ((p0+p4)+(p2+p6)) + ((p1+p5)+(p3+p7)); the other groups are +0.
    Every step uses numpy binary32 scalar arithmetic."""
    f = np.float32
    with np.errstate(all="ignore"):
        p = [f(np.float64(v) * np.float64(v)) for v in x] + [f(0.0)] * (8 - len(x))
        g0 = (p[0] + p[4]) + (p[2] + p[6])
        g1 = (p[1] + p[5]) + (p[3] + p[7])
        w0 = g0 + g1
        ss = (w0 + f(0.0)) + (f(0.0) + f(0.0))
        m = ss / f(len(x))
        t = m + f(eps)
        r = np.sqrt(t)
        inv = f(1.0) / r
        return np.array([(xi * inv) * wi for xi, wi in zip(x, w)], dtype=np.float32)


def _tiny_rows():
    g = np.random.Generator(np.random.PCG64(20240607))
    specials = [0.0, -0.0, 1.0, -1.0, 2.0 ** -70, -(2.0 ** 60), 1.5e-41, -3e-44,
                1.8e19, -1.9e19, 3.4e38, 7.0, 1e-3, 65504.0]
    rows = []
    for n in range(1, 9):
        for k in range(40):
            x = (g.standard_normal(n) * 10.0 ** g.uniform(-4, 4)).astype(np.float32)
            if k % 3 == 1:
                x[g.integers(0, n)] = np.float32(specials[g.integers(0, len(specials))])
            if k % 5 == 2:
                x[:] = np.float32(specials[g.integers(0, len(specials))])
            w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
            eps = np.float32([1e-6, 0.0, 1e-5, 3.0][k % 4])
            rows.append((x, w, eps))
    return rows


def test_brute_force_tiny_widths(oracle_mod):
    for x, w, eps in _tiny_rows():
        want = closed_form_small(x, w, eps)
        got = oracle_mod.row_f32(x, w, eps)
        assert same_bits(got, want), (x, w, eps, got, want)


# ---- second transcription (R7 ii) --------------------------------------------

@pytest.mark.parametrize("n", [1, 5, 63, 255, 256, 257, 700, 1536, 4097, 7168, 19999])
def test_second_transcription_sumsq_and_row(oracle_mod, n):
    x, w = wl.misc_f32(1000 + n, n, sigma=float(10.0 ** ((n % 7) - 3)))
    eps = wl.EPS
    ss_or = oracle_mod.sumsq_f32(x)
    ss_2 = r256_second.sumsq(x)
    assert bits32(ss_or) == bits32(ss_2), (n, ss_or, ss_2)
    inv_or = oracle_mod.inv_rms(ss_or, n, eps)
    assert bits32(inv_or) == bits32(r256_second.inv_rms(ss_2, n, eps))
    if n <= 4097:
        assert same_bits(oracle_mod.row_f32(x, w, eps), r256_second.row(x, w, eps))


def test_inverse_matches_exact_epilogue(oracle_mod):
    """Steps 4-7 against exact-rational rounding over many (ss, n, eps)."""
    g = np.random.Generator(np.random.PCG64(77))
    for _ in range(3000):
        ss = np.float32(10.0 ** g.uniform(-30, 30))
        n = int(g.integers(1, 1 << 24))
        eps = np.float32([0.0, 1e-6, 1e-12, 0.5][int(g.integers(0, 4))])
        assert bits32(oracle_mod.inv_rms(ss, n, eps)) == bits32(r256_second.inv_rms(ss, n, eps))


# ---- association probes (R7 i) -----------------------------------------------

def _alt_sumsq(x, lanes=256, group=64, descending=True):
    """Neighbouring associations, each evaluated with exact-rational rounding:
    a different lane count, or ascending instead of descending halving."""
    x = np.asarray(x, dtype=np.float32)
    part = []
    for l in range(lanes):
        acc = np.float32(0.0)
        for d in range(l, len(x), lanes):
            acc = ex.fma(x[d], x[d], acc)
        part.append(acc)

    def tree(v):
        v = list(v)
        if descending:
            while len(v) > 1:
                s = len(v) // 2
                v = [ex.add(v[j], v[j + s]) for j in range(s)]
        else:
            while len(v) > 1:
                v = [ex.add(v[2 * j], v[2 * j + 1]) for j in range(len(v) // 2)]
        return v[0]
    groups = [tree(part[group * g:group * (g + 1)]) for g in range(lanes // group)]
    return tree(groups)


def _sequential_sumsq(x):
    acc = np.float32(0.0)
    for v in np.asarray(x, dtype=np.float32):
        acc = ex.fma(v, v, acc)
    return acc


def _probe_rows():
    probes = []
    # one huge square on lane 0 plus unit squares: 2^24 + 1 rounds to even,
    # so how many units meet the huge value inside one chain decides the bits
    x = np.ones(1024, dtype=np.float32)
    x[0] = 4096.0
    probes.append(x)
    # huge square placed on lane 100 of group 1, units everywhere else
    x = np.ones(768, dtype=np.float32)
    x[100] = 4096.0
    probes.append(x)
    # a tree-order probe: descending halving adds lanes 1 and 33 first (1+1=2,
    # then 2^24+2 is exact); adjacent-pair halving meets 2^24+1 first (-> 2^24)
    x = np.zeros(34, dtype=np.float32)
    x[0], x[1], x[33] = 4096.0, 1.0, 1.0
    probes.append(x)
    # a group-level probe: one group carries 2^24, units fill the others
    x = np.ones(512, dtype=np.float32)
    x[64:128] = 512.0
    probes.append(x)
    # ragged tail with mixed magnitudes
    g = np.random.Generator(np.random.PCG64(5))
    x = (g.standard_normal(1300) * np.where(g.random(1300) < 0.01, 3000.0, 1.0)).astype(np.float32)
    probes.append(x)
    return probes


def test_association_probes_discriminate(oracle_mod):
    """Each probe agrees with the second transcription of R256, and at least
    one probe tells R256 apart from every neighbouring association."""
    told_apart = {"L128": False, "L512": False, "ascending": False, "sequential": False}
    for x in _probe_rows():
        ss = oracle_mod.sumsq_f32(x)
        assert bits32(ss) == bits32(r256_second.sumsq(x))
        alts = {
            "L128": _alt_sumsq(x, lanes=128, group=32),
            "L512": _alt_sumsq(x, lanes=512, group=128),
            "ascending": _alt_sumsq(x, descending=False),
            "sequential": _sequential_sumsq(x),
        }
        for k, v in alts.items():
            if bits32(v) != bits32(ss):
                told_apart[k] = True
    assert all(told_apart.values()), told_apart


# ---- the 128-lane definition (the lecture's thread count) ---------------------

@pytest.mark.parametrize("n", [1, 7, 31, 32, 33, 127, 128, 129, 700, 1536, 7168, 9001])
def test_l128_second_transcription(oracle_mod, n):
    """The oracle's 128-lane sum and rows equal the independent transcription
    (lane lists of stride 128, four 32-lane groups, exact-rational rounding)."""
    x, w = wl.misc_f32(3000 + n, n, sigma=float(10.0 ** ((n % 5) - 2)))
    ss = oracle_mod.sumsq_lanes(x, 128)
    assert bits32(ss) == bits32(r256_second.sumsq(x, lanes=128)), n
    assert bits32(ss) == bits32(_alt_sumsq(x, lanes=128, group=32)), n
    if n <= 1536:
        assert same_bits(oracle_mod.row_lanes(x, w, wl.EPS, 128),
                         r256_second.row(x, w, wl.EPS, lanes=128))
    # lanes=256 through the same entry equals the R256 functions
    assert bits32(oracle_mod.sumsq_lanes(x, 256)) == bits32(oracle_mod.sumsq_f32(x))


def test_l128_probes_and_closed_forms(oracle_mod):
    """The probes tell the two definitions apart (R128 agrees with its own
    transcription on each); widths up to 8 have the same closed form under
    both (only the first group's lanes 0..7 hold values); zero padding is
    inert under R128 too; a bf16 row is its binary32 row rounded once."""
    differs = False
    for x in _probe_rows():
        s128 = oracle_mod.sumsq_lanes(x, 128)
        assert bits32(s128) == bits32(r256_second.sumsq(x, lanes=128))
        differs = differs or bits32(s128) != bits32(oracle_mod.sumsq_f32(x))
    assert differs
    for x, w, eps in _tiny_rows():
        assert same_bits(oracle_mod.row_lanes(x, w, eps, 128), closed_form_small(x, w, eps))
    x, _ = wl.misc_f32(11, 3000)
    base = oracle_mod.sumsq_lanes(x, 128)
    for m in (1, 127, 128, 7168):
        assert bits32(oracle_mod.sumsq_lanes(np.concatenate([x, np.zeros(m, np.float32)]), 128)) == bits32(base)
    xb, wb = wl.batch64()
    yb, _ = oracle_mod.rows(xb[:4], wb, wl.EPS, lanes=128)
    yf, _ = oracle_mod.rows(oracle_mod.bf16_to_f32(xb[:4]), oracle_mod.bf16_to_f32(wb), wl.EPS,
                            lanes=128)
    assert np.array_equal(yb, wl.to_bf16_bits(yf))
    assert bits32(oracle_mod.sumsq_lanes(xb[0], 128)) == bits32(
        oracle_mod.sumsq_lanes(oracle_mod.bf16_to_f32(xb[0]), 128))


def test_l128_float64_error(oracle_mod):
    """The 128-lane definition is as accurate as R256 on the decode widths:
    max relative error against the float64 formula below 1e-6."""
    for i, n in enumerate((7168, 1536, 512)):
        x, w = wl.misc_f32(4000 + i, n)
        y = oracle_mod.row_lanes(x, w, wl.EPS, 128)
        Y = oracle_mod.float64_reference(x, w, wl.EPS)
        nz = Y != 0
        assert np.max(np.abs(y[nz] - Y[nz]) / np.abs(Y[nz])) < 1e-6


def test_wave_totals_match_second_transcription(oracle_mod):
    x, _ = wl.misc_f32(7, 5000)
    W = oracle_mod.wave_totals_f32(x)
    lists = r256_second.lane_lists(len(x))
    part = []
    for idx in lists:
        acc = np.float32(0.0)
        for d in idx:
            acc = ex.fma(x[d], x[d], acc)
        part.append(acc)
    for g in range(4):
        assert bits32(W[g]) == bits32(r256_second.halve(part[64 * g:64 * (g + 1)]))


# ---- zero padding (R2) -------------------------------------------------------

@pytest.mark.parametrize("pad", [1, 255, 256, 7168])
def test_zero_padding_leaves_sum_bits(oracle_mod, pad):
    for n in (1, 100, 256, 1000, 7168):
        x, _ = wl.misc_f32(2000 + n, n)
        ss = oracle_mod.sumsq_f32(x)
        xp = np.concatenate([x, np.zeros(pad, dtype=np.float32)])
        assert bits32(oracle_mod.sumsq_f32(xp)) == bits32(ss)
        xn = np.concatenate([x, -np.zeros(pad, dtype=np.float32)])
        assert bits32(oracle_mod.sumsq_f32(xn)) == bits32(ss)


# ---- power-of-two scaling (R3: I1-I4) ------------------------------------------

def test_power_of_two_scaling_is_exact(oracle_mod):
    g = np.random.Generator(np.random.PCG64(11))
    for trial in range(40):
        n = int(g.integers(1, 9000))
        x, w = wl.misc_f32(3000 + trial, n)
        eps = np.float32(10.0 ** g.uniform(-8, -2))
        k = int(g.integers(-20, 21))
        j = int(g.integers(-20, 21))
        sx = (x * np.float32(2.0 ** k)).astype(np.float32)
        # I1: ss(2^k x) = 4^k ss(x)
        ss = oracle_mod.sumsq_f32(x)
        assert bits32(oracle_mod.sumsq_f32(sx)) == bits32(np.float32(ss * np.float32(4.0 ** k)))
        # I2: y(2^k x; 4^k eps) == y(x; eps)
        y = oracle_mod.row_f32(x, w, eps)
        y2 = oracle_mod.row_f32(sx, w, np.float32(eps * np.float32(4.0 ** k)))
        assert same_bits(y, y2)
        # I3: y(x; 2^j w) == 2^j y(x; w)
        y3 = oracle_mod.row_f32(x, (w * np.float32(2.0 ** j)).astype(np.float32), eps)
        assert same_bits(y3, (y * np.float32(2.0 ** j)).astype(np.float32))
        # I4: with eps = 0, y(2^k x) == y(x)
        assert same_bits(oracle_mod.row_f32(sx, w, np.float32(0)), oracle_mod.row_f32(x, w, np.float32(0)))
        # I3 in bf16 (power-of-two weights scale bf16 outputs exactly too)
        xb, wb = wl.to_bf16_bits(x), wl.to_bf16_bits(w)
        wb2 = wl.to_bf16_bits(oracle_mod.bf16_to_f32(wb) * np.float32(2.0 ** j))
        yb = oracle_mod.bf16_to_f32(oracle_mod.row_bf16(xb, wb, eps))
        yb2 = oracle_mod.bf16_to_f32(oracle_mod.row_bf16(xb, wb2, eps))
        assert same_bits(yb2, (yb * np.float32(2.0 ** j)).astype(np.float32))


# ---- constant rows (R4) and unit rows (R6) ----------------------------------------

def test_constant_row_closed_form(oracle_mod):
    """|y| = |w| / sqrt(1 + eps/c^2); for c = +-2^k the sum and mean are exact
    and the result is within 6 units in the last place."""
    u = 2.0 ** -24
    for k in range(-10, 11, 2):
        for sign in (1.0, -1.0):
            for n in (1, 3, 256, 7168, 10001):
                c = sign * 2.0 ** k
                x = np.full(n, c, dtype=np.float32)
                w = wl.weight_f32(wl.WL_MISC, n, item=k + 50)
                eps = wl.EPS
                assert oracle_mod.sumsq_f32(x) == np.float32(n * c * c)
                y = oracle_mod.row_f32(x, w, eps)
                want = np.abs(w.astype(np.float64)) / np.sqrt(1.0 + float(eps) / (c * c))
                rel = np.abs(np.abs(y.astype(np.float64)) - want) / want
                assert rel.max() <= 6 * u, (k, n, rel.max())
                assert np.all(np.sign(y) == np.sign(c) * np.sign(w))


@pytest.mark.parametrize("n", [1, 2, 255, 7168, 65537, (1 << 22) + 3])
def test_unit_rows_give_plus_minus_w(oracle_mod, n):
    """x in {+1,-1}, eps = 0: ss = n exactly, m = 1, inv = 1, so y = x * w."""
    g = np.random.Generator(np.random.PCG64(n))
    x = np.where(g.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)
    assert oracle_mod.sumsq_f32(x) == np.float32(n)
    assert same_bits(oracle_mod.row_f32(x, w, np.float32(0)), x * w)


def test_unit_rows_full_width_limit(oracle_mod):
    n = 1 << 24
    x = np.ones(n, dtype=np.float32)
    x[1::3] = -1.0
    assert oracle_mod.sumsq_f32(x) == np.float32(n)


# ---- float64 reference (R1) ---------------------------------------------------

def _max_rel(y32, Y):
    Y = np.asarray(Y, dtype=np.float64)
    nz = Y != 0
    return float(np.max(np.abs(y32.astype(np.float64)[nz] - Y[nz]) / np.abs(Y[nz]))) if nz.any() else 0.0


def test_float64_reference_single_and_decode(oracle_mod):
    worst = 0.0
    x, w = wl.single()
    worst = max(worst, _max_rel(oracle_mod.row_f32(x, w, wl.EPS), oracle_mod.float64_reference(x, w, wl.EPS)))
    for x, w in wl.decode():
        worst = max(worst, _max_rel(oracle_mod.row_f32(x, w, wl.EPS), oracle_mod.float64_reference(x, w, wl.EPS)))
    assert worst <= 1e-6, worst


def test_float64_reference_sweep(oracle_mod):
    for x, w in wl.sweep():
        r = _max_rel(oracle_mod.row_f32(x, w, wl.EPS), oracle_mod.float64_reference(x, w, wl.EPS))
        assert r <= 1e-6, (len(x), r)


def _bf16_check(oracle_mod, xb, wb, yb):
    """|y_bf16 - Y| <= half a bf16 ulp of max(|Y|,|y|) + 1e-6 |Y| elementwise."""
    Y = oracle_mod.float64_reference(oracle_mod.bf16_to_f32(xb), oracle_mod.bf16_to_f32(wb), wl.EPS)
    y = oracle_mod.bf16_to_f32(yb).astype(np.float64)
    mag = np.maximum(np.abs(Y), np.abs(y))
    ulp = np.ldexp(1.0, np.frexp(mag)[1] - 8)       # bf16 has 8 significant bits
    err = np.abs(y - Y)
    assert np.all(err <= 0.5 * ulp + 1e-6 * np.abs(Y))


def test_float64_reference_bf16_workloads(oracle_mod):
    xb, wb = wl.batch64()
    yb, _ = oracle_mod.rows(xb, wb, wl.EPS)
    _bf16_check(oracle_mod, xb, wb, yb)
    ids = list(range(0, 8192, 61))
    xb, wb = wl.prefill(ids)
    yb, _ = oracle_mod.rows(xb, wb, wl.EPS)
    _bf16_check(oracle_mod, xb, wb, yb)
    # the binary32 values before the final rounding meet the 1e-6 bar too
    xf, wf = oracle_mod.bf16_to_f32(xb), oracle_mod.bf16_to_f32(wb)
    yf, _ = oracle_mod.rows(xf, wf, wl.EPS)
    assert _max_rel(yf, oracle_mod.float64_reference(xf, wf, wl.EPS)) <= 1e-6


# ---- bf16 rounding and widening ------------------------------------------------

def test_bf16_rounding_matches_torch_rne(oracle_mod):
    import torch
    g = np.random.Generator(np.random.PCG64(3))
    pats = g.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (g.integers(0, 1 << 16, size=2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    edge = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x00008000, 0x00018000,
                     0x0000FFFF, 0x80008000, 0x3F808000, 0x3F818000, 0x7F800000, 0xFF800000,
                     0x00000000, 0x80000000, 0x007FFFFF, 0x00800000], dtype=np.uint32)
    allp = np.concatenate([pats, ties, edge])
    v = allp.view(np.float32)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for k in range(len(v)):
        got = oracle_mod.f32_to_bf16_scalar(v[k])
        if np.isnan(v[k]):
            assert got == (0x7FC0 | ((int(allp[k]) >> 16) & 0x8000))
        else:
            assert got == int(ref[k]), hex(int(allp[k]))


def test_bf16_range_narrowing_matches_torch_rne(oracle_mod):
    """The oracle's narrowing over a run of consecutive bit patterns (the form
    the device's conversion is checked against) equals torch's RNE cast on
    every non-NaN pattern of three 2^20-pattern windows: around 1.0, across the
    largest finite values into infinity and NaN, and over the subnormals."""
    import torch
    for first in (0x3F780000, 0x7F700000, 0x00000000, 0x807F0000):
        got = oracle_mod.f32_to_bf16_range(first, 1 << 20)
        pats = (np.arange(1 << 20, dtype=np.uint64) + first).astype(np.uint32)
        v = pats.view(np.float32)
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(v)
        assert np.array_equal(got[~nan], ref[~nan]), hex(first)
        assert np.all(got[nan] == (0x7FC0 | ((pats[nan] >> 16) & 0x8000)))


def test_bf16_row_is_f32_row_rounded(oracle_mod):
    """The bf16 path equals the binary32 path on widened inputs, rounded once
    (torch's cast), i.e. no intermediate bf16 rounding."""
    xb, wb = wl.batch64()
    yb, _ = oracle_mod.rows(xb[:8], wb, wl.EPS)
    yf, _ = oracle_mod.rows(oracle_mod.bf16_to_f32(xb[:8]), oracle_mod.bf16_to_f32(wb), wl.EPS)
    assert np.array_equal(yb, wl.to_bf16_bits(yf))


# ---- host logic: threading does not change bits --------------------------------

def test_rows_threads_bit_identical(oracle_mod):
    xb, wb = wl.prefill(range(40))
    y1, used1 = oracle_mod.rows(xb, wb, wl.EPS, nthreads=1)
    y4, used4 = oracle_mod.rows(xb, wb, wl.EPS, nthreads=4)
    assert used1 == 1 and used4 == 4
    assert np.array_equal(y1, y4)
