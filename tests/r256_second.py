"""A second, deliberately naive transcription of the R256 row normalisation.

Independent of the C oracle: it builds an explicit list of element indices
for each of the 256 lanes, accumulates each list with an exactly rounded
fused multiply-add, reduces each 64-lane group and then the four group totals
with one recursive halving function, and evaluates every step with
exact-rational rounding (tests/exact_f32.py). Slow; meant for rows of at most
a few tens of thousands of elements.

Definition followed: Lecture 04 "Launch Geometry: Grids, Occupancy, and 327
Norms per Token", section 2.1 (narrow sum of squares; block sum; inverse of
sqrt(ss/(float)n + eps); wide apply), with the lane count, tree order and the
correctly rounded sqrt-then-divide that this library fixes. `lanes=128` gives
the same definition with the lecture's 128 summing threads: 128 lane lists
and four groups of 32.
"""
import numpy as np

import exact_f32 as ex

LANES = 256
GROUP = 64


def lane_lists(n, lanes=LANES):
    lists = [[] for _ in range(lanes)]
    for d in range(n):
        lists[d % lanes].append(d)
    return lists


def halve(vals):
    """Descending halving: pair element j with element j + len/2."""
    if len(vals) == 1:
        return vals[0]
    s = len(vals) // 2
    return halve([ex.add(vals[j], vals[j + s]) for j in range(s)])


def sumsq(x, lanes=LANES):
    x = np.asarray(x, dtype=np.float32)
    group = lanes // 4
    partial = []
    for idx in lane_lists(len(x), lanes):
        acc = np.float32(0.0)
        for d in idx:
            acc = ex.fma(x[d], x[d], acc)
        partial.append(acc)
    groups = [halve(partial[group * g: group * (g + 1)]) for g in range(4)]
    return halve(groups)


def inv_rms(ss, n, eps):
    m = ex.div(ss, np.float32(n))
    t = ex.add(m, np.float32(eps))
    r = ex.sqrt(t)
    return ex.div(np.float32(1.0), r)


def row(x, w, eps, lanes=LANES):
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    inv = inv_rms(sumsq(x, lanes), len(x), eps)
    return np.array([ex.mul(ex.mul(x[d], inv), w[d]) for d in range(len(x))], dtype=np.float32)
