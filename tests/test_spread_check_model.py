"""CPU model of the rank step in the persistent launch's overlap check.

The spread launch puts the rows' outputs in order of start address before it
tests which rows meet. Each row's key is start * 2^16 + row (unique), and its
rank among all keys is found in two steps (quarter_ranks):

* the rows fall into four quarters of q = ceil(count / 4) consecutive rows;
  wavefront v ranks the keys of its quarter among themselves and writes them
  in that order into slots [v P, v P + n_v) of a sorted array, padding the
  rest of its P slots (P a power of two, at least q) with the largest key;
* each key's rank is its rank within its own quarter plus the number of keys
  below it in each other quarter, found by a branch-free binary search:
  steps P/2, P/4, ..., 1 each add the step when the slot before the
  candidate holds a smaller key, and a last comparison adds one.

The model restates those steps and checks that the ranks are exactly the
positions of the keys in sorted order, at every count from 1 to 40, around
the quarter and slot boundaries, and at the largest table (1024 rows).
"""
import random

import pytest

WAVES, LANES = 4, 64


def quarter_ranks(keys):
    count = len(keys)
    q = (count + 3) // 4
    P = 1
    while P < q:
        P *= 2
    big = (1 << 64) - 1
    sorted_ = [None] * (WAVES * P)
    for v in range(WAVES):
        q0 = v * q
        qn = max(0, min(q, count - q0))
        own = keys[q0:q0 + qn]
        for idx in range(P):
            sorted_[v * P + idx] = big
        for idx, k in enumerate(own):
            sorted_[v * P + sum(1 for kk in own if kk < k)] = k
    ranks = []
    for j, k in enumerate(keys):
        v = j // q
        own = keys[v * q:v * q + q]
        total = sum(1 for kk in own if kk < k)
        for u in range(WAVES):
            if u == v:
                continue
            at, step = 0, P // 2
            while step > 0:
                at += step if sorted_[u * P + at + step - 1] < k else 0
                step //= 2
            total += at + (1 if sorted_[u * P + at] < k else 0)
        ranks.append(total)
    return ranks


def keys_for(rng, count, ordered=0.0):
    """Output starts of a table (some in address order, some equal, some the
    empty-row marker), as the kernel keys them."""
    starts = []
    for j in range(count):
        r = rng.random()
        if j and r < ordered and starts[-1] < 1 << 47:
            starts.append(starts[-1] + rng.choice([64, 2048, 28672]))
        elif j and r < ordered + 0.05:
            starts.append(starts[rng.randrange(j)])                # the same output twice
        elif r < ordered + 0.08:
            starts.append(0xFFFFFFFFFFFF)                           # a row that writes nothing
        else:
            starts.append(rng.randrange(1 << 47))
    return [(s << 16) | j for j, s in enumerate(starts)]


@pytest.mark.parametrize("count", list(range(1, 41)) + [63, 64, 65, 127, 128, 129, 255, 256, 257,
                                                        327, 511, 512, 513, 1000, 1023, 1024])
def test_ranks_are_the_sorted_positions(count):
    rng = random.Random(1000 + count)
    for ordered in (0.0, 0.97):
        keys = keys_for(rng, count, ordered)
        ranks = quarter_ranks(keys)
        want = {k: i for i, k in enumerate(sorted(keys))}
        assert ranks == [want[k] for k in keys]
        assert sorted(ranks) == list(range(count))


def test_a_wrong_search_would_be_caught():
    """Control: dropping the last comparison of the binary search (a
    plausible off-by-one) breaks the permutation when a quarter fills its P
    slots (256 rows: quarters of 64, no padding)."""
    rng = random.Random(5)
    keys = keys_for(rng, 256)
    q = (len(keys) + 3) // 4
    P = 1
    while P < q:
        P *= 2
    sorted_ = []
    for v in range(WAVES):
        own = sorted(keys[v * q:(v + 1) * q])
        sorted_ += own + [(1 << 64) - 1] * (P - len(own))
    broken = []
    for k in keys:
        total = 0
        for u in range(WAVES):
            at, step = 0, P // 2
            while step > 0:
                at += step if sorted_[u * P + at + step - 1] < k else 0
                step //= 2
            total += at
        broken.append(total)
    assert sorted(broken) != list(range(len(keys)))
