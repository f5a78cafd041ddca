"""Seeded synthetic inputs for the row-wise RMSNorm workloads.

This module holds no part of the normalisation's arithmetic: it only draws
random numbers and shapes them into rows. It is the one piece shared by the
CPU oracle's tests and the GPU parity tests / benchmark, so both sides see
identical inputs.

Generator: numpy's PCG64, one independent stream per (workload, item, tensor)
seeded with ``0x524D534E00000000 | workload<<24 | item<<4 | tensor``
(tensor 0 = x, 1 = w, 2 = scale / outlier mask). Normals are drawn in float64
and rounded once to float32; bf16 inputs are then rounded float32 -> bf16 by
torch's round-to-nearest-even conversion (a library routine, not the
library-under-test's rounding code).

Workloads (widths and counts from the 327-norms-per-token decode step of
Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per Token",
section 2; widths up to the hidden size 7168):

* ``single``   fp32, 1 x 7168, x ~ N(0,1), w = 1 + 0.1 N(0,1)
* ``decode``   327 fp32 single rows: per layer (93 layers) a 7168 norm, a
               1536 norm, a 512 norm on even layers only (47 of 93), a second
               7168 norm; then one final 7168 norm (186 + 93 + 47 + 1)
* ``sweep``    fp32 rows at widths 1, 3, 64, 129, 1000, 4097, 7167, 7168,
               x = N(0,1) * 10^U, U ~ Uniform[-3, 3) drawn once per row
* ``batch64``  bf16 64 x 7168, x ~ N(0, 2) (variance 2), w as above
* ``prefill``  bf16 8192 x 7168, x ~ N(0,1) with each entry independently
               (probability 0.001) replaced by +100 or -100 (equal odds)
"""
import numpy as np

EPS = np.float32(1e-6)
HIDDEN = 7168

WL_SINGLE, WL_DECODE, WL_SWEEP, WL_BATCH64, WL_PREFILL, WL_MISC = 1, 2, 3, 4, 5, 6
SWEEP_WIDTHS = (1, 3, 64, 129, 1000, 4097, 7167, 7168)
BATCH64_SHAPE = (64, HIDDEN)
PREFILL_SHAPE = (8192, HIDDEN)
OUTLIER_P = 0.001
OUTLIER_VALUE = 100.0


def seed_of(workload, item, tensor):
    return 0x524D534E00000000 | (workload << 24) | (item << 4) | tensor


def rng(workload, item, tensor):
    return np.random.Generator(np.random.PCG64(seed_of(workload, item, tensor)))


def to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16), via torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_f32(g, size, sigma=1.0):
    return (g.standard_normal(size) * sigma).astype(np.float32)


def weight_f32(workload, n, item=0):
    """w = 1 + 0.1 * N(0,1), evaluated in float64, rounded once to float32."""
    z = rng(workload, item, 1).standard_normal(n)
    return (1.0 + 0.1 * z).astype(np.float32)


# ---- the five workloads ----------------------------------------------------

def single():
    x = normal_f32(rng(WL_SINGLE, 0, 0), HIDDEN)
    w = weight_f32(WL_SINGLE, HIDDEN)
    return x, w


def decode_widths():
    """The 327 widths of one decode step, in execution order."""
    ws = []
    for layer in range(93):
        ws.append(HIDDEN)
        ws.append(1536)
        if layer % 2 == 0:
            ws.append(512)
        ws.append(HIDDEN)
    ws.append(HIDDEN)
    assert len(ws) == 327
    return ws


def decode():
    """List of (x, w) float32 rows, one per norm of the decode step."""
    out = []
    for i, n in enumerate(decode_widths()):
        x = normal_f32(rng(WL_DECODE, i, 0), n)
        w = weight_f32(WL_DECODE, n, item=i)
        out.append((x, w))
    return out


def sweep_row(i, n):
    g = rng(WL_SWEEP, i, 2)
    u = g.uniform(-3.0, 3.0)
    z = rng(WL_SWEEP, i, 0).standard_normal(n)
    x = (z * 10.0 ** u).astype(np.float32)
    w = weight_f32(WL_SWEEP, n, item=i)
    return x, w


def sweep():
    return [sweep_row(i, n) for i, n in enumerate(SWEEP_WIDTHS)]


def batch64():
    rows, n = BATCH64_SHAPE
    x = np.empty((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r] = normal_f32(rng(WL_BATCH64, r, 0), n, sigma=np.sqrt(2.0))
    w = weight_f32(WL_BATCH64, n)
    return to_bf16_bits(x), to_bf16_bits(w)


def prefill_rows_f32(row_ids, n=HIDDEN):
    """float32 values of the requested prefill rows before the bf16 cast."""
    x = np.empty((len(row_ids), n), dtype=np.float32)
    for k, r in enumerate(row_ids):
        z = rng(WL_PREFILL, int(r), 0).standard_normal(n)
        g = rng(WL_PREFILL, int(r), 2)
        hit = g.random(n) < OUTLIER_P
        sign = np.where(g.integers(0, 2, size=int(hit.sum())) == 0, -1.0, 1.0)
        z[hit] = sign * OUTLIER_VALUE
        x[k] = z.astype(np.float32)
    return x


def prefill(row_ids=None):
    """bf16 bits (x rows, w). row_ids selects a subset (same values as in the
    full batch, since every row has its own stream)."""
    if row_ids is None:
        row_ids = range(PREFILL_SHAPE[0])
    x = prefill_rows_f32(list(row_ids))
    w = weight_f32(WL_PREFILL, PREFILL_SHAPE[1])
    return to_bf16_bits(x), to_bf16_bits(w)


def misc_f32(item, n, sigma=1.0):
    """Extra seeded float32 rows for tests (workload id 6)."""
    x = normal_f32(rng(WL_MISC, item, 0), n, sigma)
    w = weight_f32(WL_MISC, n, item=item)
    return x, w
