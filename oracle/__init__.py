"""CPU oracle for the row-wise RMSNorm -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

Two references live here:

* the binary32 oracle (``rmsn_ref.c``, loaded with ctypes): the fixed
  association R256 spelled out step by step -- the bit-exact contract;
* ``float64_reference``: the real-number formula of Lecture 04 "Launch
  Geometry: Grids, Occupancy, and 327 Norms per Token", section 2.1
  (y = x * w / sqrt(sum(x^2)/n + eps)) evaluated in float64 with numpy,
  independent of any association; it bounds the oracle's rounding error.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librmsn_ref.so")
_lib = None

F32 = 0
BF16 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build(verbose=False)
    lib = ctypes.CDLL(_LIB_PATH)
    c_i64, c_f, c_vp, c_int = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    lib.rmsn_ref_sumsq_f32.argtypes = [c_vp, c_i64]
    lib.rmsn_ref_sumsq_f32.restype = c_f
    lib.rmsn_ref_sumsq_bf16.argtypes = [c_vp, c_i64]
    lib.rmsn_ref_sumsq_bf16.restype = c_f
    lib.rmsn_ref_inv.argtypes = [c_f, c_i64, c_f]
    lib.rmsn_ref_inv.restype = c_f
    lib.rmsn_ref_wave_totals_f32.argtypes = [c_vp, c_i64, c_vp]
    lib.rmsn_ref_wave_totals_f32.restype = None
    lib.rmsn_ref_row_f32.argtypes = [c_vp, c_vp, c_vp, c_i64, c_f]
    lib.rmsn_ref_row_f32.restype = None
    lib.rmsn_ref_row_bf16.argtypes = [c_vp, c_vp, c_vp, c_i64, c_f]
    lib.rmsn_ref_row_bf16.restype = None
    lib.rmsn_ref_rows.argtypes = [c_int, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_f, c_int]
    lib.rmsn_ref_rows.restype = c_int
    lib.rmsn_ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.rmsn_ref_bf16_to_f32.restype = c_f
    lib.rmsn_ref_f32_to_bf16.argtypes = [c_f]
    lib.rmsn_ref_f32_to_bf16.restype = ctypes.c_uint16
    lib.rmsn_ref_sumsq_lanes.argtypes = [c_int, c_vp, c_i64, c_int]
    lib.rmsn_ref_sumsq_lanes.restype = c_f
    lib.rmsn_ref_rows_lanes.argtypes = [c_int, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_f,
                                        c_int, c_int]
    lib.rmsn_ref_rows_lanes.restype = c_int
    lib.rmsn_ref_f32_to_bf16_range.argtypes = [ctypes.c_uint32, c_i64, c_vp]
    lib.rmsn_ref_f32_to_bf16_range.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def sumsq_f32(x):
    """R256 steps 1-3 on a binary32 row; returns a numpy float32."""
    x = _f32(x)
    return np.float32(_load().rmsn_ref_sumsq_f32(_ptr(x), x.size))


def sumsq_bf16(x_bits):
    x = _u16(x_bits)
    return np.float32(_load().rmsn_ref_sumsq_bf16(_ptr(x), x.size))


def wave_totals_f32(x):
    """The four 64-lane tree totals W[0..3] (R256 step 2)."""
    x = _f32(x)
    out = np.zeros(4, dtype=np.float32)
    _load().rmsn_ref_wave_totals_f32(_ptr(x), x.size, _ptr(out))
    return out


def inv_rms(ss, n, eps):
    """R256 steps 4-7."""
    return np.float32(_load().rmsn_ref_inv(float(np.float32(ss)), int(n), float(np.float32(eps))))


def row_f32(x, w, eps):
    x, w = _f32(x), _f32(w)
    assert x.shape == w.shape and x.ndim == 1
    y = np.empty_like(x)
    _load().rmsn_ref_row_f32(_ptr(x), _ptr(w), _ptr(y), x.size, float(np.float32(eps)))
    return y


def row_bf16(x_bits, w_bits, eps):
    x, w = _u16(x_bits), _u16(w_bits)
    assert x.shape == w.shape and x.ndim == 1
    y = np.empty_like(x)
    _load().rmsn_ref_row_bf16(_ptr(x), _ptr(w), _ptr(y), x.size, float(np.float32(eps)))
    return y


def rows(x, w, eps, nthreads=1, out=None, lanes=256):
    """Every row of a 2-D array (float32, or uint16 bf16 bit patterns) against
    one weight row. Returns (y, threads_used). lanes: 256 (R256) or 128 (the
    same definition with 128 lane chains in four 32-lane groups)."""
    if x.dtype == np.float32:
        dt, x, w = F32, _f32(x), _f32(w)
    elif x.dtype == np.uint16:
        dt, x, w = BF16, _u16(x), _u16(w)
    else:
        raise TypeError("rows: float32 or uint16 (bf16 bits) expected")
    assert x.ndim == 2 and w.shape == (x.shape[1],)
    assert lanes in (128, 256)
    y = np.empty_like(x) if out is None else out
    if lanes == 256:
        used = _load().rmsn_ref_rows(dt, _ptr(x), x.shape[1], _ptr(w), _ptr(y), y.shape[1],
                                     x.shape[0], x.shape[1], float(np.float32(eps)), int(nthreads))
    else:
        used = _load().rmsn_ref_rows_lanes(dt, _ptr(x), x.shape[1], _ptr(w), _ptr(y), y.shape[1],
                                           x.shape[0], x.shape[1], float(np.float32(eps)),
                                           int(lanes), int(nthreads))
    return y, used


def sumsq_lanes(x, lanes):
    """Steps 1-3 with `lanes` lane chains (128 or 256) on a float32 row or a
    uint16 bf16 row."""
    if x.dtype == np.uint16:
        x = _u16(x)
        return np.float32(_load().rmsn_ref_sumsq_lanes(BF16, _ptr(x), x.size, int(lanes)))
    x = _f32(x)
    return np.float32(_load().rmsn_ref_sumsq_lanes(F32, _ptr(x), x.size, int(lanes)))


def row_lanes(x, w, eps, lanes):
    """One row (float32 or uint16 bf16 bits) under the `lanes`-lane definition."""
    y, _ = rows(np.asarray(x)[None, :], np.asarray(w), eps, lanes=lanes)
    return y[0]


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16 array) to float32."""
    b = _u16(bits)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_scalar(v):
    return int(_load().rmsn_ref_f32_to_bf16(float(np.float32(v))))


def f32_to_bf16_range(first_bits, count, out=None):
    """Step 8's narrowing of the binary32 bit patterns first_bits,
    first_bits + 1, ... (count of them), as a uint16 array."""
    if out is None:
        out = np.empty(int(count), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size >= count
    _load().rmsn_ref_f32_to_bf16_range(int(first_bits), int(count), _ptr(out))
    return out[:count]


def float64_reference(x, w, eps):
    """Y = x * w / sqrt(sum(x^2)/n + eps) in float64 for each row (1-D or 2-D);
    eps is the binary32 eps widened exactly, as the oracle uses it."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    eps64 = float(np.float32(eps))
    n = x64.shape[-1]
    ms = np.sum(x64 * x64, axis=-1, keepdims=True) / n
    return x64 * w64 / np.sqrt(ms + eps64)
