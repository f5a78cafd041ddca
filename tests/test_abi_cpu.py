"""Host-side checks of the C ABI, runnable without a GPU.

* the built library loads and exports every function include/rmsnorm.h declares
* every invalid argument is rejected with RMSN_EINVAL before any HIP call
  (on a machine without a GPU any HIP call would fail with RMSN_EHIP instead)
* the launch plan: paths, register buckets, rows per workgroup, grid
* process-wide options
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm.h")


@pytest.fixture(scope="module")
def rn():
    import row_wise_rmsnorm_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(rmsnorm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("rmsnorm_f32", "rmsnorm_bf16", "rmsnorm_batched_rows",
                 "rmsnorm_sequence_graph_create", "rmsnorm_sequence_graph_launch",
                 "rmsnorm_sequence_graph_destroy", "rmsnorm_sequence_eager"):
        assert name in fns


def test_library_exports_every_declared_symbol(rn):
    lib = ctypes.CDLL(rn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(rn.EXPORTED)


def test_l128_build_exports_the_same_abi(rn):
    lib = rn.bind(rn.LIB128_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.rmsnorm_association_lanes() == 128
    assert rn.association_lanes() == 256


def test_l128_build_plans_and_options(rn):
    """The 128-lane build: one workgroup per row whatever the shape or the
    path option, block = the apply width (default 1024); the apply-width
    option exists only there."""
    import ctypes
    lib = rn.bind(rn.LIB128_PATH)
    info = rn._PlanInfo()

    def plan(dtype, rows, n, align=16):
        assert lib.rmsnorm_plan_query(dtype, rows, n, align, ctypes.byref(info)) == rn.RMSN_OK
        return (info.path, info.chunks, info.block, info.grid, info.loads)

    assert plan(rn.BF16, 8192, 7168) == (rn.PATH_BLOCK, 0, 1024, 8192, 0)
    assert plan(rn.F32, 1, 1 << 24, 0) == (rn.PATH_BLOCK, 0, 1024, 1, 0)
    v = ctypes.c_int()
    try:
        assert lib.rmsnorm_set_option(rn.OPT_PATH, rn.PATH_SPLIT) == rn.RMSN_OK
        assert plan(rn.BF16, 8192, 7168)[0] == rn.PATH_BLOCK
        for b in (128, 256, 512, 1024):
            assert lib.rmsnorm_set_option(rn.OPT_APPLY_THREADS, b) == rn.RMSN_OK
            assert lib.rmsnorm_get_option(rn.OPT_APPLY_THREADS, ctypes.byref(v)) == rn.RMSN_OK
            assert v.value == b and plan(rn.F32, 3, 7168)[2] == b
        for bad in (64, 100, 2048, -1):
            assert lib.rmsnorm_set_option(rn.OPT_APPLY_THREADS, bad) == rn.RMSN_EINVAL
    finally:
        lib.rmsnorm_set_option(rn.OPT_APPLY_THREADS, 0)
        lib.rmsnorm_set_option(rn.OPT_PATH, rn.PATH_AUTO)
    # the default build has no apply-width option
    with pytest.raises(rn.RmsnormError):
        rn.set_option(rn.OPT_APPLY_THREADS, 256)
    assert rn.get_option(rn.OPT_APPLY_THREADS) == 0
    # argument validation is the same code in both builds
    assert lib.rmsnorm_batched_rows(0, 0, 64, B16, C16, 64, 2, 64, 1e-6, None) == rn.RMSN_EINVAL


def test_desc_layout_is_32_bytes():
    text = open(HEADER).read()
    assert re.search(r"const void\* x;\s*const void\* w;\s*void\* y;\s*int64_t n;", text)


# ---- argument validation ------------------------------------------------------

A16 = 0x10000          # fake, never dereferenced device addresses
B16 = 0x20000
C16 = 0x30000


def call_rows(rn, dtype=0, x=A16, xs=64, w=B16, y=C16, ys=64, rows=2, n=64, eps=1e-6):
    return rn.lib().rmsnorm_batched_rows(dtype, x, xs, w, y, ys, rows, n, eps, None)


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(dtype=-1),
    dict(x=0), dict(w=0), dict(y=0),
    dict(n=0), dict(n=-5), dict(n=(1 << 24) + 1),
    dict(rows=0), dict(rows=-1),
    dict(xs=63), dict(ys=10),
    dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(x=A16 + 2), dict(dtype=1, x=A16 + 1), dict(w=B16 + 1), dict(y=C16 + 3),
    dict(y=A16 + 4),                        # partial x / y overlap
    dict(y=A16, ys=128, xs=64),             # same base, different strides
    dict(w=C16 + 8),                        # w inside y
    dict(xs=1 << 62, rows=1 << 20),         # extent overflow
])
def test_batched_rows_rejects(rn, kw):
    assert call_rows(rn, **kw) == rn.RMSN_EINVAL
    assert rn.last_error() != ""


def test_single_row_entry_points_reject(rn):
    L = rn.lib()
    assert L.rmsnorm_f32(0, B16, C16, 64, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_f32(A16, B16, C16, 0, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_f32(A16 + 1, B16, C16, 8, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_f32(A16, B16, C16, 8, -1.0, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_bf16(A16, B16, C16, 1 << 25, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_bf16(A16 + 1, B16, C16, 8, 1e-6, None) == rn.RMSN_EINVAL


def test_in_place_is_accepted_by_validation(rn):
    # y == x with equal strides passes validation; without a GPU the launch
    # itself then fails with a HIP error, never with EINVAL.
    st = call_rows(rn, y=A16, ys=64)
    assert st != rn.RMSN_EINVAL


def test_sequence_validation(rn):
    L = rn.lib()
    w3 = (ctypes.c_int64 * 3)(7168, 1536, 512)
    bad = (ctypes.c_int64 * 3)(7168, 0, 512)
    assert L.rmsnorm_sequence_eager(0, None, w3, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16, None, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16, w3, 0, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16, bad, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16 + 4, w3, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(5, A16, w3, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16, w3, 3, float("nan"), None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_eager(0, A16, w3, 70000, 1e-6, None) == rn.RMSN_EINVAL
    h = ctypes.c_void_p(1234)
    assert L.rmsnorm_sequence_graph_create(0, A16, bad, 3, 1e-6, ctypes.byref(h)) == rn.RMSN_EINVAL
    assert h.value is None
    assert L.rmsnorm_sequence_graph_create(0, A16, w3, 3, 1e-6, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_graph_launch(None, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_sequence_graph_destroy(None) == rn.RMSN_OK
    v = ctypes.c_int64()
    assert L.rmsnorm_graph_node_count(None, ctypes.byref(v)) == rn.RMSN_EINVAL


def test_positioned_sequence_validation(rn):
    import ctypes
    L = rn.lib()
    w3 = (ctypes.c_int64 * 3)(7168, 1536, 512)
    P = rn._Position

    def pos(d=C16 + 0x1000, xp=4096, yp=4096, period=4):
        return ctypes.byref(P(ctypes.c_void_p(d), xp, yp, period))

    eager = L.rmsnorm_sequence_eager_positioned
    assert eager(0, A16, w3, 3, 1e-6, None, None) == rn.RMSN_EINVAL       # no position
    for bad in (dict(d=0), dict(d=C16 + 4), dict(period=0), dict(period=-3), dict(xp=-4),
                dict(xp=6), dict(yp=2), dict(xp=1 << 61, period=1 << 20)):
        assert eager(0, A16, w3, 3, 1e-6, pos(**bad), None) == rn.RMSN_EINVAL, bad
        assert rn.last_error() != ""
    assert eager(1, A16, w3, 3, 1e-6, pos(xp=2, yp=6), None) != rn.RMSN_EINVAL  # bf16: 2-byte pitches
    bad = (ctypes.c_int64 * 3)(7168, 0, 512)
    assert eager(0, A16, bad, 3, 1e-6, pos(), None) == rn.RMSN_EINVAL
    h = ctypes.c_void_p(1234)
    create = L.rmsnorm_sequence_graph_create_positioned
    assert create(0, A16, w3, 3, 1e-6, None, ctypes.byref(h)) == rn.RMSN_EINVAL
    assert h.value is None
    assert create(0, A16, w3, 3, 1e-6, pos(period=0), ctypes.byref(h)) == rn.RMSN_EINVAL
    assert create(0, A16, w3, 3, 1e-6, pos(), None) == rn.RMSN_EINVAL
    rec = ctypes.c_int(7)
    assert L.rmsnorm_sequence_graph_update(None, w3, 3, ctypes.byref(rec)) == rn.RMSN_EINVAL
    assert rec.value == 0


def test_persistent_sequence_validation(rn):
    import ctypes
    L = rn.lib()
    P = rn._Position
    f = L.rmsnorm_sequence_persistent
    assert f(2, A16, 3, 1e-6, None, None) == rn.RMSN_EINVAL
    assert f(0, 0, 3, 1e-6, None, None) == rn.RMSN_EINVAL
    assert f(0, A16 + 4, 3, 1e-6, None, None) == rn.RMSN_EINVAL
    assert f(0, A16, 0, 1e-6, None, None) == rn.RMSN_EINVAL
    assert f(0, A16, 70000, 1e-6, None, None) == rn.RMSN_EINVAL
    assert f(0, A16, 3, float("nan"), None, None) == rn.RMSN_EINVAL
    bad = P(ctypes.c_void_p(C16), 4096, 4096, 0)
    assert f(0, A16, 3, 1e-6, ctypes.byref(bad), None) == rn.RMSN_EINVAL
    assert rn.last_error() != ""


def test_diag_validation(rn):
    L = rn.lib()
    assert L.rmsnorm_diag_bf16(0xFFFFFFFF, 2, A16, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_bf16(0, 16, 0, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_bf16(0, 16, A16 + 1, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_bf16(0, -1, A16, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_inverse(0xFFFFFFFF, 2, 1, 0.0, A16, B16, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_inverse(0, 16, 0, 0.0, A16, B16, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_inverse(0, 16, 1, -1.0, A16, B16, None) == rn.RMSN_EINVAL
    assert L.rmsnorm_diag_inverse(0, 16, 1, 0.0, 0, B16, None) == rn.RMSN_EINVAL


# ---- planning -------------------------------------------------------------------

def test_plan_paths_and_buckets(rn):
    # many 16-byte aligned rows: a workgroup of 7 wavefronts per row, two 1 KB
    # slices (16-byte loads) per wavefront; a 235 MB launch streams (non-temporal)
    p = rn.plan_query(rn.BF16, 8192, 7168, aligned=True)
    assert p == {"path": rn.PATH_SPLIT, "chunks": 4, "rows_per_block": 1, "streaming": 1,
                 "block": 448, "grid": 8192, "loads": 2, "parts": 1}
    # binary32: 28 slices, four per wavefront
    p = rn.plan_query(rn.F32, 8192, 7168)
    assert (p["path"], p["loads"], p["block"], p["chunks"]) == (rn.PATH_SPLIT, 4, 448, 4)
    # many wide rows in a launch under 64 MiB (29 MB here): GROUP, default caching
    p = rn.plan_query(rn.BF16, 1024, 7168)
    assert p["path"] == rn.PATH_GROUP and p["streaming"] == 0
    assert rn.plan_query(rn.BF16, 2048, 7168)["path"] == rn.PATH_GROUP      # 58.7 MB
    assert rn.plan_query(rn.BF16, 3072, 7168)["path"] == rn.PATH_SPLIT      # 88 MB
    # rows under 1 KB at any size, and rows of 1-4 KB under 32 MiB: WAVE
    assert rn.plan_query(rn.BF16, 245760, 256)["path"] == rn.PATH_WAVE      # 252 MB, 512 B rows
    assert rn.plan_query(rn.BF16, 2730, 1536)["path"] == rn.PATH_WAVE       # 16.8 MB, 3 KB rows
    assert rn.plan_query(rn.BF16, 8533, 1536)["path"] == rn.PATH_SPLIT      # 52 MB
    assert rn.plan_query(rn.F32, 25600, 256)["path"] == rn.PATH_SPLIT       # 52 MB, 1 KB rows
    p = rn.plan_query(rn.BF16, 122880, 512)                                 # 252 MB, 1 KB rows
    assert (p["path"], p["loads"], p["block"]) == (rn.PATH_SPLIT, 1, 64)
    p = rn.plan_query(rn.BF16, 40960, 1536)                                 # 3 slices: two per wavefront
    assert (p["path"], p["loads"], p["block"]) == (rn.PATH_SPLIT, 2, 128)
    # rows aligned to 8 bytes only: one wavefront per row, eight rows per
    # workgroup sharing one LDS copy of w
    p = rn.plan_query(rn.BF16, 8192, 7168, align=8)
    assert p == {"path": rn.PATH_WAVE, "chunks": 28, "rows_per_block": 8, "streaming": 1,
                 "block": 512, "grid": 1024, "loads": 0, "parts": 1}
    # fewer than 2048 rows: 4 per workgroup
    p = rn.plan_query(rn.BF16, 1024, 1536, align=8)   # 3 KB rows, 6 MB
    assert p["path"] == rn.PATH_WAVE and p["rows_per_block"] == 4 and p["grid"] == 256
    # a width that is not a whole number of 16-byte vectors: WAVE
    assert rn.plan_query(rn.BF16, 4096, 7164)["path"] == rn.PATH_WAVE
    # few rows: a 256-thread workgroup per row, group segments read with
    # vector loads (GROUP); element loads (BLOCK) when the rows are not
    # quad-aligned or the width is not a whole number of quads
    p = rn.plan_query(rn.BF16, 64, 7168, aligned=True)
    assert p == {"path": rn.PATH_GROUP, "chunks": 28, "rows_per_block": 1, "streaming": 0,
                 "block": 256, "grid": 64, "loads": 7, "parts": 1}
    p = rn.plan_query(rn.BF16, 64, 7168, aligned=False)
    assert p == {"path": rn.PATH_BLOCK, "chunks": 28, "rows_per_block": 1, "streaming": 0,
                 "block": 256, "grid": 64, "loads": 0, "parts": 1}
    assert rn.plan_query(rn.BF16, 64, 7166)["path"] == rn.PATH_BLOCK
    # single rows
    assert rn.plan_query(rn.F32, 1, 7168)["path"] == rn.PATH_GROUP
    assert rn.plan_query(rn.F32, 1, 7168, align=0)["chunks"] == 28
    assert rn.plan_query(rn.F32, 1, 1536, align=0)["chunks"] == 6
    assert rn.plan_query(rn.F32, 1, 512, align=0)["chunks"] == 2
    # descriptor rows of the decode step: BLOCK instances by width
    assert rn.plan_query(rn.F32, 1, 7168, align=-1) == {
        "path": rn.PATH_BLOCK, "chunks": 28, "rows_per_block": 1, "streaming": 0,
        "block": 256, "grid": 1, "loads": 0, "parts": 1}
    assert rn.plan_query(rn.F32, 1, 1536, align=-1)["chunks"] == 6
    assert rn.plan_query(rn.F32, 1, 512, align=-1)["chunks"] == 2
    # unaligned rows never take the WAVE, SPLIT or GROUP path
    assert rn.plan_query(rn.F32, 4096, 7168, aligned=False)["path"] == rn.PATH_BLOCK
    assert rn.plan_query(rn.F32, 4096, 7168, align=4)["path"] == rn.PATH_BLOCK
    assert rn.plan_query(rn.F32, 4096, 7168, align=24)["path"] == rn.PATH_BLOCK  # 8 B
    assert rn.plan_query(rn.BF16, 4096, 7168, align=24)["path"] == rn.PATH_WAVE
    # beyond 8192 elements: SPLIT up to 128 KB rows of whole vectors, else streamed
    p = rn.plan_query(rn.F32, 3, 8193)
    assert p["path"] == rn.PATH_STREAM and p["chunks"] == 0 and p["grid"] == 3
    p = rn.plan_query(rn.F32, 3, 8196)                                      # 33 slices
    assert p["path"] == rn.PATH_SPLIT and p["loads"] == 4 and p["block"] == 576
    p = rn.plan_query(rn.BF16, 2, 65536)
    assert p["path"] == rn.PATH_SPLIT and p["loads"] == 8 and p["block"] == 1024
    assert rn.plan_query(rn.BF16, 2, 65544)["path"] == rn.PATH_STREAM
    p = rn.plan_query(rn.F32, 1, 1 << 24)
    assert p["path"] == rn.PATH_STREAM


@pytest.mark.parametrize("n,es", [(4, 4), (8, 2), (256, 4), (1000, 2), (2056, 2), (7168, 2),
                                  (7168, 4), (8196, 4), (12000, 4), (20000, 2), (32768, 4),
                                  (65536, 2)])
def test_split_geometry(rn, n, es):
    """Every SPLIT plan: one slice per wavefront for a one-slice row, two below
    16 slices, four from 16 (eight where four would need more than 16
    wavefronts), and a forced slice count honoured when it fits."""
    dtype = rn.F32 if es == 4 else rn.BF16
    slices = -(-n * es // 1024)
    try:
        rn.set_option(rn.OPT_PATH, rn.PATH_SPLIT)
        p = rn.plan_query(dtype, 5, n)
        assert p["path"] == rn.PATH_SPLIT
        u = 1 if slices <= 1 else 2 if slices < 16 else 4
        while -(-slices // u) > 16:
            u *= 2
        assert p["loads"] == u
        assert p["block"] == 64 * -(-slices // p["loads"])
        assert p["chunks"] == p["loads"] * 1024 // (256 * es)
        for u in (1, 2, 4, 8):
            rn.set_option(rn.OPT_SPLIT_LOADS, u)
            q = rn.plan_query(dtype, 5, n)
            want = u if -(-slices // u) <= 16 else p["loads"]
            assert q["loads"] == want and q["block"] == 64 * -(-slices // want)
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        rn.set_option(rn.OPT_SPLIT_LOADS, 0)


@pytest.mark.parametrize("n", [1, 255, 256, 257, 511, 512, 513, 1024, 1535, 1536, 2049, 3072,
                               4096, 5000, 6144, 6145, 7167, 7168, 8191, 8192])
def test_plan_bucket_holds_row_and_previous_does_not(rn, n):
    buckets = [1, 2, 4, 6, 8, 12, 16, 20, 24, 28, 32]
    c = rn.plan_query(rn.F32, 1, n, align=0)["chunks"]
    assert c in buckets and 256 * c >= n
    i = buckets.index(c)
    if i > 0:
        assert 256 * buckets[i - 1] < n


def test_plan_rejects(rn):
    for args in [(2, 1, 10), (0, 0, 10), (0, 1, 0), (0, 1, (1 << 24) + 1)]:
        with pytest.raises(rn.RmsnormError):
            rn.plan_query(*args)


def test_options_roundtrip_and_force_paths(rn):
    try:
        rn.set_option(rn.OPT_PATH, rn.PATH_STREAM)
        assert rn.get_option(rn.OPT_PATH) == rn.PATH_STREAM
        assert rn.plan_query(rn.BF16, 8192, 7168)["path"] == rn.PATH_STREAM
        rn.set_option(rn.OPT_PATH, rn.PATH_BLOCK)
        assert rn.plan_query(rn.BF16, 8192, 7168)["path"] == rn.PATH_BLOCK
        rn.set_option(rn.OPT_PATH, rn.PATH_WAVE)
        assert rn.plan_query(rn.BF16, 3, 7168)["path"] == rn.PATH_WAVE
        assert rn.plan_query(rn.BF16, 8192, 7168)["path"] == rn.PATH_WAVE
        # ineligible: falls back to the automatic choice
        assert rn.plan_query(rn.BF16, 3, 7168, aligned=False)["path"] == rn.PATH_BLOCK
        assert rn.plan_query(rn.BF16, 3, 7168, align=4)["path"] == rn.PATH_BLOCK
        assert rn.plan_query(rn.BF16, 3, 9000)["path"] == rn.PATH_SPLIT
        assert rn.plan_query(rn.BF16, 3, 9001)["path"] == rn.PATH_STREAM
        rn.set_option(rn.OPT_PATH, rn.PATH_SPLIT)
        assert rn.plan_query(rn.BF16, 3, 7168)["path"] == rn.PATH_SPLIT
        assert rn.plan_query(rn.BF16, 3, 7167)["path"] == rn.PATH_BLOCK
        assert rn.plan_query(rn.BF16, 3, 7168, align=8)["path"] == rn.PATH_GROUP
        rn.set_option(rn.OPT_PATH, rn.PATH_GROUP)
        p = rn.plan_query(rn.BF16, 64, 7168, align=8)
        assert p == {"path": rn.PATH_GROUP, "chunks": 28, "rows_per_block": 1, "streaming": 0,
                     "block": 256, "grid": 64, "loads": 7, "parts": 1}
        assert rn.plan_query(rn.F32, 1, 1536)["loads"] == 2
        assert rn.plan_query(rn.F32, 1, 4)["loads"] == 1
        assert rn.plan_query(rn.F32, 1, 1025, align=16)["path"] == rn.PATH_BLOCK   # not whole quads
        assert rn.plan_query(rn.F32, 1, 1024, align=8)["path"] == rn.PATH_BLOCK    # f32 quads need 16 B
        assert rn.plan_query(rn.F32, 1, 8196)["path"] != rn.PATH_GROUP             # > 8192
        # descriptor rows (alignment checked by the kernel when it runs)
        assert rn.plan_query(rn.F32, 1, 1536, align=-1)["path"] == rn.PATH_GROUP
        assert rn.plan_query(rn.F32, 1, 1537, align=-1)["path"] == rn.PATH_BLOCK
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        rn.set_option(rn.OPT_ROWS_PER_BLOCK, 4)
        p = rn.plan_query(rn.BF16, 8191, 7168, align=8)
        assert p["rows_per_block"] == 4 and p["grid"] == 2048 and p["block"] == 256
        rn.set_option(rn.OPT_STREAMING, 0)
        assert rn.plan_query(rn.BF16, 8191, 7168)["streaming"] == 0
        assert rn.plan_query(rn.BF16, 8191, 7168, align=8)["streaming"] == 0
        rn.set_option(rn.OPT_STREAMING, 1)
        assert rn.plan_query(rn.BF16, 1024, 256)["streaming"] == 1
        assert rn.get_option(rn.OPT_STREAMING) == 1
        rn.set_option(rn.OPT_SPLIT_LOADS, 4)
        assert rn.get_option(rn.OPT_SPLIT_LOADS) == 4
        p = rn.plan_query(rn.BF16, 8192, 7168)
        assert p["loads"] == 4 and p["block"] == 256
        for bad in ((rn.OPT_ROWS_PER_BLOCK, 3), (rn.OPT_ROWS_PER_BLOCK, 1),
                    (rn.OPT_STREAMING, 2), (rn.OPT_STREAMING, -2),
                    (rn.OPT_SPLIT_LOADS, 3), (rn.OPT_SPLIT_LOADS, 16), (rn.OPT_SPLIT_LOADS, -1)):
            with pytest.raises(rn.RmsnormError):
                rn.set_option(*bad)
        with pytest.raises(rn.RmsnormError):
            rn.set_option(rn.OPT_PATH, 7)
        with pytest.raises(rn.RmsnormError):
            rn.set_option(rn.OPT_PATH, -2)
        # WIDE needs a workspace: forced, the plain plan falls back to the
        # automatic choice and the workspace plan takes it for any shape
        rn.set_option(rn.OPT_PATH, rn.PATH_WIDE)
        assert rn.plan_query(rn.BF16, 3, 7168)["path"] == rn.PATH_GROUP
        assert rn.workspace_query(rn.BF16, 3, 100)[0]["path"] == rn.PATH_WIDE
        assert rn.workspace_query(rn.BF16, 5000, 7168)[1] == 16 * 5000
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        with pytest.raises(rn.RmsnormError):
            rn.set_option(99, 0)
        # the persistent launch: 0 automatic (free rows spread), 1 one workgroup
        assert rn.get_option(rn.OPT_PERSISTENT_WORKGROUPS) == 0
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1)
        assert rn.get_option(rn.OPT_PERSISTENT_WORKGROUPS) == 1
        for bad in (2, -1, 256):
            with pytest.raises(rn.RmsnormError):
                rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, bad)
        assert rn.get_option(rn.OPT_PERSISTENT_WORKGROUPS) == 1
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        rn.set_option(rn.OPT_ROWS_PER_BLOCK, 0)
        rn.set_option(rn.OPT_STREAMING, -1)
        rn.set_option(rn.OPT_SPLIT_LOADS, 0)
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)


def test_error_messages_are_per_thread(rn):
    """Several host threads rejecting different arguments at once: each reads
    back its own reason (the message is kept per thread)."""
    import threading
    lib = rn.lib()
    errors = {}
    barrier = threading.Barrier(4)

    def worker(k):
        barrier.wait()
        for _ in range(200):
            if k % 2 == 0:   # width 0
                st = lib.rmsnorm_batched_rows(0, 16, 0, 16, 16, 0, 1, 0, ctypes.c_float(1e-6), None)
                want = "n must be"
            else:            # negative eps
                st = lib.rmsnorm_batched_rows(0, 16, 8, 16, 64, 8, 1, 8, ctypes.c_float(-1.0), None)
                want = "eps must be"
            msg = lib.rmsnorm_last_error().decode()
            if st != 1 or want not in msg:
                errors[k] = (st, msg)
                return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU only; asking for more exits with status 2 and
    says so, before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_binding_refuses_host_tensors(rn):
    """The binding takes device tensors only; a host tensor is refused before
    the library is called (there is no CPU path)."""
    import torch
    x = torch.ones(8)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.rmsnorm_f32(x, x, 1e-6)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.rmsnorm_batched_rows(x.view(2, 4), x[:4], 1e-6)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.make_table([(x, x, x)])


def test_workspace_query(rn):
    """WIDE (and a workspace of 16 bytes per row) for at most 64 rows of at
    least 64 KB; everything else needs none and plans as rmsnorm_plan_query."""
    for dt in (rn.F32, rn.BF16):
        es = 4 if dt == rn.F32 else 2
        for rows, n, wide in ((1, 65536 // es, True), (1, 65536 // es - 1, False),
                              (1, 1 << 24, True), (64, 65536, True), (65, 65536, False),
                              (1, 8192, False), (1, 9000, False), (8192, 7168, False),
                              (3, 100, False)):
            plan, need = rn.workspace_query(dt, rows, n)
            assert (plan["path"] == rn.PATH_WIDE) == wide, (dt, rows, n, plan)
            if wide:
                assert need == 16 * rows
                assert plan["grid"] == 4 * rows and plan["block"] == 64
                assert plan["loads"] == -(-n // 4096)
            else:
                assert need == 0 and plan == rn.plan_query(dt, rows, n)
    # descriptor-row alignment never takes WIDE; bad arguments are refused
    assert rn.workspace_query(rn.F32, 1, 1 << 20, align=-1)[0]["path"] != rn.PATH_WIDE
    with pytest.raises(rn.RmsnormError):
        rn.workspace_query(rn.F32, 0, 100)
    L = rn.lib()
    assert L.rmsnorm_workspace_query(0, 1, 100, 16, None, None) == rn.RMSN_EINVAL


def test_workspace_rejects(rn):
    """A WIDE launch refuses a missing, small, misaligned or overlapping
    workspace before anything is launched (fake, never dereferenced
    addresses); the plain checks apply first."""
    L = rn.lib()
    n = 1 << 16                                   # 256 KB rows: WIDE for a few rows
    X, W, Y, WS = 0x1000000, 0x2000000, 0x3000000, 0x4000000

    def call(ws, nbytes, rows=2, x=X, y=Y, xs=n, ys=n):
        return L.rmsnorm_batched_rows_ws(0, x, xs, W, y, ys, rows, n, 1e-6, ws, nbytes, None)

    assert call(0, 64) == rn.RMSN_EINVAL and "workspace" in rn.last_error()
    assert call(WS + 2, 64) == rn.RMSN_EINVAL and "workspace" in rn.last_error()
    assert call(WS, 31) == rn.RMSN_EINVAL and "needs 32" in rn.last_error()
    assert call(X + 4 * n, 64) == rn.RMSN_EINVAL and "overlaps" in rn.last_error()   # in x's row 1
    assert call(W + 8, 64) == rn.RMSN_EINVAL and "overlaps" in rn.last_error()
    assert call(Y, 64) == rn.RMSN_EINVAL and "overlaps" in rn.last_error()
    assert call(WS, 64, xs=n - 1) == rn.RMSN_EINVAL and "stride" in rn.last_error()
    # a launch that needs no workspace ignores it: validation passes, and
    # without a GPU the launch then fails with a HIP error, never EINVAL
    assert L.rmsnorm_batched_rows_ws(0, X, 64, W, Y, 64, 2, 64, 1e-6, 0, 0, None) \
        != rn.RMSN_EINVAL


def test_build_scripts_load_without_the_package():
    # On a fresh checkout the library is not built yet, and the package refuses
    # to import; the build entry must reach the build scripts without it.
    import subprocess
    import sys
    code = (
        "import sys\n"
        "class Block:\n"
        "    def find_spec(self, name, path=None, target=None):\n"
        "        if name.split('.')[0] == 'row_wise_rmsnorm_amd':\n"
        "            raise ImportError('package imported before the build')\n"
        "        return None\n"
        "sys.meta_path.insert(0, Block())\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import __graft_entry__ as g\n"
        "import os\n"
        "h = g._load_script(os.path.join('row_wise_rmsnorm_amd', 'build.py'))\n"
        "o = g._load_script(os.path.join('oracle', 'build.py'))\n"
        "assert callable(h.build) and callable(o.build)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_descriptor_kernels_built_both_ways():
    """The descriptor kernels are compiled twice (rmsn_desc.hip): with their
    arguments preloaded into SGPRs (the launches a sequence graph records) and
    loading their own (eager launches); the build lists both objects, and the
    built library carries both kernel families. Every other object is built
    with preloading except the host-only plan code."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "rmsn_build_check", os.path.join(ROOT, "row_wise_rmsnorm_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    desc = [extra for src, extra in b.UNITS if src == "rmsn_desc.hip"]
    assert len(desc) == 2
    assert sorted("-DRMSN_DESC_PRELOADED=1" in e for e in desc) == [False, True]
    for e in desc:
        assert ("-DRMSN_DESC_PRELOADED=1" in e) == all(f in e for f in b.PRELOAD)
    for src, extra in b.UNITS:
        if src.endswith(".hip") and src != "rmsn_desc.hip":
            assert all(f in extra for f in b.PRELOAD), src
    with open(os.path.join(ROOT, "row_wise_rmsnorm_amd", "librmsnorm_amd.so"), "rb") as f:
        blob = f.read()
    # the kernels' mangled names: namespace rmsn::desc_preloaded / rmsn::desc_loaded
    assert b"14desc_preloaded" in blob and b"11desc_loaded" in blob


def test_noalloc_rejects(rn):
    """The allocation-free entry point checks its arguments as the plain one
    does, and refuses a launch whose group totals would not fit the library's
    64 KB workspace (only reachable with the WIDE path forced) before any HIP
    call; a launch that fits gets past validation (without a GPU it then
    fails with a HIP error, never EINVAL)."""
    L = rn.lib()
    n = 1 << 14                                   # 64 KB binary32 rows
    X, W, Y = 0x10000000, 0x20000000, 0x30000000

    def call(rows, x=X, w=W, y=Y, xs=n, ys=n, eps=1e-6, dtype=0):
        return L.rmsnorm_batched_rows_noalloc(dtype, x, xs, w, y, ys, rows, n, eps, None)

    assert call(2, x=0) == rn.RMSN_EINVAL and "null" in rn.last_error()
    assert call(2, xs=n - 1) == rn.RMSN_EINVAL and "stride" in rn.last_error()
    assert call(2, eps=-1.0) == rn.RMSN_EINVAL and "eps" in rn.last_error()
    assert call(2, dtype=7) == rn.RMSN_EINVAL
    rn.set_option(rn.OPT_PATH, rn.PATH_WIDE)
    try:
        assert rn.workspace_query(rn.F32, 4097, n)[1] == 16 * 4097
        assert call(4097) == rn.RMSN_EINVAL
        assert "65536" in rn.last_error() and "4096 rows" in rn.last_error()
        assert call(4096) != rn.RMSN_EINVAL
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    assert call(2) != rn.RMSN_EINVAL


def test_replica_plan(rn):
    """REPLICA (forced only): `parts` GROUP workgroups per row, parts from the
    option (default 4), capped at the row's 1024-element blocks; the grid is
    rows x parts; rows GROUP cannot take and descriptor rows fall back to the
    automatic choice."""
    try:
        rn.set_option(rn.OPT_PATH, rn.PATH_REPLICA)
        p = rn.plan_query(rn.F32, 1, 7168)
        assert (p["path"], p["parts"], p["grid"], p["loads"], p["block"]) == \
            (rn.PATH_REPLICA, 4, 4, 7, 256)
        p = rn.plan_query(rn.BF16, 64, 7168)
        assert (p["path"], p["parts"], p["grid"]) == (rn.PATH_REPLICA, 4, 256)
        for parts, want in ((1, 1), (2, 2), (7, 7), (8, 7)):
            rn.set_option(rn.OPT_REPLICA_PARTS, parts)
            assert rn.get_option(rn.OPT_REPLICA_PARTS) == parts
            p = rn.plan_query(rn.BF16, 64, 7168)
            assert (p["parts"], p["grid"]) == (want, 64 * want), parts
        assert rn.plan_query(rn.F32, 3, 512)["parts"] == 1        # one block: one part
        assert rn.plan_query(rn.F32, 3, 8190)["path"] == rn.PATH_BLOCK   # n % 4: BLOCK
        assert rn.plan_query(rn.F32, 1, 7168, align=-1)["path"] != rn.PATH_REPLICA
        for bad in (-1, 9):
            with pytest.raises(rn.RmsnormError):
                rn.set_option(rn.OPT_REPLICA_PARTS, bad)
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        rn.set_option(rn.OPT_REPLICA_PARTS, 0)
    assert rn.plan_query(rn.F32, 1, 7168)["path"] == rn.PATH_GROUP


def test_walk_spin_cap_option_and_diagnostics_reject(rn):
    """The ordered walk's spin cap: 0 (default) or 1..2^30, round-trips;
    the timeout counter needs an output; the diagnostic copy refuses bad
    pointers, sizes, vector counts and blocks before any HIP call."""
    assert rn.get_option(rn.OPT_WALK_SPIN_CAP) == 0
    try:
        for v in (1, 1000, 1 << 30):
            rn.set_option(rn.OPT_WALK_SPIN_CAP, v)
            assert rn.get_option(rn.OPT_WALK_SPIN_CAP) == v
        for bad in (-1, (1 << 30) + 1):
            with pytest.raises(rn.RmsnormError):
                rn.set_option(rn.OPT_WALK_SPIN_CAP, bad)
    finally:
        rn.set_option(rn.OPT_WALK_SPIN_CAP, 0)
    L = rn.lib()
    assert L.rmsnorm_diag_walk_timeouts(None, 0) == rn.RMSN_EINVAL
    S, D = 0x100000, 0x900000
    good = dict(src=S, dst=D, nbytes=1 << 20, v=1, b=64)

    def call(**kw):
        a = dict(good, **kw)
        return L.rmsnorm_diag_copy(a["src"], a["dst"], a["nbytes"], a["v"], a["b"], None)

    for kw in (dict(src=0), dict(dst=0), dict(src=S + 8), dict(dst=D + 4), dict(nbytes=0),
               dict(nbytes=100), dict(nbytes=-16), dict(dst=S + 4096), dict(v=3), dict(v=0),
               dict(b=32), dict(b=96), dict(b=2048)):
        assert call(**kw) == rn.RMSN_EINVAL, kw
    assert call() != rn.RMSN_EINVAL          # valid: without a GPU the launch itself fails
