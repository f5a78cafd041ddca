"""The 128-lane build (librmsnorm_amd_l128.so) on the GPU.

Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per Token",
section 2.1, makes two claims about its norm kernel: the thread count of the
sum of squares is part of the result's bits, the width of the elementwise
apply is not. With both builds loaded side by side:
* the 128-lane build equals the oracle's 128-lane definition bit for bit, at
  every apply width (128, 256, 512, 1024 threads), on aligned and misaligned
  rows, in place, and through the eager and captured sequence;
* `cmp` on the output bytes: the 128-lane build at apply widths 128 and 1024
  (and every width between) writes identical files; the 128- and 256-lane
  builds do not.
"""
import ctypes
import subprocess

import numpy as np
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

import oracle
import workloads as wl
from gpu_util import (assert_bits_bf16, assert_bits_f32, bf16_host, dev, f32_host, say,
                      to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu

APPLY = (128, 256, 512, 1024)


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    m.set_option(m.OPT_PATH, m.PATH_AUTO)
    return m


@pytest.fixture(scope="module")
def l128(rn):
    lib = rn.bind(rn.LIB128_PATH)
    assert lib.rmsnorm_association_lanes() == 128
    return lib


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def rows_call(lib, rn, x, w, y, dtype, eps):
    """rmsnorm_batched_rows of one build on 2-D device tensors (any strides)."""
    es = x.element_size()
    st = lib.rmsnorm_batched_rows(dtype, ctypes.c_void_p(x.data_ptr()), x.stride(0),
                                  ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  y.stride(0), x.shape[0], x.shape[1], float(eps), stream())
    assert st == rn.RMSN_OK, (st, lib.rmsnorm_last_error())
    assert es in (2, 4)


def set_apply(lib, rn, b):
    assert lib.rmsnorm_set_option(rn.OPT_APPLY_THREADS, b) == rn.RMSN_OK


def dev_rows(x, kind):
    return to_dev_f32(x) if kind == "f32" else to_dev_bf16(x)


def host_rows(t, kind):
    return f32_host(t) if kind == "f32" else bf16_host(t)


def assert_rows(got, want, kind, what):
    (assert_bits_f32 if kind == "f32" else assert_bits_bf16)(got, want, what)


def _inputs(rows, n, kind, item):
    x = np.empty((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r], w = wl.misc_f32(90000 + item * 131 + r, n, sigma=float(10.0 ** ((r % 5) - 2)))
    if kind == "bf16":
        return wl.to_bf16_bits(x), wl.to_bf16_bits(w)
    return x, w


CASES = [(1, 7168, "f32"), (6, 1536, "f32"), (9, 512, "f32"), (64, 7168, "bf16"),
         (5, 1, "f32"), (7, 33, "bf16"), (4, 127, "f32"), (4, 129, "f32"), (3, 1000, "bf16"),
         (3, 4097, "f32"), (2, 9000, "bf16"), (2, 20001, "f32")]


@pytest.mark.parametrize("rows,n,kind", CASES)
def test_l128_matches_its_oracle_at_every_apply_width(rn, l128, rows, n, kind):
    say(f"128 lanes: {rows} x {n} {kind}")
    dtype = rn.F32 if kind == "f32" else rn.BF16
    x, w = _inputs(rows, n, kind, n)
    want, _ = oracle.rows(x, w, wl.EPS, lanes=128)
    xd, wd = dev_rows(x, kind), dev_rows(w, kind)
    try:
        for b in APPLY:
            set_apply(l128, rn, b)
            yd = torch.empty_like(xd)
            rows_call(l128, rn, xd, wd.view(1, -1), yd, dtype, wl.EPS)
            torch.cuda.synchronize()
            assert_rows(host_rows(yd, kind), want, kind, f"apply width {b}")
    finally:
        set_apply(l128, rn, 0)


def test_l128_misaligned_strided_and_in_place(rn, l128):
    """Rows at element offsets (the element apply loop) and strided, and in
    place; same bits as the oracle."""
    say("128 lanes: offsets, strides, in place")
    for kind in ("f32", "bf16"):
        dtype = rn.F32 if kind == "f32" else rn.BF16
        x, w = _inputs(5, 3000, kind, 5)
        want, _ = oracle.rows(x, w, wl.EPS, lanes=128)
        tdt = torch.float32 if kind == "f32" else torch.bfloat16
        bx = torch.zeros(5, 3011, dtype=tdt, device=dev())
        by = torch.zeros(5, 3013, dtype=tdt, device=dev())
        bw = torch.zeros(3005, dtype=tdt, device=dev())
        bx[:, 1:3001].copy_(dev_rows(x, kind))
        bw[3:3003].copy_(dev_rows(w, kind))
        rows_call(l128, rn, bx[:, 1:3001], bw[3:3003].view(1, -1), by[:, 2:3002], dtype, wl.EPS)
        torch.cuda.synchronize()
        assert_rows(host_rows(by[:, 2:3002], kind), want, kind, f"offsets {kind}")
        t = dev_rows(x, kind)
        rows_call(l128, rn, t, dev_rows(w, kind).view(1, -1), t, dtype, wl.EPS)
        torch.cuda.synchronize()
        assert_rows(host_rows(t, kind), want, kind, f"in place {kind}")


def test_l128_sequence_eager_and_graph(rn, l128):
    """The 327-norm decode step on the 128-lane build, eager and captured
    (three replays on rewritten tables), against the 128-lane oracle."""
    say("128 lanes: decode-step sequence")
    rows = wl.decode()
    xs = [to_dev_f32(x) for x, _ in rows]
    ws = [to_dev_f32(w) for _, w in rows]
    ys = [torch.empty_like(t) for t in xs]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    arr = (ctypes.c_int64 * len(widths))(*widths)
    want = [oracle.row_lanes(x, w, wl.EPS, 128) for x, w in rows]

    def check(what):
        for i, (y, wv) in enumerate(zip(ys, want)):
            assert_bits_f32(f32_host(y), wv, f"{what}: norm {i}")

    for y in ys:
        y.fill_(float("nan"))
    assert l128.rmsnorm_sequence_eager(rn.F32, ctypes.c_void_p(table.data_ptr()), arr,
                                       len(widths), float(wl.EPS), stream()) == rn.RMSN_OK
    torch.cuda.synchronize()
    check("eager")
    h = ctypes.c_void_p()
    st = l128.rmsnorm_sequence_graph_create(rn.F32, ctypes.c_void_p(table.data_ptr()), arr,
                                            len(widths), float(wl.EPS), ctypes.byref(h))
    assert st == rn.RMSN_OK, l128.rmsnorm_last_error()
    n = ctypes.c_int64()
    assert l128.rmsnorm_graph_node_count(h, ctypes.byref(n)) == rn.RMSN_OK and n.value == 327
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        assert l128.rmsnorm_sequence_graph_launch(h, stream()) == rn.RMSN_OK
        torch.cuda.synchronize()
        check(f"graph replay {rep}")
    assert l128.rmsnorm_sequence_graph_destroy(h) == rn.RMSN_OK
    for y in ys:
        y.fill_(float("nan"))
    assert l128.rmsnorm_sequence_persistent(rn.F32, ctypes.c_void_p(table.data_ptr()),
                                            len(widths), float(wl.EPS), None,
                                            stream()) == rn.RMSN_OK
    torch.cuda.synchronize()
    check("persistent")


def _dump(path, arrays):
    with open(path, "wb") as f:
        for a in arrays:
            f.write(np.ascontiguousarray(a).tobytes())


def _cmp(a, b):
    r = subprocess.run(["cmp", str(a), str(b)], capture_output=True, text=True)
    return r.returncode, (r.stdout + r.stderr).strip()


def test_cmp_apply_width_is_inert_lane_count_is_not(rn, l128, tmp_path):
    """The lecture's claim, shown with `cmp` on the output bytes of the whole
    decode step (327 binary32 norms) and the 64-row bf16 batch."""
    say("cmp: apply width vs lane count")
    rows = wl.decode()
    xs = [to_dev_f32(x) for x, _ in rows]
    ws = [to_dev_f32(w) for _, w in rows]
    xb, wb = wl.batch64()
    xbd, wbd = to_dev_bf16(xb), to_dev_bf16(wb)

    def outputs(lib):
        out = []
        for x, w in zip(xs, ws):
            y = torch.empty_like(x)
            rows_call(lib, rn, x.view(1, -1), w.view(1, -1), y.view(1, -1), rn.F32, wl.EPS)
            out.append(y)
        yb = torch.empty_like(xbd)
        rows_call(lib, rn, xbd, wbd.view(1, -1), yb, rn.BF16, wl.EPS)
        torch.cuda.synchronize()
        return [f32_host(y) for y in out] + [bf16_host(yb)]

    files = {}
    try:
        for b in APPLY:
            set_apply(l128, rn, b)
            files[f"l128_apply{b}"] = tmp_path / f"l128_apply{b}.bin"
            _dump(files[f"l128_apply{b}"], outputs(l128))
    finally:
        set_apply(l128, rn, 0)
    files["l256"] = tmp_path / "l256.bin"
    o256 = outputs(rn.lib())
    _dump(files["l256"], o256)
    # the oracle's two definitions, written the same way
    o_or = {lanes: [oracle.row_lanes(x, w, wl.EPS, lanes) for x, w in rows]
            + [oracle.rows(xb, wb, wl.EPS, lanes=lanes)[0]] for lanes in (128, 256)}
    for lanes in (128, 256):
        files[f"oracle{lanes}"] = tmp_path / f"oracle{lanes}.bin"
        _dump(files[f"oracle{lanes}"], o_or[lanes])
    for b in APPLY:
        rc, msg = _cmp(files["l128_apply128"], files[f"l128_apply{b}"])
        say(f"cmp l128_apply128 l128_apply{b}: exit {rc} {msg}")
        assert rc == 0, msg
    rc, msg = _cmp(files["l128_apply1024"], files["oracle128"])
    assert rc == 0, msg
    rc, msg = _cmp(files["l256"], files["oracle256"])
    assert rc == 0, msg
    rc, msg = _cmp(files["l128_apply1024"], files["l256"])
    say(f"cmp l128_apply1024 l256: exit {rc} {msg}")
    assert rc == 1 and "differ" in msg, (rc, msg)
    # how much: elements that differ, and by how many units in the last place
    a = np.concatenate([v.view(np.uint32) for v in o_or[128][:-1]]).astype(np.int64)
    c = np.concatenate([v.view(np.uint32) for v in o256[:-1]]).astype(np.int64)
    d = np.abs(a - c)
    say(f"decode step: {int((d != 0).sum())} of {d.size} binary32 outputs differ between 128 and "
        f"256 lanes, by at most {int(d.max())} ulp")
    assert (d != 0).sum() > 0
