"""Python binding of the gfx950 row-wise RMSNorm library (librmsnorm_amd.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/rmsnorm.h. torch supplies device memory
and the stream; nothing here computes a result, and there is no CPU fallback.
Importing this module without the built library raises ImportError.

Function names follow the C entry points:
    rmsnorm_f32(x, w, eps, out=None)           one binary32 row
    rmsnorm_bf16(x, w, eps, out=None)          one bf16 row
    rmsnorm_batched_rows(x, w, eps, out=None)  2-D, rows share w
    rmsnorm_batched_rows_ws(x, w, eps, out=None, workspace=None)
                                               the same with a device workspace
                                               (few very wide rows over many CUs)
    rmsnorm_batched_rows_noalloc(x, w, eps, out=None)
                                               the same with the library's own
                                               workspace (allocates nothing)
    rmsnorm_sequence_eager(table, widths, eps, dtype)
    SequenceGraph(table, widths, eps, dtype)   captured sequence (.launch())
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_amd.so")
# the 128-lane build (same C ABI; rmsnorm_association_lanes() == 128)
LIB128_PATH = os.path.join(_HERE, "librmsnorm_amd_l128.so")

RMSN_OK, RMSN_EINVAL, RMSN_EHIP, RMSN_ECAPTURE, RMSN_ENOMEM = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
PATH_AUTO, PATH_WAVE, PATH_BLOCK, PATH_STREAM, PATH_SPLIT, PATH_GROUP, PATH_WIDE = \
    -1, 0, 1, 2, 3, 4, 5
PATH_REPLICA = 6
OPT_PATH, OPT_ROWS_PER_BLOCK, OPT_STREAMING, OPT_SPLIT_LOADS, OPT_APPLY_THREADS = 1, 2, 3, 4, 5
OPT_PERSISTENT_WORKGROUPS = 6
OPT_REPLICA_PARTS = 7
OPT_WALK_SPIN_CAP = 8
MAX_N = 1 << 24
DESC_BYTES = 32


class RmsnormError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"rmsnorm status {status}: {message}")
        self.status = status


class _PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("chunks", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("block", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("streaming", ctypes.c_int32),
                ("loads", ctypes.c_int32), ("parts", ctypes.c_int32)]


class _Position(ctypes.Structure):
    _fields_ = [("d_pos", ctypes.c_void_p), ("x_pitch", ctypes.c_int64),
                ("y_pitch", ctypes.c_int64), ("period", ctypes.c_int64)]


def _position(position):
    """(d_pos int64 device tensor, x_pitch bytes, y_pitch bytes, period) -> struct."""
    import torch
    d_pos, x_pitch, y_pitch, period = position
    _device_tensor(d_pos, "d_pos")
    if d_pos.dtype != torch.int64 or d_pos.numel() < 1:
        raise ValueError("d_pos must be an int64 device tensor of at least one element")
    return _Position(ctypes.c_void_p(d_pos.data_ptr()), int(x_pitch), int(y_pitch), int(period))


def bind(path):
    """Load one build of the library (LIB_PATH or LIB128_PATH) and declare the
    C signatures; returns the ctypes handle."""
    if not os.path.exists(path):
        raise ImportError(f"row_wise_rmsnorm_amd: {path} is not built "
                          "(run __graft_entry__.build() or row_wise_rmsnorm_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_uint32
    c_int = ctypes.c_int
    sig = {
        "rmsnorm_f32": [vp, vp, vp, i64, f, vp],
        "rmsnorm_bf16": [vp, vp, vp, i64, f, vp],
        "rmsnorm_batched_rows": [c_int, vp, i64, vp, vp, i64, i64, i64, f, vp],
        "rmsnorm_batched_rows_ws": [c_int, vp, i64, vp, vp, i64, i64, i64, f, vp, i64, vp],
        "rmsnorm_batched_rows_noalloc": [c_int, vp, i64, vp, vp, i64, i64, i64, f, vp],
        "rmsnorm_diag_walk_timeouts": [ctypes.POINTER(u32), c_int],
        "rmsnorm_diag_copy": [vp, vp, i64, c_int, c_int, vp],
        "rmsnorm_workspace_query": [c_int, i64, i64, c_int, ctypes.POINTER(_PlanInfo),
                                    ctypes.POINTER(i64)],
        "rmsnorm_sequence_eager": [c_int, vp, vp, i32, f, vp],
        "rmsnorm_sequence_graph_create": [c_int, vp, vp, i32, f, ctypes.POINTER(vp)],
        "rmsnorm_sequence_graph_launch": [vp, vp],
        "rmsnorm_sequence_graph_destroy": [vp],
        "rmsnorm_graph_node_count": [vp, ctypes.POINTER(i64)],
        "rmsnorm_graph_is_fallback": [vp, ctypes.POINTER(c_int)],
        "rmsnorm_plan_query": [c_int, i64, i64, c_int, ctypes.POINTER(_PlanInfo)],
        "rmsnorm_set_option": [c_int, c_int],
        "rmsnorm_get_option": [c_int, ctypes.POINTER(c_int)],
        "rmsnorm_diag_inverse": [u32, i64, i64, f, vp, vp, vp],
        "rmsnorm_diag_bf16": [u32, i64, vp, vp],
        "rmsnorm_sequence_eager_positioned": [c_int, vp, vp, i32, f, ctypes.POINTER(_Position), vp],
        "rmsnorm_sequence_graph_create_positioned": [c_int, vp, vp, i32, f,
                                                     ctypes.POINTER(_Position), ctypes.POINTER(vp)],
        "rmsnorm_sequence_graph_update": [vp, vp, i32, ctypes.POINTER(c_int)],
        "rmsnorm_sequence_persistent": [c_int, vp, i32, f, ctypes.POINTER(_Position), vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int
    lib.rmsnorm_last_error.argtypes = []
    lib.rmsnorm_last_error.restype = ctypes.c_char_p
    lib.rmsnorm_association_lanes.argtypes = []
    lib.rmsnorm_association_lanes.restype = c_int
    return lib


_lib = bind(LIB_PATH)

EXPORTED = ("rmsnorm_f32", "rmsnorm_bf16", "rmsnorm_batched_rows", "rmsnorm_sequence_eager",
            "rmsnorm_sequence_graph_create", "rmsnorm_sequence_graph_launch",
            "rmsnorm_sequence_graph_destroy", "rmsnorm_graph_node_count",
            "rmsnorm_graph_is_fallback", "rmsnorm_last_error", "rmsnorm_plan_query",
            "rmsnorm_set_option", "rmsnorm_get_option", "rmsnorm_diag_inverse",
            "rmsnorm_diag_bf16", "rmsnorm_sequence_eager_positioned",
            "rmsnorm_sequence_graph_create_positioned", "rmsnorm_sequence_graph_update",
            "rmsnorm_association_lanes", "rmsnorm_sequence_persistent",
            "rmsnorm_batched_rows_ws", "rmsnorm_workspace_query",
            "rmsnorm_batched_rows_noalloc", "rmsnorm_diag_walk_timeouts", "rmsnorm_diag_copy")


def lib():
    """The ctypes handle of the loaded library."""
    return _lib


def last_error():
    return (_lib.rmsnorm_last_error() or b"").decode()


def association_lanes():
    """Lane chains of the association the loaded library computes (256)."""
    return _lib.rmsnorm_association_lanes()


def _check(status):
    if status != RMSN_OK:
        raise RmsnormError(status, last_error())
    return status


def _stream_ptr(stream, device=None):
    """The HIP stream handle: `stream`, else the current stream of `device`
    (of the current device when None)."""
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(device):
    """Context that makes `device` current, so the library launches there."""
    import torch
    return torch.cuda.device(device)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"float32 or bfloat16 tensor expected, got {t.dtype}")


def _device_tensor(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _out_like(x, out):
    import torch
    if out is None:
        return torch.empty_like(x)
    _device_tensor(out, "out")
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    return out


def _weight(x, w, n):
    """w must be one contiguous row of n elements of x's dtype on x's device:
    the kernels read n elements of that type from it."""
    _device_tensor(w, "w")
    if w.dtype != x.dtype or w.device != x.device:
        raise ValueError(f"w must have x's dtype and device (x: {x.dtype} on {x.device}, "
                         f"w: {w.dtype} on {w.device})")
    if w.dim() != 1 or w.numel() != n or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous 1-D tensor of {n} elements, got shape "
                         f"{tuple(w.shape)}")
    return w


def _single_row(x, w, out, dtype):
    import torch
    _device_tensor(x, "x")
    if x.dtype != dtype:
        raise TypeError(f"{dtype} tensor expected, got {x.dtype}")
    if x.dim() != 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 1-D tensor")
    _weight(x, w, x.numel())
    y = _out_like(x, out)
    if not y.is_contiguous():
        raise ValueError("out must be contiguous")
    return y


def rmsnorm_f32(x, w, eps, out=None, stream=None):
    """One binary32 row (1-D contiguous float32 tensors of one width)."""
    import torch
    y = _single_row(x, w, out, torch.float32)
    with _on(x.device):
        _check(_lib.rmsnorm_f32(x.data_ptr(), w.data_ptr(), y.data_ptr(), x.numel(),
                                float(eps), _stream_ptr(stream, x.device)))
    return y


def rmsnorm_bf16(x, w, eps, out=None, stream=None):
    """One bf16 row (1-D contiguous bfloat16 tensors of one width)."""
    import torch
    y = _single_row(x, w, out, torch.bfloat16)
    with _on(x.device):
        _check(_lib.rmsnorm_bf16(x.data_ptr(), w.data_ptr(), y.data_ptr(), x.numel(),
                                 float(eps), _stream_ptr(stream, x.device)))
    return y


def rmsnorm_batched_rows(x, w, eps, out=None, stream=None):
    """Every row of a 2-D tensor (unit stride along a row) against w."""
    _device_tensor(x, "x")
    code = _dtype_code(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("2-D tensor with unit stride along rows expected")
    rows, n = x.shape
    _weight(x, w, n)
    y = _out_like(x, out)
    if y.stride(1) != 1:
        raise ValueError("out must have unit stride along rows")
    # a single row's stride is never used; torch may report 0 for a size-1 axis
    xs = x.stride(0) if rows > 1 else n
    ys = y.stride(0) if rows > 1 else n
    with _on(x.device):
        _check(_lib.rmsnorm_batched_rows(code, x.data_ptr(), xs, w.data_ptr(), y.data_ptr(), ys,
                                         rows, n, float(eps), _stream_ptr(stream, x.device)))
    return y


def _rows_alignment(x, w, y, xs, ys):
    """The byte alignment (power of two, at most 16) shared by every row start
    and w, as the library computes it for a launch."""
    es = x.element_size()
    bits = x.data_ptr() | w.data_ptr() | y.data_ptr() | (xs * es) | (ys * es) | 16
    return bits & -bits


def workspace_query(dtype, rows, n, align=16):
    """(plan dict, workspace bytes) that rmsnorm_batched_rows_ws would use."""
    info = _PlanInfo()
    b = ctypes.c_int64()
    _check(_lib.rmsnorm_workspace_query(int(dtype), int(rows), int(n), int(align),
                                        ctypes.byref(info), ctypes.byref(b)))
    return _plan_dict(info), b.value


def rmsnorm_batched_rows_ws(x, w, eps, out=None, workspace=None, stream=None):
    """rmsnorm_batched_rows with a device workspace, so that few very wide
    rows spread over many CUs (RMSN_PATH_WIDE); same bits. `workspace`: a
    contiguous uint8 device tensor of at least the queried bytes, or None to
    take one from torch's allocator when the launch needs it."""
    import torch
    _device_tensor(x, "x")
    code = _dtype_code(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("2-D tensor with unit stride along rows expected")
    rows, n = x.shape
    _weight(x, w, n)
    y = _out_like(x, out)
    if y.stride(1) != 1:
        raise ValueError("out must have unit stride along rows")
    xs = x.stride(0) if rows > 1 else n
    ys = y.stride(0) if rows > 1 else n
    _, need = workspace_query(code, rows, n, _rows_alignment(x, w, y, xs, ys))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _device_tensor(workspace, "workspace")
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or \
            workspace.device != x.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    with _on(x.device):
        _check(_lib.rmsnorm_batched_rows_ws(code, x.data_ptr(), xs, w.data_ptr(), y.data_ptr(),
                                            ys, rows, n, float(eps), workspace.data_ptr(),
                                            workspace.numel(), _stream_ptr(stream, x.device)))
    return y


def rmsnorm_batched_rows_noalloc(x, w, eps, out=None, stream=None):
    """rmsnorm_batched_rows_ws with the library's own per-GPU workspace
    instead of a caller's: nothing is allocated (pass `out` for that), same
    bits. Calls that overlap in time on one GPU share that workspace and must
    not be issued."""
    _device_tensor(x, "x")
    code = _dtype_code(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("2-D tensor with unit stride along rows expected")
    rows, n = x.shape
    _weight(x, w, n)
    y = _out_like(x, out)
    if y.stride(1) != 1:
        raise ValueError("out must have unit stride along rows")
    xs = x.stride(0) if rows > 1 else n
    ys = y.stride(0) if rows > 1 else n
    with _on(x.device):
        _check(_lib.rmsnorm_batched_rows_noalloc(code, x.data_ptr(), xs, w.data_ptr(),
                                                 y.data_ptr(), ys, rows, n, float(eps),
                                                 _stream_ptr(stream, x.device)))
    return y


def make_table(rows, device=None):
    """Device descriptor table from a list of (x, w, y) GPU tensors: each
    1-D and contiguous, one dtype and one device for the whole table, and
    within a row one width. Returns (table tensor, host widths list). The
    table holds raw pointers: the tensors must outlive every launch that
    reads it."""
    import struct
    import torch
    if len(rows) == 0:
        raise ValueError("a table needs at least one row")
    first = rows[0][0]
    _device_tensor(first, "x")
    _dtype_code(first)
    buf = bytearray()
    widths = []
    for i, (x, w, y) in enumerate(rows):
        for name, t in (("x", x), ("w", w), ("y", y)):
            _device_tensor(t, f"row {i} {name}")
            if t.dtype != first.dtype or t.device != first.device:
                raise ValueError(f"row {i} {name}: every tensor of a table must be "
                                 f"{first.dtype} on {first.device}")
            if t.dim() != 1 or not t.is_contiguous() or t.numel() != x.numel():
                raise ValueError(f"row {i} {name}: contiguous 1-D tensors of one width "
                                 "expected")
        buf += struct.pack("<QQQq", x.data_ptr(), w.data_ptr(), y.data_ptr(), x.numel())
        widths.append(int(x.numel()))
    host = torch.frombuffer(buf, dtype=torch.uint8)
    dev = device if device is not None else first.device
    return host.to(dev), widths


def _table(table, count):
    """A device descriptor table of at least `count` records (see make_table)."""
    import torch
    _device_tensor(table, "table")
    if table.dtype != torch.uint8 or not table.is_contiguous() or \
            table.numel() < DESC_BYTES * int(count):
        raise ValueError(f"table must be a contiguous uint8 device tensor of at least "
                         f"{DESC_BYTES} * {int(count)} bytes")
    return ctypes.c_void_p(table.data_ptr())


def _widths_array(widths):
    arr = (ctypes.c_int64 * len(widths))(*[int(v) for v in widths])
    return arr


def rmsnorm_sequence_eager(table, widths, eps, dtype, stream=None, position=None):
    """Issue len(widths) dependent launches reading descriptors from `table`.
    position: None, or (d_pos tensor, x_pitch bytes, y_pitch bytes, period)
    for a positioned sequence (rows taken at the device-resident position,
    which the sequence then advances by one)."""
    arr = _widths_array(widths)
    tp = _table(table, len(widths))
    with _on(table.device):
        if position is None:
            _check(_lib.rmsnorm_sequence_eager(int(dtype), tp, arr, len(widths), float(eps),
                                               _stream_ptr(stream, table.device)))
        else:
            pos = _position(position)
            _check(_lib.rmsnorm_sequence_eager_positioned(
                int(dtype), tp, arr, len(widths), float(eps), ctypes.byref(pos),
                _stream_ptr(stream, table.device)))


def rmsnorm_sequence_persistent(table, count, eps, dtype, stream=None, position=None):
    """All `count` norms of the table, in order, in one kernel launch."""
    tp = _table(table, count)
    pos = ctypes.byref(_position(position)) if position is not None else None
    with _on(table.device):
        _check(_lib.rmsnorm_sequence_persistent(int(dtype), tp, int(count), float(eps), pos,
                                                _stream_ptr(stream, table.device)))


class SequenceGraph:
    """A decode step's norms captured as one HIP graph (or, if capture failed,
    an eager replay with the same kernels). `status` is RMSN_OK or
    RMSN_ECAPTURE."""

    def __init__(self, table, widths, eps, dtype, position=None):
        self._h = ctypes.c_void_p()
        tp = _table(table, len(widths))
        self._table = table  # keep the descriptor table alive with the graph
        self._position = position
        self._device = table.device
        arr = _widths_array(widths)
        h = ctypes.c_void_p()
        with _on(table.device):
            if position is None:
                st = _lib.rmsnorm_sequence_graph_create(int(dtype), tp, arr, len(widths),
                                                        float(eps), ctypes.byref(h))
            else:
                pos = _position(position)
                st = _lib.rmsnorm_sequence_graph_create_positioned(
                    int(dtype), tp, arr, len(widths), float(eps), ctypes.byref(pos),
                    ctypes.byref(h))
        if st not in (RMSN_OK, RMSN_ECAPTURE):
            raise RmsnormError(st, last_error())
        self.status = st
        self.capture_error = last_error() if st == RMSN_ECAPTURE else ""
        self._h = h

    def launch(self, stream=None):
        with _on(self._device):
            _check(_lib.rmsnorm_sequence_graph_launch(self._h, _stream_ptr(stream, self._device)))

    def update(self, widths):
        """New capture-time widths; returns (status, recaptured)."""
        arr = _widths_array(widths)
        rec = ctypes.c_int()
        with _on(self._device):
            st = _lib.rmsnorm_sequence_graph_update(self._h, arr, len(widths), ctypes.byref(rec))
        if st not in (RMSN_OK, RMSN_ECAPTURE):
            raise RmsnormError(st, last_error())
        return st, bool(rec.value)

    def node_count(self):
        v = ctypes.c_int64()
        _check(_lib.rmsnorm_graph_node_count(self._h, ctypes.byref(v)))
        return v.value

    def is_fallback(self):
        v = ctypes.c_int()
        _check(_lib.rmsnorm_graph_is_fallback(self._h, ctypes.byref(v)))
        return bool(v.value)

    def destroy(self):
        if self._h:
            _check(_lib.rmsnorm_sequence_graph_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def plan_query(dtype, rows, n, aligned=True, align=None):
    """The launch plan for `rows` rows of width n. `align`: byte alignment
    shared by the row starts and w (default 16 if `aligned`, else element
    alignment only)."""
    if align is None:
        align = 16 if aligned else 0
    info = _PlanInfo()
    _check(_lib.rmsnorm_plan_query(int(dtype), int(rows), int(n), int(align), ctypes.byref(info)))
    return _plan_dict(info)


def _plan_dict(info):
    return {"path": info.path, "chunks": info.chunks, "rows_per_block": info.rows_per_block,
            "streaming": info.streaming, "block": info.block, "grid": info.grid,
            "loads": info.loads, "parts": info.parts}


def set_option(key, value):
    _check(_lib.rmsnorm_set_option(int(key), int(value)))


def get_option(key):
    v = ctypes.c_int()
    _check(_lib.rmsnorm_get_option(int(key), ctypes.byref(v)))
    return v.value


def diag_bf16(first_bits, count, out, stream=None):
    """Step 8's bf16 narrowing of the kernels over consecutive bit patterns
    (diagnostic); `out`: a contiguous device tensor of 2-byte elements, at
    least `count` of them."""
    _device_tensor(out, "out")
    if out.element_size() != 2 or not out.is_contiguous() or out.numel() < int(count):
        raise ValueError(f"out must be a contiguous device tensor of at least {int(count)} "
                         "2-byte elements")
    with _on(out.device):
        _check(_lib.rmsnorm_diag_bf16(int(first_bits), int(count),
                                      ctypes.c_void_p(out.data_ptr()),
                                      _stream_ptr(stream, out.device)))


def diag_copy(src, dst, vectors=1, block=64, stream=None):
    """Streaming copy of src's bytes into dst (contiguous device tensors of
    equal byte size, a multiple of 16): `vectors` 16-byte vectors per lane,
    `block` threads per workgroup (diagnostic: the copy-pattern ceiling)."""
    for name, t in (("src", src), ("dst", dst)):
        _device_tensor(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or src.device != dst.device:
        raise ValueError("src and dst must hold the same number of bytes on one device")
    with _on(src.device):
        _check(_lib.rmsnorm_diag_copy(ctypes.c_void_p(src.data_ptr()),
                                      ctypes.c_void_p(dst.data_ptr()), nbytes, int(vectors),
                                      int(block), _stream_ptr(stream, src.device)))


def diag_walk_timeouts(reset=False, device=None):
    """Ordered waits of the persistent launch that ran out of polls on the
    device since the last reset (synchronous); reset=True clears the count."""
    import torch
    v = ctypes.c_uint32()
    with _on(torch.cuda.current_device() if device is None else device):
        _check(_lib.rmsnorm_diag_walk_timeouts(ctypes.byref(v), 1 if reset else 0))
    return v.value


def diag_inverse(first_bits, count, n, eps, r_out, inv_out, stream=None):
    """Steps 4-7 of the kernels over consecutive bit patterns (diagnostic);
    r_out, inv_out: contiguous float32 device tensors of at least `count`
    elements."""
    import torch
    for name, t in (("r_out", r_out), ("inv_out", inv_out)):
        _device_tensor(t, name)
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < int(count):
            raise ValueError(f"{name} must be a contiguous float32 device tensor of at least "
                             f"{int(count)} elements")
    with _on(r_out.device):
        _check(_lib.rmsnorm_diag_inverse(int(first_bits), int(count), int(n), float(eps),
                                         ctypes.c_void_p(r_out.data_ptr()),
                                         ctypes.c_void_p(inv_out.data_ptr()),
                                         _stream_ptr(stream, r_out.device)))
