"""The Python binding refuses operands the kernels would misread.

The C ABI takes raw pointers, so it cannot know a buffer's size or element
type; the binding checks them before any launch: the dtype the entry point
computes in, w of x's dtype, device and width, `out` like x, descriptor rows of
one width, dtype and device, a table large enough for `count` records, the
position counter's type, and diagnostic outputs large enough for `count`
results. Each case raises on the host; nothing is launched.
"""
import pytest
import torch  # imported at collection: the first import on a fresh machine is slow

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import row_wise_rmsnorm_amd as m
    return m


def _t(n, dtype=torch.float32):
    return torch.ones(n, dtype=dtype, device=dev())


def test_single_row_operands(rn):
    x, w = _t(64), _t(64)
    with pytest.raises(TypeError):
        rn.rmsnorm_f32(_t(64, torch.bfloat16), _t(64, torch.bfloat16), 1e-6)
    with pytest.raises(TypeError):
        rn.rmsnorm_bf16(x, w, 1e-6)
    with pytest.raises(ValueError, match="dtype"):
        rn.rmsnorm_f32(x, _t(64, torch.bfloat16), 1e-6)      # would read 2x past w
    with pytest.raises(ValueError, match="64 elements"):
        rn.rmsnorm_f32(x, _t(63), 1e-6)                       # would read past w
    with pytest.raises(ValueError, match="64 elements"):
        rn.rmsnorm_f32(x, _t(128)[::2], 1e-6)                 # strided w
    with pytest.raises(ValueError, match="out must match"):
        rn.rmsnorm_f32(x, w, 1e-6, out=_t(32))
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.rmsnorm_f32(x, torch.ones(64), 1e-6)
    y = rn.rmsnorm_f32(x, w, 0.0)                  # the valid call still works: y = w exactly
    torch.cuda.synchronize()
    assert bool((y == 1).all())


def test_batched_rows_operands(rn):
    x = torch.ones(8, 64, device=dev())
    with pytest.raises(ValueError, match="64 elements"):
        rn.rmsnorm_batched_rows(x, _t(32), 1e-6)
    with pytest.raises(ValueError, match="64 elements"):
        rn.rmsnorm_batched_rows(x, torch.ones(2, 32, device=dev()), 1e-6)
    with pytest.raises(ValueError, match="dtype"):
        rn.rmsnorm_batched_rows(x, _t(64, torch.bfloat16), 1e-6)
    with pytest.raises(TypeError):
        rn.rmsnorm_batched_rows(x.half(), _t(64).half(), 1e-6)


def test_table_and_sequence_operands(rn):
    a, b, c = _t(64), _t(64), _t(64)
    with pytest.raises(ValueError, match="one width"):
        rn.make_table([(a, b, _t(32))])
    with pytest.raises(ValueError, match="every tensor"):
        rn.make_table([(a, b, c), (_t(64, torch.bfloat16),) * 3])
    with pytest.raises(ValueError, match="at least one row"):
        rn.make_table([])
    table, widths = rn.make_table([(a, b, c), (a, b, c)])
    with pytest.raises(ValueError, match="32 \\* 3"):
        rn.rmsnorm_sequence_eager(table, widths + [64], 1e-6, rn.F32)
    with pytest.raises(ValueError, match="32 \\* 3"):
        rn.rmsnorm_sequence_persistent(table, 3, 1e-6, rn.F32)
    with pytest.raises(ValueError, match="32 \\* 3"):
        rn.SequenceGraph(table, widths + [64], 1e-6, rn.F32)
    bad_pos = (torch.zeros(1, dtype=torch.int32, device=dev()), 256, 256, 2)
    with pytest.raises(ValueError, match="int64"):
        rn.rmsnorm_sequence_eager(table, widths, 1e-6, rn.F32, position=bad_pos)


def test_diagnostic_outputs(rn):
    with pytest.raises(ValueError, match="2-byte"):
        rn.diag_bf16(0, 100, torch.empty(99, dtype=torch.int16, device=dev()))
    with pytest.raises(ValueError, match="2-byte"):
        rn.diag_bf16(0, 100, torch.empty(100, dtype=torch.float32, device=dev()))
    r, i = torch.empty(100, device=dev()), torch.empty(99, device=dev())
    with pytest.raises(ValueError, match="inv_out"):
        rn.diag_inverse(0x3F800000, 100, 1, 0.0, r, i)
