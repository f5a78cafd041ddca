"""Helpers for the GPU tests: numpy <-> device tensors and bitwise comparison.

Only data movement lives here; every expected value comes from the CPU oracle.
"""
import numpy as np


def dev():
    import torch
    return torch.device("cuda", 0)


def to_dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_dev_bf16(bits):
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).to(dev()).view(torch.bfloat16)


def f32_host(t):
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def bf16_host(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bits_f32(got, want, what=""):
    """Bitwise equality; two NaNs compare equal (payloads are not specified)."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    g, w = got.view(np.uint32)[~gn], want.view(np.uint32)[~wn]
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} elements differ; first at "
                           f"{bad[0]}: got {g[bad[0]]:#010x} want {w[bad[0]]:#010x}")


def assert_bits_bf16(got, want, what=""):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gn = ((got & 0x7FFF) > 0x7F80)
    wn = ((want & 0x7FFF) > 0x7F80)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    bad = np.flatnonzero(got[~gn] != want[~wn])
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} elements differ; first at "
                           f"{bad[0]}: got {got[~gn][bad[0]]:#06x} want {want[~wn][bad[0]]:#06x}")


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
