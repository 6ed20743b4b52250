"""Helpers for the GPU parity tests: device upload/download of seeded numpy inputs.

The GPU side is reached only through the C ABI (the ctypes binding); expected values
come only from the CPU oracle on the same seeded inputs.
"""

from __future__ import annotations

import sys

import numpy as np


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """numpy -> contiguous device tensor (uint16 travels as int16, bit for bit)."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).to("cuda")


def host(t, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    t = torch()
    m = {np.int8: t.int8, np.int32: t.int32, np.float32: t.float32, np.uint16: t.int16,
         np.uint8: t.uint8}
    return t.empty(shape, dtype=m[dtype], device="cuda")


def zeros(shape, dtype):
    return empty(shape, dtype).zero_()


def dev_weight(w: np.ndarray, layout: int):
    """Uploads an INT8 [N, K] weight; in the tiled layout it is regrouped on the device by
    the library's own pack kernel (a layout change only, checked separately)."""
    from w8a8_quantized_decode_amd import binding as B
    t = dev(w)
    if layout == B.LAYOUT_ROWMAJOR:
        return t
    out = torch().empty_like(t)
    B.a8w8_pack_weight(t, out)
    return out


def qw(w: np.ndarray, s: np.ndarray, layout: int):
    return (dev_weight(w, layout), dev(s), layout)


def announce(msg: str) -> None:
    """Names the GPU case on stdout before it runs (so a failure names its case)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between FP32 arrays (same sign assumed)."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def assert_bf16_close(got_bits: np.ndarray, want_bits: np.ndarray, rtol=1e-2, atol=1e-2):
    """BF16 outputs: relative error <= rtol, or absolute <= atol where |want| < 1."""
    from oracle import bf16_to_f32
    g = bf16_to_f32(got_bits).astype(np.float64)
    w = bf16_to_f32(want_bits).astype(np.float64)
    err = np.abs(g - w)
    ok = np.where(np.abs(w) < 1.0, err <= atol, err <= rtol * np.abs(w))
    bad = np.nonzero(~ok)
    pairs = [(tuple(int(i) for i in idx), float(g[idx]), float(w[idx]))
             for idx in list(zip(*bad))[:5]]
    assert ok.all(), f"{bad[0].size} BF16 outputs out of tolerance: (index, got, want) {pairs}"
