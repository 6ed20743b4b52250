"""Pins of the oracle's FP32 -> BF16 round-to-nearest-even narrowing.

The reference used here is independent of the oracle's bit trick: it takes the two BF16
neighbours of the exact value (truncation toward zero and the next magnitude up),
measures both distances exactly in FP64, and breaks ties toward the even pattern.
"""

import os

import numpy as np
import pytest

from oracle import bf16_to_f32, rne_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rne_bf16_vectors.txt")


def nearest_bf16_reference(u32: np.ndarray) -> np.ndarray:
    """Nearest BF16 (ties to even) of finite FP32 patterns, by exact FP64 distances."""
    u32 = np.asarray(u32, dtype=np.uint32)
    x = u32.view(np.float32).astype(np.float64)
    lo_b = (u32 >> np.uint32(16)).astype(np.uint32)
    hi_b = lo_b + np.uint32(1)
    lo = (lo_b << np.uint32(16)).view(np.float32).astype(np.float64)
    hi_mag_bits = hi_b & np.uint32(0x7FFF)
    hi = np.where(hi_mag_bits == 0x7F80,
                  np.where(lo_b & 0x8000, -(2.0 ** 128), 2.0 ** 128),
                  (hi_b << np.uint32(16)).view(np.float32).astype(np.float64))
    dlo = np.abs(x - lo)
    dhi = np.abs(hi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo_b & 1) == 1))
    return np.where(pick_hi, hi_b, lo_b).astype(np.uint16)


def _finite(u):
    return (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)


def test_golden_vectors():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), int(b, 16)))
    u = np.array([r[0] for r in rows], dtype=np.uint32)
    want = np.array([r[1] for r in rows], dtype=np.uint16)
    got = rne_bf16(u.view(np.float32))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(u[i]), hex(got[i]), hex(want[i])) for i in bad]


def test_all_high_halves_with_decisive_low_halves():
    hi = np.arange(1 << 16, dtype=np.uint32)
    rng = np.random.default_rng(7)
    lows = np.unique(np.concatenate([
        np.array([0, 1, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF, 0x4000, 0xC000],
                 dtype=np.uint32),
        rng.integers(0, 1 << 16, size=54, dtype=np.uint32)]))
    u = ((hi[:, None] << np.uint32(16)) | lows[None, :]).ravel()
    u = u[_finite(u)]
    got = rne_bf16(u.view(np.float32))
    want = nearest_bf16_reference(u)
    assert np.array_equal(got, want)


def test_all_low_halves_for_sampled_high_halves():
    rng = np.random.default_rng(11)
    highs = np.unique(np.concatenate([
        np.array([0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F,
                  0xFF7F, 0xBF80, 0x4049], dtype=np.uint32),
        rng.integers(0, 1 << 16, size=116, dtype=np.uint32)]))
    lows = np.arange(1 << 16, dtype=np.uint32)
    u = ((highs[:, None] << np.uint32(16)) | lows[None, :]).ravel()
    u = u[_finite(u)]
    got = rne_bf16(u.view(np.float32))
    want = nearest_bf16_reference(u)
    assert np.array_equal(got, want)


def test_non_finite():
    u = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FFFFFFF],
                 dtype=np.uint32)
    got = rne_bf16(u.view(np.float32))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    back = bf16_to_f32(got[2:])
    assert np.all(np.isnan(back))
    assert np.all((got[2:] & 0x0040) != 0)  # quiet


def test_round_trip_of_bf16_values_is_exact():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[_finite(b.astype(np.uint32) << np.uint32(16))]
    assert np.array_equal(rne_bf16(bf16_to_f32(b)), b)


@pytest.mark.slow
def test_exhaustive_all_fp32_patterns():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        u = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        u = u[_finite(u)]
        if u.size == 0:
            continue
        assert np.array_equal(rne_bf16(u.view(np.float32)), nearest_bf16_reference(u)), hex(start)
