"""Pins of the oracle's per-row dynamic INT8 quantizer.

pypto-lib PR #810, What changed > Gate/Up INT8 path (dynamic per-row quantization with
FP32 row scales).  Checked by invariants that hold for any input, the quantize /
dequantize error bound (at most half a scale step, plus the FP32 rounding of the
quotient), a hand-worked tie row, and the degenerate rows.
"""

import os

import numpy as np
import pytest

from oracle import quantize_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_tie_row.txt")


def _rows(seed, M=8, K=5120):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((M, K)).astype(np.float32)
    v *= rng.uniform(1e-3, 1e3, size=(M, 1)).astype(np.float32)
    v[1, 17] = -50 * np.abs(v[1]).max()          # one dominant negative outlier
    v[2, :] = np.abs(v[2])                        # one-signed row
    return v


@pytest.mark.parametrize("seed", range(4))
def test_invariants_and_error_bound(seed):
    v = _rows(seed)
    q, s = quantize_rows(v)
    assert q.dtype == np.int8 and s.dtype == np.float32 and q.shape == v.shape
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    for m in range(v.shape[0]):
        assert np.max(np.abs(q[m].astype(np.int32))) == 127
        sg = np.sign(q[m])
        assert np.all((sg == np.sign(v[m])) | (sg == 0))
        # |v - q*s| <= s * (1/2 + 2**-16): half a step plus the FP32 rounding of v/s
        err = np.abs(v[m].astype(np.float64) - q[m].astype(np.float64) * np.float64(s[m]))
        assert np.max(err) <= np.float64(s[m]) * (0.5 + 2.0**-16)
        # the scale maps the row's absolute maximum onto 127 (within one FP32 rounding)
        a = np.float64(np.max(np.abs(v[m])))
        assert abs(np.float64(s[m]) * 127 - a) <= a * 2.0**-23


def test_golden_tie_row():
    with open(GOLDEN) as f:
        lines = [ln for ln in f.read().splitlines() if ln and not ln.startswith("#")]
    v = np.array([float(t) for t in lines[0].split()], dtype=np.float32)[None, :]
    s_want = np.float32(float(lines[1]))
    q_want = np.array([int(t) for t in lines[2].split()], dtype=np.int8)
    q, s = quantize_rows(v)
    assert s[0] == s_want
    assert np.array_equal(q[0], q_want)


def test_zero_and_underflowing_rows():
    v = np.zeros((3, 64), dtype=np.float32)
    v[1, 5] = np.float32(1e-44)      # a/127 underflows to 0 in FP32
    v[2, :] = 0.25
    q, s = quantize_rows(v)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert s[1] == 0 and np.all(q[1] == 0)
    assert np.all(q[2] == 127) and s[2] == np.float32(np.float32(0.25) / np.float32(127))


def test_rounding_is_to_nearest_not_truncation():
    # absmax 127 -> s = 1: codes are the nearest integers of the values
    v = np.array([[127.0, 0.7, -0.7, 5.49, -5.51, 99.999]], dtype=np.float32)
    q, s = quantize_rows(v)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 1, -1, 5, -6, 100]


def test_empty():
    q, s = quantize_rows(np.zeros((0, 32), np.float32))
    assert q.shape == (0, 32) and s.shape == (0,)
