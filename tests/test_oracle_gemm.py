"""Pins of the oracle's INT8 x INT8 -> INT32 GEMM, dequantization and split-K.

Brute force in Python integers on tiny shapes, closed forms, and the exact split-K
identity the Down projection relies on (pypto-lib PR #810, What changed > Decode
scheduling: Down is split two ways along K, each part with its own accumulator).
"""

import numpy as np
import pytest

from oracle import dequant, down_split, int_gemm, split_k_ranges


def brute(q, w):
    M, K = q.shape
    N = w.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(q[m, k]) * int(w[n, k])
            out[m, n] = s
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 4))
    N = int(rng.integers(1, 9))
    K = int(rng.integers(1, 131))
    q = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    assert np.array_equal(int_gemm(q, w), brute(q, w))


def test_closed_forms():
    for K in (64, 5120, 17408):
        q = np.full((2, K), 127, dtype=np.int8)
        w = np.stack([np.full(K, 127, np.int8), np.full(K, -127, np.int8)])
        acc = int_gemm(q, w)
        assert acc[0, 0] == 16129 * K and acc[1, 1] == -16129 * K
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, size=(3, 40), dtype=np.int8)
    w = np.zeros((5, 40), dtype=np.int8)
    cols = [0, 7, 39, 13, 21]
    for n, c in enumerate(cols):
        w[n, c] = 1
    acc = int_gemm(q, w)
    assert np.array_equal(acc, q[:, cols].astype(np.int64))


def test_many_rows_blocked_path():
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(4, 96), dtype=np.int8)
    w = rng.integers(-127, 128, size=(1100, 96), dtype=np.int8)
    want = np.einsum("mk,nk->mn", q.astype(np.int64), w.astype(np.int64))
    assert np.array_equal(int_gemm(q, w), want)


def test_empty_rows():
    w = np.ones((4, 64), dtype=np.int8)
    assert int_gemm(np.zeros((0, 64), np.int8), w).shape == (0, 4)


def test_split_k_identity_every_split_point():
    rng = np.random.default_rng(9)
    K = 130
    q = rng.integers(-127, 128, size=(2, K), dtype=np.int8)
    w = rng.integers(-127, 128, size=(6, K), dtype=np.int8)
    full = int_gemm(q, w)
    for p in range(1, K):
        assert np.array_equal(int_gemm(q[:, :p], w[:, :p]) + int_gemm(q[:, p:], w[:, p:]), full)


@pytest.mark.parametrize("split_k", [1, 2, 4, 8])
def test_down_split_partitions(split_k):
    rng = np.random.default_rng(split_k)
    K, N, M = 512, 24, 3
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    w = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s_h = rng.uniform(0.1, 2, size=M).astype(np.float32)
    s_d = rng.uniform(1e-3, 1e-2, size=N).astype(np.float32)
    accs, ps = down_split(q, s_h, w, s_d, split_k)
    assert len(accs) == split_k
    assert np.array_equal(sum(accs), int_gemm(q, w))
    ranges = split_k_ranges(K, split_k)
    assert ranges[0][0] == 0 and ranges[-1][1] == K
    assert all(b - a == K // split_k for a, b in ranges)
    for (k0, k1), acc in zip(ranges, accs):
        assert np.array_equal(acc, brute(q[:, k0:k1], w[:, k0:k1]))
    with pytest.raises(ValueError):
        split_k_ranges(K + 1, 2)


def test_dequant_error_bound_and_channel_broadcast():
    rng = np.random.default_rng(21)
    M, N = 4, 64
    acc = rng.integers(-(2**31) + 1, 2**31 - 1, size=(M, N), dtype=np.int64)
    acc[0, :8] = rng.integers(-2**20, 2**20, size=8)
    s_row = rng.uniform(1e-3, 3.0, size=M).astype(np.float32)
    s_w = rng.uniform(1e-3, 1e-2, size=N).astype(np.float32)
    y = dequant(acc, s_row, s_w).astype(np.float64)
    exact = acc.astype(np.float64) * s_row.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]
    # three roundings (INT32->FP32, two products): relative error <= 3 * 2**-24 (+ tiny)
    rel = np.abs(y - exact) / np.abs(exact)
    assert np.max(rel) <= 3.0001 * 2.0**-24
