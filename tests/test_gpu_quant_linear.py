"""GPU parity of a8w8_quantize_rows and a8w8_linear against the CPU oracle.

Expected values come only from the oracle on the same seeded inputs.  INT8 codes, row
scales, INT32 accumulators, the FP32 RMSNorm output and the BF16 outputs are compared
bit for bit: every FP32 step on both sides is the same correctly rounded operation,
so they agree exactly (the only order-dependent step, the FP64 sum of squares, would
need an FP64 rounding error to straddle an FP32 rounding boundary, probability about
2**-26 per row).
"""

import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import announce, dev, dev_weight, empty, host, zeros
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,ldx,rms", [(1, 256, 256, True), (3, 5120, 5120, True),
                                          (16, 5120, 5120, False), (16, 5120, 7168, False),
                                          (7, 17408, 17408, True), (256, 5120, 5120, True),
                                          (2, 8, 8, True)])
def test_quantize_rows(M, K, ldx, rms):
    announce(f"quantize_rows M={M} K={K} ldx={ldx} rms={rms}")
    x = synth.normal_bf16(100 + M, (M, ldx))
    gamma = synth.uniform_bf16(200 + K, (K,), 0.5, 1.5)
    if rms:
        xn = O.rmsnorm(x[:, :K], gamma, 1e-6)
    else:
        xn = O.bf16_to_f32(x[:, :K])
    q_want, s_want = O.quantize_rows(xn)
    q = empty((M, K), np.int8)
    s = empty((M,), np.float32)
    xt = empty((M, K), np.float32)
    B.a8w8_quantize_rows(dev(x), q, s, gamma=dev(gamma) if rms else None, eps=1e-6,
                         xn_tap=xt, K=K)
    np.testing.assert_array_equal(host(s), s_want)
    np.testing.assert_array_equal(host(q), q_want)
    np.testing.assert_array_equal(host(xt).view(np.uint32), xn.view(np.uint32))


def test_quantize_rows_edge_rows():
    announce("quantize_rows edge rows")
    K = 64
    rows = np.zeros((4, K), np.float32)
    rows[1, :10] = [127.0, 2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0, 0.0, 3.25]  # ties
    rows[2, :] = 1e-40                                # subnormal row: s underflows to 0
    rows[3, 5] = -2.0                                 # single nonzero
    x = O.rne_bf16(rows)
    q_want, s_want = O.quantize_rows(O.bf16_to_f32(x))
    q = empty((4, K), np.int8)
    s = empty((4,), np.float32)
    B.a8w8_quantize_rows(dev(x), q, s)
    np.testing.assert_array_equal(host(s), s_want)
    np.testing.assert_array_equal(host(q), q_want)
    assert host(q)[1, :10].tolist() == [127, 2, -4, 0, 0, 2, 126, -127, 0, 3]


def test_quantize_rows_empty_is_noop():
    q = zeros((0, 64), np.int8)
    s = zeros((0,), np.float32)
    B.a8w8_quantize_rows(zeros((0, 64), np.uint16), q, s)


LINEAR_CASES = [(1, 16, 64), (1, 7168, 5120), (5, 48, 320), (16, 5120, 5120), (17, 64, 128),
                (100, 32, 192), (64, 256, 17408), (1, 5120, 17408), (33, 80, 8704),
                (3, 96, 2048), (16, 64, 1024), (12, 4096, 3072)]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
@pytest.mark.parametrize("with_res", [False, True])
@pytest.mark.parametrize("layout", [B.LAYOUT_ROWMAJOR, B.LAYOUT_TILED])
def test_linear(M, N, K, with_res, layout):
    announce(f"linear M={M} N={N} K={K} res={with_res} layout={layout}")
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    s_x = rng.uniform(1e-3, 1.0, size=M).astype(np.float32)
    s_w = rng.uniform(1e-3, 1e-2, size=N).astype(np.float32)
    res = synth.normal_bf16(M + N, (M, N)) if with_res else None
    y_want, acc_want = O.linear_decode(q, s_x, w, s_w, res)
    y = empty((M, N), np.uint16)
    acc = empty((M, N), np.int32)
    B.a8w8_linear(dev(q), dev(s_x), dev_weight(w, layout), dev(s_w), y,
                  residual=dev(res) if with_res else None, acc_tap=acc, layout=layout)
    np.testing.assert_array_equal(host(acc), acc_want)
    np.testing.assert_array_equal(host(y, np.uint16), y_want)


@pytest.mark.parametrize("N,K", [(16, 64), (48, 320), (7168, 5120)])
def test_pack_weight_layout(N, K):
    """The tiled layout is the documented regrouping of the row-major bytes."""
    announce(f"pack_weight N={N} K={K}")
    rng = np.random.default_rng(N + K)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    t = dev(w)
    out = dev(np.zeros_like(w))
    B.a8w8_pack_weight(t, out)
    got = host(out).reshape(-1)
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    pos = (n // 16) * 16 * K + (k // 64) * 1024 + 16 * ((n % 16) + 16 * ((k % 64) // 16)) + k % 16
    want = np.empty(N * K, np.int8)
    want[pos.ravel()] = w.ravel()
    np.testing.assert_array_equal(got, want)


def _rne_probe_values():
    rng = np.random.default_rng(17)
    hi = np.arange(1 << 16, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = ((hi[:, None] << np.uint32(16)) | lows[None, :]).ravel()
    u = np.concatenate([u, rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)])
    u = u[(u & 0x7F800000) != 0x7F800000]           # finite only
    u = u[: (u.size // 16) * 16]
    return u.view(np.float32)


def test_bf16_narrowing_through_linear():
    """y = rne_bf16(fl32(fl32(f(1) * 1) * s_w[n])) = rne_bf16(s_w[n]): with a one-hot
    activation and one-hot weight rows the output of a8w8_linear is the RNE narrowing
    of the channel scale itself, for every probed FP32 pattern (ties, carries,
    overflow to Inf, subnormals).  (With acc = 1 and s_x = 1 both association orders of
    the dequantization agree, so the order is tested elsewhere: on the FP32 Down
    partials of the MLP block, test_mlp_dequant_order_is_observable.)"""
    announce("linear RNE probe")
    vals = _rne_probe_values()
    N, K = vals.size, 64
    q = np.zeros((1, K), np.int8)
    q[0, 0] = 1
    w = np.zeros((N, K), np.int8)
    w[:, 0] = 1
    y = empty((1, N), np.uint16)
    B.a8w8_linear(dev(q), dev(np.ones(1, np.float32)), dev(w), dev(vals), y)
    np.testing.assert_array_equal(host(y, np.uint16)[0], O.rne_bf16(vals))


def test_linear_int32_to_fp32_conversion_rounding():
    """Accumulators above 2**24 convert to FP32 with ties to even (s_x = s_w = 1)."""
    announce("linear INT32->FP32 conversion")
    K = 17408
    rng = np.random.default_rng(5)
    N = 64
    w = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    w[:8] = 127
    q = np.full((1, K), 127, np.int8)
    q[0, : K // 2] = rng.integers(-127, 128, size=K // 2)
    ones = np.ones(N, np.float32)
    y_want, acc_want = O.linear_decode(q, np.ones(1, np.float32), w, ones)
    assert np.abs(acc_want).max() > 2**24
    y = empty((1, N), np.uint16)
    acc = empty((1, N), np.int32)
    B.a8w8_linear(dev(q), dev(np.ones(1, np.float32)), dev(w), dev(ones), y, acc_tap=acc)
    np.testing.assert_array_equal(host(acc), acc_want)
    np.testing.assert_array_equal(host(y, np.uint16), y_want)
