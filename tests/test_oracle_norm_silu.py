"""Pins of the oracle's RMSNorm and SiLU(gate)*up.

RMSNorm: closed forms that are exact in FP32, scale invariance, and the FP64 formula
within the error of the FP32 rounding chain.  SiLU*up: the FP64 formula within a few
FP32 roundings, plus its exact special cases.
"""

import numpy as np
import pytest

from oracle import bf16_to_f32, exp_f32, rmsnorm, rne_bf16, silu_mul
from w8a8_quantized_decode_amd import synth

U = 2.0 ** -24  # unit roundoff of FP32


def _bf(v):
    return rne_bf16(np.asarray(v, dtype=np.float32))


@pytest.mark.parametrize("c", [1.0, 2.0, 0.5, 4.0, -8.0])
def test_constant_power_of_two_rows_give_gamma(c):
    K = 96
    gamma = synth.uniform_bf16(3, (K,), 0.5, 1.5)
    x = np.full((1, K), _bf(c)[()] if np.ndim(_bf(c)) == 0 else _bf([c])[0], dtype=np.uint16)
    xn = rmsnorm(x, gamma, 0.0)
    assert np.array_equal(xn[0], np.sign(c) * bf16_to_f32(gamma))


def test_alternating_signs_and_mean_not_sum():
    K = 128
    gamma = _bf(np.ones(K))
    x = _bf(np.where(np.arange(K) % 2 == 0, 3.0, -3.0))[None, :]
    xn = rmsnorm(x, gamma, 0.0)
    # mean of squares is 9 -> r = 1/3; 3 * fl32(1/3) rounds back to 1 exactly
    assert np.array_equal(np.abs(xn[0]), np.ones(K, np.float32))


def test_scale_invariance_exact_without_eps():
    x = synth.normal_bf16(4, (3, 256))
    gamma = synth.uniform_bf16(5, (256,), 0.5, 1.5)
    x2 = _bf(2.0 * bf16_to_f32(x))  # doubling a BF16 value is exact
    assert np.array_equal(rmsnorm(x, gamma, 0.0), rmsnorm(x2, gamma, 0.0))


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_against_fp64_formula(eps):
    x = synth.normal_bf16(6, (5, 5120))
    x[3] = _bf(bf16_to_f32(x[3]) * np.float32(1e-3))  # small row: eps matters
    gamma = synth.uniform_bf16(7, (5120,), 0.5, 1.5)
    xn = rmsnorm(x, gamma, eps).astype(np.float64)
    xf = bf16_to_f32(x).astype(np.float64)
    gf = bf16_to_f32(gamma).astype(np.float64)
    ref = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + np.float64(np.float32(eps))) * gf
    # ms, t, sqrt, 1/x, two products: at most ~5.5 units of FP32 roundoff
    assert np.all(np.abs(xn - ref) <= 6 * U * np.abs(ref) + 1e-300)


def test_silu_mul_against_fp64():
    rng = np.random.default_rng(8)
    g = (rng.standard_normal(20000) * 30).astype(np.float32)
    u = (rng.standard_normal(20000) * 30).astype(np.float32)
    h = silu_mul(g, u).astype(np.float64)
    gd, ud = g.astype(np.float64), u.astype(np.float64)
    ref = gd / (1.0 + np.exp(-gd)) * ud
    # below -ln(FLT_MAX) ~ -88.72, exp(-g) overflows FP32: silu(g) becomes a signed zero
    # where the exact value is below 1e-33 in magnitude
    over = g < -88.72
    assert np.all(h[over] == 0) and np.all(np.abs(ref[over]) < 1e-33)
    ok = ~over
    assert np.all(np.abs(h[ok] - ref[ok]) <= 4 * 2 * U * np.abs(ref[ok]) + 1e-37)


def test_silu_special_cases():
    u = np.array([3.0, -2.0, 7.5], dtype=np.float32)
    assert np.all(silu_mul(np.zeros(3, np.float32), u) == 0)
    g = np.array([40.0, 100.0, 1e6], dtype=np.float32)  # exp(-g) < 2**-24: silu(g) == g
    assert np.array_equal(silu_mul(g, u), g * u)
    big_neg = silu_mul(np.array([-1e4], np.float32), np.array([1.0], np.float32))
    assert big_neg[0] == 0
    # silu(g) - silu(-g) == g up to a few roundings
    gg = np.linspace(-20, 20, 4001).astype(np.float32)
    one = np.ones_like(gg)
    d = silu_mul(gg, one).astype(np.float64) - silu_mul(-gg, one).astype(np.float64)
    assert np.all(np.abs(d - gg) <= 8 * U * np.abs(gg) + 1e-30)


def test_exp_f32_is_correctly_rounded_on_a_grid():
    x = np.linspace(-80, 80, 100001).astype(np.float32)
    e = exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.all(np.abs(e - ref) <= U * ref * (1 + 1e-9))
