"""The oracle's composed decode blocks against a scalar brute force on tiny shapes.

The stage functions of the oracle are pinned one by one elsewhere; this pins how they
are put together (which scale meets which accumulator, the requantization of h, the
split-K partials and the residual, the Q slice that feeds O, h1 as both input and
residual of the MLP).  The brute force below computes the whole MLP block and the layer
linears element by element with Python scalars, from the readings the oracle documents
(RMSNorm, quantization, dequantization, SiLU, the Down reduction), and calls nothing
from the oracle.  FP32 operations are numpy float32 scalar operations (one rounding
each); sums of squares are exact rationals rounded once; integer products are Python
integers; BF16 narrowing is done on the bit pattern.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from w8a8_quantized_decode_amd import synth

F = np.float32


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def from_bf16(b: int) -> np.float32:
    return np.frombuffer(struct.pack("<I", (int(b) & 0xFFFF) << 16), dtype=np.float32)[0]


def to_bf16(x) -> int:
    """Round-to-nearest-even of an FP32 value to BF16 (bit pattern), on the integer bits."""
    u = f32_bits(x)
    keep, rest = u >> 16, u & 0xFFFF
    if rest > 0x8000 or (rest == 0x8000 and keep & 1):
        keep += 1
    return keep & 0xFFFF


def bf16_row_values(bits_row):
    return [from_bf16(b) for b in bits_row]


def rmsnorm_row(xb, gb, eps):
    x = bf16_row_values(xb)
    g = bf16_row_values(gb)
    S = float(sum(Fraction(float(v)) ** 2 for v in x))   # exact, rounded once to FP64
    ms = F(S / len(x))
    t = F(ms + F(eps))
    r = F(F(1.0) / F(np.sqrt(t)))
    return [F(F(v * r) * gv) for v, gv in zip(x, g)]


def quantize_row(v):
    a = F(0.0)
    for e in v:
        a = max(a, F(abs(e)))
    s = F(a / F(127.0))
    if s == 0:
        return [0] * len(v), s
    q = []
    for e in v:
        t = float(F(e / s))
        c = round(t)                 # ties to even on Python floats
        q.append(max(-127, min(127, int(c))))
    return q, s


def int_dot(q, w_row):
    return sum(int(a) * int(b) for a, b in zip(q, w_row))


def dequant_one(acc, s_row, s_w):
    return F(F(F(acc) * s_row) * s_w)


def silu_times(g, u):
    e = F(math.exp(-float(g)))                      # exp in FP64, rounded once
    return F(F(g / F(F(1.0) + e)) * u)


def mlp_block_brute(xb, gb, eps, wg, sg, wu, su, wd, sd, resb, split_k):
    """Returns the output bits [M][H] and the intermediates: g, u, h [M][I] (FP32), the h
    codes and scales, and the Down partials [split_k][M][H] (FP32)."""
    M, H = len(xb), len(xb[0])
    I = len(wg)
    out, st = [], dict(xn=[], g=[], u=[], h=[], q_h=[], s_h=[], p=[[] for _ in range(split_k)])
    for m in range(M):
        xn = rmsnorm_row(xb[m], gb, eps)
        st["xn"].append(xn)
        qx, sx = quantize_row(xn)
        gs, us, h = [], [], []
        for n in range(I):
            g = dequant_one(int_dot(qx, wg[n]), sx, F(sg[n]))
            u = dequant_one(int_dot(qx, wu[n]), sx, F(su[n]))
            gs.append(g)
            us.append(u)
            h.append(silu_times(g, u))
        qh, sh = quantize_row(h)
        for k, v in (("g", gs), ("u", us), ("h", h), ("q_h", qh), ("s_h", sh)):
            st[k].append(v)
        cut = I // split_k
        row, prow = [], [[] for _ in range(split_k)]
        for n in range(H):
            parts = []
            for j in range(split_k):
                acc = int_dot(qh[j * cut:(j + 1) * cut], wd[n][j * cut:(j + 1) * cut])
                parts.append(dequant_one(acc, sh, F(sd[n])))
                prow[j].append(parts[-1])
            tot = parts[0]
            for p in parts[1:]:
                tot = F(tot + p)
            row.append(to_bf16(F(tot + from_bf16(resb[m][n]))))
        out.append(row)
        for j in range(split_k):
            st["p"][j].append(prow[j])
    return out, st


def _same_bits(a, b):
    np.testing.assert_array_equal(np.asarray(a, np.float32).view(np.uint32),
                                  np.asarray(b, np.float32).view(np.uint32))


TINY = synth.Config(0, "tiny block", 2, 64, 128, "mlp", n_q_heads=2, n_kv_heads=1,
                    head_dim=32)


def _lists(d):
    return {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in d.items()}


@pytest.mark.parametrize("split_k", [1, 2, 4])
@pytest.mark.parametrize("M", [1, 3])
def test_mlp_block_composition_brute_force(M, split_k):
    d = synth.mlp_inputs(TINY, M=M)
    want, st = O.mlp_block_decode(d["x"], d["gamma_post"], TINY.eps, d["w_gate"], d["s_gate"],
                                  d["w_up"], d["s_up"], d["w_down"], d["s_down"], d["res"],
                                  split_k=split_k)
    L = _lists(d)
    out, bt = mlp_block_brute(L["x"], L["gamma_post"], TINY.eps, L["w_gate"], L["s_gate"],
                              L["w_up"], L["s_up"], L["w_down"], L["s_down"], L["res"],
                              split_k)
    for k in ("xn", "g", "u", "h", "s_h"):
        _same_bits(bt[k], st[k])
    np.testing.assert_array_equal(np.array(bt["q_h"], np.int8), st["q_h"])
    for j in range(split_k):
        _same_bits(bt["p"][j], st["p_down"][j])
    np.testing.assert_array_equal(np.array(out, np.uint16), want)


def test_layer_linears_composition_brute_force():
    cfg, M = TINY, 2
    d = synth.layer_inputs(cfg, layer=0, M=M)
    want, st = O.layer_linears_decode(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                      d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"],
                                      d["s_gate"], d["w_up"], d["s_up"], d["w_down"],
                                      d["s_down"], cfg.n_q_heads, cfg.head_dim, cfg.split_k)
    L = _lists(d)
    n_q = cfg.n_q_heads * cfg.head_dim
    h1 = []
    for m in range(M):
        xn = rmsnorm_row(L["x"][m], L["gamma_in"], cfg.eps)
        qx, sx = quantize_row(xn)
        qkv = [to_bf16(dequant_one(int_dot(qx, L["w_qkv"][n]), sx, F(L["s_qkv"][n])))
               for n in range(len(L["w_qkv"]))]
        qa, sa = quantize_row(bf16_row_values(qkv[:n_q]))
        row = []
        for n in range(cfg.H):
            y = dequant_one(int_dot(qa, L["w_o"][n]), sa, F(L["s_o"][n]))
            row.append(to_bf16(F(y + from_bf16(L["x"][m][n]))))
        h1.append(row)
        np.testing.assert_array_equal(np.array(qkv, np.uint16), st["qkv"][m])
    np.testing.assert_array_equal(np.array(h1, np.uint16), st["h1"])
    out, _ = mlp_block_brute(h1, L["gamma_post"], cfg.eps, L["w_gate"], L["s_gate"],
                             L["w_up"], L["s_up"], L["w_down"], L["s_down"], h1,
                             cfg.split_k)
    np.testing.assert_array_equal(np.array(out, np.uint16), want)


def test_brute_force_sees_a_miswired_composition():
    """A plausible wiring mistake (the residual of the MLP taken from the layer input
    instead of h1) changes the brute force's output, so the comparison above can fail."""
    cfg, M = TINY, 2
    d = _lists(synth.layer_inputs(cfg, layer=0, M=M))
    d2 = _lists(synth.mlp_inputs(cfg, M=M))
    a, _ = mlp_block_brute(d2["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                           d["w_up"], d["s_up"], d["w_down"], d["s_down"], d2["x"], 2)
    b, _ = mlp_block_brute(d2["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                           d["w_up"], d["s_up"], d["w_down"], d["s_down"], d2["res"], 2)
    assert a != b


# ----------------------------------------------------------------------------- prefill

def weight_bf16(w_row, s):
    """A weight row converted for the prefill matrix cores: BF16 of the FP32 product."""
    return [from_bf16(to_bf16(F(F(int(w)) * F(s)))) for w in w_row]


def bf16_dot(a_vals, w_vals):
    """Products of BF16 values are exact in FP64; their sum is taken exactly (fsum, one
    rounding to FP64) and then rounded to FP32."""
    return F(math.fsum(float(a) * float(w) for a, w in zip(a_vals, w_vals)))


def prefill_mlp_brute(xb, gb, eps, wg, sg, wu, su, wd, sd, resb):
    M, H = len(xb), len(xb[0])
    I = len(wg)
    Wg = [weight_bf16(wg[n], sg[n]) for n in range(I)]
    Wu = [weight_bf16(wu[n], su[n]) for n in range(I)]
    Wd = [weight_bf16(wd[n], sd[n]) for n in range(H)]
    out, hs = [], []
    for m in range(M):
        a = [from_bf16(to_bf16(v)) for v in rmsnorm_row(xb[m], gb, eps)]
        h = [from_bf16(to_bf16(silu_times(bf16_dot(a, Wg[n]), bf16_dot(a, Wu[n]))))
             for n in range(I)]
        hs.append([to_bf16(v) for v in h])
        out.append([to_bf16(F(bf16_dot(h, Wd[n]) + from_bf16(resb[m][n]))) for n in range(H)])
    return out, hs


def test_prefill_mlp_composition_brute_force():
    cfg, M = TINY, 3
    d = synth.mlp_inputs(cfg, M=M)
    want, st = O.prefill_mlp(d["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                             d["w_up"], d["s_up"], d["w_down"], d["s_down"], d["res"])
    L = _lists(d)
    out, h = prefill_mlp_brute(L["x"], L["gamma_post"], cfg.eps, L["w_gate"], L["s_gate"],
                               L["w_up"], L["s_up"], L["w_down"], L["s_down"], L["res"])
    np.testing.assert_array_equal(np.array(h, np.uint16), st["h"])
    np.testing.assert_array_equal(np.array(out, np.uint16), want)


def test_prefill_layer_composition_brute_force():
    cfg, M = TINY, 2
    d = synth.layer_inputs(cfg, layer=0, M=M)
    want, st = O.layer_linears_prefill(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                       d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"],
                                       d["s_gate"], d["w_up"], d["s_up"], d["w_down"],
                                       d["s_down"], cfg.n_q_heads, cfg.head_dim)
    L = _lists(d)
    n_q = cfg.n_q_heads * cfg.head_dim
    Wqkv = [weight_bf16(L["w_qkv"][n], L["s_qkv"][n]) for n in range(len(L["w_qkv"]))]
    Wo = [weight_bf16(L["w_o"][n], L["s_o"][n]) for n in range(cfg.H)]
    h1 = []
    for m in range(M):
        a = [from_bf16(to_bf16(v)) for v in rmsnorm_row(L["x"][m], L["gamma_in"], cfg.eps)]
        qkv = [to_bf16(bf16_dot(a, Wqkv[n])) for n in range(len(Wqkv))]
        np.testing.assert_array_equal(np.array(qkv, np.uint16), st["qkv"][m])
        attn = bf16_row_values(qkv[:n_q])
        h1.append([to_bf16(F(bf16_dot(attn, Wo[n]) + from_bf16(L["x"][m][n])))
                   for n in range(cfg.H)])
    np.testing.assert_array_equal(np.array(h1, np.uint16), st["h1"])
    out, _ = prefill_mlp_brute(h1, L["gamma_post"], cfg.eps, L["w_gate"], L["s_gate"],
                               L["w_up"], L["s_up"], L["w_down"], L["s_down"], h1)
    np.testing.assert_array_equal(np.array(out, np.uint16), want)
