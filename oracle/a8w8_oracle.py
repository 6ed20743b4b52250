"""Plain CPU oracle for the A8W8 decode linears of a Qwen3-14B-shaped layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct statement of
what the GPU path computes.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python
binding) never imports, links or calls anything here, and this module shares no code
with it.

Sources (the four pages this method is described on):

* [PR810] pypto-lib PR #810, "perf(qwen3-a8w8): optimize decode scheduling and data
  paths": "What changed" (Decode scheduling; Gate/Up INT8 path), "Validation", the
  CodeRabbit walkthrough table ("Decode activation and gate/up quantization",
  "Split down projection accumulation"), the Gemini review (narrowing with
  mode="rint") and the CodeRabbit nitpick on the down-projection constants.
* [PR48] pypto-serving PR #48, "Add native Qwen3 14B A8W8 serving path": CodeRabbit
  inline comment on ``_hf_linear_to_bf16`` (scale broadcasts over output channels),
  PR body "Compatibility and boundaries" (explicit RNE narrowing).
* [ISSUE52] pypto-serving issue #52, "[Feature] Add native Qwen3-14B A8W8 serving
  path": "Measurement basis" (MLP gate/up/silu/down).

Where the pages leave a step open the reading taken is stated at the function.  Every
FP32 step is one IEEE-754 binary32 operation rounded to nearest-even (numpy float32
arithmetic; no fused multiply-add); constants are cast to float32 explicitly.

Notation: ``f()`` is exact conversion of INT32/BF16 to FP32 (INT32 values above 2**24
round to nearest-even); ``fl32(.)`` is one FP32 operation.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against brute force,
closed forms, invariants or error bounds.  The end-to-end compositions
(``mlp_block_decode``, ``layer_linears_decode``, ``prefill_mlp``,
``layer_linears_prefill``) are pinned beyond their stage pins by an element-by-element
scalar brute force on tiny shapes (``tests/test_oracle_composed.py``), written from the
same readings without calling this module and compared bit for bit, intermediates
included, and by an error bound against exact (unquantized) FP64 math; the pages print
no worked example of a whole block.  ``decode_layer`` (the layer with real attention)
is pinned beyond its stages by the one-position context, the identity-attention
layer's QKV and h1, and the cache slot it writes.
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32
_INT32_MAX = 2**31 - 1


# ----------------------------------------------------------------------------- BF16

def bf16_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> exact FP32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rne_bf16(x) -> np.ndarray:
    """FP32 -> BF16 with round-to-nearest, ties to even; returns uint16 bit patterns.

    [PR810] Validation: every FP32->BF16 narrowing site rounds to nearest-even (the
    Gemini review asks for ``mode="rint"`` on every such cast); [PR48] body,
    "Compatibility and boundaries": explicit RNE narrowing.

    On the FP32 bit pattern ``u``: add 0x7FFF plus the lowest kept bit, keep the top 16
    bits.  Values past the largest finite BF16 by half an ulp or more become +-Inf.
    NaN maps to a quiet NaN with the same sign (non-finite inputs are outside the
    method's domain and only kept NaN so that they stay visible).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    if np.any(nan):
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return r


# ----------------------------------------------------------------------------- steps

def rmsnorm(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """RMSNorm of BF16 rows, FP32 result ``xn[m,k] = fl32(fl32(f(x[m,k]) * r[m]) * f(g[k]))``.

    [PR810] What changed > Gate/Up INT8 path: the post-attention RMSNorm output is what
    gets quantized per row.  The pages give no precision for the norm; reading taken:
    ``S = sum_k f(x_k)**2`` summed exactly and rounded once to FP64 (each square of a
    BF16 value is exact in FP64), ``ms = fl32(S / K)`` (one FP64 division rounded to
    FP32), ``t = fl32(ms + eps)``, ``r = fl32(1 / fl32(sqrt(t)))`` with correctly
    rounded square root and division.
    """
    x = bf16_to_f32(x_bits)
    g = bf16_to_f32(gamma_bits)
    if x.ndim != 2 or g.shape != (x.shape[1],):
        raise ValueError("rmsnorm: x must be [M,K] and gamma [K]")
    M, K = x.shape
    out = np.empty((M, K), dtype=np.float32)
    eps32 = F32(eps)
    for m in range(M):
        row64 = x[m].astype(np.float64)
        S = math.fsum(row64 * row64)
        ms = F32(S / K)
        t = F32(ms + eps32)
        sq = F32(np.sqrt(t))
        r = F32(F32(1.0) / sq)
        out[m] = (x[m] * r) * g
    return out


def quantize_rows(v) -> tuple[np.ndarray, np.ndarray]:
    """Per-row dynamic symmetric INT8 quantization of FP32 rows.

    [PR810] What changed > Decode scheduling (activation quantization batched over all
    decode rows) and > Gate/Up INT8 path (dynamic quantization once per row); the
    CodeRabbit walkthrough (decode activations carry per-row scales).

    Readings (the pages name row scales but give no formula): symmetric, no zero point;
    ``a = max_k |v_k|``; ``s = fl32(a / 127)``; ``q_k = clamp(rint(fl32(v_k / s)), -127,
    127)`` with ties to even (the pages' rounding policy is RNE).  If ``s == 0`` (an
    all-zero row, or a row so small that ``a / 127`` underflows) every code is 0.
    Returns ``(q int8 [M,K], s float32 [M])``.
    """
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("quantize_rows: v must be [M,K]")
    M, K = v.shape
    q = np.zeros((M, K), dtype=np.int8)
    s = np.zeros((M,), dtype=np.float32)
    for m in range(M):
        a = np.max(np.abs(v[m])) if K else F32(0)
        sm = F32(F32(a) / F32(127.0))
        s[m] = sm
        if sm == 0:
            continue
        t = v[m] / sm
        q[m] = np.clip(np.rint(t), -127, 127).astype(np.int8)
    return q, s


def int_gemm(q, w) -> np.ndarray:
    """INT8 x INT8 -> INT32 accumulators ``acc[m,n] = sum_k q[m,k] * w[n,k]``.

    [PR810] What changed > Gate/Up INT8 path (INT8 x INT8 -> INT32 matmuls).  Weights
    are ``[N_out, K_in]`` row-major.  Computed as an FP64 matrix product of the integer
    values, in row blocks: every partial sum is an integer of magnitude below
    128*128*K < 2**53, so the result is exact in any summation order.  Returns int64
    (values are checked to fit INT32).
    """
    q = np.asarray(q)
    w = np.asarray(w)
    if q.ndim != 2 or w.ndim != 2 or q.shape[1] != w.shape[1]:
        raise ValueError("int_gemm: q [M,K] and w [N,K] required")
    M, K = q.shape
    N = w.shape[0]
    if 128 * 128 * K >= 2**53:
        raise ValueError("int_gemm: K too large for exact FP64 accumulation")
    qf = q.astype(np.float64)
    out = np.empty((M, N), dtype=np.float64)
    rows = 512
    buf = np.empty((min(rows, max(N, 1)), K), dtype=np.float64)
    for r0 in range(0, N, rows):
        r1 = min(N, r0 + rows)
        b = buf[: r1 - r0]
        np.copyto(b, w[r0:r1])
        out[:, r0:r1] = qf @ b.T
    acc = out.astype(np.int64)
    if acc.size and np.max(np.abs(acc)) > _INT32_MAX:
        raise OverflowError("int_gemm: accumulator exceeds INT32")
    return acc


def dequant(acc, s_row, s_w) -> np.ndarray:
    """``y[m,n] = fl32(fl32(f(acc[m,n]) * s_row[m]) * s_w[n])``.

    [PR810] What changed > Gate/Up INT8 path: the activation-row and weight-channel
    scales are applied when the INT32 results are dequantized; [PR48] CodeRabbit on
    ``_hf_linear_to_bf16``: a weight scale belongs to an output channel (row n of
    ``[N,K]``), not to the last axis.  Reading: activation scale first, then weight
    scale, in the order the page lists them.
    """
    a = np.asarray(acc, dtype=np.int64).astype(np.float32)
    sr = np.asarray(s_row, dtype=np.float32)
    sw = np.asarray(s_w, dtype=np.float32)
    return (a * sr[:, None]) * sw[None, :]


def exp_f32(x) -> np.ndarray:
    """``exp`` rounded to FP32: evaluated in FP64 and rounded once to FP32 (reading)."""
    with np.errstate(over="ignore"):
        return np.exp(np.asarray(x, dtype=np.float32).astype(np.float64)).astype(np.float32)


def silu_mul(g, u) -> np.ndarray:
    """``h = fl32(silu(g) * u)`` with ``silu(g) = fl32(g / fl32(1 + exp_f32(-g)))``.

    [ISSUE52] Measurement basis names the MLP as gate/up/silu/down; SiLU(gate) times up
    is the gated MLP of the model family.  The pages give no formula; this is the
    textbook SiLU, x * sigmoid(x), written as a division.
    """
    g = np.asarray(g, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    e = exp_f32(-g)
    den = F32(1.0) + e
    return (g / den) * u


def split_k_ranges(K: int, split_k: int) -> list[tuple[int, int]]:
    """Contiguous, equal K partitions ``[j*K/split_k, (j+1)*K/split_k)``.

    [PR810] What changed > Decode scheduling (the Down projection is split two ways
    along K, each part with an accumulator of its own) and the CodeRabbit nitpick (the
    intermediate size has to be a multiple of the number of K splits).
    """
    if split_k < 1 or K % split_k:
        raise ValueError("split_k must divide K")
    c = K // split_k
    return [(j * c, (j + 1) * c) for j in range(split_k)]


def down_split(q_h, s_h, w_d, s_d, split_k: int):
    """Down projection in ``split_k`` independent K partitions.

    [PR810] CodeRabbit walkthrough, "Split down projection accumulation": Down's work
    is divided over K partitions whose results are kept as FP32 partials.  Each partition
    is an exact INT32 sum ``acc_j``, dequantized on its own with the row-global scale
    ``s_h`` (reading: one row scale covers the whole row) into ``p_j``.
    Returns ``(acc list of int64 [M,H], p list of float32 [M,H])``.
    """
    K = np.asarray(w_d).shape[1]
    accs, ps = [], []
    for k0, k1 in split_k_ranges(K, split_k):
        acc = int_gemm(np.asarray(q_h)[:, k0:k1], np.asarray(w_d)[:, k0:k1])
        accs.append(acc)
        ps.append(dequant(acc, s_h, s_d))
    return accs, ps


def reduce_residual_bf16(ps, res_bits) -> np.ndarray:
    """``out = rne_bf16(fl32(fl32(p_0 + p_1 + ...) + f(res)))``, partials summed in index order.

    [PR810] CodeRabbit walkthrough: the FP32 partials are summed, the residual is
    added, and the result is narrowed to BF16 by RNE ([PR810] Validation).
    """
    tot = np.asarray(ps[0], dtype=np.float32)
    for p in ps[1:]:
        tot = tot + np.asarray(p, dtype=np.float32)
    return rne_bf16(tot + bf16_to_f32(res_bits))


# ----------------------------------------------------------------------------- blocks

def linear_decode(q, s_row, w, s_w, residual_bits=None):
    """One A8W8 linear on quantized input: INT32 GEMM, dequant, optional BF16 residual, RNE.

    ``y = rne_bf16(dequant(acc))`` or ``rne_bf16(fl32(dequant(acc) + f(res)))``.
    Returns ``(y uint16 [M,N], acc int64 [M,N])``.
    """
    acc = int_gemm(q, w)
    y = dequant(acc, s_row, s_w)
    if residual_bits is not None:
        y = y + bf16_to_f32(residual_bits)
    return rne_bf16(y), acc


def mlp_block_decode(x_bits, gamma_bits, eps, w_g, s_g, w_u, s_u, w_d, s_d, res_bits,
                     split_k: int = 2):
    """The A8W8 decode MLP block, every stage returned for stage-wise comparison.

    RMSNorm -> per-row INT8 quant -> Gate/Up INT32 GEMMs -> dequant -> SiLU(g)*u ->
    per-row requant of h over the full intermediate row (reading: the Down projection
    runs on INT8 codes; the pages only state Gate/Up are INT8) -> split-K Down ->
    partials + residual -> RNE BF16.
    """
    xn = rmsnorm(x_bits, gamma_bits, eps)
    q_x, s_x = quantize_rows(xn)
    acc_g = int_gemm(q_x, w_g)
    acc_u = int_gemm(q_x, w_u)
    g = dequant(acc_g, s_x, s_g)
    u = dequant(acc_u, s_x, s_u)
    h = silu_mul(g, u)
    q_h, s_h = quantize_rows(h)
    acc_d, p_d = down_split(q_h, s_h, w_d, s_d, split_k)
    out = reduce_residual_bf16(p_d, res_bits)
    return out, dict(xn=xn, q_x=q_x, s_x=s_x, acc_g=acc_g, acc_u=acc_u, g=g, u=u, h=h,
                     q_h=q_h, s_h=s_h, acc_down=acc_d, p_down=p_d, out=out)


def layer_linears_decode(x_bits, gamma_in_bits, gamma_post_bits, eps, w_qkv, s_qkv, w_o,
                         s_o, w_g, s_g, w_u, s_u, w_d, s_d, n_q_heads: int,
                         head_dim: int, split_k: int = 2):
    """All linears of one decode layer with attention replaced by identity.

    Readings (the pages only say the decode layer is A8W8 with INT8 weights and
    activation/weight scales): pre-norm layer, input RMSNorm before QKV;
    ``attn = qkv[:, :n_q_heads*head_dim]`` (the Q slice, BF16); O output plus the layer
    input as residual, ``h1 = rne_bf16(fl32(y_o + f(x)))``; then the MLP block with
    ``x = res = h1``.  Each projection quantizes its input rows dynamically.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    xn_in = rmsnorm(x_bits, gamma_in_bits, eps)
    q_in, s_in = quantize_rows(xn_in)
    acc_qkv = int_gemm(q_in, w_qkv)
    qkv = rne_bf16(dequant(acc_qkv, s_in, s_qkv))
    attn = qkv[:, : n_q_heads * head_dim]
    q_a, s_a = quantize_rows(bf16_to_f32(attn))
    acc_o = int_gemm(q_a, w_o)
    h1 = rne_bf16(dequant(acc_o, s_a, s_o) + bf16_to_f32(x_bits))
    out, mlp = mlp_block_decode(h1, gamma_post_bits, eps, w_g, s_g, w_u, s_u, w_d, s_d, h1,
                                split_k)
    st = dict(xn_in=xn_in, q_in=q_in, s_in=s_in, acc_qkv=acc_qkv, qkv=qkv, q_attn=q_a,
              s_attn=s_a, acc_o=acc_o, h1=h1)
    st.update({"mlp_" + k: v for k, v in mlp.items()})
    st["out"] = out
    return out, st


# ----------------------------------------------------------------------------- prefill

def dequant_weight_bf16(w, s) -> np.ndarray:
    """``W'[n,k] = rne_bf16(fl32(f(w[n,k]) * s[n]))`` (uint16 bits).

    [PR810] What changed > Gate/Up INT8 path.  The prefill GEMMs read the same INT8
    weights as decode; each weight becomes a BF16 value on the way in: the weight times
    its channel scale as one FP32 product, then rounded to BF16 with ties to even.
    Both roundings belong to the definition.
    """
    wf = np.asarray(w, dtype=np.int8).astype(np.float32)
    return rne_bf16(wf * np.asarray(s, dtype=np.float32)[:, None])


def _bf16_matmul_f64_to_f32(a_bits, w_bits) -> np.ndarray:
    """``fl32(sum_k f(a[m,k]) * f(w[n,k]))`` accumulated in FP64, rounded once to FP32."""
    a = bf16_to_f32(a_bits).astype(np.float64)
    wb = np.asarray(w_bits, dtype=np.uint16)
    N, K = wb.shape
    out = np.empty((a.shape[0], N), dtype=np.float64)
    rows = 512
    for r0 in range(0, N, rows):
        r1 = min(N, r0 + rows)
        out[:, r0:r1] = a @ bf16_to_f32(wb[r0:r1]).astype(np.float64).T
    return out.astype(np.float32)


def prefill_mlp(x_bits, gamma_bits, eps, w_g, s_g, w_u, s_u, w_d, s_d, res_bits):
    """W8A16 prefill MLP on the shared INT8 weights.

    ``a = rne_bf16(RMSNorm(x))``; ``g, u`` = BF16 products accumulated in FP64 and
    rounded once to FP32; ``h = rne_bf16(silu(g) * u)``; ``d`` likewise from ``h`` and
    ``W'_d``; ``out = rne_bf16(fl32(d + f(res)))``.  No split-K here: the sum is one
    FP64 accumulation (the GPU may split it; its FP32 accumulation is compared within
    an error bound).
    """
    xn = rmsnorm(x_bits, gamma_bits, eps)
    a = rne_bf16(xn)
    wg = dequant_weight_bf16(w_g, s_g)
    wu = dequant_weight_bf16(w_u, s_u)
    wd = dequant_weight_bf16(w_d, s_d)
    g = _bf16_matmul_f64_to_f32(a, wg)
    u = _bf16_matmul_f64_to_f32(a, wu)
    h = rne_bf16(silu_mul(g, u))
    d = _bf16_matmul_f64_to_f32(h, wd)
    out = rne_bf16(d + bf16_to_f32(res_bits))
    return out, dict(xn=xn, a=a, g=g, u=u, h=h, d=d, out=out)


def prefill_linear(a_bits, w, s, residual_bits=None):
    """One W8A16 linear: ``y = rne_bf16(fl32(sum_k f(a) * f(W')) [+ f(res)])``.

    ``W' = dequant_weight_bf16(w, s)``; the dot products are accumulated in FP64 and
    rounded once to FP32, the residual (when given) is one FP32 add, and the result is
    narrowed with RNE ([PR810] What changed > Gate/Up INT8 path: prefill reads the INT8
    weights that decode uses, turned into BF16 tile by tile; the Gemini review: narrowing with
    ``mode="rint"``).
    """
    y = _bf16_matmul_f64_to_f32(a_bits, dequant_weight_bf16(w, s))
    if residual_bits is not None:
        y = y + bf16_to_f32(residual_bits)
    return rne_bf16(y)


def layer_linears_prefill(x_bits, gamma_in_bits, gamma_post_bits, eps, w_qkv, s_qkv, w_o,
                          s_o, w_g, s_g, w_u, s_u, w_d, s_d, n_q_heads: int, head_dim: int):
    """All linears of one prefill layer, W8A16, attention replaced by identity.

    The decode layer's readings (``layer_linears_decode``) with the prefill linear in place
    of the A8W8 one: ``a = rne_bf16(RMSNorm(x, gamma_in))``;
    ``qkv = prefill_linear(a, W_qkv)``; ``attn = qkv[:, :n_q_heads*head_dim]`` (the Q
    slice, already BF16, so it is the next operand as it stands);
    ``h1 = prefill_linear(attn, W_o, residual=x)``; then ``prefill_mlp`` with
    ``x = res = h1``.  The pages name prefill on the shared INT8 weights ([PR810] What
    changed > Gate/Up INT8 path) and a prefill hidden-state path in the serving PR; the
    layer composition is a reading of those passages.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    xn_in = rmsnorm(x_bits, gamma_in_bits, eps)
    a = rne_bf16(xn_in)
    qkv = prefill_linear(a, w_qkv, s_qkv)
    attn = qkv[:, : n_q_heads * head_dim]
    h1 = prefill_linear(attn, w_o, s_o, residual_bits=x_bits)
    out, mlp = prefill_mlp(h1, gamma_post_bits, eps, w_g, s_g, w_u, s_u, w_d, s_d, h1)
    st = dict(xn_in=xn_in, a=a, qkv=qkv, h1=h1)
    st.update({"mlp_" + k: v for k, v in mlp.items()})
    st["out"] = out
    return out, st


# ------------------------------------------------------------- QK-norm, RoPE, KV write

def rope_rotate_half(x, cos, sin) -> np.ndarray:
    """Rotary position embedding, rotate-half form, on FP32 vectors ``x [..., d]`` with
    ``cos, sin [..., d/2]`` (broadcast): for ``i < d/2``,
    ``o[i] = fl32(fl32(x[i]*c[i]) - fl32(x[i+d/2]*s[i]))`` and
    ``o[i+d/2] = fl32(fl32(x[i+d/2]*c[i]) + fl32(x[i]*s[i]))``.

    The pages name RoPE on Q and K before the BF16 KV-cache write ([ISSUE52] Current
    behavior: the fused QK-norm path and its Q RoPE; [PR810] walkthrough, BF16 cache and
    interface contracts: RoPE writes use BF16 KV caches) but not its form; rotate-half is
    the Qwen3 family's, and the angle tables are inputs (both sides read the same values).
    """
    x = np.asarray(x, dtype=F32)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=F32)
    s_ = np.asarray(sin, dtype=F32)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s_, x2 * c + x1 * s_], axis=-1).astype(F32)


def qk_norm_rope_kv(qkv_bits, n_q_heads: int, n_kv_heads: int, head_dim: int, q_gamma_bits,
                    k_gamma_bits, eps, cos_table, sin_table, positions, block_table,
                    k_cache_bits, v_cache_bits):
    """QK-norm, RoPE and the BF16 KV-cache write that follow the QKV projection.

    ``qkv [M, (n_q + 2 n_kv) * d]`` holds the Q heads, then the K heads, then the V heads.
    Per row ``m`` at position ``p = positions[m]``:
    * each Q head ``q = rne_bf16(rope(RMSNorm_d(q, q_gamma), cos[p], sin[p]))`` (the
      attention input);
    * each K head likewise with ``k_gamma``, written to the cache slot of position ``p``;
    * each V head copied to the same slot of the V cache.
    RMSNorm over one head is ``rmsnorm`` above on a row of ``d`` values.  The cache is
    paged: ``cache[b, o, h, :]`` with ``b = block_table[m, p // block_size]``,
    ``o = p % block_size`` ([PR48] runner: paged KV cache with a block table and bounds
    validated before dispatch).  Readings: QK-norm gains shared by the heads of each kind
    (one ``[d]`` vector each) and the paged layout ``[blocks, block_size, n_kv, d]``.
    Returns the Q output and new copies of the two caches.
    """
    qkv = np.asarray(qkv_bits, dtype=np.uint16)
    M = qkv.shape[0]
    d = head_dim
    kc = np.array(k_cache_bits, dtype=np.uint16, copy=True)
    vc = np.array(v_cache_bits, dtype=np.uint16, copy=True)
    bs = kc.shape[1]
    q_out = np.empty((M, n_q_heads * d), dtype=np.uint16)
    for m in range(M):
        p = int(positions[m])
        c, s_ = cos_table[p], sin_table[p]
        for h in range(n_q_heads):
            v = qkv[m : m + 1, h * d : (h + 1) * d]
            q_out[m, h * d : (h + 1) * d] = rne_bf16(rope_rotate_half(rmsnorm(v, q_gamma_bits, eps), c, s_))[0]
        b = int(block_table[m, p // bs])
        o = p % bs
        for h in range(n_kv_heads):
            k0 = (n_q_heads + h) * d
            v0 = (n_q_heads + n_kv_heads + h) * d
            kv = qkv[m : m + 1, k0 : k0 + d]
            kc[b, o, h] = rne_bf16(rope_rotate_half(rmsnorm(kv, k_gamma_bits, eps), c, s_))[0]
            vc[b, o, h] = qkv[m, v0 : v0 + d]
    return q_out, kc, vc


# ------------------------------------------------------------------ decode attention

def decode_attention(q_bits, n_q_heads: int, n_kv_heads: int, head_dim: int, k_cache_bits,
                     v_cache_bits, block_table, context_lens, scale):
    """Decode attention over the paged BF16 KV cache, defined exactly (FP64), then RNE.

    Row ``m`` attends to its positions ``0 .. L-1`` (``L = context_lens[m]``), read from
    the cache slots ``(block_table[m, j // block_size], j % block_size)``.  Q head ``h``
    uses KV head ``h // (n_q / n_kv)`` (grouped-query attention; consecutive Q heads share
    a KV head).  ``o = sum_j softmax_j(scale * q . k_j) v_j`` over exact real numbers
    (FP64 here), and the output is ``rne_bf16(o)``.  The pages place attention over a BF16
    KV cache between QKV and O ([PR810] walkthrough: attention loads use BF16 KV caches;
    [PR48] runner: paged KV cache with a block table) but give none of its arithmetic;
    this is the plain definition, and a GPU computing it in FP32 is held to the stated
    BF16 output tolerance.  A position whose block number lies outside ``[0, num_blocks)``
    is left out of the softmax (the library's stated behaviour for a hole in the block
    table); a row with no position left gets zeros.
    """
    q = bf16_to_f32(np.asarray(q_bits, dtype=np.uint16)).astype(np.float64)
    kc = bf16_to_f32(np.asarray(k_cache_bits, dtype=np.uint16)).astype(np.float64)
    vc = bf16_to_f32(np.asarray(v_cache_bits, dtype=np.uint16)).astype(np.float64)
    M = q.shape[0]
    d = head_dim
    bs = kc.shape[1]
    group = n_q_heads // n_kv_heads
    out = np.empty((M, n_q_heads * d), dtype=np.uint16)
    for m in range(M):
        L = int(context_lens[m])
        j = np.arange(L)
        blocks = np.asarray(block_table[m], dtype=np.int64)[j // bs]
        keep = (blocks >= 0) & (blocks < kc.shape[0])
        j, blocks = j[keep], blocks[keep]
        for h in range(n_q_heads):
            if j.size == 0:
                out[m, h * d : (h + 1) * d] = 0
                continue
            g = h // group
            k = kc[blocks, j % bs, g]                     # [L, d]
            v = vc[blocks, j % bs, g]
            s_ = float(scale) * (k @ q[m, h * d : (h + 1) * d])
            w = np.exp(s_ - s_.max())
            o = (w / w.sum()) @ v
            out[m, h * d : (h + 1) * d] = rne_bf16(o.astype(np.float32))
    return out


# ------------------------------------------------------------ decode layer, real attention

def o_projection(attn_bits, x_bits, w_o, s_o) -> np.ndarray:
    """O on the attention output with the layer input as residual, as in
    ``layer_linears_decode``: each attention row gets INT8 codes and one scale, is multiplied
    in INT32 and dequantized, and ``h1 = rne_bf16(fl32(y_o + f(x)))``."""
    q_a, s_a = quantize_rows(bf16_to_f32(np.asarray(attn_bits, dtype=np.uint16)))
    acc_o = int_gemm(q_a, w_o)
    return rne_bf16(dequant(acc_o, s_a, s_o) + bf16_to_f32(np.asarray(x_bits, dtype=np.uint16)))


def decode_layer(x_bits, gamma_in_bits, gamma_post_bits, eps, w_qkv, s_qkv, w_o, s_o, w_g,
                 s_g, w_u, s_u, w_d, s_d, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 split_k, q_gamma_bits, k_gamma_bits, qk_eps, cos_table, sin_table,
                 positions, context_lens, block_table, k_cache_bits, v_cache_bits, scale):
    """One decode layer with real attention, in the layer order the pages give ([PR810]
    walkthrough: QKV, QK-norm/RoPE, the BF16 KV cache and attention, O, the post-attention
    norm and the MLP): QKV as in ``layer_linears_decode``; ``qk_norm_rope_kv`` writes the
    new token's K and V to the cache and rotates Q; ``decode_attention`` over the updated
    cache; ``o_projection`` (+ x) gives h1; ``mlp_block_decode`` on h1.  Returns the
    output and the stages (qkv, q_rot, the two caches, attn, h1)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    q_in, s_in = quantize_rows(rmsnorm(x_bits, gamma_in_bits, eps))
    qkv = rne_bf16(dequant(int_gemm(q_in, w_qkv), s_in, s_qkv))
    q_rot, kc, vc = qk_norm_rope_kv(qkv, n_q_heads, n_kv_heads, head_dim, q_gamma_bits,
                                    k_gamma_bits, qk_eps, cos_table, sin_table, positions,
                                    block_table, k_cache_bits, v_cache_bits)
    attn = decode_attention(q_rot, n_q_heads, n_kv_heads, head_dim, kc, vc, block_table,
                            context_lens, scale)
    h1 = o_projection(attn, x_bits, w_o, s_o)
    out, _ = mlp_block_decode(h1, gamma_post_bits, eps, w_g, s_g, w_u, s_u, w_d, s_d, h1,
                              split_k)
    return out, dict(qkv=qkv, q_rot=q_rot, k_cache=kc, v_cache=vc, attn=attn, h1=h1)
