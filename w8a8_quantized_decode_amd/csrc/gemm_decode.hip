// Decode-batch INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, with fused activation
// quantization (prologue) and fused dequant / SiLU / residual / split-K epilogues.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path (INT8 x INT8 -> INT32 Gate/Up matmuls, the
// activation-row and weight-channel scales applied at dequantization, the
// post-attention RMSNorm output quantized once per row) and > Decode scheduling (Down
// split two ways along K with independent accumulators), plus the CodeRabbit
// walkthrough row on the split Down projection (FP32 partials summed and narrowed
// together with the residual).  QKV and O reuse the same pattern.
//
// Shape of the work.  At decode batch sizes the weights dominate the traffic, so the
// kernel is a weight stream: every weight byte is read from HBM exactly once.
//   * A 16-channel output tile is computed with v_mfma_i32_16x16x64_i8: the weights are
//     the A operand (16 channels x 64 k), the activation codes the B operand (64 k x 16
//     rows of M; rows beyond the batch are zeros).  Lane l feeds channel l%16 with the
//     16 bytes at k-offset 16*(l/16) of the 64-byte step; its result holds channels
//     4*(l/16)+r (r = 0..3) of row l%16.
//   * Weights in the tiled layout store each such 1 KB operand block contiguously, so a
//     wave's load instruction reads 1 KB of consecutive bytes and a wave's K range is
//     one contiguous run; the row-major layout is also accepted (64 bytes from each of
//     16 rows per load, measurably slower on HBM).
//   * A workgroup owns one tile and one K range; its waves split the range, keep U
//     steps of weight loads in flight (double-buffered in registers), and meet in LDS
//     with exact INT32 sums.
//   * When a tile's K is spread over several workgroups (ranges > 1) the partial sums
//     go to a device-scope INT32 accumulator with atomic adds; the last workgroup to
//     arrive (per-tile counter) reads the sums and runs the epilogue.  Integer addition
//     is exact, so the result is the same bit for bit in any arrival order.  These
//     accumulators are zeroed by an earlier kernel of the same call.
//   * Fused prologues: each workgroup re-derives the row statistics (RMSNorm sum of
//     squares, absolute maximum) from the whole input row and quantizes only its own K
//     range into LDS.  The weight loads of the first batch are issued before the
//     prologue so HBM stays busy while it runs.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 ld16(const int8_t* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// Dequantized value: fl32(fl32(f(acc) * sa) * sw).
__device__ __forceinline__ float dq(int32_t acc, float sa, float sw) {
  return (static_cast<float>(acc) * sa) * sw;
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)), exp evaluated in FP64 and rounded once.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = static_cast<float>(exp(-static_cast<double>(g)));
  const float den = 1.0f + e;
  return (g / den) * u;
}

// Workgroup reductions: each wave reduces, lane 0 posts to its slot, and after one
// barrier every thread combines the slots in wave order (same bits in every thread).
template <int NW>
__device__ __forceinline__ double block_sum_f64(double v, double* slots) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += slots[w];
  return s;
}

template <int NW>
__device__ __forceinline__ float block_max_f32(float v, float* slots) {
  v = wave_max_f32(v);
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s = fmaxf(s, slots[w]);
  return s;
}

__device__ __forceinline__ void load8_bf16(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ void load8_f32(const float* p, float (&v)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

__device__ __forceinline__ u32x2 codes8(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t(quant_code(v[i], s)) & 0xFFu) << (8 * i);
      hi |= (uint32_t(quant_code(v[4 + i], s)) & 0xFFu) << (8 * i);
    }
  }
  return u32x2{lo, hi};
}

// Shared scratch of one workgroup (besides the dynamic activation buffer).
template <int NW, int NMAT, int MB>
struct Smem {
  i32x4 red[NW][NMAT][MB][kWave];
  double sum_slots[kFuseMaxRows][NW];
  float max_slots[kFuseMaxRows][NW];
  float row_scale[kFuseMaxRows];
  int last;
};

// Fused prologue: codes of this workgroup's K steps for every row, into LDS act[m][.].
// The local step index ls = part * ns + (t - rs0) addresses 64-byte groups.
template <int NW, int PRO, typename SM>
__device__ void fused_prologue(const DecodeGemmArgs& p, SM& sm, int8_t* act, int act_ld,
                               int P, int64_t Kp, int rs0, int ns, bool write_taps) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
  const int nloc = P * ns * 64;
  for (int m = 0; m < p.M; ++m) {
    float s;
    float r = 1.0f;
    if constexpr (PRO == PRO_QUANT_BF16) {
      const uint16_t* xr = p.x + int64_t(m) * p.ldx;
      if (p.gamma) {
        double ss = 0.0;
        for (int64_t k = int64_t(tid) * 8; k < p.K; k += NT * 8) {
          float v[8];
          load8_bf16(xr + k, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) ss += double(v[i]) * double(v[i]);
        }
        const double S = block_sum_f64<NW>(ss, sm.sum_slots[m]);
        const float ms = static_cast<float>(S / static_cast<double>(p.K));
        const float t = ms + p.eps;
        const float sq = __builtin_sqrtf(t);
        r = 1.0f / sq;
      }
      float amax = 0.0f;
      for (int64_t k = int64_t(tid) * 8; k < p.K; k += NT * 8) {
        float v[8];
        load8_bf16(xr + k, v);
        if (p.gamma) {
          float g[8];
          load8_bf16(p.gamma + k, g);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (v[i] * r) * g[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
      amax = block_max_f32<NW>(amax, sm.max_slots[m]);
      s = amax / 127.0f;
    } else {  // PRO_REQUANT_F32: the row maximum comes from per-tile partial maxima
      float amax = 0.0f;
      for (int i = tid; i < p.npmax; i += NT) amax = fmaxf(amax, p.pmax[int64_t(i) * p.M + m]);
      amax = block_max_f32<NW>(amax, sm.max_slots[m]);
      s = amax / 127.0f;
    }
    if (tid == 0) {
      sm.row_scale[m] = s;
      if (write_taps && p.tap_s) p.tap_s[m] = s;
    }
    for (int e = tid * 8; e < nloc; e += NT * 8) {
      const int ls = e >> 6, off = e & 63;
      const int pp = ls / ns, tt = rs0 + ls % ns;
      const int64_t k = int64_t(pp) * Kp + int64_t(tt) * 64 + off;
      float v[8];
      if constexpr (PRO == PRO_QUANT_BF16) {
        load8_bf16(p.x + int64_t(m) * p.ldx + k, v);
        if (p.gamma) {
          float g[8];
          load8_bf16(p.gamma + k, g);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (v[i] * r) * g[i];
        }
      } else {
        load8_f32(p.hin + int64_t(m) * p.ldhin + k, v);
      }
      const u32x2 c = codes8(v, s);
      *reinterpret_cast<u32x2*>(act + m * act_ld + e) = c;
      if (write_taps) {
        if (p.tap_q) *reinterpret_cast<u32x2*>(p.tap_q + int64_t(m) * p.K + k) = c;
        if (p.tap_xn) {
          f32x4* t = reinterpret_cast<f32x4*>(p.tap_xn + int64_t(m) * p.K + k);
          t[0] = f32x4{v[0], v[1], v[2], v[3]};
          t[1] = f32x4{v[4], v[5], v[6], v[7]};
        }
      }
    }
  }
  __syncthreads();
}

// EPI: epilogue, NMAT: weights per tile (2 for Gate/Up), NW: waves per workgroup,
// MB: 16-row blocks of M (1 with a fused prologue), P: K partitions (EPI_DOWN),
// LAYOUT: weight layout, PRO: prologue.
template <int EPI, int NMAT, int NW, int MB, int P, int LAYOUT, int PRO>
__global__ __launch_bounds__(NW * kWave) void decode_gemm_kernel(DecodeGemmArgs p) {
  constexpr int NSETS = (EPI == EPI_DOWN) ? P : NMAT;
  constexpr int wpp = NW / P;                 // waves per partition
  constexpr bool kFused = PRO != PRO_CODES;
  constexpr int U = 8 / NMAT;                 // k steps per load batch
  __shared__ Smem<NW, NMAT, MB> sm;
  extern __shared__ __align__(16) int8_t act[];

  const int tid = threadIdx.x;
  // The wave index lives in a scalar register so that every loop bound below is
  // wave-uniform: the MFMA guards must be real branches, since a matrix instruction
  // does not honour a partial lane mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int row16 = lane & 15, kg = lane >> 4;
  const int R = p.ranges;
  const int tile = blockIdx.x / R, r = blockIdx.x % R;
  const int mg = blockIdx.y;
  const int64_t n0 = int64_t(tile) * 16;
  const int64_t m0 = int64_t(mg) * MB * 16;
  const int part = wave / wpp, wl = wave % wpp;
  const int64_t Kp = p.K / P;                 // bytes per partition
  const int Sp = static_cast<int>(Kp / 64);   // steps per partition
  const int rs0 = static_cast<int>(int64_t(r) * Sp / R);
  const int rs1 = static_cast<int>(int64_t(r + 1) * Sp / R);
  const int ns = rs1 - rs0;
  const int ws0 = rs0 + ns * wl / wpp, ws1 = rs0 + ns * (wl + 1) / wpp;
  const int act_ld = P * ((Sp + R - 1) / R) * 64;

  // Weight operand addresses (step t is a step within this wave's partition).
  const int8_t* wbase[NMAT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i) {
    const int8_t* w = (i == 0) ? p.w0 : p.w1;
    if (LAYOUT == LAYOUT_TILED)
      wbase[i] = w + int64_t(tile) * 16 * p.K + int64_t(part) * Sp * 1024 + lane * 16;
    else
      wbase[i] = w + (n0 + row16) * p.K + int64_t(part) * Kp + kg * 16;
  }
  constexpr int64_t kStep = (LAYOUT == LAYOUT_TILED) ? 1024 : 64;

  // Activation operand (B) sources.
  const int8_t* abase[MB];
  bool aval[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + mb * 16 + row16;
    aval[mb] = m < p.M;
    // Lanes of rows beyond the batch read row 0 (in bounds) and feed zeros instead.
    abase[mb] = kFused ? act + (aval[mb] ? row16 : 0) * act_ld + (part * ns - rs0) * 64 + kg * 16
                       : p.a + (aval[mb] ? m : 0) * p.lda + int64_t(part) * Kp + kg * 16;
  }

  i32x4 acc[NMAT][MB];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[i][mb] = i32x4{0, 0, 0, 0};

  // Batches of U steps, ping-ponged between two register sets so that the next batch
  // is in flight while the current one feeds the matrix cores.  Loads are issued
  // unconditionally (steps past the wave's range re-read its last step, an L2 hit) and
  // the activation operand of those steps is zero, so the loop has no data-dependent
  // branches and the compiler can wait for exactly the batch it consumes.
  const int nsteps = ws1 - ws0;
  const int nb = (nsteps + U - 1) / U;
  auto load_batch = [&](i32x4 (&wv)[U][NMAT], i32x4 (&bv)[U][MB], int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = min(t + u, ws1 - 1);
#pragma unroll
      for (int i = 0; i < NMAT; ++i) wv[u][i] = ld16(wbase[i] + int64_t(tt) * kStep);
      if (!kFused) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) bv[u][mb] = ld16(abase[mb] + int64_t(tt) * 64);
      }
    }
  };
  auto compute = [&](const i32x4 (&wv)[U][NMAT], const i32x4 (&bv)[U][MB], int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = t + u < ws1;
      const int tt = min(t + u, ws1 - 1);
      i32x4 b[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 v = kFused ? *reinterpret_cast<const i32x4*>(abase[mb] + tt * 64) : bv[u][mb];
        b[mb] = (live && aval[mb]) ? v : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma_i8(wv[u][i], b[mb], acc[i][mb]);
    }
  };

  i32x4 wA[U][NMAT], bA[U][MB], wB[U][NMAT], bB[U][MB];
  if (nb > 0) load_batch(wA, bA, ws0);

  // Zero the accumulators of the call's later kernels (grid-stride, 16 bytes a store).
  if (p.zero_ptr) {
    const int64_t nwg = int64_t(gridDim.x) * gridDim.y;
    const int64_t wg = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t n16 = int64_t(p.zero_bytes / 16);
    u32x4* z = static_cast<u32x4*>(p.zero_ptr);
    for (int64_t i = wg * (NW * kWave) + tid; i < n16; i += nwg * (NW * kWave))
      z[i] = u32x4{0u, 0u, 0u, 0u};
  }

  if (kFused)
    fused_prologue<NW, PRO>(p, sm, act, act_ld, P, Kp, rs0, ns, tile == 0);

  for (int bi = 0; bi < nb; bi += 2) {
    const int t = ws0 + bi * U;
    load_batch(wB, bB, t + U);
    compute(wA, bA, t);
    if (bi + 1 >= nb) break;
    load_batch(wA, bA, t + 2 * U);
    compute(wB, bB, t + U);
  }

#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sm.red[wave][i][mb][lane] = acc[i][mb];
  __syncthreads();

  // One epilogue thread per (16-row block, lane): it owns 4 channels of one row.
  const bool active = tid < MB * kWave;
  const int emb = tid / kWave, eln = tid & (kWave - 1);
  const int64_t em = m0 + emb * 16 + (eln & 15);
  const int64_t en = n0 + 4 * (eln >> 4);
  const bool mval = active && em < p.M;

  i32x4 sum[NSETS];
#pragma unroll
  for (int s = 0; s < NSETS; ++s) sum[s] = i32x4{0, 0, 0, 0};
  if (active) {
    if constexpr (EPI == EPI_DOWN) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int w = s * wpp; w < (s + 1) * wpp; ++w) sum[s] += sm.red[w][0][emb][eln];
    } else {
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int w = 0; w < NW; ++w) sum[i] += sm.red[w][i][emb][eln];
    }
  }

  if (R > 1) {
    // Cross-workgroup INT32 reduction.  Accumulator layout [set][M][N].
    const int64_t MN = p.M * p.N;
    int32_t seen = 0;
    if (mval) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        int32_t* base = p.wacc + s * MN + em * p.N + en;
#pragma unroll
        for (int c = 0; c < 4; ++c) seen |= atomic_add_dev(base + c, sum[s][c]);
      }
    }
    // Using the returned values forces every add to complete before the barrier.
    if (seen == 0x7FFFFFFF) sm.last = 2;
    __syncthreads();
    if (tid == 0) {
      int32_t* cnt = p.wcnt + int64_t(mg) * (p.N / 16) + tile;
      sm.last = (atomic_add_dev(cnt, 1) == R - 1) ? 1 : 0;
    }
    __syncthreads();
    if (sm.last != 1) return;
    if (mval) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        int32_t* base = p.wacc + s * MN + em * p.N + en;
#pragma unroll
        for (int c = 0; c < 4; ++c) sum[s][c] = atomic_take(base + c);
      }
    }
  }

  float sa = 0.0f;
  if (mval) sa = kFused ? sm.row_scale[em] : p.sa[em];

  if constexpr (EPI == EPI_BF16 || EPI == EPI_BF16_RES) {
    if (!mval) return;
    if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = sum[0];
    float y[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = dq(sum[0][c], sa, p.sw0[en + c]);
    if constexpr (EPI == EPI_BF16_RES) {
      const u32x2 rr = *reinterpret_cast<const u32x2*>(p.res + em * p.ldr + en);
      y[0] = y[0] + bf16_lo(rr[0]);
      y[1] = y[1] + bf16_hi(rr[0]);
      y[2] = y[2] + bf16_lo(rr[1]);
      y[3] = y[3] + bf16_hi(rr[1]);
    }
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(y[0])) | (uint32_t(f32_to_bf16_rne(y[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(y[2])) | (uint32_t(f32_to_bf16_rne(y[3])) << 16);
    *reinterpret_cast<u32x2*>(p.out + em * p.ldo + en) = o;
  } else if constexpr (EPI == EPI_SILU) {
    f32x4 h = {0.f, 0.f, 0.f, 0.f};
    if (mval) {
      if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = sum[0];
      if (p.tap_acc1) *reinterpret_cast<i32x4*>(p.tap_acc1 + em * p.N + en) = sum[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float g = dq(sum[0][c], sa, p.sw0[en + c]);
        const float u = dq(sum[1][c], sa, p.sw1[en + c]);
        h[c] = silu_mul(g, u);
      }
      *reinterpret_cast<f32x4*>(p.h + em * p.ldh + en) = h;
      if (p.tap_h) *reinterpret_cast<f32x4*>(p.tap_h + em * p.N + en) = h;
    }
    if (p.pmax_out && active) {
      // Absolute maximum of the tile's 16 channels of row em: the four lanes that
      // share eln % 16 hold them.
      float mx = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if (mval && (eln >> 4) == 0) p.pmax_out[int64_t(tile) * p.M + em] = mx;
    }
  } else {  // EPI_DOWN
    if (!mval) return;
    const int64_t MN = p.M * p.N;
    float tot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + s * MN + em * p.N + en) = sum[s];
      f32x4 pv;
#pragma unroll
      for (int c = 0; c < 4; ++c) pv[c] = dq(sum[s][c], sa, p.sw0[en + c]);
      if (p.tap_p) *reinterpret_cast<f32x4*>(p.tap_p + s * MN + em * p.N + en) = pv;
#pragma unroll
      for (int c = 0; c < 4; ++c) tot[c] = (s == 0) ? pv[c] : tot[c] + pv[c];
    }
    const u32x2 rr = *reinterpret_cast<const u32x2*>(p.res + em * p.ldr + en);
    tot[0] = tot[0] + bf16_lo(rr[0]);
    tot[1] = tot[1] + bf16_hi(rr[0]);
    tot[2] = tot[2] + bf16_lo(rr[1]);
    tot[3] = tot[3] + bf16_hi(rr[1]);
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(tot[0])) | (uint32_t(f32_to_bf16_rne(tot[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(tot[2])) | (uint32_t(f32_to_bf16_rne(tot[3])) << 16);
    *reinterpret_cast<u32x2*>(p.out + em * p.ldo + en) = o;
  }
}

// Tiled-layout packing: one thread moves one 16-byte operand chunk.
__global__ __launch_bounds__(256) void pack_tiled_kernel(const int8_t* w, int64_t N, int64_t K,
                                                         int8_t* out) {
  const int64_t chunks = N * K / 16;
  const int64_t per_tile = K;  // 16 rows * K bytes / 16 bytes per chunk
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += int64_t(gridDim.x) * blockDim.x) {
    const int64_t tile = c / per_tile, rem = c % per_tile;
    const int64_t t = rem / 64, l = rem % 64;
    const int64_t row = tile * 16 + (l & 15);
    const int64_t k = t * 64 + (l >> 4) * 16;
    *reinterpret_cast<i32x4*>(out + c * 16) = ld16(w + row * K + k);
  }
}

constexpr int kWavesDefault = 4;
// Resident workgroups targeted when K is spread over workgroups: 256 CUs x 5.
constexpr int kTargetWorkgroups = 1280;

int waves_for(int epi, int parts) { return (epi == EPI_DOWN && parts == 8) ? 8 : kWavesDefault; }

template <int EPI, int NMAT, int NW, int MB, int P, int PRO>
hipError_t launch_layout(const DecodeGemmArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const dim3 block(NW * kWave);
  if (a.layout == LAYOUT_TILED)
    hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, MB, P, LAYOUT_TILED, PRO>), grid, block,
                       lds, s, a);
  else
    hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, MB, P, LAYOUT_ROWMAJOR, PRO>), grid,
                       block, lds, s, a);
  return hipGetLastError();
}

template <int EPI, int NMAT, int NW, int P>
hipError_t launch_codes(const DecodeGemmArgs& a, int mb, dim3 grid, hipStream_t s) {
  switch (mb) {
    case 1: return launch_layout<EPI, NMAT, NW, 1, P, PRO_CODES>(a, grid, 0, s);
    case 2: return launch_layout<EPI, NMAT, NW, 2, P, PRO_CODES>(a, grid, 0, s);
    case 3: return launch_layout<EPI, NMAT, NW, 3, P, PRO_CODES>(a, grid, 0, s);
    default: return launch_layout<EPI, NMAT, NW, 4, P, PRO_CODES>(a, grid, 0, s);
  }
}

template <int P>
hipError_t launch_down(const DecodeGemmArgs& a, int mb, dim3 grid, size_t lds, hipStream_t s) {
  constexpr int NW = (P == 8) ? 8 : kWavesDefault;
  if (a.prologue == PRO_REQUANT_F32)
    return launch_layout<EPI_DOWN, 1, NW, 1, P, PRO_REQUANT_F32>(a, grid, lds, s);
  return launch_codes<EPI_DOWN, 1, NW, P>(a, mb, grid, s);
}

}  // namespace

DecodeGemmPlan plan_decode_gemm(int epi, int64_t M, int64_t N, int64_t K, int parts,
                                bool first) {
  DecodeGemmPlan pl{};
  pl.tiles = static_cast<int>(N / 16);
  pl.mgroups = static_cast<int>((M + 63) / 64);
  pl.waves = waves_for(epi, parts);
  const int P = (epi == EPI_DOWN) ? parts : 1;
  const int64_t steps = K / P / 64;                 // 64-byte steps per partition
  int R = 1;
  if (!first) {
    // Spread K over workgroups until the grid reaches the resident target, keeping at
    // least 8 steps (8 KB of weights) per wave.
    const int64_t per_wave_min = 8 * (pl.waves / P);
    while (int64_t(pl.tiles) * pl.mgroups * (R + 1) <= kTargetWorkgroups &&
           steps / (R + 1) >= per_wave_min)
      ++R;
  }
  pl.ranges = R;
  const int sets = (epi == EPI_DOWN) ? P : (epi == EPI_SILU ? 2 : 1);
  pl.acc_elems = R > 1 ? size_t(sets) * size_t(M) * size_t(N) : 0;
  pl.cnt_elems = R > 1 ? size_t(pl.tiles) * pl.mgroups : 0;
  return pl;
}

hipError_t launch_decode_gemm(const DecodeGemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int mgroups = static_cast<int>((a.M + 63) / 64);
  const dim3 grid(static_cast<unsigned>((a.N / 16) * a.ranges), static_cast<unsigned>(mgroups));
  const int64_t b = (a.M + 15) / 16;
  const int mb = static_cast<int>(b > 4 ? 4 : b);
  const bool fused = a.prologue != PRO_CODES;
  if (fused && a.M > kFuseMaxRows) return hipErrorInvalidValue;
  size_t lds = 0;
  if (fused) {
    const int P = (a.epi == EPI_DOWN) ? a.parts : 1;
    const int64_t Sp = a.K / P / 64;
    lds = size_t(a.M) * P * ((Sp + a.ranges - 1) / a.ranges) * 64;
  }
  switch (a.epi) {
    case EPI_BF16:
      if (fused)
        return launch_layout<EPI_BF16, 1, kWavesDefault, 1, 1, PRO_QUANT_BF16>(a, grid, lds, stream);
      return launch_codes<EPI_BF16, 1, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_BF16_RES:
      if (fused)
        return launch_layout<EPI_BF16_RES, 1, kWavesDefault, 1, 1, PRO_QUANT_BF16>(a, grid, lds,
                                                                                  stream);
      return launch_codes<EPI_BF16_RES, 1, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_SILU:
      if (fused)
        return launch_layout<EPI_SILU, 2, kWavesDefault, 1, 1, PRO_QUANT_BF16>(a, grid, lds, stream);
      return launch_codes<EPI_SILU, 2, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_DOWN:
      switch (a.parts) {
        case 1: return launch_down<1>(a, mb, grid, lds, stream);
        case 2: return launch_down<2>(a, mb, grid, lds, stream);
        case 4: return launch_down<4>(a, mb, grid, lds, stream);
        case 8: return launch_down<8>(a, mb, grid, lds, stream);
        default: return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pack_tiled(const int8_t* w, int64_t N, int64_t K, int8_t* out,
                             hipStream_t stream) {
  const int64_t chunks = N * K / 16;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_tiled_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     w, N, K, out);
  return hipGetLastError();
}

}  // namespace a8w8
