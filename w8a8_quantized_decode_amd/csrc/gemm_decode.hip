// Decode-batch INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, with fused epilogues.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path (INT8 x INT8 -> INT32 Gate/Up matmuls,
// activation-row and weight-channel scales applied at dequantization) and > Decode
// scheduling (Down split two ways along K with independent accumulators), plus the
// CodeRabbit walkthrough row on the split Down projection (FP32 partials summed and
// narrowed together with the residual).  QKV and O reuse the same pattern.
//
// Shape of the work.  At decode batch sizes the weights dominate the traffic, so the
// kernel is a weight stream: every weight byte is read from HBM exactly once.
//   * A 16-channel tile of the output is computed with v_mfma_i32_16x16x64_i8: the
//     weights are the A operand (16 output channels x 64 k), the activation codes the
//     B operand (64 k x 16 rows of M).  Lane l feeds channel l%16 with the 16 bytes at
//     k-offset 16*(l/16) of the current 64-byte step, so one load instruction reads
//     64 contiguous bytes from each of 16 weight rows; rows of M beyond the batch are
//     fed zeros.  Lane l's result holds channels 4*(l/16)+r (r = 0..3) of row l%16.
//   * A workgroup owns one tile and one K range; its waves split the range, and their
//     INT32 partial sums meet in LDS (exact, order-free).
//   * When a tile's K is spread over several workgroups (ranges > 1) the partial sums
//     go to a device-scope INT32 accumulator with atomic adds; the last workgroup to
//     arrive (per-tile counter) takes the sums, clears the accumulator and counter,
//     and runs the epilogue.  Integer addition is exact, so the result is the same
//     bit for bit in any arrival order.
//   * EPI_DOWN: the waves of a workgroup are divided among the K partitions; each
//     partition keeps its own accumulator up to its own FP32 partial.
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

// NMAT: weights per tile (2 for Gate/Up), NW: waves per workgroup, MB: 16-row blocks of
// M, P: K partitions (EPI_DOWN only; 1 otherwise).
template <int EPI, int NMAT, int NW, int MB, int P>
__global__ __launch_bounds__(NW * kWave) void decode_gemm_kernel(DecodeGemmArgs p) {
  constexpr int NSETS = (EPI == EPI_DOWN) ? P : NMAT;
  constexpr int wpp = NW / P;             // waves per partition
  __shared__ i32x4 red[NW][NMAT][MB][kWave];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int row16 = lane & 15, kg = lane >> 4;
  const int R = p.ranges;
  const int tile = blockIdx.x / R, r = blockIdx.x % R;
  const int mg = blockIdx.y;
  const int64_t n0 = int64_t(tile) * 16;
  const int64_t m0 = int64_t(mg) * MB * 16;
  const int part = wave / wpp, wl = wave % wpp;
  const int64_t Kp = p.K / P;             // bytes per partition
  const int Sp = static_cast<int>(Kp / 64);
  const int rs0 = static_cast<int>(int64_t(r) * Sp / R);
  const int rs1 = static_cast<int>(int64_t(r + 1) * Sp / R);
  const int ns = rs1 - rs0;
  const int ws0 = rs0 + ns * wl / wpp, ws1 = rs0 + ns * (wl + 1) / wpp;

  const int64_t kbase = int64_t(part) * Kp + kg * 16;
  const int8_t* wrow[NMAT];
  wrow[0] = p.w0 + (n0 + row16) * p.K + kbase;
  if (NMAT > 1) wrow[NMAT - 1] = p.w1 + (n0 + row16) * p.K + kbase;
  const int8_t* arow[MB];
  bool aval[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + mb * 16 + row16;
    aval[mb] = m < p.M;
    arow[mb] = p.a + (aval[mb] ? m : 0) * p.lda + kbase;
  }

  i32x4 acc[NMAT][MB];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[i][mb] = i32x4{0, 0, 0, 0};

  constexpr int U = 4;
  int t = ws0;
  for (; t + U <= ws1; t += U) {
    i32x4 wv[U][NMAT], bv[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NMAT; ++i) wv[u][i] = ld16(wrow[i] + int64_t(t + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 v = ld16(arow[mb] + int64_t(t + u) * 64);
        bv[u][mb] = aval[mb] ? v : i32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma_i8(wv[u][i], bv[u][mb], acc[i][mb]);
  }
  for (; t < ws1; ++t) {
    i32x4 wv[NMAT], bv[MB];
#pragma unroll
    for (int i = 0; i < NMAT; ++i) wv[i] = ld16(wrow[i] + int64_t(t) * 64);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const i32x4 v = ld16(arow[mb] + int64_t(t) * 64);
      bv[mb] = aval[mb] ? v : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma_i8(wv[i], bv[mb], acc[i][mb]);
  }

#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][i][mb][lane] = acc[i][mb];
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
    if (EPI == EPI_DOWN) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int w = s * wpp; w < (s + 1) * wpp; ++w) sum[s] += red[w][0][emb][eln];
    } else {
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
        for (int w = 0; w < NW; ++w) sum[i] += red[w][i][emb][eln];
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
    if (seen == 0x7FFFFFFF) s_last = 2;
    __syncthreads();
    if (tid == 0) {
      int32_t* cnt = p.wcnt + int64_t(mg) * (p.N / 16) + tile;
      const int old = atomic_add_dev(cnt, 1);
      const bool last = old == R - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last ? 1 : 0;
    }
    __syncthreads();
    if (s_last != 1) return;
    if (mval) {
#pragma unroll
      for (int s = 0; s < NSETS; ++s) {
        int32_t* base = p.wacc + s * MN + em * p.N + en;
#pragma unroll
        for (int c = 0; c < 4; ++c) sum[s][c] = atomic_take(base + c);
      }
    }
  }
  if (!mval) return;

  const float sa = p.sa[em];
  if (EPI == EPI_BF16 || EPI == EPI_BF16_RES) {
    if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = sum[0];
    float y[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = dq(sum[0][c], sa, p.sw0[en + c]);
    if (EPI == EPI_BF16_RES) {
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
  } else if (EPI == EPI_SILU) {
    if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = sum[0];
    if (p.tap_acc1) *reinterpret_cast<i32x4*>(p.tap_acc1 + em * p.N + en) = sum[1];
    f32x4 h;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float g = dq(sum[0][c], sa, p.sw0[en + c]);
      const float u = dq(sum[1][c], sa, p.sw1[en + c]);
      h[c] = silu_mul(g, u);
    }
    *reinterpret_cast<f32x4*>(p.h + em * p.ldh + en) = h;
  } else {  // EPI_DOWN
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

constexpr int kWavesDefault = 4;
constexpr int kWavesDown = 8;
// Resident workgroups targeted per launch: 256 CUs x 5 four-wave workgroups.
constexpr int kTargetWorkgroups = 1280;

template <int EPI, int NMAT, int NW, int P>
hipError_t launch_mb(const DecodeGemmArgs& a, int mb, dim3 grid, hipStream_t stream) {
  const dim3 block(NW * kWave);
  switch (mb) {
    case 1: hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, 1, P>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, 2, P>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, 3, P>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_gemm_kernel<EPI, NMAT, NW, 4, P>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

int blocks_of_m(int64_t M) {
  const int64_t b = (M + 15) / 16;
  return static_cast<int>(b > 4 ? 4 : b);
}

}  // namespace

DecodeGemmPlan plan_decode_gemm(int epi, int64_t M, int64_t N, int64_t K, int parts,
                                bool allow_ranges) {
  DecodeGemmPlan pl{};
  pl.tiles = static_cast<int>(N / 16);
  pl.mgroups = static_cast<int>((M + 63) / 64);
  const int P = (epi == EPI_DOWN) ? parts : 1;
  const int nw = (epi == EPI_DOWN) ? kWavesDown : kWavesDefault;
  const int64_t steps = K / P / 64;                 // 64-byte steps per partition
  int R = 1;
  if (allow_ranges) {
    // Spread K over workgroups until the grid reaches the resident target, keeping
    // at least 4 steps per wave.
    const int64_t per_wave_min = 4 * (nw / P);
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
  const int mb = blocks_of_m(a.M);
  switch (a.epi) {
    case EPI_BF16: return launch_mb<EPI_BF16, 1, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_BF16_RES: return launch_mb<EPI_BF16_RES, 1, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_SILU: return launch_mb<EPI_SILU, 2, kWavesDefault, 1>(a, mb, grid, stream);
    case EPI_DOWN:
      switch (a.parts) {
        case 1: return launch_mb<EPI_DOWN, 1, kWavesDown, 1>(a, mb, grid, stream);
        case 2: return launch_mb<EPI_DOWN, 1, kWavesDown, 2>(a, mb, grid, stream);
        case 4: return launch_mb<EPI_DOWN, 1, kWavesDown, 4>(a, mb, grid, stream);
        case 8: return launch_mb<EPI_DOWN, 1, kWavesDown, 8>(a, mb, grid, stream);
        default: return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace a8w8
