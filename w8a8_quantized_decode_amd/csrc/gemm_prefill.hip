// Prefill-shaped W8A16 GEMMs on gfx950 BF16 matrix cores, on the shared INT8 weights.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path: prefill keeps the INT8 checkpoint weights
// and dequantizes each weight tile to BF16 before the matrix multiply.  Here every tile
// element becomes W' = rne_bf16(fl32(w * s[n])) in registers, the activations are BF16,
// products accumulate in FP32 (v_mfma_f32_16x16x32_bf16).
//
// Work shape.  A workgroup of 4 waves owns 64 rows of M and 4 * 16 * CB output
// channels; each wave owns 16 * CB channels (CB blocks of 16) of NMAT weights.
//   * Weights come from the tiled layout: one 1 KB block = 16 channels x 64 k, lane l
//     holding channel l%16, k-offsets 16*(l/16)..+15.  The lane dequantizes its 16
//     bytes into two BF16 operands (k-offsets +0..7 and +8..15); each feeds one
//     16x16x32 MFMA, and the activation operand is gathered with the same k order.
//   * int8 -> FP32 -> x scale uses the biased byte u = w + 128 (exact in FP32) and one
//     fused multiply-add u*s + (-128*s): the exact value is w*s, so the single rounding
//     gives fl32(w*s) bit for bit.  The FP32 -> BF16 step is the RNE conversion.
//   * Activations (BF16, row-major [M, K]) are staged per 64-k step through LDS in a
//     double buffer whose rows are padded to 144 bytes, so the 16 lanes that read one
//     column group hit 16 distinct 4-bank groups.
//   * EPI_PF_SILU: h = rne_bf16(silu(g) * u) from the Gate and Up accumulators.
//     EPI_PF_PARTIAL: FP32 partial sums of one K split, reduced by reduce_residual.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPfWaves = 4;
constexpr int kPfMt = 64;             // rows of M per workgroup
constexpr int kPfRowBytes = 144;      // LDS row pitch (128 B of data + 16 B pad)
constexpr int kPfStage = kPfMt * kPfRowBytes;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 INT8 weights of one channel -> two BF16 operands of 8, scaled by s.
__device__ __forceinline__ void dequant16(u32x4 raw, float s, bf16x8& lo, bf16x8& hi) {
  const float bias = -128.0f * s;
  float f[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = raw[d] ^ 0x80808080u;  // biased bytes w + 128
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float fu = static_cast<float>((u >> (8 * b)) & 0xFFu);
      f[4 * d + b] = __builtin_fmaf(fu, s, bias);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = static_cast<__bf16>(f[e]);
    hi[e] = static_cast<__bf16>(f[8 + e]);
  }
}

template <int EPI, int NMAT, int CB, int LAYOUT>
__global__ __launch_bounds__(kPfWaves * kWave) void prefill_gemm_kernel(PrefillGemmArgs p) {
  __shared__ __align__(16) int8_t bsm[2][kPfStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15, g4 = lane >> 4;
  constexpr int kChPerWg = kPfWaves * 16 * CB;
  const int ntile = blockIdx.x / p.splits, split = blockIdx.x % p.splits;
  const int64_t m0 = int64_t(blockIdx.y) * kPfMt;
  const int64_t ch0 = int64_t(ntile) * kChPerWg + wave * 16 * CB;  // this wave's first channel
  const int steps_total = static_cast<int>(p.K / 64);
  const int s0 = static_cast<int>(int64_t(split) * steps_total / p.splits);
  const int s1 = static_cast<int>(int64_t(split + 1) * steps_total / p.splits);

  // Weight blocks and channel scales of this lane.
  const int8_t* wblk[NMAT][CB];
  float sc[NMAT][CB];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int64_t tile16 = ch0 / 16 + c;
      const int8_t* w = (i == 0) ? p.w0 : p.w1;
      wblk[i][c] = (LAYOUT == LAYOUT_TILED) ? w + tile16 * 16 * p.K + lane * 16
                                           : w + (tile16 * 16 + r16) * p.K + g4 * 16;
      sc[i][c] = ((i == 0) ? p.sw0 : p.sw1)[tile16 * 16 + r16];
    }

  // Activation staging: a stage is 64 rows x 128 bytes (64 BF16); thread t moves the
  // 32 bytes (16 BF16) at quarter t%4 of row t/4.
  const int srow = tid >> 2, squart = tid & 3;
  const bool srow_ok = m0 + srow < p.M;
  const uint16_t* asrc = p.act + (srow_ok ? (m0 + srow) : 0) * p.lda + squart * 16;
  auto stage_load = [&](int t, u32x4 (&v)[2]) {
    const uint16_t* s = asrc + int64_t(t) * 64;
    v[0] = *reinterpret_cast<const u32x4*>(s);
    v[1] = *reinterpret_cast<const u32x4*>(s + 8);
    if (!srow_ok) v[0] = v[1] = u32x4{0u, 0u, 0u, 0u};
  };
  auto stage_store = [&](int buf, const u32x4 (&v)[2]) {
    int8_t* d = &bsm[buf][srow * kPfRowBytes + squart * 32];
    reinterpret_cast<u32x4*>(d)[0] = v[0];
    reinterpret_cast<u32x4*>(d)[1] = v[1];
  };

  f32x4 acc[NMAT][CB][4];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[i][c][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int64_t kStep = (LAYOUT == LAYOUT_TILED) ? 1024 : 64;
  auto load_w = [&](u32x4 (&wv)[NMAT][CB], int t) {
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int c = 0; c < CB; ++c)
        wv[i][c] = *reinterpret_cast<const u32x4*>(wblk[i][c] + int64_t(t) * kStep);
  };
  const int nsteps = s1 - s0;
  // One 64-k step: prefetch the next weights and activation stage, multiply the
  // current one, then publish the next stage to LDS.
  u32x4 sv[2];
  auto step = [&](int it, const u32x4 (&wc)[NMAT][CB], u32x4 (&wn)[NMAT][CB]) {
    const int cur = it & 1;
    const bool more = it + 1 < nsteps;
    if (more) {
      stage_load(s0 + it + 1, sv);
      load_w(wn, s0 + it + 1);
    }
    bf16x8 b[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int8_t* rp = &bsm[cur][(mb * 16 + r16) * kPfRowBytes + g4 * 32];
      b[mb][0] = *reinterpret_cast<const bf16x8*>(rp);
      b[mb][1] = *reinterpret_cast<const bf16x8*>(rp + 16);
    }
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        bf16x8 alo, ahi;
        dequant16(wc[i][c], sc[i][c], alo, ahi);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          acc[i][c][mb] = mfma_bf16(alo, b[mb][0], acc[i][c][mb]);
          acc[i][c][mb] = mfma_bf16(ahi, b[mb][1], acc[i][c][mb]);
        }
      }
    if (more) stage_store(cur ^ 1, sv);
    __syncthreads();
  };

  u32x4 wA[NMAT][CB], wB[NMAT][CB];
  if (nsteps > 0) {
    stage_load(s0, sv);
    load_w(wA, s0);
    stage_store(0, sv);
  }
  __syncthreads();
  for (int it = 0; it < nsteps; it += 2) {
    step(it, wA, wB);
    if (it + 1 >= nsteps) break;
    step(it + 1, wB, wA);
  }

  // Epilogue.  Lane l holds channels 4*(l/16)+r of row l%16 for each block.
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int64_t m = m0 + mb * 16 + r16;
      if (m >= p.M) continue;
      const int64_t n = ch0 + c * 16 + 4 * g4;
      if constexpr (EPI == EPI_PF_SILU) {
        const f32x4 g = acc[0][c][mb], u = acc[NMAT - 1][c][mb];
        if (p.tap_g) *reinterpret_cast<f32x4*>(p.tap_g + m * p.N + n) = g;
        if (p.tap_u) *reinterpret_cast<f32x4*>(p.tap_u + m * p.N + n) = u;
        u32x2 o;
        o[0] = uint32_t(f32_to_bf16_rne(silu_mul(g[0], u[0]))) |
               (uint32_t(f32_to_bf16_rne(silu_mul(g[1], u[1]))) << 16);
        o[1] = uint32_t(f32_to_bf16_rne(silu_mul(g[2], u[2]))) |
               (uint32_t(f32_to_bf16_rne(silu_mul(g[3], u[3]))) << 16);
        *reinterpret_cast<u32x2*>(p.out_bf16 + m * p.ldo + n) = o;
      } else {
        *reinterpret_cast<f32x4*>(p.part + (int64_t(split) * p.M + m) * p.N + n) = acc[0][c][mb];
      }
    }
}

// out = rne_bf16(fl32(sum_s part[s]) + res), partial sums added in split order.
__global__ __launch_bounds__(256) void reduce_residual_kernel(const float* part, int splits,
                                                              int64_t MN, const uint16_t* res,
                                                              uint16_t* out, float* tap_d) {
  for (int64_t i4 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i4 < MN / 4;
       i4 += int64_t(gridDim.x) * blockDim.x) {
    f32x4 s = reinterpret_cast<const f32x4*>(part)[i4];
    for (int j = 1; j < splits; ++j) s += reinterpret_cast<const f32x4*>(part + j * MN)[i4];
    if (tap_d) reinterpret_cast<f32x4*>(tap_d)[i4] = s;
    const u32x2 rr = reinterpret_cast<const u32x2*>(res)[i4];
    const float y0 = s[0] + bf16_lo(rr[0]), y1 = s[1] + bf16_hi(rr[0]);
    const float y2 = s[2] + bf16_lo(rr[1]), y3 = s[3] + bf16_hi(rr[1]);
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(y0)) | (uint32_t(f32_to_bf16_rne(y1)) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(y2)) | (uint32_t(f32_to_bf16_rne(y3)) << 16);
    reinterpret_cast<u32x2*>(out)[i4] = o;
  }
}

}  // namespace

int prefill_channels_per_wg(int epi) { return kPfWaves * 16 * (epi == EPI_PF_SILU ? 2 : 4); }

hipError_t launch_prefill_gemm(const PrefillGemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int chw = prefill_channels_per_wg(a.epi);
  const dim3 grid(static_cast<unsigned>((a.N / chw) * a.splits),
                  static_cast<unsigned>((a.M + kPfMt - 1) / kPfMt));
  const dim3 block(kPfWaves * kWave);
  const bool tiled = a.layout == LAYOUT_TILED;
  if (a.epi == EPI_PF_SILU) {
    if (tiled)
      hipLaunchKernelGGL((prefill_gemm_kernel<EPI_PF_SILU, 2, 2, LAYOUT_TILED>), grid, block, 0,
                         stream, a);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<EPI_PF_SILU, 2, 2, LAYOUT_ROWMAJOR>), grid, block,
                         0, stream, a);
  } else {
    if (tiled)
      hipLaunchKernelGGL((prefill_gemm_kernel<EPI_PF_PARTIAL, 1, 4, LAYOUT_TILED>), grid, block,
                         0, stream, a);
    else
      hipLaunchKernelGGL((prefill_gemm_kernel<EPI_PF_PARTIAL, 1, 4, LAYOUT_ROWMAJOR>), grid,
                         block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_residual(const float* part, int splits, int64_t M, int64_t N,
                                  const uint16_t* res, uint16_t* out, float* tap_d,
                                  hipStream_t stream) {
  const int64_t n4 = M * N / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(reduce_residual_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, part, splits, M * N, res, out, tap_d);
  return hipGetLastError();
}

}  // namespace a8w8
