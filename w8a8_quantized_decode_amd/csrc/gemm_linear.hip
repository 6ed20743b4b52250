// Standalone INT8 x INT8 -> INT32 linear on given activation codes (a8w8_linear), on
// gfx950 matrix cores, with the dequant (+ residual) -> RNE BF16 epilogue.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path (INT8 x INT8 products summed in INT32, the
// sums turned into FP32 with the row scale and the channel scale).
//
// This entry point takes no workspace, so every 16-channel output tile is owned by one
// workgroup: its waves split K, keep U steps of weight loads in flight (two register
// sets), and add their INT32 partial sums in LDS.  The v_mfma_i32_16x16x64_i8 operands:
// the weights are A (16 channels x 64 k, lane l feeds channel l%16 with the 16 bytes at
// k-offset 16*(l/16)), the codes are B (64 k x 16 rows of M, missing rows are zero);
// the result of lane l holds channels 4*(l/16)+r of row l%16.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

constexpr int kLinWaves = 4;

template <int EPI, int MB, int LAYOUT>
__global__ __launch_bounds__(kLinWaves * kWave) void linear_kernel(LinearArgs p) {
  constexpr int NW = kLinWaves;
  constexpr int U = MB == 1 ? 8 : (MB == 2 ? 4 : 2);  // k steps per load batch
  __shared__ i32x4 red[NW][MB][kWave];

  const int tid = threadIdx.x;
  // Wave index in a scalar register: every loop bound below is wave-uniform, because a
  // matrix instruction ignores a partial lane mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int row16 = lane & 15, kg = lane >> 4;
  const int tile = blockIdx.x;
  const int64_t n0 = int64_t(tile) * 16;
  const int64_t m0 = int64_t(blockIdx.y) * MB * 16;
  const int S = static_cast<int>(p.K / 64);
  const int ws0 = S * wave / NW, ws1 = S * (wave + 1) / NW;

  const int8_t* wbase = (LAYOUT == LAYOUT_TILED)
                            ? p.w0 + int64_t(tile) * 16 * p.K + lane * 16
                            : p.w0 + (n0 + row16) * p.K + kg * 16;
  constexpr int64_t kStep = (LAYOUT == LAYOUT_TILED) ? 1024 : 64;
  const int8_t* abase[MB];
  bool aval[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + mb * 16 + row16;
    aval[mb] = m < p.M;
    abase[mb] = p.a + (aval[mb] ? m : 0) * p.lda + kg * 16;  // missing rows read row 0
  }

  i32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = i32x4{0, 0, 0, 0};

  // Unconditional, clamped loads and a zero operand on dead steps keep the loop free
  // of data-dependent branches, so each wait covers exactly the batch being consumed.
  const int nb = (ws1 - ws0 + U - 1) / U;
  auto load_batch = [&](i32x4 (&wv)[U], i32x4 (&bv)[U][MB], int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = min(t + u, ws1 - 1);
      wv[u] = ld16_stream(wbase + int64_t(tt) * kStep);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) bv[u][mb] = ld16(abase[mb] + int64_t(tt) * 64);
    }
  };
  auto compute = [&](const i32x4 (&wv)[U], const i32x4 (&bv)[U][MB], int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = t + u < ws1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 b = (live && aval[mb]) ? bv[u][mb] : i32x4{0, 0, 0, 0};
        acc[mb] = mfma_i8(wv[u], b, acc[mb]);
      }
    }
  };
  i32x4 wA[U], bA[U][MB], wB[U], bB[U][MB];
  if (nb > 0) load_batch(wA, bA, ws0);
  for (int bi = 0; bi < nb; bi += 2) {
    const int t = ws0 + bi * U;
    load_batch(wB, bB, t + U);
    compute(wA, bA, t);
    if (bi + 1 >= nb) break;
    load_batch(wA, bA, t + 2 * U);
    compute(wB, bB, t + U);
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();

  // One epilogue thread per (16-row block, lane): 4 channels of one row.
  if (tid >= MB * kWave) return;
  const int emb = tid / kWave, eln = tid & (kWave - 1);
  const int64_t em = m0 + emb * 16 + (eln & 15);
  const int64_t en = n0 + 4 * (eln >> 4);
  if (em >= p.M) return;
  i32x4 sum = {0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < NW; ++w) sum += red[w][emb][eln];
  if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = sum;
  const float sa = p.sa[em];
  float y[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) y[c] = dq(sum[c], sa, p.sw0[en + c]);
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
}

template <int EPI, int MB>
hipError_t launch_mb(const LinearArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(kLinWaves * kWave);
  if (a.layout == LAYOUT_TILED)
    hipLaunchKernelGGL((linear_kernel<EPI, MB, LAYOUT_TILED>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((linear_kernel<EPI, MB, LAYOUT_ROWMAJOR>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const LinearArgs& a, hipStream_t s) {
  const int64_t blocks16 = (a.M + 15) / 16;
  const int mb = static_cast<int>(blocks16 > 4 ? 4 : blocks16);
  const dim3 grid(static_cast<unsigned>(a.N / 16), static_cast<unsigned>((a.M + 16 * mb - 1) / (16 * mb)));
  switch (mb) {
    case 1: return launch_mb<EPI, 1>(a, grid, s);
    case 2: return launch_mb<EPI, 2>(a, grid, s);
    case 3: return launch_mb<EPI, 3>(a, grid, s);
    default: return launch_mb<EPI, 4>(a, grid, s);
  }
}

}  // namespace

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.epi == EPI_BF16) return launch_epi<EPI_BF16>(a, stream);
  if (a.epi == EPI_BF16_RES) return launch_epi<EPI_BF16_RES>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace a8w8
