// Per-row dynamic INT8 quantization with optional fused RMSNorm (gfx950).
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Decode scheduling (one batched activation-quantization pass
// over all decode rows) and > Gate/Up INT8 path (each row of normalized activations after
// attention gets its own INT8 codes and one FP32 scale).
//
// One workgroup per row.  A row of up to kRegChunks * 4096 values is read once into
// registers (all its loads in flight together) and the three passes (sum of squares,
// absolute maximum, codes) run on the registers; a longer row is read three times from
// L2, recomputing the normalized value each time with the same operations.  Either way
// every thread takes its values in the same order and the reductions use a fixed tree,
// so the result does not depend on the variant or on scheduling.
//
// Per row (readings where the pages leave the formula open):
//   S  = sum f(x_k)^2 in FP64 (squares of BF16 are exact in FP64)
//   ms = fl32(S / K); t = fl32(ms + eps); r = fl32(1 / fl32(sqrt(t)))
//   v_k = fl32(fl32(x_k * r) * gamma_k)           (v_k = x_k without the norm)
//   s  = fl32(max_k |v_k| / 127); q_k = clamp(rint(v_k / s), -127, 127), 0 if s == 0
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

constexpr int kQuantThreads = 512;
constexpr int kQuantWaves = kQuantThreads / kWave;

template <bool kF32In>
struct RowLoader;

// 8 BF16 values per 16-byte load.
template <>
struct RowLoader<false> {
  static constexpr int kVec = 8;
  __device__ static void load(const void* row, int64_t k, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};

// 4 FP32 values per 16-byte load (two loads fill 8).
template <>
struct RowLoader<true> {
  static constexpr int kVec = 8;
  __device__ static void load(const void* row, int64_t k, float (&v)[8]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + k);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
};

__device__ __forceinline__ void load_gamma(const uint16_t* g, int64_t k, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(g + k);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

constexpr int kRegChunks = 5;  // rows of up to 5 * 512 * 8 = 20480 values stay in registers

template <bool kRms, bool kF32In>
__global__ __launch_bounds__(kQuantThreads) void quant_rows_reg_kernel(QuantRowsArgs p) {
  using L = RowLoader<kF32In>;
  constexpr int V = L::kVec;
  __shared__ double s_sum[kQuantWaves];
  __shared__ float s_max[kQuantWaves];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.x;
  const int64_t K = p.K;
  const char* xrow = static_cast<const char*>(p.x) +
                     row * p.ldx * (kF32In ? sizeof(float) : sizeof(uint16_t));
  // Chunk c of this thread starts at k = (c * kQuantThreads + tid) * V, the order the
  // looping kernel visits them in.
  // The gain is requested with the row: its loads then overlap the row's.
  float v[kRegChunks][V];
  float gm[kRms ? kRegChunks : 1][V];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int64_t k = (int64_t(c) * kQuantThreads + tid) * V;
    if (k < K) {
      L::load(xrow, k, v[c]);
      if constexpr (kRms) load_gamma(p.gamma, k, gm[c]);
    }
  }

  if (kRms) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      const int64_t k = (int64_t(c) * kQuantThreads + tid) * V;
      if (k >= K) break;
#pragma unroll
      for (int i = 0; i < V; ++i) ss += double(v[c][i]) * double(v[c][i]);
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) s_sum[wave] = ss;
    __syncthreads();
    double S = 0.0;
    for (int w = 0; w < kQuantWaves; ++w) S += s_sum[w];
    const float ms = static_cast<float>(S / static_cast<double>(K));
    const float t = ms + p.eps;
    const float sq = __builtin_sqrtf(t);
    const float r = 1.0f / sq;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      const int64_t k = (int64_t(c) * kQuantThreads + tid) * V;
      if (k >= K) break;
#pragma unroll
      for (int i = 0; i < V; ++i) v[c][i] = (v[c][i] * r) * gm[c][i];
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int64_t k = (int64_t(c) * kQuantThreads + tid) * V;
    if (k >= K) break;
#pragma unroll
    for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    if (p.xn_tap) {
      f32x4* t = reinterpret_cast<f32x4*>(p.xn_tap + row * K + k);
      t[0] = f32x4{v[c][0], v[c][1], v[c][2], v[c][3]};
      t[1] = f32x4{v[c][4], v[c][5], v[c][6], v[c][7]};
    }
    if (p.a_bf16 || p.a_bf16_tap) {
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = uint32_t(f32_to_bf16_rne(v[c][2 * i])) |
                (uint32_t(f32_to_bf16_rne(v[c][2 * i + 1])) << 16);
      if (p.a_bf16)
        *reinterpret_cast<u32x4*>(p.a_bf16 + (p.a_bf16_tiled ? prefill_operand_index(row, k, K)
                                                             : row * K + k)) = pk;
      if (p.a_bf16_tap) *reinterpret_cast<u32x4*>(p.a_bf16_tap + row * K + k) = pk;
    }
  }
  if (!p.write_codes) return;
  amax = wave_max_f32(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  float a = 0.0f;
  for (int w = 0; w < kQuantWaves; ++w) a = fmaxf(a, s_max[w]);
  const float s = a / 127.0f;
  if (tid == 0) {
    p.s[row] = s;
    if (p.s_tap) p.s_tap[row] = s;
  }
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int64_t k = (int64_t(c) * kQuantThreads + tid) * V;
    if (k >= K) break;
    uint32_t lo = 0, hi = 0;
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (uint32_t(quant_code(v[c][i], s)) & 0xFFu) << (8 * i);
        hi |= (uint32_t(quant_code(v[c][4 + i], s)) & 0xFFu) << (8 * i);
      }
    }
    const u32x2 pk = {lo, hi};
    *reinterpret_cast<u32x2*>(p.q + (p.q_tiled ? tiled_code_index(row, k) : row * K + k)) = pk;
    if (p.q_tap) *reinterpret_cast<u32x2*>(p.q_tap + row * K + k) = pk;
  }
}

template <bool kRms, bool kF32In>
__global__ __launch_bounds__(kQuantThreads) void quant_rows_kernel(QuantRowsArgs p) {
  using L = RowLoader<kF32In>;
  constexpr int V = L::kVec;
  __shared__ double s_sum[kQuantWaves];
  __shared__ float s_max[kQuantWaves];
  __shared__ float s_bcast[2];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.x;
  const int64_t K = p.K;
  const char* xrow = static_cast<const char*>(p.x) +
                     row * p.ldx * (kF32In ? sizeof(float) : sizeof(uint16_t));

  float r = 1.0f;
  if (kRms) {
    double ss = 0.0;
    for (int64_t k = int64_t(tid) * V; k < K; k += int64_t(kQuantThreads) * V) {
      float v[V];
      L::load(xrow, k, v);
#pragma unroll
      for (int i = 0; i < V; ++i) ss += double(v[i]) * double(v[i]);
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) s_sum[wave] = ss;
    __syncthreads();
    if (tid == 0) {
      double S = 0.0;
      for (int w = 0; w < kQuantWaves; ++w) S += s_sum[w];
      const float ms = static_cast<float>(S / static_cast<double>(K));
      const float t = ms + p.eps;
      const float sq = __builtin_sqrtf(t);
      s_bcast[0] = 1.0f / sq;
    }
    __syncthreads();
    r = s_bcast[0];
  }

  // Pass 2: normalized values, their absolute maximum, optional FP32 / BF16 taps.
  float amax = 0.0f;
  for (int64_t k = int64_t(tid) * V; k < K; k += int64_t(kQuantThreads) * V) {
    float v[V];
    L::load(xrow, k, v);
    if (kRms) {
      float g[V];
      load_gamma(p.gamma, k, g);
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = (v[i] * r) * g[i];
    }
#pragma unroll
    for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if (p.xn_tap) {
      f32x4* t = reinterpret_cast<f32x4*>(p.xn_tap + row * K + k);
      t[0] = f32x4{v[0], v[1], v[2], v[3]};
      t[1] = f32x4{v[4], v[5], v[6], v[7]};
    }
    if (p.a_bf16 || p.a_bf16_tap) {
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = uint32_t(f32_to_bf16_rne(v[2 * i])) | (uint32_t(f32_to_bf16_rne(v[2 * i + 1])) << 16);
      if (p.a_bf16)
        *reinterpret_cast<u32x4*>(p.a_bf16 + (p.a_bf16_tiled ? prefill_operand_index(row, k, K)
                                                             : row * K + k)) = pk;
      if (p.a_bf16_tap) *reinterpret_cast<u32x4*>(p.a_bf16_tap + row * K + k) = pk;
    }
  }
  if (!p.write_codes) return;
  amax = wave_max_f32(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  if (tid == 0) {
    float a = 0.0f;
    for (int w = 0; w < kQuantWaves; ++w) a = fmaxf(a, s_max[w]);
    const float s = a / 127.0f;
    s_bcast[1] = s;
    p.s[row] = s;
    if (p.s_tap) p.s_tap[row] = s;
  }
  __syncthreads();
  const float s = s_bcast[1];

  // Pass 3: codes, 8 per thread per step, stored as one 8-byte word.
  for (int64_t k = int64_t(tid) * V; k < K; k += int64_t(kQuantThreads) * V) {
    float v[V];
    L::load(xrow, k, v);
    if (kRms) {
      float g[V];
      load_gamma(p.gamma, k, g);
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = (v[i] * r) * g[i];
    }
    uint32_t lo = 0, hi = 0;
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (uint32_t(quant_code(v[i], s)) & 0xFFu) << (8 * i);
        hi |= (uint32_t(quant_code(v[4 + i], s)) & 0xFFu) << (8 * i);
      }
    }
    const u32x2 pk = {lo, hi};
    *reinterpret_cast<u32x2*>(p.q + (p.q_tiled ? tiled_code_index(row, k) : row * K + k)) = pk;
    if (p.q_tap) *reinterpret_cast<u32x2*>(p.q_tap + row * K + k) = pk;
  }
}

// Requantization of FP32 rows whose absolute maxima are given per 16-column tile (the
// partial maxima written by the Gate/Up epilogue): the scale needs no pass over the row
// (the maximum of the partial maxima is the row's absolute maximum), so each row is cut
// into chunks of kRqChunk values, one workgroup each, and every workgroup derives the
// scale itself.  Codes as in the kernels above.
constexpr int kRqThreads = 256;
constexpr int kRqChunk = kRqThreads * 8;

__global__ __launch_bounds__(kRqThreads) void requant_pmax_kernel(QuantRowsArgs p) {
  __shared__ float s_max[kRqThreads / kWave];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.y;
  const int64_t K = p.K;
  const int64_t k = int64_t(blockIdx.x) * kRqChunk + int64_t(tid) * 8;
  float v[8];
  if (k < K) RowLoader<true>::load(static_cast<const float*>(p.x) + row * p.ldx, k, v);
  float a = 0.0f;
  for (int64_t t = tid; t < p.npmax; t += kRqThreads) a = fmaxf(a, p.pmax[t * p.M + row]);
  a = wave_max_f32(a);
  if (lane == 0) s_max[wave] = a;
  __syncthreads();
  a = 0.0f;
#pragma unroll
  for (int w = 0; w < kRqThreads / kWave; ++w) a = fmaxf(a, s_max[w]);
  const float s = a / 127.0f;
  if (blockIdx.x == 0 && tid == 0) {
    p.s[row] = s;
    if (p.s_tap) p.s_tap[row] = s;
  }
  if (k >= K) return;
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t(quant_code(v[i], s)) & 0xFFu) << (8 * i);
      hi |= (uint32_t(quant_code(v[4 + i], s)) & 0xFFu) << (8 * i);
    }
  }
  const u32x2 pk = {lo, hi};
  *reinterpret_cast<u32x2*>(p.q + (p.q_tiled ? tiled_code_index(row, k) : row * K + k)) = pk;
  if (p.q_tap) *reinterpret_cast<u32x2*>(p.q_tap + row * K + k) = pk;
}

}  // namespace

hipError_t launch_requant_pmax(const QuantRowsArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.M > 65535 || !a.x_is_f32 || a.gamma || !a.pmax || a.K % 8) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((a.K + kRqChunk - 1) / kRqChunk),
                  static_cast<unsigned>(a.M)),
      block(kRqThreads);
  hipLaunchKernelGGL(requant_pmax_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  // One workgroup per row.
  const dim3 grid(static_cast<unsigned>(a.M)), block(kQuantThreads);
  const bool rms = a.gamma != nullptr;
  if (a.K <= int64_t(kRegChunks) * kQuantThreads * 8) {
    if (rms && !a.x_is_f32)
      hipLaunchKernelGGL((quant_rows_reg_kernel<true, false>), grid, block, 0, stream, a);
    else if (!rms && !a.x_is_f32)
      hipLaunchKernelGGL((quant_rows_reg_kernel<false, false>), grid, block, 0, stream, a);
    else if (!rms && a.x_is_f32)
      hipLaunchKernelGGL((quant_rows_reg_kernel<false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((quant_rows_reg_kernel<true, true>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  if (rms && !a.x_is_f32)
    hipLaunchKernelGGL((quant_rows_kernel<true, false>), grid, block, 0, stream, a);
  else if (!rms && !a.x_is_f32)
    hipLaunchKernelGGL((quant_rows_kernel<false, false>), grid, block, 0, stream, a);
  else if (!rms && a.x_is_f32)
    hipLaunchKernelGGL((quant_rows_kernel<false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((quant_rows_kernel<true, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace a8w8
