// QK-norm, rotate-half RoPE and the paged BF16 KV-cache write that follow the QKV
// projection (pypto-serving issue #52, Current behavior: the fused QK-norm path and its
// Q RoPE; pypto-lib PR #810 walkthrough, BF16 cache and interface contracts: RoPE writes
// into BF16 KV caches).
//
// One wave per (row, head).  Lane l holds the rotate-half pairs (i, i + d/2) for
// i = l, l + 64, ...; the sum of squares of a head is accumulated in FP64 (squares of
// BF16 values are exact) and reduced across the wave, so each head's RMSNorm needs no
// barrier.  All FP32 steps are single IEEE operations in the stated order (the library
// is built without contraction), so the result is the oracle's bit for bit.  Rows whose
// position or cache block lies outside the given tables are skipped.
#include "device_common.h"
#include "attention_args.h"
#include "internal.h"

namespace a8w8 {
namespace {

constexpr int kRopeMaxPairsPerLane = 4;  // head_dim <= 512

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__global__ __launch_bounds__(kWave) void qk_rope_kernel(QkRopeArgs p) {
  const int64_t m = blockIdx.x;
  const int head = static_cast<int>(blockIdx.y);
  const int lane = threadIdx.x;
  const int d = p.head_dim, h2 = d / 2;
  const int32_t pos = p.positions[m];
  if (pos < 0 || pos >= p.max_pos) return;
  const bool is_q = head < p.n_q;
  const bool is_k = !is_q && head < p.n_q + p.n_kv;
  const uint16_t* src = p.qkv + m * p.ld_qkv + int64_t(head) * d;

  // Cache slot of this row's position; a row without a valid slot is skipped by every
  // head (its Q output included).
  int64_t slot = -1;
  if (p.n_kv > 0) {
    const int64_t bi = pos / p.block_size;
    if (bi >= p.blocks_per_seq) return;
    const int32_t blk = p.block_table[m * p.blocks_per_seq + bi];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int kvh = is_q ? 0 : (is_k ? head - p.n_q : head - p.n_q - p.n_kv);
    slot = ((int64_t(blk) * p.block_size + pos % p.block_size) * p.n_kv + kvh) * d;
  }
  if (!is_q && !is_k) {  // V: copied as it is
    for (int i = lane; i < d; i += kWave) p.v_cache[slot + i] = src[i];
    return;
  }

  float x1[kRopeMaxPairsPerLane], x2[kRopeMaxPairsPerLane];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < kRopeMaxPairsPerLane; ++j) {
    const int i = lane + j * kWave;
    x1[j] = 0.0f;
    x2[j] = 0.0f;
    if (i < h2) {
      x1[j] = bf16_bits_to_f32(src[i]);
      x2[j] = bf16_bits_to_f32(src[i + h2]);
      ss += double(x1[j]) * double(x1[j]) + double(x2[j]) * double(x2[j]);
    }
  }
  const double S = wave_sum_f64(ss);
  const float ms = static_cast<float>(S / static_cast<double>(d));
  const float t = ms + p.eps;
  const float r = 1.0f / __builtin_sqrtf(t);
  const uint16_t* g = is_q ? p.q_gamma : p.k_gamma;
  const float* cs = p.cos_table + int64_t(pos) * h2;
  const float* sn = p.sin_table + int64_t(pos) * h2;
  uint16_t* dst = is_q ? p.q_out + m * p.ld_q + int64_t(head) * d : p.k_cache + slot;
#pragma unroll
  for (int j = 0; j < kRopeMaxPairsPerLane; ++j) {
    const int i = lane + j * kWave;
    if (i < h2) {
      const float a = (x1[j] * r) * bf16_bits_to_f32(g[i]);
      const float b = (x2[j] * r) * bf16_bits_to_f32(g[i + h2]);
      const float c = cs[i], s = sn[i];
      const float o1 = a * c - b * s;
      const float o2 = b * c + a * s;
      dst[i] = f32_to_bf16_rne(o1);
      dst[i + h2] = f32_to_bf16_rne(o2);
    }
  }
}

}  // namespace

hipError_t launch_qk_rope(const QkRopeArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.M), static_cast<unsigned>(a.n_q + 2 * a.n_kv));
  hipLaunchKernelGGL(qk_rope_kernel, grid, dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace a8w8
