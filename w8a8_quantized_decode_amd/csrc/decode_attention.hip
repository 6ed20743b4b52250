// Decode attention over the paged BF16 KV cache, between QKV and O (pypto-lib PR #810
// walkthrough: attention loads use BF16 KV caches; pypto-serving PR #48: paged KV cache
// with a block table).
//
// One workgroup of 16 waves per (row, KV head) serves the group's Q heads (grouped-
// query attention: Q head h reads KV head h / (n_q / n_kv)).  The query rows sit in LDS
// (every lane reads them as broadcasts).  The waves take chunks of 64 positions in turn:
//   * scores: lane l takes position j = chunk + l, reads its whole key row and forms the
//     scaled dot product with every Q head of the group (FP32);
//   * online softmax: per head, the chunk's maximum and sum across the wave update the
//     wave's running maximum and normalizer, rescaling its output accumulators;
//   * values: lane l owns head dimensions l, l + 64, ...; the chunk's weights go through
//     LDS and each value row is read once, coalesced.
// At the end the waves' states are combined through LDS and the output is narrowed
// to BF16 with RNE.  FP32 throughout; the oracle is the exact definition.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

constexpr int kAttWaves = 16;      // a chunk of 64 positions per wave at a time
constexpr int kAttMaxGroup = 8;    // Q heads per KV head
constexpr int kAttMaxDim = 128;    // head_dim
constexpr int kAttDimPerLane = kAttMaxDim / kWave;

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__global__ __launch_bounds__(kAttWaves * kWave) void decode_attention_kernel(AttnArgs p) {
  __shared__ float qs[kAttMaxGroup][kAttMaxDim];
  __shared__ float pw[kAttWaves][kAttMaxGroup][kWave];
  __shared__ int64_t pslot[kAttWaves][kWave];  // cache slot of each chunk position (-1: none)
  __shared__ float st_m[kAttWaves][kAttMaxGroup], st_l[kAttWaves][kAttMaxGroup];
  __shared__ float st_o[kAttWaves][kAttMaxGroup][kAttMaxDim];

  const int64_t m = blockIdx.x;
  const int kvh = static_cast<int>(blockIdx.y);
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int d = p.head_dim, G = p.group;
  const int32_t L = p.context_lens[m];
  if (L <= 0 || int64_t(L) > p.blocks_per_seq * p.block_size) return;

  for (int e = tid; e < G * d; e += kAttWaves * kWave) {
    const int h = e / d, i = e % d;
    qs[h][i] = bf16_bits_to_f32(p.q[m * p.ld_q + int64_t(kvh * G + h) * d + i]);
  }
  __syncthreads();

  float run_m[kAttMaxGroup], run_l[kAttMaxGroup], acc[kAttMaxGroup][kAttDimPerLane];
#pragma unroll
  for (int h = 0; h < kAttMaxGroup; ++h) {
    run_m[h] = -INFINITY;
    run_l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < kAttDimPerLane; ++c) acc[h][c] = 0.0f;
  }
  const int32_t* bt = p.block_table + m * p.blocks_per_seq;
  const int64_t row_stride = int64_t(p.n_kv) * d;  // one (block, offset) slot
  for (int32_t base = wave * kWave; base < L; base += kAttWaves * kWave) {
    // Scores: lane l takes position base + l.
    const int32_t j = base + lane;
    bool live = j < L;
    int64_t slot = 0;
    if (live) {
      const int32_t blk = bt[j / p.block_size];
      live = blk >= 0 && blk < p.num_blocks;
      slot = (int64_t(blk) * p.block_size + j % p.block_size) * row_stride + int64_t(kvh) * d;
    }
    pslot[wave][lane] = live ? slot : -1;
    float s[kAttMaxGroup];
#pragma unroll
    for (int h = 0; h < kAttMaxGroup; ++h) s[h] = 0.0f;
    {
      // The key row in groups of 64 elements: eight 16-byte loads issued together, then
      // used (a lane without a position reads row 0 and its scores are discarded).
      const uint16_t* kr = p.k_cache + (live ? slot : 0);
      for (int i0 = 0; i0 < d; i0 += 64) {
        u32x4 kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = *reinterpret_cast<const u32x4*>(kr + i0 + 8 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float kf[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[2 * c] = bf16_lo(kv[u][c]);
            kf[2 * c + 1] = bf16_hi(kv[u][c]);
          }
#pragma unroll
          for (int h = 0; h < kAttMaxGroup; ++h)
            if (h < G)
#pragma unroll
              for (int c = 0; c < 8; ++c) s[h] = fmaf(qs[h][i0 + 8 * u + c], kf[c], s[h]);
        }
      }
    }
    // Online softmax per head.
    float scale_old[kAttMaxGroup];
#pragma unroll
    for (int h = 0; h < kAttMaxGroup; ++h) {
      if (h >= G) break;
      const float sh = live ? s[h] * p.scale : -INFINITY;
      const float cmax = wave_max_f32(sh);
      const float nm = fmaxf(run_m[h], cmax);
      const float w = live ? __expf(sh - nm) : 0.0f;
      pw[wave][h][lane] = w;
      scale_old[h] = (run_m[h] == -INFINITY) ? 0.0f : __expf(run_m[h] - nm);
      run_l[h] = run_l[h] * scale_old[h] + wave_sum_f32(w);
      run_m[h] = nm;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's weights are in LDS
    __builtin_amdgcn_wave_barrier();
    // Values: lane owns dims lane, lane + 64, ...
#pragma unroll
    for (int h = 0; h < kAttMaxGroup; ++h) {
      if (h >= G) break;
#pragma unroll
      for (int c = 0; c < kAttDimPerLane; ++c) acc[h][c] *= scale_old[h];
    }
    // Eight positions per step: their slots come from LDS, all their value loads are
    // issued before any is used (a position without a slot reads row 0 of the cache and
    // has weight 0).
    const int32_t nj = (L - base) < kWave ? (L - base) : kWave;
    for (int32_t jj = 0; jj < nj; jj += 8) {
      float vf[8][kAttDimPerLane];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t sl = (jj + u < nj) ? pslot[wave][jj + u] : -1;
        const uint16_t* vr = p.v_cache + (sl >= 0 ? sl : 0);
#pragma unroll
        for (int c = 0; c < kAttDimPerLane; ++c) {
          const int i = lane + c * kWave;
          vf[u][c] = i < d ? bf16_bits_to_f32(vr[i]) : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (jj + u >= nj) break;
#pragma unroll
        for (int h = 0; h < kAttMaxGroup; ++h) {
          if (h >= G) break;
          const float w = pw[wave][h][jj + u];
#pragma unroll
          for (int c = 0; c < kAttDimPerLane; ++c) acc[h][c] = fmaf(w, vf[u][c], acc[h][c]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // Combine the waves.
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      st_m[wave][h] = run_m[h];
      st_l[wave][h] = run_l[h];
    }
#pragma unroll
    for (int c = 0; c < kAttDimPerLane; ++c) {
      const int i = lane + c * kWave;
      if (i < d) st_o[wave][h][i] = acc[h][c];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * d; e += kAttWaves * kWave) {
    const int h = e / d, i = e % d;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) mx = fmaxf(mx, st_m[w][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
      if (st_m[w][h] == -INFINITY) continue;
      const float f = __expf(st_m[w][h] - mx);
      o = fmaf(st_o[w][h][i], f, o);
      l = fmaf(st_l[w][h], f, l);
    }
    p.out[m * p.ld_q + int64_t(kvh * G + h) * d + i] = f32_to_bf16_rne(l > 0.0f ? o / l : 0.0f);
  }
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_attention_kernel, dim3(static_cast<unsigned>(a.M),
                                                   static_cast<unsigned>(a.n_kv)),
                     dim3(kAttWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace a8w8
