// Decode attention over the paged BF16 KV cache, between QKV and O (pypto-lib PR #810
// walkthrough: attention loads use BF16 KV caches; pypto-serving PR #48: paged KV cache
// with a block table).
//
// The context of each (row, KV head) is cut into splits of split_len positions; one
// workgroup per (split, KV head, row) serves the group's Q heads (grouped-query
// attention: Q head h reads KV head h / (n_q / n_kv)) and walks its split in chunks of
// 64 positions.  Three shapes of workgroup, chosen by the host from the problem size:
//   * one wave (large grids: every workgroup stays resident at once);
//   * four waves, each taking a quarter of every chunk with its own online-softmax
//     state (small grids: shorter dependent chains per wave);
//   * eight waves on whole chunks of one unsplit context (short contexts: no partials
//     and no merge kernel).
// Per chunk:
//   * scores: a key row of D BF16 values is read by D/8 lanes, 16 bytes each, so one
//     load instruction covers 64/(D/8) rows.  Each lane keeps the matching 8 query
//     values of every head in registers, forms 8-term partial dot products, and the
//     row's lanes add them with DPP row permutations (no LDS traffic);
//   * online softmax: per head, the chunk's maximum and sum over the wave update the
//     running maximum and normalizer and rescale the output accumulators;
//   * values: value rows are read like key rows; each lane accumulates its 8 output
//     dimensions over the rows it reads, with the weights taken from a 64-entry LDS
//     table, and the row groups are summed once at the end of the split.
// The waves' states are merged through LDS.  With one split the workgroup writes
// rne_bf16(o / l) directly; otherwise it writes the split's FP32 (max, normalizer,
// unnormalized output) and a second kernel merges the splits of each (row, Q head).
// FP32 throughout; the oracle is the exact definition.
#include "device_common.h"
#include "attention_args.h"
#include "internal.h"

namespace a8w8 {
namespace {

// DPP control words (row = 16 lanes): quad_perm(1,0,3,2), quad_perm(2,3,0,1), row
// half-mirror (lane i of each 8 reads lane 7-i), row mirror (lane i reads lane 15-i).
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141,
              kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of kLanes (8 or 16) lanes; every lane of the group ends
// with the same value (each step adds two equal-order partial sums).
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (kLanes == 16) v += dpp_f32<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  return fmaxf(v, __shfl_xor(v, 32, kWave));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16, kWave);
  return v + __shfl_xor(v, 32, kWave);
}

__device__ __forceinline__ void unpack8(const u32x4& w, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

// kWhole: each wave takes whole chunks (wave w the chunks w, w + W, ...), with its own
// slot table and wave-level waits inside the chunk loop; otherwise the waves share each
// chunk, a quarter of its load instructions each.
template <int D, int G, int kAttnWaves, bool kWhole>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_split_kernel(AttnArgs p) {
  constexpr int LPR = D / 8;        // lanes per cache row
  constexpr int RG = kWave / LPR;   // rows per load instruction
  constexpr int T = LPR;            // load instructions per chunk (T * RG == 64)
  constexpr int TW = kWhole ? T : T / kAttnWaves;  // load instructions of each wave per chunk
  static_assert(kWhole || TW * kAttnWaves == T, "the chunk's loads split evenly over the waves");
  constexpr int kStride = kWhole ? kAttnWaves * kWave : kWave;  // positions between a wave's chunks
  __shared__ int64_t pslot[kWhole ? kAttnWaves : 1][kWave];  // cache offset of each chunk position (-1: none)
  __shared__ float pw[kAttnWaves][G][RG][TW];  // weight of position RG * (w*TW + u) + g
  __shared__ float st_m[kAttnWaves][G], st_l[kAttnWaves][G];
  __shared__ float st_o[kAttnWaves][G][D];

  const int64_t m = blockIdx.z;
  const int kvh = static_cast<int>(blockIdx.y);
  const int tid = threadIdx.x;
  const int wave = kAttnWaves == 1 ? 0 : tid / kWave;
  const int lane = tid % kWave;
  const int r = lane % LPR, g = lane / LPR;
  const int t0 = kWhole ? 0 : wave * TW;  // this wave's first load instruction
  const bool slot_thread = kWhole || kAttnWaves == 1 || tid < kWave;  // fills the chunk's slots
  const int ps = kWhole ? wave : 0;       // this wave's slot table
  // The context length, the query and the block number of the first position are
  // requested together (the table entry exists whenever the position is below
  // blocks_per_seq * block_size, which the host keeps below 2^30).
  const int32_t bs = static_cast<int32_t>(p.block_size);
  const int32_t max_ctx = static_cast<int32_t>(p.blocks_per_seq * p.block_size);
  const int32_t* bt = p.block_table + m * p.blocks_per_seq;
  const int32_t begin = static_cast<int32_t>(int64_t(blockIdx.x) * p.split_len);
  const int32_t first = kWhole ? begin + wave * kWave : begin;  // this wave's first chunk
  const int32_t L = p.context_lens[m];
  int32_t blk_next = (slot_thread && first + lane < max_ctx) ? bt[(first + lane) / bs] : -1;
  u32x4 qraw[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qraw[h] = *reinterpret_cast<const u32x4*>(p.q + m * p.ld_q + int64_t(kvh * G + h) * D + r * 8);
  if (L <= 0 || L > max_ctx || begin >= L) return;
  const int32_t end = static_cast<int32_t>(begin + p.split_len < L ? begin + p.split_len : L);

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) unpack8(qraw[h], qf[h]);
  float run_m[G], run_l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    run_m[h] = -INFINITY;
    run_l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.0f;
  }
  const int64_t row_stride = int64_t(p.n_kv) * D;
  // Lane (g, r) of wave w holds the scores of position RG * r + g when w * TW <= r <
  // (w + 1) * TW; its other lanes hold none.
  const bool owner = kWhole || (r >= t0 && r < t0 + TW);
  // Waits between a chunk's LDS writes and reads: the whole workgroup when the waves
  // share the chunk; the wave alone when it has the chunk to itself (the waves then run
  // different numbers of chunks).
  auto chunk_sync = [] {
    if constexpr (kWhole) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    } else {
      __syncthreads();
    }
  };

  for (int32_t base = first; base < end; base += kStride) {
    if (slot_thread) {
      const int32_t j = base + lane;
      const int32_t blk = blk_next;
      int64_t slot = -1;
      if (j < end && blk >= 0 && blk < p.num_blocks)
        slot = (int64_t(blk) * bs + j % bs) * row_stride + int64_t(kvh) * D;
      pslot[ps][lane] = slot;
      // the next chunk's block number is requested before this chunk's rows
      const int32_t jn = j + kStride;
      blk_next = (jn < end) ? bt[jn / bs] : -1;
    }
    chunk_sync();

    // Scores.  Load instruction t = t0 + u reads chunk position RG * t + g; the key
    // loads are in flight together, and the value loads are issued as soon as the keys
    // are used, so their latency overlaps the softmax.
    float sel[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sel[h] = 0.0f;
    bool has[TW];
    u32x4 kv[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int64_t sl = pslot[ps][RG * (t0 + u) + g];
      has[u] = sl >= 0;
      kv[u] = *reinterpret_cast<const u32x4*>(p.k_cache + (has[u] ? sl : 0) + r * 8);
    }
    u32x4 vv[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      float kf[8];
      unpack8(kv[u], kf);
      // the value row of the same position reuses this lane's address
      const int64_t sl = pslot[ps][RG * (t0 + u) + g];
      vv[u] = *reinterpret_cast<const u32x4*>(p.v_cache + (has[u] ? sl : 0) + r * 8);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qf[h][c], kf[c], s);
        s = group_sum<LPR>(s);
        sel[h] = (r == t0 + u) ? s : sel[h];
      }
    }
    const bool live = owner && pslot[ps][RG * r + g] >= 0;

    // Online softmax per head over this wave's positions.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sh = live ? sel[h] * p.scale : -INFINITY;
      const float nm = fmaxf(run_m[h], wave_max(sh));
      const float w = live ? __expf(sh - nm) : 0.0f;
      if (owner) pw[wave][h][g][r - t0] = w;
      const float f = (run_m[h] == -INFINITY) ? 0.0f : __expf(run_m[h] - nm);
      run_l[h] = run_l[h] * f + wave_sum(w);
      run_m[h] = nm;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= f;
    }
    chunk_sync();

    // Values: a position without a slot contributes nothing (its row is not used,
    // whatever row 0 of the cache holds).
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      if (!has[u]) continue;
      float vf[8];
      unpack8(vv[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = pw[wave][h][g][u];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(w, vf[c], acc[h][c]);
      }
    }
    chunk_sync();
  }

  // Sum the row groups (lanes with the same r hold the same output dimensions), then
  // hand each wave's state to LDS.
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] += __shfl_xor(acc[h][c], o, kWave);
  if constexpr (kAttnWaves == 1) {
    // One wave: its state is the split's; lanes 0 .. LPR-1 write it from registers.
    if (g != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (p.n_split == 1) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = run_l[h] > 0.0f ? acc[h][2 * i] / run_l[h] : 0.0f;
          const float b = run_l[h] > 0.0f ? acc[h][2 * i + 1] / run_l[h] : 0.0f;
          o[i] = uint32_t(f32_to_bf16_rne(a)) | (uint32_t(f32_to_bf16_rne(b)) << 16);
        }
        *reinterpret_cast<u32x4*>(p.out + m * p.ld_q + int64_t(kvh * G + h) * D + r * 8) = o;
      } else {
        const int64_t idx = (m * p.n_q + kvh * G + h) * p.n_split + blockIdx.x;
        float* o = p.ws_o + idx * D + r * 8;
        *reinterpret_cast<f32x4*>(o) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
        if (lane == 0) {
          p.ws_ml[2 * idx] = run_m[h];
          p.ws_ml[2 * idx + 1] = run_l[h];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      st_m[wave][h] = run_m[h];
      st_l[wave][h] = run_l[h];
    }
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) st_o[wave][h][r * 8 + c] = acc[h][c];
    }
  }
  __syncthreads();

  // Merge the waves; with one split the result is the output, otherwise the split's
  // partial (max, normalizer, unnormalized output).
  for (int e = tid; e < G * D; e += kAttnWaves * kWave) {
    const int h = e / D, i = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mx = fmaxf(mx, st_m[w][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      if (st_m[w][h] == -INFINITY) continue;
      const float f = __expf(st_m[w][h] - mx);
      o = fmaf(st_o[w][h][i], f, o);
      l = fmaf(st_l[w][h], f, l);
    }
    if (p.n_split == 1) {
      p.out[m * p.ld_q + int64_t(kvh * G + h) * D + i] = f32_to_bf16_rne(l > 0.0f ? o / l : 0.0f);
    } else {
      const int64_t idx = (m * p.n_q + kvh * G + h) * p.n_split + blockIdx.x;
      p.ws_o[idx * D + i] = o;
      if (i == 0) {
        p.ws_ml[2 * idx] = mx;
        p.ws_ml[2 * idx + 1] = l;
      }
    }
  }
}

// Merge the splits of one (row, Q head): o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Lane s of each group of 64 splits forms that split's factor and the factors go through
// LDS; each lane sums its output dimensions over the splits with 32 splits' loads in
// flight, the first 32 requested before the maxima are known.
template <int D>
__global__ __launch_bounds__(kWave) void attn_combine_kernel(AttnArgs p) {
  constexpr int DPL = D / kWave;  // output dimensions per lane
  constexpr int kB = 32;          // splits per batch of loads
  __shared__ float fs[kWave];
  const int64_t m = blockIdx.y;
  const int hq = static_cast<int>(blockIdx.x);
  const int lane = threadIdx.x;
  const int32_t L = p.context_lens[m];
  if (L <= 0 || int64_t(L) > p.blocks_per_seq * p.block_size) return;
  const int64_t ns = (int64_t(L) + p.split_len - 1) / p.split_len;
  const int64_t idx0 = (m * p.n_q + hq) * p.n_split;
  const float* ml = p.ws_ml + 2 * idx0;
  const float* po = p.ws_o + idx0 * D + lane;
  float v[kB][DPL];
#pragma unroll
  for (int u = 0; u < kB; ++u)
#pragma unroll
    for (int c = 0; c < DPL; ++c) v[u][c] = (u < ns) ? po[int64_t(u) * D + c * kWave] : 0.0f;
  float mx = -INFINITY;
  for (int64_t s = lane; s < ns; s += kWave) mx = fmaxf(mx, ml[2 * s]);
  mx = wave_max(mx);
  float l = 0.0f, o[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) o[c] = 0.0f;
  for (int64_t s0 = 0; s0 < ns; s0 += kWave) {
    float f = 0.0f;
    if (s0 + lane < ns) {
      const float ms = ml[2 * (s0 + lane)];
      if (ms != -INFINITY) {
        f = __expf(ms - mx);
        l = fmaf(ml[2 * (s0 + lane) + 1], f, l);
      }
    }
    fs[lane] = f;
    __syncthreads();
    const int nb = static_cast<int>(ns - s0 < kWave ? ns - s0 : kWave);
    for (int u0 = 0; u0 < nb; u0 += kB) {
      if (s0 + u0 > 0) {
#pragma unroll
        for (int u = 0; u < kB; ++u)
#pragma unroll
          for (int c = 0; c < DPL; ++c)
            v[u][c] = (u0 + u < nb) ? po[(s0 + u0 + u) * D + c * kWave] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u)
#pragma unroll
        for (int c = 0; c < DPL; ++c) o[c] = fmaf(fs[(u0 + u) & (kWave - 1)], v[u][c], o[c]);
    }
    __syncthreads();
  }
  l = wave_sum(l);
#pragma unroll
  for (int c = 0; c < DPL; ++c)
    p.out[m * p.ld_q + int64_t(hq) * D + lane + c * kWave] =
        f32_to_bf16_rne(l > 0.0f ? o[c] / l : 0.0f);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_split), static_cast<unsigned>(a.n_kv),
                  static_cast<unsigned>(a.M));
  switch (a.group * 16 + a.waves) {
#define A8W8_ATTN_CASE(GG)                                                                  \
  case GG * 16 + 1:                                                                         \
    hipLaunchKernelGGL((attn_split_kernel<D, GG, 1, false>), grid, dim3(kWave), 0, stream, a); \
    break;                                                                                  \
  case GG * 16 + 4:                                                                         \
    hipLaunchKernelGGL((attn_split_kernel<D, GG, 4, false>), grid, dim3(4 * kWave), 0, stream, a); \
    break;                                                                                  \
  case GG * 16 + 8:                                                                         \
    hipLaunchKernelGGL((attn_split_kernel<D, GG, 8, true>), grid, dim3(8 * kWave), 0, stream, a); \
    break;
    A8W8_ATTN_CASE(1) A8W8_ATTN_CASE(2) A8W8_ATTN_CASE(3) A8W8_ATTN_CASE(4)
    A8W8_ATTN_CASE(5) A8W8_ATTN_CASE(6) A8W8_ATTN_CASE(7) A8W8_ATTN_CASE(8)
#undef A8W8_ATTN_CASE
    default: return hipErrorInvalidValue;
  }
  if (a.n_split > 1)
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(static_cast<unsigned>(a.n_q),
                                                      static_cast<unsigned>(a.M)),
                       dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace a8w8
