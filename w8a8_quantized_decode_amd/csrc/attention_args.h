// Kernel arguments of the attention side of the decode layer: QK-norm + RoPE + paged
// KV-cache write, and decode attention over the paged cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace a8w8 {

// ---------------------------------------------------------------- QK-norm + RoPE + KV
struct QkRopeArgs {
  const uint16_t* qkv;      // [M, ld_qkv] BF16: Q heads, then K heads, then V heads
  int64_t M, ld_qkv;
  int n_q, n_kv, head_dim;
  const uint16_t* q_gamma;  // [head_dim] BF16 QK-norm gains
  const uint16_t* k_gamma;
  float eps;
  const float* cos_table;   // [max_pos, head_dim / 2]
  const float* sin_table;
  int64_t max_pos;
  const int32_t* positions;    // [M]
  const int32_t* block_table;  // [M, blocks_per_seq]
  int64_t blocks_per_seq;
  uint16_t* k_cache;        // [num_blocks, block_size, n_kv, head_dim] BF16
  uint16_t* v_cache;
  int64_t num_blocks, block_size;
  uint16_t* q_out;          // [M, ld_q] BF16
  int64_t ld_q;
};
hipError_t launch_qk_rope(const QkRopeArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- decode attention
struct AttnArgs {
  const uint16_t* q;        // [M, ld_q] BF16, n_q heads of head_dim
  int64_t M, ld_q;
  int n_q, n_kv, group, head_dim;
  const uint16_t* k_cache;  // [num_blocks, block_size, n_kv, head_dim] BF16
  const uint16_t* v_cache;
  int64_t num_blocks, block_size;
  const int32_t* block_table;   // [M, blocks_per_seq]
  int64_t blocks_per_seq;
  const int32_t* context_lens;  // [M]
  float scale;
  uint16_t* out;            // [M, ld_q] BF16
  int64_t split_len;        // positions per split (a multiple of 64)
  int64_t n_split;          // splits per row: ceil(blocks_per_seq * block_size / split_len)
  int waves;                // waves per workgroup: 1 or 4 sharing each chunk, 8 on whole chunks
  float* ws_o;              // [M, n_q, n_split, head_dim] FP32 partial outputs (n_split > 1)
  float* ws_ml;             // [M, n_q, n_split, 2] FP32 partial (max, normalizer)
};
hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace a8w8
