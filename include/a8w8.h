/*
 * a8w8.h -- C ABI of liba8w8: the A8W8 decode-step linears of a Qwen3-14B-shaped
 * transformer layer on MI355X (gfx950), with the attention side of the decode layer
 * (QK-norm + RoPE + paged BF16 KV-cache write, decode attention over the paged cache)
 * and the whole decode layer built from them.
 *
 * What is computed (sources: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode
 * scheduling and data paths", sections What changed > Decode scheduling and > Gate/Up
 * INT8 path, Validation, and its CodeRabbit walkthrough table; pypto-serving PR #48
 * "Add native Qwen3 14B A8W8 serving path", CodeRabbit comment on _hf_linear_to_bf16
 * and the PR body section Compatibility and boundaries):
 *
 *   RMSNorm -> per-row dynamic INT8 quantization (FP32 row scale) -> INT8 x INT8 ->
 *   INT32 GEMM against INT8 weights with per-output-channel FP32 scales -> dequant
 *   (activation-row scale, then weight-channel scale) -> SiLU(gate) * up -> per-row
 *   requantization -> Down projection split along K into independent partitions, each
 *   dequantized to an FP32 partial -> partials summed, BF16 residual added, narrowed
 *   to BF16 with round-to-nearest-even.  QKV and O use the same quantize -> INT8 GEMM ->
 *   dequant pattern.  A W8A16 prefill mode dequantizes INT8 weight tiles to BF16 for
 *   BF16 matrix cores (PR #810, Gate/Up INT8 path: prefill keeps the shared INT8
 *   weights by dequantizing each tile to BF16).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are caller-owned DEVICE memory on the current HIP device.
 *     The library allocates nothing and keeps no pointer after a call returns.
 *   - BF16 values travel as uint16_t bit patterns.  Tensors are row-major and dense
 *     unless a leading dimension says otherwise.  Every pointer must be 16-byte aligned.
 *   - Weights are [N_out, K_in] row-major INT8; the FP32 scale has one entry per output
 *     channel (per row of the weight).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work;
 *     buffers must stay alive until the stream has passed it.
 *   - All arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a status other than A8W8_OK is returned.  M == 0 is
 *     a valid no-op.  No exception crosses the ABI and nothing aborts.  Values are not
 *     checked: non-finite inputs give unspecified outputs.  Kernel faults surface at
 *     the caller's next synchronization, as for any HIP kernel.
 *   - No output may alias an input except where stated.
 */
#ifndef A8W8_H
#define A8W8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum a8w8_status {
  A8W8_OK = 0,
  A8W8_ERR_NULL = 1,        /* a required pointer is NULL                          */
  A8W8_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or not
                               a multiple the kernels need                          */
  A8W8_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                     */
  A8W8_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than a8w8_workspace_bytes  */
  A8W8_ERR_UNSUPPORTED = 5, /* valid request the library does not implement          */
  A8W8_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed           */
} a8w8_status;

typedef enum a8w8_mode {
  A8W8_MODE_DECODE_A8W8 = 0,   /* INT8 activations x INT8 weights, INT32 accumulate */
  A8W8_MODE_PREFILL_W8A16 = 1  /* BF16 activations x BF16-dequantized weight tiles  */
} a8w8_mode;

typedef enum a8w8_op {
  A8W8_OP_MLP_BLOCK = 0,
  A8W8_OP_LAYER_LINEARS = 1
} a8w8_op;

/*
 * Weight layouts.  ROWMAJOR: w[n * K + k].  TILED: the same bytes regrouped into
 * 16-row tiles, one 1 KB block per 64-byte K step, each block in the operand order of
 * the gfx950 INT8 matrix instruction (v_mfma_i32_16x16x64_i8):
 *   tiled[(n / 16) * 16 * K + (k / 64) * 1024 + 16 * (n % 16 + 16 * ((k % 64) / 16))
 *         + k % 16] = w[n * K + k].
 * In the tiled layout every load instruction of the decode kernels reads 1 KB of
 * consecutive bytes, which streams HBM faster than 64-byte pieces of 16 rows.  The
 * serving loader converts checkpoint layouts once at load time (pypto-serving PR #48,
 * loader walkthrough), which is where a8w8_pack_weight belongs.
 */
typedef enum a8w8_layout {
  A8W8_LAYOUT_ROWMAJOR = 0,
  A8W8_LAYOUT_TILED = 1
} a8w8_layout;

/* One quantized weight: w [N_out, K_in] INT8 in `layout`, scale [N_out] FP32. */
typedef struct a8w8_qweight {
  const int8_t* w;
  const float* scale;
  int layout; /* a8w8_layout */
} a8w8_qweight;

/*
 * Kernel roles, for the timing hook (ev_kernel).  Which kernels a call launches depends
 * on M: with M <= 4 rows the GEMMs quantize their inputs in their prologues (roles 1, 3,
 * 5, 7 only); with more rows separate row-quantization kernels (0, 2, 4, 6) run first.
 */
typedef enum a8w8_kernel {
  A8W8_KERNEL_QUANT_IN = 0,    /* RMSNorm(gamma_in) + quantization before QKV     */
  A8W8_KERNEL_QKV = 1,
  A8W8_KERNEL_QUANT_ATTN = 2,  /* quantization of the attention output before O  */
  A8W8_KERNEL_O = 3,
  A8W8_KERNEL_QUANT_POST = 4,  /* post-attention RMSNorm + quantization          */
  A8W8_KERNEL_GATE_UP = 5,
  A8W8_KERNEL_REQUANT = 6,     /* requantization of silu(g) * u before Down       */
  A8W8_KERNEL_DOWN = 7,
  A8W8_KERNEL_REDUCE = 8       /* reserved: no current path launches this role     */
} a8w8_kernel;

/*
 * Diagnostic taps of the MLP block.  Every member may be NULL; a non-NULL device
 * pointer receives that intermediate (written in addition to the normal work).  Sizes
 * use the call's M, H (hidden), I (intermediate) and split_k.
 *
 * Decode mode:
 *   xn [M,H] FP32 RMSNorm output; q_x [M,H] INT8 codes; s_x [M] row scales;
 *   acc_gate, acc_up [M,I] INT32; h [M,I] FP32 = silu(g)*u; q_h [M,I] INT8; s_h [M];
 *   acc_down [split_k,M,H] INT32 per K partition; p_down [split_k,M,H] FP32 partials.
 * Prefill mode:
 *   xn [M,H] FP32; a_bf16 [M,H] BF16 activations; g, u [M,I] FP32 accumulators;
 *   h_bf16 [M,I] BF16; d [M,H] FP32 Down accumulator (before the residual).
 *
 * Timing hook: when ev_start and ev_stop are non-NULL hipEvent_t handles, the call
 * records ev_start right before and ev_stop right after launching the kernel whose role
 * (a8w8_kernel) is ev_kernel, on `stream`; nothing is recorded if the call launches no
 * kernel of that role.
 */
typedef struct a8w8_mlp_taps {
  float* xn;
  int8_t* q_x;
  float* s_x;
  int32_t* acc_gate;
  int32_t* acc_up;
  float* h;
  int8_t* q_h;
  float* s_h;
  int32_t* acc_down;
  float* p_down;
  uint16_t* a_bf16;
  float* g;
  float* u;
  uint16_t* h_bf16;
  float* d;
  void* ev_start;
  void* ev_stop;
  int ev_kernel;
} a8w8_mlp_taps;

/*
 * Diagnostic taps of the layer linears (decode).  Same rules as a8w8_mlp_taps.
 *   xn_in [M,H] FP32; q_in [M,H]; s_in [M]; acc_qkv [M,n_qkv] INT32;
 *   qkv [M,n_qkv] BF16; q_attn [M,n_q*head_dim]; s_attn [M]; acc_o [M,H] INT32;
 *   h1 [M,H] BF16 (attention-block output = MLP input and residual); mlp = MLP taps.
 * The timing hook of a layer call lives in mlp.ev_start / mlp.ev_stop / mlp.ev_kernel.
 */
typedef struct a8w8_layer_taps {
  float* xn_in;
  int8_t* q_in;
  float* s_in;
  int32_t* acc_qkv;
  uint16_t* qkv;
  int8_t* q_attn;
  float* s_attn;
  int32_t* acc_o;
  uint16_t* h1;
  a8w8_mlp_taps mlp;
} a8w8_layer_taps;

/*
 * Converts a row-major weight [N, K] into the tiled layout (see a8w8_layout) on the
 * device.  N % 16 == 0, K % 64 == 0; w and w_tiled do not overlap.  One kernel.
 * The scale vector is unchanged by the layout.
 */
a8w8_status a8w8_pack_weight(const int8_t* w, int64_t N, int64_t K, int8_t* w_tiled,
                             void* stream);

/*
 * Per-row dynamic INT8 quantization of BF16 rows, optionally after RMSNorm.
 *   x_bf16 [M, ldx] BF16 (row stride ldx elements, ldx >= K, ldx % 8 == 0);
 *   gamma_bf16 [K] BF16 RMSNorm gain, or NULL for no norm (eps is then ignored);
 *   q_out [M, K] INT8 codes; row_scale_out [M] FP32; xn_tap [M, K] FP32 or NULL.
 * Per row: v = RMSNorm(x) (or x); a = max|v|; s = a/127; q = clamp(rint(v/s), -127,
 * 127) with ties to even; s == 0 gives all-zero codes.  K > 0, K % 8 == 0.
 * (PR #810 What changed: activation quantization once per row, batched over all
 * decode rows.)  One kernel.
 */
a8w8_status a8w8_quantize_rows(const uint16_t* x_bf16, int64_t ldx,
                               const uint16_t* gamma_bf16, float eps, int64_t M,
                               int64_t K, int8_t* q_out, float* row_scale_out,
                               float* xn_tap, void* stream);

/*
 * One A8W8 linear on already-quantized rows.
 *   q [M, K] INT8 codes, row_scale [M] FP32, W = {w [N, K] INT8, scale [N] FP32};
 *   residual_bf16 [M, N] BF16 or NULL; y_bf16 [M, N] BF16 output;
 *   acc_i32_tap [M, N] INT32 or NULL.
 * y = rne_bf16((f32(acc) * row_scale[m]) * scale[n] [+ residual]).
 * K % 64 == 0, 0 < K <= 131072 (INT32 accumulators cannot overflow), N % 16 == 0,
 * M <= 65535 * 64 (one grid row per 64 rows).  y may alias residual_bf16.  One kernel.
 * (pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data paths",
 * What changed > Gate/Up INT8 path: INT8 x INT8 products summed in INT32, the sums turned
 * into FP32 with the row scale and the channel scale; the decode layer's QKV and output
 * projections use the same arithmetic, What changed > Decode scheduling.)
 */
a8w8_status a8w8_linear(const int8_t* q, const float* row_scale, a8w8_qweight W,
                        const uint16_t* residual_bf16, int64_t M, int64_t N,
                        int64_t K, uint16_t* y_bf16, int32_t* acc_i32_tap,
                        void* stream);

/*
 * Workspace size in bytes for a8w8_mlp_block (op = A8W8_OP_MLP_BLOCK, n_qkv ignored)
 * or a8w8_layer_linears (op = A8W8_OP_LAYER_LINEARS).  Returns 0 for invalid
 * arguments.  (Caller-owned device scratch, allocated once and reused across calls, the
 * way the runner of pypto-serving PR #61 "Add Qwen3 A8W8 L2 runner foundation", Summary,
 * caches its worker-side tensor allocations.)  The workspace is scratch: its contents on entry do not matter and are
 * unspecified on return.  Its first 256 bytes hold two tag words that the decode GEMMs
 * advance on the device (each GEMM reads one and writes the next value to the other);
 * partial sums exchanged between workgroups carry that tag, so nothing is cleared
 * between calls, and a call captured into a HIP graph stays correct when replayed (the
 * tags move on every replay).  A zero-filled workspace is the usual start; any other
 * content works except with negligible probability (a stale word matching a 32-bit tag).
 * A workspace can serve later calls of any size it fits; calls that share a workspace
 * must not overlap in time.  The workspace must be 256-byte aligned.
 */
size_t a8w8_workspace_bytes(int op, int64_t M, int64_t H, int64_t I, int64_t n_qkv,
                            int split_k, int mode);

/*
 * The MLP block of one layer.
 *   x_bf16 [M, H] BF16 input; gamma_bf16 [H] post-attention RMSNorm gain; eps;
 *   gate, up: W [I, H]; down: W [H, I]; residual_bf16 [M, H]; out_bf16 [M, H].
 *   split_k in {1, 2, 4, 8}: Down is computed in split_k contiguous K partitions of
 *   I/split_k, each dequantized to its own FP32 partial (PR #810 What changed >
 *   Decode scheduling and the CodeRabbit walkthrough row on the split Down
 *   projection); out = rne_bf16((p_0 + p_1 + ...) + residual).
 *   mode: A8W8_MODE_DECODE_A8W8 or A8W8_MODE_PREFILL_W8A16 (prefill ignores split_k
 *   for its numerics: Down is one FP32-accumulated sum).
 *   workspace: ws_bytes >= a8w8_workspace_bytes(A8W8_OP_MLP_BLOCK, ...), 256-byte
 *   aligned scratch.  taps: a8w8_mlp_taps or NULL.
 * Shapes: H % 64 == 0, I % (64 * split_k) == 0, H and I <= 131072, M <= 65535 * 64.
 * out may alias
 * residual_bf16 or x_bf16.
 * Prefill mode (any M; built for M in the hundreds): a = rne_bf16(RMSNorm(x)); every
 * weight tile is dequantized to W' = rne_bf16(fl32(w * s)) on the fly; Gate/Up
 * accumulate in FP32 on BF16 matrix cores; h = rne_bf16(silu(g) * u); Down accumulates
 * in FP32 (a K range split between workgroups is added back in K order, so results
 * are reproducible run to run); out = rne_bf16(d + residual).  Additionally needs
 * H % 256 == 0, I % 256 == 0 and M * max(H, I) < 2^31.  Kernels: QUANT_POST (norm),
 * GATE_UP, DOWN (with the residual add).
 */
a8w8_status a8w8_mlp_block(const uint16_t* x_bf16, const uint16_t* gamma_bf16, float eps,
                           a8w8_qweight gate, a8w8_qweight up, a8w8_qweight down,
                           const uint16_t* residual_bf16, uint16_t* out_bf16, int64_t M,
                           int64_t H, int64_t I, int split_k, int mode, void* workspace,
                           size_t ws_bytes, const a8w8_mlp_taps* taps, void* stream);

/*
 * All linears of one decode layer, attention replaced by identity (decode mode).
 *   x_bf16 [M, H]; gamma_in, gamma_post [H]; qkv: W [n_qkv, H] with
 *   n_qkv = (n_q_heads + 2 * n_kv_heads) * head_dim and n_q_heads * head_dim == H;
 *   o: W [H, H]; gate/up/down as in a8w8_mlp_block.
 * Steps: RMSNorm(gamma_in) -> quant -> QKV -> qkv = rne_bf16(dequant) -> the Q slice
 * qkv[:, :H] stands in for the attention output -> quant -> O -> h1 = rne_bf16(dequant
 * + x) -> MLP block with input h1 and residual h1.
 * (pypto-serving issue #52 "[Feature] Add native Qwen3-14B A8W8 serving path", Proposed
 * behavior: the A8W8 decode layer; its linears in the order of the CodeRabbit
 * walkthrough of pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and
 * data paths".)
 *   qkv_out_bf16 [M, n_qkv] receives qkv, or NULL to keep it in the workspace;
 *   out_bf16 [M, H]; workspace from a8w8_workspace_bytes(A8W8_OP_LAYER_LINEARS, ...).
 * out may alias x_bf16.
 */
a8w8_status a8w8_layer_linears(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                               const uint16_t* gamma_post_bf16, float eps,
                               a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                               a8w8_qweight up, a8w8_qweight down, int64_t M, int64_t H,
                               int64_t I, int n_q_heads, int n_kv_heads, int head_dim,
                               int split_k, uint16_t* qkv_out_bf16, uint16_t* out_bf16,
                               void* workspace, size_t ws_bytes,
                               const a8w8_layer_taps* taps, void* stream);

/*
 * a8w8_layer_linears without a workspace argument, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and errors as a8w8_layer_linears;
 * the workspace is a device array inside the library, one per GPU, of
 * a8w8_layer_linears_static_max_workspace() bytes (16 MiB: Qwen3-14B shapes up to
 * M = 16 need about 8.7 MB), kept until the process ends.  A call whose workspace
 * would exceed it returns A8W8_ERR_WORKSPACE before anything is enqueued.  The call
 * itself allocates nothing; its first call on a device looks up that device's array
 * (A8W8_ERR_HIP if the lookup fails).  Every call on one GPU shares the array, which
 * keeps the previous call's contents (none of which need clearing, as for any
 * workspace): calls that overlap in time on one GPU race and must be serialized by
 * the caller, e.g. by issuing them on one stream.
 */
size_t a8w8_layer_linears_static_max_workspace(void);
a8w8_status a8w8_layer_linears_static(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                                      const uint16_t* gamma_post_bf16, float eps,
                                      a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                                      a8w8_qweight up, a8w8_qweight down, int64_t M, int64_t H,
                                      int64_t I, int n_q_heads, int n_kv_heads, int head_dim,
                                      int split_k, uint16_t* qkv_out_bf16, uint16_t* out_bf16,
                                      const a8w8_layer_taps* taps, void* stream);

/*
 * All linears of one prefill layer, W8A16 on the shared INT8 weights (pypto-lib PR #810,
 * What changed > Gate/Up INT8 path: prefill turns each INT8 weight tile into BF16 values; the
 * layer composition is the decode layer's with that linear).  Same shapes as
 * a8w8_layer_linears; attention replaced by identity.
 * Steps: a = rne_bf16(RMSNorm(x, gamma_in)) -> qkv = rne_bf16(a W'_qkv^T) -> the Q slice
 * qkv[:, :H] -> h1 = rne_bf16(attn W'_o^T + x) -> the prefill MLP block (a8w8_mlp_block in
 * A8W8_MODE_PREFILL_W8A16) with input h1 and residual h1.  W' = rne_bf16(w * scale) per
 * tile; products accumulate in FP32 on BF16 matrix cores.
 *   qkv_out_bf16 [M, n_qkv] receives qkv, h1_out_bf16 [M, H] receives h1 (each may be
 *   NULL: kept in the workspace); out_bf16 [M, H] (may alias x_bf16); workspace from
 *   a8w8_workspace_bytes(A8W8_OP_LAYER_LINEARS, M, H, I, n_qkv, 2,
 *   A8W8_MODE_PREFILL_W8A16).
 * Needs H % 256 == 0, I % 256 == 0, n_qkv % 128 == 0, M * max(H, I, n_qkv) < 2^31.
 * Errors as a8w8_layer_linears (shape errors before any launch).  Kernels: row norm,
 * QKV GEMM, Q-slice copy to the operand layout, O GEMM, then the prefill MLP's kernels.
 */
a8w8_status a8w8_layer_linears_prefill(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                                       const uint16_t* gamma_post_bf16, float eps,
                                       a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                                       a8w8_qweight up, a8w8_qweight down, int64_t M,
                                       int64_t H, int64_t I, int n_q_heads, int n_kv_heads,
                                       int head_dim, uint16_t* qkv_out_bf16,
                                       uint16_t* h1_out_bf16, uint16_t* out_bf16,
                                       void* workspace, size_t ws_bytes, void* stream);

/*
 * QK-norm, rotate-half RoPE and the paged BF16 KV-cache write after the QKV projection
 * (pypto-serving issue #52, Current behavior: the fused QK-norm path and its Q RoPE;
 * pypto-lib PR #810 walkthrough, BF16 cache and interface contracts: RoPE writes into
 * BF16 KV caches; pypto-serving PR #48: paged KV cache with a block table).
 *   qkv_bf16 [M, (n_q + 2 n_kv) * d]: Q heads, then K heads, then V heads (the QKV
 *   projection's output); q_gamma, k_gamma [d] BF16 (shared by the heads of each kind);
 *   cos_table, sin_table [max_pos, d/2] FP32 (4-byte aligned; the caller's angles);
 *   positions [M] int32; block_table [M, blocks_per_seq] int32;
 *   k_cache, v_cache [num_blocks, block_size, n_kv, d] BF16; q_out [M, n_q * d] BF16.
 * Per row m at position p: each Q head -> rne_bf16(rope(RMSNorm_d(q, q_gamma))) into
 * q_out; each K head likewise with k_gamma, and each V head as it is, into the cache slot
 * (block_table[m, p / block_size], p % block_size).  RMSNorm over a head as in
 * a8w8_quantize_rows; rope: o[i] = x[i] c - x[i+d/2] s, o[i+d/2] = x[i+d/2] c + x[i] s
 * with c, s = cos/sin_table[p, i], each product and sum one FP32 operation.
 * Shapes: d even and <= 512, n_q > 0, n_kv >= 0 (k_gamma, block_table and the caches may
 * be NULL when n_kv == 0), M <= 65535.  A row whose position is outside [0, max_pos) or
 * whose block index or block number is out of range is skipped (its outputs are not
 * written).  One kernel.
 */
a8w8_status a8w8_qk_norm_rope_kv(const uint16_t* qkv_bf16, int64_t M, int n_q_heads,
                                 int n_kv_heads, int head_dim, const uint16_t* q_gamma_bf16,
                                 const uint16_t* k_gamma_bf16, float eps,
                                 const float* cos_table, const float* sin_table,
                                 int64_t max_pos, const int32_t* positions,
                                 const int32_t* block_table, int64_t blocks_per_seq,
                                 uint16_t* k_cache_bf16, uint16_t* v_cache_bf16,
                                 int64_t num_blocks, int64_t block_size, uint16_t* q_out_bf16,
                                 void* stream);

/*
 * Decode attention over the paged BF16 KV cache, between QKV (after
 * a8w8_qk_norm_rope_kv) and O (pypto-lib PR #810 walkthrough: attention loads use BF16
 * KV caches; pypto-serving PR #48: paged KV cache with a block table).
 *   q_bf16 [M, n_q * d] and out_bf16 [M, n_q * d] (16-byte aligned);
 *   k_cache, v_cache [num_blocks, block_size, n_kv, d] BF16 (16-byte aligned);
 *   block_table [M, blocks_per_seq] int32; context_lens [M] int32.
 * Row m attends to its positions 0 .. L-1 (L = context_lens[m]) at the cache slots
 * (block_table[m, j / block_size], j % block_size); Q head h uses KV head
 * h / (n_q / n_kv).  out = rne_bf16(sum_j softmax_j(scale * q . k_j) v_j), computed in
 * FP32 with an online softmax.  Shapes: n_q % n_kv == 0, n_q / n_kv <= 8, d in {64, 128},
 * M <= 65535, blocks_per_seq * block_size <= 2^30.  A row with L outside
 * [1, blocks_per_seq * block_size] is skipped (its output is not written); a position
 * whose block number is out of range is left out of the softmax, and a row with no
 * position left gets zeros.
 * workspace: NULL, or ws_bytes >= a8w8_decode_attention_workspace_bytes(M, n_q, n_kv,
 * d, blocks_per_seq * block_size), 256-byte aligned scratch (contents on entry do not
 * matter; calls that share a workspace must not overlap in time).  The size query
 * returns 0 for invalid shapes and when the context needs no split.  With a workspace
 * the context of each row is cut into splits that separate workgroups take (one kernel
 * for the splits, one that merges them; the merge runs only when there is more than
 * one split); with NULL one workgroup per (row, KV head) walks the whole context (one
 * kernel; slow for long contexts at small M).  Errors: A8W8_ERR_SHAPE, _NULL, _ALIGN
 * (q, out, the caches or the workspace misaligned), _WORKSPACE (too small).
 */
size_t a8w8_decode_attention_workspace_bytes(int64_t M, int n_q_heads, int n_kv_heads,
                                             int head_dim, int64_t max_context);
a8w8_status a8w8_decode_attention(const uint16_t* q_bf16, int64_t M, int n_q_heads,
                                  int n_kv_heads, int head_dim, const uint16_t* k_cache_bf16,
                                  const uint16_t* v_cache_bf16, int64_t num_blocks,
                                  int64_t block_size, const int32_t* block_table,
                                  int64_t blocks_per_seq, const int32_t* context_lens,
                                  float scale, uint16_t* out_bf16, void* workspace,
                                  size_t ws_bytes, void* stream);

/*
 * Inputs and buffers of the attention step inside a8w8_decode_layer: the arguments of
 * a8w8_qk_norm_rope_kv and a8w8_decode_attention that the layer does not already hold.
 *   q_gamma_bf16, k_gamma_bf16 [d]; qk_eps; cos_table, sin_table [max_pos, d/2] FP32;
 *   positions [M] (the new token's position), context_lens [M] (positions attended,
 *   normally positions + 1); block_table [M, blocks_per_seq]; k_cache, v_cache
 *   [num_blocks, block_size, n_kv, d] BF16 (the step writes the new token's K and V);
 *   scale; q_rot_bf16 [M, n_q * d] and attn_bf16 [M, n_q * d] caller buffers that
 *   receive the rotated Q and the attention output (O's input); attn_workspace /
 *   attn_ws_bytes as the workspace of a8w8_decode_attention (may be NULL).
 */
typedef struct a8w8_attention_step {
  const uint16_t* q_gamma_bf16;
  const uint16_t* k_gamma_bf16;
  float qk_eps;
  const float* cos_table;
  const float* sin_table;
  int64_t max_pos;
  const int32_t* positions;
  const int32_t* context_lens;
  const int32_t* block_table;
  int64_t blocks_per_seq;
  uint16_t* k_cache_bf16;
  uint16_t* v_cache_bf16;
  int64_t num_blocks;
  int64_t block_size;
  float scale;
  uint16_t* q_rot_bf16;
  uint16_t* attn_bf16;
  void* attn_workspace;
  size_t attn_ws_bytes;
} a8w8_attention_step;

/*
 * One decode layer with real attention: QKV (as in a8w8_layer_linears), QK-norm + RoPE +
 * KV-cache write (a8w8_qk_norm_rope_kv), decode attention over the paged cache
 * (a8w8_decode_attention), then O on the attention output with the layer input as
 * residual -> h1, then the MLP block (PR #810 walkthrough: the layer's order QKV ->
 * QK-norm/RoPE -> BF16 KV cache and attention -> O -> post-attention norm -> MLP).
 * Arguments as in a8w8_layer_linears (workspace sized by a8w8_workspace_bytes with
 * A8W8_OP_LAYER_LINEARS) and a8w8_attention_step; attn must not be NULL and its shapes
 * follow the two steps' rules (d in {64, 128}, n_q / n_kv <= 8).  qkv_out_bf16 [M, n_qkv]
 * and h1_out_bf16 [M, H] are optional outputs (NULL: kept in the workspace).  Every
 * argument is checked before anything is enqueued.
 */
a8w8_status a8w8_decode_layer(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                              const uint16_t* gamma_post_bf16, float eps, a8w8_qweight qkv,
                              a8w8_qweight o, a8w8_qweight gate, a8w8_qweight up,
                              a8w8_qweight down, int64_t M, int64_t H, int64_t I,
                              int n_q_heads, int n_kv_heads, int head_dim, int split_k,
                              const a8w8_attention_step* attn, uint16_t* qkv_out_bf16,
                              uint16_t* h1_out_bf16, uint16_t* out_bf16, void* workspace,
                              size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* a8w8_status_string(a8w8_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int a8w8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* A8W8_H */
