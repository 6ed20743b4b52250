// Internal interface between the C-ABI layer (a8w8_api.cpp) and the kernel files.
// Host-only declarations; no torch or Python types anywhere in the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace a8w8 {

// ---------------------------------------------------------------- row quantization
struct QuantRowsArgs {
  const void* x;            // [M, ldx] BF16 bits (uint16) or FP32
  int64_t ldx;              // row stride in elements
  int x_is_f32;             // 0: BF16 input, 1: FP32 input
  const uint16_t* gamma;    // [K] BF16 RMSNorm gain or nullptr (no norm)
  float eps;
  int64_t M, K;
  int8_t* q;                // [M, K] codes (row stride K)
  float* s;                 // [M] row scales
  float* xn_tap;            // [M, K] FP32 or nullptr
  int8_t* q_tap;            // [M, K] or nullptr (copy of q)
  float* s_tap;             // [M] or nullptr (copy of s)
  uint16_t* a_bf16;         // [M, K] rne_bf16(v) or nullptr (prefill activations)
  uint16_t* a_bf16_tap;     // [M, K] or nullptr
  int write_codes;          // 0: skip the INT8 codes (prefill only needs a_bf16)
  // Extra workgroups beyond the M row workgroups zero this region (16-byte aligned,
  // a multiple of 16 bytes): the split-K accumulators and counters of the GEMMs that
  // follow in the same call.
  void* zero_ptr;
  size_t zero_bytes;
};
hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- weight layouts
// LAYOUT_ROWMAJOR: w[n * K + k].
// LAYOUT_TILED: 16-row tiles, one 1 KB block per 64-byte k step, each block in the
// operand order of v_mfma_i32_16x16x64_i8:
//   byte (n/16) * 16K + (k/64) * 1024 + 16 * lane + b, lane = (n % 16) + 16 * ((k % 64) / 16),
//   b = k % 16.
enum WeightLayout : int { LAYOUT_ROWMAJOR = 0, LAYOUT_TILED = 1 };
hipError_t launch_pack_tiled(const int8_t* w, int64_t N, int64_t K, int8_t* out,
                             hipStream_t stream);

// ---------------------------------------------------------------- decode GEMM
enum DecodeEpilogue : int {
  EPI_BF16 = 0,       // y = rne_bf16(dequant(acc))
  EPI_BF16_RES = 1,   // y = rne_bf16(dequant(acc) + res)
  EPI_SILU = 2,       // two weights: h = silu(dequant(acc_g)) * dequant(acc_u), FP32
  EPI_DOWN = 3        // K partitions: out = rne_bf16(sum_j dequant(acc_j) + res)
};

enum DecodePrologue : int {
  PRO_CODES = 0,        // INT8 codes and row scales are given (a, lda, sa)
  PRO_QUANT_BF16 = 1,   // quantize BF16 rows x (optionally after RMSNorm) in-kernel
  PRO_REQUANT_F32 = 2   // quantize FP32 rows hin with the scale from partial maxima
};

// Rows a fused-prologue launch handles (the prologue re-derives each row per workgroup).
constexpr int kFuseMaxRows = 4;

struct DecodeGemmArgs {
  int epi, layout, prologue;
  int64_t M, N, K;
  int parts;                // K partitions (EPI_DOWN: split_k), else 1
  int ranges;               // K ranges per partition spread over workgroups
  // PRO_CODES
  const int8_t* a;          // [M, lda] INT8 codes
  int64_t lda;
  const float* sa;          // [M] activation row scales
  // PRO_QUANT_BF16
  const uint16_t* x;        // [M, ldx] BF16
  int64_t ldx;
  const uint16_t* gamma;    // [K] RMSNorm gain or nullptr
  float eps;
  // PRO_REQUANT_F32
  const float* hin;         // [M, ldhin] FP32
  int64_t ldhin;
  const float* pmax;        // [npmax, M] partial absolute maxima of hin's rows
  int npmax;
  // weights
  const int8_t* w0;
  const float* sw0;         // [N]
  const int8_t* w1;         // second weight (EPI_SILU) or nullptr
  const float* sw1;
  // outputs
  uint16_t* out;            // [M, ldo] BF16
  int64_t ldo;
  const uint16_t* res;      // [M, ldr] BF16 residual or nullptr
  int64_t ldr;
  float* h;                 // [M, ldh] FP32 (EPI_SILU)
  int64_t ldh;
  float* pmax_out;          // EPI_SILU: [N/16, M] absolute maximum of h per 16-channel tile
  int32_t* wacc;            // ranges > 1: [sets, M, N] INT32 accumulators, zero on entry
  int32_t* wcnt;            // ranges > 1: [tiles * mgroups] arrival counters, zero on entry
  void* zero_ptr;           // region this kernel zeroes for later kernels (16 B multiple)
  size_t zero_bytes;
  // taps (nullptr = off)
  int32_t* tap_acc0;        // [M, N] (EPI_DOWN: [parts, M, N])
  int32_t* tap_acc1;        // [M, N] (EPI_SILU up accumulator)
  float* tap_p;             // EPI_DOWN: [parts, M, N] FP32 partials
  float* tap_h;             // EPI_SILU: [M, N] copy of h
  float* tap_xn;            // fused prologue: [M, K] normalized FP32 rows
  int8_t* tap_q;            // fused prologue: [M, K] codes
  float* tap_s;             // fused prologue: [M] row scales
};

// Launch shape chosen for a problem; the host needs it to size the workspace.
struct DecodeGemmPlan {
  int ranges;        // K ranges per partition (1 = no cross-workgroup reduction)
  int waves;         // waves per workgroup
  int mgroups;       // grid.y: groups of up to 64 rows
  int tiles;         // N / 16
  size_t acc_elems;  // INT32 accumulator elements needed (0 when ranges == 1)
  size_t cnt_elems;  // counters needed
};
// first: the call's first GEMM (its accumulators cannot be pre-zeroed, so ranges = 1).
DecodeGemmPlan plan_decode_gemm(int epi, int64_t M, int64_t N, int64_t K, int parts,
                                bool first);
hipError_t launch_decode_gemm(const DecodeGemmArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- prefill GEMM
enum PrefillEpilogue : int {
  EPI_PF_SILU = 10,     // two weights: h = rne_bf16(silu(g) * u) -> out_bf16
  EPI_PF_PARTIAL = 11   // one weight, K split `splits` ways: FP32 partials -> part
};

struct PrefillGemmArgs {
  int epi, layout;
  int64_t M, N, K;
  int splits;               // K splits (EPI_PF_PARTIAL), else 1
  const uint16_t* act;      // [M, lda] BF16 activations
  int64_t lda;
  const int8_t* w0;
  const float* sw0;
  const int8_t* w1;         // EPI_PF_SILU: the Up weight
  const float* sw1;
  uint16_t* out_bf16;       // EPI_PF_SILU: [M, ldo]
  int64_t ldo;
  float* part;              // EPI_PF_PARTIAL: [splits, M, N]
  float* tap_g;             // EPI_PF_SILU taps: [M, N] FP32 accumulators or nullptr
  float* tap_u;
};
// Output channels one workgroup covers (N must be a multiple of it).
int prefill_channels_per_wg(int epi);
hipError_t launch_prefill_gemm(const PrefillGemmArgs& a, hipStream_t stream);
// out = rne_bf16(sum_s part[s] + res) over [M, N] (M * N % 4 == 0); tap_d gets the sum.
hipError_t launch_reduce_residual(const float* part, int splits, int64_t M, int64_t N,
                                  const uint16_t* res, uint16_t* out, float* tap_d,
                                  hipStream_t stream);

}  // namespace a8w8
