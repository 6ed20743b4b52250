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
};
hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- decode GEMM
enum DecodeEpilogue : int {
  EPI_BF16 = 0,       // y = rne_bf16(dequant(acc))
  EPI_BF16_RES = 1,   // y = rne_bf16(dequant(acc) + res)
  EPI_SILU = 2,       // two weights: h = silu(dequant(acc_g)) * dequant(acc_u), FP32
  EPI_DOWN = 3        // K partitions: out = rne_bf16(sum_j dequant(acc_j) + res)
};

struct DecodeGemmArgs {
  int epi;
  const int8_t* a;          // [M, lda] INT8 codes
  int64_t lda;
  const float* sa;          // [M] activation row scales
  const int8_t* w0;         // [N, K]
  const float* sw0;         // [N]
  const int8_t* w1;         // [N, K] second weight (EPI_SILU) or nullptr
  const float* sw1;
  int64_t M, N, K;
  int parts;                // K partitions (EPI_DOWN: split_k), else 1
  int ranges;               // K ranges per partition spread over workgroups
  uint16_t* out;            // [M, ldo] BF16
  int64_t ldo;
  const uint16_t* res;      // [M, ldr] BF16 residual or nullptr
  int64_t ldr;
  float* h;                 // [M, ldh] FP32 (EPI_SILU)
  int64_t ldh;
  int32_t* wacc;            // ranges > 1: [sets, M, N] INT32 accumulators, zero on entry
  int32_t* wcnt;            // ranges > 1: [tiles * mgroups] arrival counters, zero on entry
  int32_t* tap_acc0;        // [M, N] (EPI_DOWN: [parts, M, N]) or nullptr
  int32_t* tap_acc1;        // [M, N] (EPI_SILU up accumulator) or nullptr
  float* tap_p;             // EPI_DOWN: [parts, M, N] FP32 partials or nullptr
};

// Workgroup shape used for a given problem; the host needs it to size the workspace.
struct DecodeGemmPlan {
  int ranges;        // K ranges per partition (1 = no cross-workgroup reduction)
  int mgroups;       // grid.y: groups of up to 64 rows
  int tiles;         // N / 16
  size_t acc_elems;  // INT32 accumulator elements needed (0 when ranges == 1)
  size_t cnt_elems;  // counters needed
};
DecodeGemmPlan plan_decode_gemm(int epi, int64_t M, int64_t N, int64_t K, int parts,
                                bool allow_ranges);
hipError_t launch_decode_gemm(const DecodeGemmArgs& a, hipStream_t stream);

}  // namespace a8w8
