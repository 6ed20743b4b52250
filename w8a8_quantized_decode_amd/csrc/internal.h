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
  int8_t* q;                // [M, K] codes (row stride K), or tiled (q_tiled)
  int q_tiled;              // 1: q in the 16-row tiled operand order (M <= 16, 16 * K bytes)
  float* s;                 // [M] row scales
  float* xn_tap;            // [M, K] FP32 or nullptr
  int8_t* q_tap;            // [M, K] or nullptr (copy of q)
  float* s_tap;             // [M] or nullptr (copy of s)
  uint16_t* a_bf16;         // rne_bf16(v) or nullptr (prefill activations)
  int a_bf16_tiled;         // a_bf16 layout: 0 row-major [M, K]; 1 prefill operand layout
  uint16_t* a_bf16_tap;     // [M, K] or nullptr
  int write_codes;          // 0: skip the INT8 codes (prefill only needs a_bf16)
  const float* pmax;        // launch_requant_pmax: [npmax, M] absolute maxima of x's rows per tile
  int64_t npmax;
};
hipError_t launch_quant_rows(const QuantRowsArgs& a, hipStream_t stream);
// FP32 rows (x_is_f32, no gain) with their absolute maxima given as pmax: M <= 65535.
hipError_t launch_requant_pmax(const QuantRowsArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- weight layouts
// LAYOUT_ROWMAJOR: w[n * K + k].
// LAYOUT_TILED: 16-row tiles, one 1 KB block per 64-byte k step, each block in the
// operand order of v_mfma_i32_16x16x64_i8:
//   byte (n/16) * 16K + (k/64) * 1024 + 16 * lane + b, lane = (n % 16) + 16 * ((k % 64) / 16),
//   b = k % 16.
enum WeightLayout : int { LAYOUT_ROWMAJOR = 0, LAYOUT_TILED = 1 };
hipError_t launch_pack_tiled(const int8_t* w, int64_t N, int64_t K, int8_t* out,
                             hipStream_t stream);

// ---------------------------------------------------------------- decode GEMMs
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

// Rows a fused-prologue launch handles (each workgroup re-derives every row).
constexpr int kFuseMaxRows = 4;

// Standalone linear on given codes (a8w8_linear): one workgroup per 16-channel tile, no
// workspace.
struct LinearArgs {
  int epi, layout;          // EPI_BF16 or EPI_BF16_RES
  int64_t M, N, K;
  const int8_t* a;          // [M, lda] INT8 codes
  int64_t lda;
  const float* sa;          // [M] row scales
  const int8_t* w0;
  const float* sw0;         // [N]
  uint16_t* out;            // [M, ldo]
  int64_t ldo;
  const uint16_t* res;      // [M, ldr] or nullptr
  int64_t ldr;
  int32_t* tap_acc0;        // [M, N] or nullptr
};
hipError_t launch_linear(const LinearArgs& a, hipStream_t stream);

// Division of n < 2^31 by a divisor d in [1, 2^31) fixed per launch, by multiply-high
// and shift (the round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
  FastDiv() : d(1), m(1), l(0) {}
  explicit FastDiv(uint32_t dd) : d(dd), m(0), l(0) {
    while ((uint64_t(1) << l) < d) ++l;
    m = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  }
  __host__ __device__ uint32_t div(uint32_t n) const {
    const uint32_t hi = static_cast<uint32_t>((uint64_t(n) * m) >> 32);
    return static_cast<uint32_t>((uint64_t(hi) + n) >> l);
  }
};

// Stream-K decode GEMM of the MLP block and layer chains.
//
// The work is the sequence of 64-byte K steps of every 16-channel tile, ordered by K
// chunk, then tile, then step: for the tiled layout each (chunk, tile) segment is one
// contiguous run of weight bytes.  The sequence is dealt out evenly, in order, to every
// wave of the grid.  A workgroup writes the INT32 partial sums of each shared segment
// to its own slot, each value paired with the call's tag in one 64-bit word; a wave that
// finds the call's tag in every word of a tile's pieces adds them (integer sums: exact
// in any order) and runs the epilogue.  The tags make clearing unnecessary.
// Geometry of the step sequence (all counts below 2^31).  Waves w < r take q + 1 steps,
// the others q, in order: wave w starts at w * q + min(w, r).
struct StreamKGeom {
  int32_t tiles;            // T = N / 16
  int32_t steps_tile;       // K / 64
  int32_t steps_seg;        // Ss = steps_tile / chunks
  int32_t chunks;           // C
  int32_t total;            // T * steps_tile
  int32_t waves;            // W, per 64-row group
  int32_t q, r;             // total = q * W + r
  FastDiv by_seg, by_tiles, by_q, by_q1;  // divisors Ss, T, q (1 if q == 0), q + 1
};

struct StreamKArgs {
  int epi, layout, prologue;
  int64_t M, N, K;
  int parts;                // K partitions (EPI_DOWN: split_k), else 1
  int64_t act_row;          // bytes of codes per row one workgroup keeps in LDS (fused prologue)
  int64_t red_off;          // byte offset of the workgroup-combine area in dynamic LDS
  // Call tags live on the device: this GEMM's tag is *epoch_in; workgroup (0, 0)
  // writes *epoch_in + 1 to epoch_out, the word the next GEMM of the chain reads.
  const uint32_t* epoch_in;
  uint32_t* epoch_out;
  StreamKGeom g;
  // Workgroups b >= wgs1 run a second geometry g2 over tiles [toff2, toff2 + g2.tiles),
  // as workgroup b - wgs1 of it (wgs1 = grid.x: one geometry).
  StreamKGeom g2;
  int32_t wgs1, toff2;
  // PRO_CODES
  const int8_t* a;          // [M, lda] INT8 codes (DecodeGeom::gcodes: 16-row tiled, 16 * K bytes)
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
  int64_t npmax;
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
  float* pmax_out;          // EPI_SILU: [N/16, M] absolute maximum of h per tile
  int32_t* slots;           // tagged partial-sum slots (StreamKPlan::slot_elems INT32)
  uint64_t* dones;          // [mgroups, tiles] done words (used when `once`)
  int once;                 // the output may overwrite the residual: one epilogue per tile
  // taps (nullptr = off)
  int32_t* tap_acc0;        // [M, N] (EPI_DOWN: [parts, M, N])
  int32_t* tap_acc1;        // [M, N] (EPI_SILU up accumulator)
  float* tap_p;             // EPI_DOWN: [parts, M, N] FP32 partials
  float* tap_h;             // EPI_SILU: [M, N] copy of h
  float* tap_xn;            // fused prologue: [M, K] normalized FP32 rows
  int8_t* tap_q;            // fused prologue: [M, K] codes
  float* tap_s;             // fused prologue: [M] row scales
};

// Decode GEMM with one 16-wave workgroup per CU and whole tiles per workgroup
// (gemm_decode.hip), used for fused-prologue shapes it covers.
struct DecodeGeom {
  int32_t tiles, steps_tile, steps_seg, grid;
  int32_t whole_q, whole_r;  // workgroup b: q (+1 if b < r) whole tiles from b*q + min(b, r)
  int32_t leftover;          // 1: tiles grid*q .. grid*q + grid/4 - 1 are cut in K quarters,
                             // quarter b % 4 of tile grid*q + b/4 computed by workgroup b
  int32_t gcodes;            // 1: the given codes are read from global memory in the 16-row
                             // tiled operand order (tiled_code_index), not staged in LDS
  int32_t act_ld;            // bytes of codes per row in LDS (= K)
  int32_t acc_off, lred_off; // LDS offsets of the segment accumulators and the control waves' partials
  int32_t stage_g;           // offset of the staged RMSNorm gain from acc_off (the staging area)
  int32_t lds;               // dynamic LDS bytes
};
// False when the shape is not covered (then the stream-K kernel runs).  codes_in: the
// input codes and row scales are given (PRO_CODES) instead of quantized in the kernel.
bool plan_decode(int epi, int64_t M, int64_t N, int64_t K, int parts, bool codes_in,
                 DecodeGeom& g);
size_t decode_slot_elems(const DecodeGeom& g, int nmat);

struct StreamKPlan {
  int use_decode;      // 1: launch the decode kernel of gemm_decode.hip with `dec`
  DecodeGeom dec;
  int waves;           // waves per workgroup
  int wgs;             // grid.x: workgroups per 64-row group
  int mgroups;         // grid.y
  int mb;              // 16-row blocks per group (1 with a fused prologue)
  StreamKGeom geom;
  StreamKGeom geom2;   // second geometry for workgroups >= wgs1 (see StreamKArgs)
  int wgs1, toff2;
  int64_t act_row;
  size_t slot_elems;   // INT32 elements of partial-sum slots
  size_t done_elems;   // 64-bit done words
  size_t red_off;      // dynamic LDS: codes first (fused), workgroup-combine area here
  size_t lds;          // dynamic LDS bytes
};
StreamKPlan plan_streamk(int epi, int64_t M, int64_t N, int64_t K, int parts, bool fused);
// Whether a fused-prologue plan fits (rows, LDS, prologue registers); K_in is the row
// length a BF16 prologue normalizes (bf16_rows), else the requantized row.
bool streamk_fusable(const StreamKPlan& pl, int64_t M, int64_t K_in, bool bf16_rows);
hipError_t launch_streamk(const StreamKArgs& a, const StreamKPlan& pl, hipStream_t stream);
hipError_t launch_decode(const StreamKArgs& a, const DecodeGeom& g, hipStream_t stream);

// ---------------------------------------------------------------- prefill GEMM
// W8A16 GEMM over tiles of 256 rows x 64 (Gate/Up: 64 Gate + the same 64 Up channels)
// or 128 (Down) channels.  Each of at most kPrefillGrid workgroups first runs whole tiles
// (tiles / grid of them); the leftover tiles' quads (4 steps of 64 k) are dealt evenly
// over all workgroups, and a reduction kernel completes the tiles split that way.
// Needs K % 256 == 0 and N a multiple of prefill_tile_channels(epi).
enum PrefillEpilogue : int {
  EPI_PF_SILU = 10,     // two weights: h = rne_bf16(silu(g) * u) -> out
  EPI_PF_RES = 11       // one weight: out = rne_bf16(acc + res)
};
constexpr int32_t kPrefillGrid = 256;

struct PrefillPlan {
  int32_t mtiles, ntiles, tiles;  // tiles along M and N, and in all
  int32_t quads;                  // quads per tile
  int32_t grid;                   // workgroups
  int32_t dp_per_wg, tiles_dp;    // whole tiles per workgroup; tiles run whole
  int32_t q, r;                   // leftover quads: workgroups w < r take q + 1, others q
};
PrefillPlan plan_prefill(int epi, int64_t M, int64_t N, int64_t K);
int prefill_tile_channels(int epi);
// FP32 elements of one exchange slot; a launch uses 2 * grid slots.
size_t prefill_slot_floats();

struct PrefillGemmArgs {
  int epi, layout;
  int64_t M, N, K;
  const uint16_t* act;      // BF16 activations, prefill operand layout, K columns
  const int8_t* w0;
  const float* sw0;
  const int8_t* w1;         // EPI_PF_SILU: the Up weight
  const float* sw1;
  uint16_t* out;            // EPI_PF_SILU: h, prefill operand layout (N columns);
  int64_t ldo;              // EPI_PF_RES: [M, ldo] BF16 block output
  const uint16_t* res;      // EPI_PF_RES: [M, ldr] BF16 residual (may alias out) or nullptr
  int64_t ldr;
  uint16_t* tap_h;          // EPI_PF_SILU tap: [M, N] row-major h or nullptr
  float* tap_g;             // EPI_PF_SILU taps: [M, N] FP32 accumulators or nullptr
  float* tap_u;
  float* tap_d;             // EPI_PF_RES tap: [M, N] FP32 accumulator or nullptr
  float* slots;             // partial sums of split tiles (2 * grid slots)
  // Filled in by launch_prefill_gemm from plan_prefill.
  int32_t mtiles, quads, tiles, grid, dp_per_wg, tiles_dp, q, r;
  FastDiv by_quads, by_mtiles;
};
// Launches the GEMM and, when tiles were split, the reduction kernel.
hipError_t launch_prefill_gemm(const PrefillGemmArgs& a, hipStream_t stream);

}  // namespace a8w8
