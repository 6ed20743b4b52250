// Decode GEMM with one 16-wave workgroup per CU: INT8 x INT8 -> INT32 on gfx950 matrix
// cores with the fused input quantization (RMSNorm + per-row quantization, or the
// requantization of h for Down) and the fused dequant / SiLU / residual / split-K
// epilogues.  It serves the layer chain and the MLP block at decode batch sizes
// (M <= kFuseMaxRows) for the shapes it covers (plan_decode), and, with the input codes
// given (row-quantization kernels before it), up to kDcMaxRows rows: the codes are
// copied into LDS at the start, or (QKV and O above 4 rows, Down when they do not fit)
// read from global memory beside the weights in the tiled order (template argument GC).
// The stream-K kernel in gemm_streamk.hip serves the other shapes.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path (Gate/Up as INT8 x INT8 products summed in
// INT32, the sums turned into FP32 with the row scale and the channel scale, the
// normalized activations after attention given one INT8 scale per row) and > Decode scheduling (Down
// split two ways along K into independent accumulators), with the CodeRabbit walkthrough
// row "Split down projection accumulation" (FP32 partials summed, the residual added,
// the sum narrowed with round-to-nearest-even).  QKV and O reuse the pattern.
//
// Why this shape.  At decode batch sizes the kernel is a weight stream: every weight
// byte is read once.  What a plain stream does not have is the dependency of every
// matrix instruction on the input row's statistics.  Measured on MI355X: a row read by
// a wave that has weight loads queued (its own or other waves' on the same CU) waits
// behind them, 2.5-7 us; the same row read before any weight load by waves that issue
// none arrives in 0.5-1 us.  So the 16 waves are split by role:
//   * waves 0-3 (control): request the input row(s) before anything else, then compute
//     the row statistics and the INT8 codes of the whole row into LDS; then prefetch the
//     epilogue inputs into LDS and, for the "leftover" tiles (below), stream their
//     quarter of a shared tile and publish it;
//   * waves 4-15 (stream): wait at one barrier until the row requests are out, issue two
//     deep batches of weight loads, wait for the codes, then stream the workgroup's whole
//     tiles through the matrix cores.
// Every workgroup owns whole tiles (16 output channels over all of K), so a tile's partial
// sums meet in LDS and the kernel's tail has no exchange between workgroups.  When the
// tile count is G*q + G/4 (Gate/Up: 1088 = 256*4 + 64; Down: 320 = 256 + 64), the last
// G/4 tiles are cut into K quarters, one per workgroup; each quarter is computed early by
// the control waves and published as tagged words, and the owner of quarter 0 adds the
// four and runs that tile's epilogue long before the stream ends.  Otherwise the tiles
// are dealt whole, q or q + 1 per workgroup; QKV and O take a smaller grid that divides
// their tiles (448 = 224 x 2, 320 = 160 x 2), so every workgroup has the same share.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

constexpr int kDcWaves = 16;
constexpr int kDcCtl = 4;                        // control waves
constexpr int kDcStream = kDcWaves - kDcCtl;     // stream waves
constexpr int kDcThreads = kDcWaves * kWave;
constexpr int kDcCtlThreads = kDcCtl * kWave;
constexpr int kDcMaxGrid = 256;
constexpr int kDcMaxTiles = 5;                   // whole tiles per workgroup
constexpr int kDcMaxRows = 16;                   // rows with given codes (one matrix-core tile)
constexpr int kBfUnits = 3;                      // BF16 row: 8-value units per control thread
constexpr int kF32Units = 18;                    // FP32 row: 4-value units per control thread
constexpr int64_t kBfMaxK = int64_t(kBfUnits) * 8 * kDcCtlThreads;   // 6144
constexpr int64_t kF32MaxK = int64_t(kF32Units) * 4 * kDcCtlThreads; // 18432
constexpr int kSlotWords = 4 * kWave;            // tagged 64-bit words per matrix per piece
constexpr size_t kDcMaxLds = 150 * 1024;
constexpr size_t kDcLdsPerCu = 160 * 1024;
// Leftover-quarter steps a control wave requests before its prologue and holds in
// registers meanwhile (the rest of its share follows after the prologue), sized within
// the register budget of a 1024-thread workgroup: Qwen3-14B has 5 steps per control wave
// (K = 5120) and 17 for Down (K = 17408).
constexpr int lo_steps(int epi) { return epi == EPI_DOWN ? 12 : 5; }
// ... and steps requested into LDS beside them (Down only: one weight matrix).
constexpr int lo_lds_steps(int epi) { return epi == EPI_DOWN ? 5 : 0; }

struct DcSmem {
  double sum_slot[kFuseMaxRows][kDcCtl];
  float max_slot[kFuseMaxRows][kDcCtl];
  float row_scale[kDcMaxRows];
  int ctl_sync;        // control-wave barrier counter
  int lo_arrive;       // control waves done with their share of the leftover quarter
  int pf_done;         // control waves done storing the epilogue inputs
  int scales_ready;    // Down, one row: the row scale is in row_scale[0]
  int task_next;       // ... next 64-chunk code task
  int task_done;       // ... code tasks finished
  int codes_ready;     // set by the control waves once the codes are in LDS
  float sw[kDcMaxTiles + 1][2][16];                 // channel scales (slot kDcMaxTiles: leftover)
  uint16_t res[kDcMaxTiles + 1][kDcMaxRows][16];    // residual
};

// Agent-coherent tagged words of the leftover exchange (64-bit: tag in the high half, an
// INT32 sum in the low half), four per lane, laid out component-major: word c * 64 + lane.
__device__ __forceinline__ void store_tagged_lanes(uint64_t* block, int lane, i32x4 v, uint32_t tag) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    __hip_atomic_store(block + c * kWave + lane, (uint64_t(tag) << 32) | uint32_t(v[c]),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ TaggedX4 load_tagged_lanes(const uint64_t* block, int lane) {
  TaggedX4 t;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    t.w[c] = __hip_atomic_load(block + c * kWave + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return t;
}

// LDS hand-offs between waves that may have global loads in flight.  The workgroup-scope
// fences and atomic loads of the memory model also wait for every outstanding global load
// (vmcnt(0)), which would drain a wave's weight stream or its early leftover loads.  The
// LDS operations of one wave execute in order, so waiting for this wave's LDS operations
// (lgkmcnt(0)) before raising a flag is the whole release, and a volatile read through an
// LDS pointer followed by a compiler barrier is the whole acquire.
__device__ __forceinline__ void lds_release_only() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __asm__ __volatile__("" ::: "memory");
}
__device__ __forceinline__ void lds_wait_flag(int* flag, int at_least) {
  const volatile __attribute__((address_space(3))) int* f =
      (const volatile __attribute__((address_space(3))) int*)(flag);
  while (*f < at_least) __builtin_amdgcn_s_sleep(1);
  __asm__ __volatile__("" ::: "memory");
}

// Adds to an LDS counter (waiting for the add to complete) and stores an LDS flag, both
// out of sight of the compiler's memory-counter tracking, which would otherwise place a
// vmcnt(0) before them while the control waves' early leftover loads are in flight.
__device__ __forceinline__ uint32_t lds_addr(int* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)(p)));
}
__device__ __forceinline__ void lds_add_sync(int* p, int v) {
  __asm__ __volatile__("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_set_flag(int* p, int v) {
  __asm__ __volatile__("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// Barrier of the four control waves only (the stream waves are in their loop): an LDS
// counter that every control wave advances once per use; waits until all have.
__device__ __forceinline__ void ctl_sync(DcSmem& sm, int& gen) {
  gen += kDcCtl;
  lds_release_only();
  if ((threadIdx.x & (kWave - 1)) == 0) lds_add_sync(&sm.ctl_sync, 1);
  lds_wait_flag(&sm.ctl_sync, gen);
}

// INT8 codes clamp(rint(v / s), -127, 127) of N values, s > 0, |v| <= 127 s (s is the
// row's absolute maximum over 127), with the correctly rounded quotient computed only
// where it can matter.  rs = fl32(1/s) and t = fl32(v * rs) carry two roundings, a
// relative error of at most 2^-23, so |t - v/s| <= |t| * 2^-22.9 and fl32(v/s) lies within
// |t| * 2^-24 of v/s.  |t| < 128, so if t is farther than 2^-14 (> |t| * 2^-21) from the
// midpoint n + 1/2 of its neighbours, fl32(v/s) rounds to the same integer as t and is no
// tie.  Otherwise (or when t is not finite: s subnormal) the exact quotient decides; that
// path runs only when some lane of the wave needs it.
template <int N>
__device__ __forceinline__ void quant_codes(const float (&v)[N], float s, float rs, int (&q)[N]) {
  bool need = false;
  float qf[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float t = v[i] * rs;
    qf[i] = rintf(t);
    need = need || !(fabsf(t - qf[i]) < 0.5f - 6.103515625e-5f);
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float t = v[i] * rs;
      if (!(fabsf(t - rintf(t)) < 0.5f - 6.103515625e-5f)) qf[i] = rintf(v[i] / s);
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) q[i] = static_cast<int>(fminf(fmaxf(qf[i], -127.0f), 127.0f));
}

__device__ __forceinline__ u32x2 codes8_fast(const float (&v)[8], float s, float rs) {
  int q[8];
  quant_codes<8>(v, s, rs, q);
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t(q[i]) & 0xFFu) << (8 * i);
      hi |= (uint32_t(q[4 + i]) & 0xFFu) << (8 * i);
    }
  }
  return u32x2{lo, hi};
}

__device__ __forceinline__ uint32_t codes4_fast(const f32x4& h, float s, float rs) {
  const float v[4] = {h[0], h[1], h[2], h[3]};
  int q[4];
  quant_codes<4>(v, s, rs, q);
  uint32_t w = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (uint32_t(q[i]) & 0xFFu) << (8 * i);
  }
  return w;
}

// Wave reductions in registers: four DPP steps leave every lane of a 16-lane row with the
// row's result (each step combines a lane with a partner that holds the mirrored partial,
// and addition and maximum are commutative, so both partners get identical bits), then
// the four rows are combined from lanes 0, 16, 32 and 48 in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(uint32_t(u)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(uint32_t(u >> 32)), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}
constexpr int kDppQuad1032 = 0xB1, kDppQuad2301 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(uint32_t(u)), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(uint32_t(u >> 32)), l);
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppQuad1032>(v));
  v = fmaxf(v, dpp_f32<kDppQuad2301>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ double wave_sum_dpp(double v) {
  v = v + dpp_f64<kDppQuad1032>(v);
  v = v + dpp_f64<kDppQuad2301>(v);
  v = v + dpp_f64<kDppHalfMirror>(v);
  v = v + dpp_f64<kDppMirror>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ------------------------------------------------------------------ control-wave prologues
// The input row is copied straight into an LDS staging area by the control waves (direct
// global-to-LDS loads take no registers), in 16-byte chunks: chunk c = u * 256 + ct of
// control thread ct lands at stage + 16 * c.  The staging area overlaps the partial-sum
// areas, which are used only after the prologue.
template <int UNITS>
__device__ __forceinline__ void stage_chunks(const void* src, int64_t nbytes, int8_t* stage) {
  // Unrolled, so the compiler counts these loads exactly when it places waits for loads
  // issued before them.
  const int ct = threadIdx.x, w = ct / kWave;
  const int8_t* s8 = static_cast<const int8_t*>(src);
#pragma unroll
  for (int u = 0; u < UNITS; ++u) {
    const int64_t c = int64_t(u) * kDcCtlThreads + ct;
    const int64_t off = c * 16 < nbytes ? c * 16 : 0;   // chunks past the row re-read chunk 0
    // Lane l of the wave writes stage + 16 * (u * 256 + 64 * w + l).
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(s8 + off),
                                     reinterpret_cast<__shared__ uint32_t*>(
                                         stage + (int64_t(u) * kDcCtlThreads + w * kWave) * 16),
                                     16, 0, 0);
  }
}

// Given codes (M rows of K bytes at a, row stride lda) copied into act[M][act_ld] with
// direct global-to-LDS loads: 1 KB units u = wave, wave + 4, ... of chunks (64 u + lane);
// a unit lies inside one row when rows are padded (K / 16 chunks a multiple of 64), and
// the rows are contiguous otherwise.  A unit past the codes' end writes into the
// accumulator area behind them (zeroed after the copy) from a clamped source.
__device__ __forceinline__ void stage_codes(const StreamKArgs& p, int8_t* act, int32_t act_ld) {
  const int ct = threadIdx.x, w = ct / kWave, l = ct & (kWave - 1);
  const int32_t cpr = static_cast<int32_t>(p.K / 16);   // 16-byte chunks per row
  const int32_t nch = static_cast<int32_t>(p.M) * cpr;
  const int32_t units = (nch + kWave - 1) / kWave;
  for (int32_t u = w; u < units; u += kDcCtl) {
    const int32_t c = u * kWave + l;
    const int32_t cc = c < nch ? c : 0;
    const int32_t m = cc / cpr;
    const int8_t* src = p.a + int64_t(m) * p.lda + int64_t(cc - m * cpr) * 16;
    const int32_t m0 = (u * kWave) / cpr;   // the unit's row (its first chunk's)
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const uint32_t*>(src),
        reinterpret_cast<__shared__ uint32_t*>(act + m0 * act_ld + (u * kWave - m0 * cpr) * 16),
        16, 0, 0);
  }
}

// RMSNorm (when gamma) and quantization of one BF16 row staged at xs (and the gain at gs)
// into codes act[0..K), scale into sm.row_scale[m]; taps (xn, q, s) when requested.
// Values k = u * 2048 + ct * 8 + i; each pass re-reads the staged row from LDS.
__device__ __forceinline__ void bf_vals(const int8_t* xs, int u, int ct, int64_t K, float (&v)[8]) {
  const bool in = int64_t(u) * 8 * kDcCtlThreads + ct * 8 < K;
  const u32x4 xr = *reinterpret_cast<const u32x4*>(xs + (int64_t(u) * kDcCtlThreads + ct) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = in ? bf16_lo(xr[i]) : 0.0f;
    v[2 * i + 1] = in ? bf16_hi(xr[i]) : 0.0f;
  }
}

__device__ void ctl_row_bf16(const StreamKArgs& p, DcSmem& sm, int8_t* act, int m,
                             const int8_t* xs, const int8_t* gs, bool taps, int& gen) {
  const int ct = threadIdx.x, wave = ct / kWave;
  const int64_t K = p.K;
  float r = 1.0f;
  if (p.gamma) {
    // Sum of squares in FP64; the square of a BF16 value is exact in FP64, so a fused
    // multiply-add rounds exactly as the product followed by the sum.  Then
    // r = 1 / sqrt(fl32(S / K) + eps) with correctly rounded steps.
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < kBfUnits; ++u) {
      float v[8];
      bf_vals(xs, u, ct, K, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = __builtin_fma(double(v[i]), double(v[i]), ss);
    }
    ss = wave_sum_dpp(ss);
    if ((ct & (kWave - 1)) == 0) sm.sum_slot[m][wave] = ss;
    ctl_sync(sm, gen);
    double S = 0.0;
#pragma unroll
    for (int w = 0; w < kDcCtl; ++w) S += sm.sum_slot[m][w];
    const float ms = static_cast<float>(S / static_cast<double>(K));
    const float t = ms + p.eps;
    r = 1.0f / __builtin_sqrtf(t);
  }
  auto norm = [&](int u, float (&v)[8]) {
    bf_vals(xs, u, ct, K, v);
    if (p.gamma) {
      const u32x4 gr = *reinterpret_cast<const u32x4*>(gs + (int64_t(u) * kDcCtlThreads + ct) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = (v[2 * i] * r) * bf16_lo(gr[i]);
        v[2 * i + 1] = (v[2 * i + 1] * r) * bf16_hi(gr[i]);
      }
    }
  };
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < kBfUnits; ++u) {
    float v[8];
    norm(u, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max_dpp(amax);
  if ((ct & (kWave - 1)) == 0) sm.max_slot[m][wave] = amax;
  ctl_sync(sm, gen);
  float a = 0.0f;
#pragma unroll
  for (int w = 0; w < kDcCtl; ++w) a = fmaxf(a, sm.max_slot[m][w]);
  const float s = a / 127.0f;
  const float rs = 1.0f / s;
  if (ct == 0) sm.row_scale[m] = s;
  if (taps && ct == 0 && p.tap_s) p.tap_s[m] = s;
#pragma unroll
  for (int u = 0; u < kBfUnits; ++u) {
    const int64_t k = int64_t(u) * 8 * kDcCtlThreads + ct * 8;
    if (k < K) {
      float v[8];
      norm(u, v);
      const u32x2 c = codes8_fast(v, s, rs);
      *reinterpret_cast<u32x2*>(act + k) = c;
      if (taps && p.tap_q) *reinterpret_cast<u32x2*>(p.tap_q + int64_t(m) * K + k) = c;
      if (taps && p.tap_xn) {
        f32x4* tx = reinterpret_cast<f32x4*>(p.tap_xn + int64_t(m) * K + k);
        tx[0] = f32x4{v[0], v[1], v[2], v[3]};
        tx[1] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// Partial maxima of |h| per 16-channel tile of the producing GEMM: [npmax, M].  The first
// kPmWords of them are copied straight into an LDS array of their own (pm_lds), words
// e = u * 1024 + ct * 4 + i at pm_lds[e]; being a separate LDS object, it does not make
// the compiler wait for these copies where it reads other LDS, and being loads it does
// not make it wait for later loads where it reads these.
constexpr int kPmUnits = 2;  // 4-value units per control thread (8 * 256 = 2048 words)
constexpr int kPmWords = kPmUnits * 4 * kDcCtlThreads;

__device__ __forceinline__ void stage_pmax(const StreamKArgs& p, float* pm_lds) {
  const int ct = threadIdx.x, w = ct / kWave;
  const int64_t n = p.npmax * p.M;
#pragma unroll
  for (int u = 0; u < kPmUnits; ++u) {
    const int64_t e = int64_t(u) * 4 * kDcCtlThreads + ct * 4;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(p.pmax + (e < n ? e : 0)),
                                     reinterpret_cast<__shared__ uint32_t*>(
                                         pm_lds + (u * kDcCtlThreads + w * kWave) * 4),
                                     16, 0, 0);
  }
}

// Row scales of the requantized input from the partial maxima (all rows at once).
__device__ void ctl_requant_scales(const StreamKArgs& p, DcSmem& sm, const float* pm_lds, bool taps,
                                   int& gen) {
  const int ct = threadIdx.x, wave = ct / kWave;
  // Word e of the [npmax, M] table belongs to row e % M (32-bit: npmax * M < 2^26).
  const uint32_t n = static_cast<uint32_t>(p.npmax * p.M), Mu = static_cast<uint32_t>(p.M);
  float mx[kFuseMaxRows];
#pragma unroll
  for (int m = 0; m < kFuseMaxRows; ++m) mx[m] = 0.0f;
#pragma unroll
  for (int u = 0; u < kPmUnits; ++u) {
    const uint32_t e0 = uint32_t(u) * 4 * kDcCtlThreads + uint32_t(ct) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(pm_lds + e0);
    uint32_t m = e0 % Mu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + i < n) {
#pragma unroll
        for (int mm = 0; mm < kFuseMaxRows; ++mm)
          if (uint32_t(mm) == m) mx[mm] = fmaxf(mx[mm], v[i]);
      }
      m = m + 1 == Mu ? 0 : m + 1;
    }
  }
  // partial maxima beyond the prefetched words (npmax * M > 2048)
  for (uint32_t e = uint32_t(kPmUnits) * 4 * kDcCtlThreads + ct; e < n; e += kDcCtlThreads) {
    const uint32_t m = e % Mu;
    const float v = p.pmax[e];
#pragma unroll
    for (int mm = 0; mm < kFuseMaxRows; ++mm)
      if (uint32_t(mm) == m) mx[mm] = fmaxf(mx[mm], v);
  }
#pragma unroll
  for (int m = 0; m < kFuseMaxRows; ++m) {
    const float w = wave_max_dpp(mx[m]);
    if ((ct & (kWave - 1)) == 0) sm.max_slot[m][wave] = w;
  }
  ctl_sync(sm, gen);
  if (ct < p.M) {
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kDcCtl; ++w) a = fmaxf(a, sm.max_slot[ct][w]);
    const float s = a / 127.0f;
    sm.row_scale[ct] = s;
    if (taps && p.tap_s) p.tap_s[ct] = s;
  }
  ctl_sync(sm, gen);
}

// One row: its scale from the partial maxima after a single exchange of the four control
// waves' maxima; every control thread derives it (the maximum is exact in any order), and
// thread 0 stores it for the stream waves and the epilogue.
__device__ float ctl_requant_scale_one(const StreamKArgs& p, DcSmem& sm, const float* pm_lds,
                                       bool taps, int& gen) {
  const int ct = threadIdx.x, wave = ct / kWave;
  const uint32_t n = static_cast<uint32_t>(p.npmax);
  float mx = 0.0f;
#pragma unroll
  for (int u = 0; u < kPmUnits; ++u) {
    const uint32_t e0 = uint32_t(u) * 4 * kDcCtlThreads + uint32_t(ct) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(pm_lds + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i < n) mx = fmaxf(mx, v[i]);
  }
  for (uint32_t e = uint32_t(kPmUnits) * 4 * kDcCtlThreads + ct; e < n; e += kDcCtlThreads)
    mx = fmaxf(mx, p.pmax[e]);
  mx = wave_max_dpp(mx);
  if ((ct & (kWave - 1)) == 0) sm.max_slot[0][wave] = mx;
  ctl_sync(sm, gen);
  float a = 0.0f;
#pragma unroll
  for (int w = 0; w < kDcCtl; ++w) a = fmaxf(a, sm.max_slot[0][w]);
  const float s = a / 127.0f;
  if (ct == 0) {
    sm.row_scale[0] = s;
    if (taps && p.tap_s) p.tap_s[0] = s;
  }
  return s;
}

// Codes of one FP32 row staged at hs into act[0..K): values k = u * 1024 + ct * 4 + i.
__device__ void ctl_row_f32(const StreamKArgs& p, const DcSmem& sm, int8_t* act, int m,
                            const int8_t* hs, bool taps) {
  const int ct = threadIdx.x;
  const float s = sm.row_scale[m];
  const float rs = 1.0f / s;
  // Unrolled by three so that the LDS reads of a group overlap; every unit of the staging
  // area is in bounds (units past the row hold re-read data and are not stored).
#pragma unroll 3
  for (int u = 0; u < kF32Units; ++u) {
    const int64_t k = int64_t(u) * 4 * kDcCtlThreads + ct * 4;
    const f32x4 h = *reinterpret_cast<const f32x4*>(hs + (int64_t(u) * kDcCtlThreads + ct) * 16);
    const uint32_t c = codes4_fast(h, s, rs);
    if (k < p.K) {
      *reinterpret_cast<uint32_t*>(act + k) = c;
      if (taps && p.tap_q) *reinterpret_cast<uint32_t*>(p.tap_q + int64_t(m) * p.K + k) = c;
    }
  }
}

// Down with one row: the codes of the staged FP32 row in tasks of 128 chunks (chunk c = the
// four values from k = 4c, staged at hs + 16c), which any wave takes from an LDS counter
// until none is left: the control waves right after the row scale, the stream waves as
// soon as their first weight batch is requested.  A wave counts its finished tasks once,
// when the counter runs out.
// Wave-level counter updates: one add per wave, made by lane 0 with the execution mask
// narrowed inside the asm block and restored there, so the caller's control flow has no
// lane-dependent branch (a loop around such a branch may be split by lane, and a copy that
// lane 0 does not run would never see the counter move).  The fetch returns lane 0's old
// value to every lane.
__device__ __forceinline__ int lds_fetch_add_wave(int* p, int v) {
  int old;
  uint64_t saved;
  __asm__ __volatile__(
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "s_nop 1\n\t"
      "ds_add_rtn_u32 %0, %2, %3\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_nop 1"
      : "=&v"(old), "=&s"(saved)
      : "v"(lds_addr(p)), "v"(v)
      : "memory");
  return __builtin_amdgcn_readlane(old, 0);
}
__device__ __forceinline__ void lds_add_wave(int* p, int v) {
  uint64_t saved;
  __asm__ __volatile__(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "s_nop 1\n\t"
      "ds_add_u32 %1, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b64 exec, %0\n\t"
      "s_nop 1"
      : "=&s"(saved)
      : "v"(lds_addr(p)), "v"(v)
      : "memory");
}

constexpr int kTaskChunks = 2 * kWave;   // chunks per code task (two per lane)

__device__ __forceinline__ int code_tasks(int64_t K) {
  return static_cast<int>((K / 4 + kTaskChunks - 1) / kTaskChunks);
}

__device__ void codes_tasks_f32(const StreamKArgs& p, DcSmem& sm, int8_t* act, const int8_t* hs,
                                bool taps, float s) {
  const int lane = threadIdx.x & (kWave - 1);
  const float rs = 1.0f / s;
  const int32_t nchunks = static_cast<int32_t>(p.K / 4);
  const int ntasks = code_tasks(p.K);
  int done = 0;
  for (;;) {
    const int t = lds_fetch_add_wave(&sm.task_next, 1);
    if (t >= ntasks) break;
#pragma unroll
    for (int j = 0; j < kTaskChunks / kWave; ++j) {
      const int32_t c = t * kTaskChunks + j * kWave + lane;
      if (c < nchunks) {
        const f32x4 h = *reinterpret_cast<const f32x4*>(hs + int64_t(c) * 16);
        const uint32_t q = codes4_fast(h, s, rs);
        *reinterpret_cast<uint32_t*>(act + int64_t(c) * 4) = q;
        if (taps && p.tap_q) *reinterpret_cast<uint32_t*>(p.tap_q + int64_t(c) * 4) = q;
      }
    }
    ++done;
  }
  // The wave's codes are written before its tasks are counted.
  lds_release_only();
  if (done > 0) lds_add_wave(&sm.task_done, done);
}

// ------------------------------------------------------------------ epilogue
// Element-wise: lane l handles output channel l % 16 of one (tile, row) pair, pair index
// pq = base + l / 16; pairs enumerate (local tile j, row m) with m fastest.  sums(j, part,
// mat, m, n) yields the INT32 sum of K partition part (EPI_DOWN) or of the whole K, for
// weight matrix mat, row m and channel n of local tile j.  tile_of(j) is the global tile and
// slot_of(j) its LDS slot of epilogue inputs.  The 16 lanes of a pair form one DPP row, so
// the tile's absolute maximum of h (Gate/Up) is a row reduction.
template <int EPI, int NMAT, typename Sums, typename TileOf, typename SlotOf>
__device__ void dc_epilogue(const StreamKArgs& p, const DcSmem& sm, int32_t npairs, int32_t pq,
                            int nparts, Sums&& sums, TileOf&& tile_of, SlotOf&& slot_of) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15;
  const bool act_pair = pq < npairs;
  const int32_t j = act_pair ? pq / static_cast<int32_t>(p.M) : 0;
  const int64_t m = act_pair ? pq - int64_t(j) * p.M : 0;
  const int32_t t = tile_of(j);
  const int slot = slot_of(j);
  const int64_t en = int64_t(t) * 16 + n;
  const float sa = sm.row_scale[m];
  const float sw0 = sm.sw[slot][0][n], sw1 = sm.sw[slot][NMAT - 1][n];
  if constexpr (EPI == EPI_BF16 || EPI == EPI_BF16_RES) {
    if (!act_pair) return;
    const int32_t acc = sums(j, 0, 0, m, n);
    if (p.tap_acc0) p.tap_acc0[m * p.N + en] = acc;
    float y = dq(acc, sa, sw0);
    if constexpr (EPI == EPI_BF16_RES) y = y + bf16_bits_to_f32(sm.res[slot][m][n]);
    p.out[m * p.ldo + en] = f32_to_bf16_rne(y);
  } else if constexpr (EPI == EPI_SILU) {
    float h = 0.0f;
    if (act_pair) {
      const int32_t ag = sums(j, 0, 0, m, n), au = sums(j, 0, NMAT - 1, m, n);
      if (p.tap_acc0) p.tap_acc0[m * p.N + en] = ag;
      if (p.tap_acc1) p.tap_acc1[m * p.N + en] = au;
      h = silu_mul(dq(ag, sa, sw0), dq(au, sa, sw1));
      p.h[m * p.ldh + en] = h;
      if (p.tap_h) p.tap_h[m * p.N + en] = h;
    }
    // Absolute maximum over the tile's 16 channels of row m, for the next requantization.
    float mx = fabsf(h);
    mx = fmaxf(mx, dpp_f32<kDppQuad1032>(mx));
    mx = fmaxf(mx, dpp_f32<kDppQuad2301>(mx));
    mx = fmaxf(mx, dpp_f32<kDppHalfMirror>(mx));
    mx = fmaxf(mx, dpp_f32<kDppMirror>(mx));
    if (p.pmax_out && act_pair && n == 0) p.pmax_out[int64_t(t) * p.M + m] = mx;
  } else {  // EPI_DOWN: partitions dequantized one by one and summed in order, then the residual
    if (!act_pair) return;
    const int64_t MN = p.M * p.N;
    float tot = 0.0f;
    for (int q = 0; q < nparts; ++q) {
      const int32_t acc = sums(j, q, 0, m, n);
      const float pv = dq(acc, sa, sw0);
      if (p.tap_acc0) p.tap_acc0[q * MN + m * p.N + en] = acc;
      if (p.tap_p) p.tap_p[q * MN + m * p.N + en] = pv;
      tot = (q == 0) ? pv : tot + pv;
    }
    p.out[m * p.ldo + en] = f32_to_bf16_rne(tot + bf16_bits_to_f32(sm.res[slot][m][n]));
  }
}

// INT32 sum of a segment accumulator kept in LDS in the matrix-instruction layout: row m,
// channel n is lane 16 * (n / 4) + m, component n % 4.
__device__ __forceinline__ int32_t acc_elem(const int32_t* seg_acc, int mat, int64_t m, int n) {
  return seg_acc[mat * kWave * 4 + ((n >> 2) * 16 + m) * 4 + (n & 3)];
}

// ------------------------------------------------------------------ the kernel
// GC: the given codes are read from global memory with the weights (codes too large for
// LDS: Down at 16 rows), one 16-byte code load per weight load, in batches of 4 steps.
template <int EPI, int NMAT, int LAYOUT, bool GC>
__global__ __launch_bounds__(kDcThreads) void decode_kernel(StreamKArgs p, DecodeGeom dg) {
  constexpr bool kReq = EPI == EPI_DOWN;   // FP32 input requantized with partial maxima
  constexpr int U = (NMAT == 2 || GC) ? 4 : 8;   // K steps per batch (8 loads of 16 bytes per lane)
  constexpr int NB = NMAT + (GC ? 1 : 0);        // loads per step: the weights (and the codes)
  __shared__ DcSmem sm;
  extern __shared__ __align__(16) int8_t lds[];
  int8_t* act = lds;                                               // [M][act_ld] codes
  int32_t* accum = reinterpret_cast<int32_t*>(lds + dg.acc_off);   // per segment, INT32 sums
  int32_t* lred = reinterpret_cast<int32_t*>(lds + dg.lred_off);   // control waves' partials
  constexpr int kPart = NMAT * 4 * kWave;                          // INT32 per partial

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int row16 = lane & 15, kg = lane >> 4;
  const int32_t b = static_cast<int32_t>(blockIdx.x);
  const int32_t St = dg.steps_tile, Ss = dg.steps_seg, P = St / Ss;
  int32_t tb0, nt;
  if (dg.leftover) {
    tb0 = b * dg.whole_q;
    nt = dg.whole_q;
  } else {
    tb0 = b * dg.whole_q + (b < dg.whole_r ? b : dg.whole_r);
    nt = dg.whole_q + (b < dg.whole_r ? 1 : 0);
  }
  const int64_t act_ld = dg.act_ld;
  const bool taps = b == 0;
  if (tid == 0) {
    sm.ctl_sync = 0;
    sm.lo_arrive = 0;
    sm.pf_done = 0;
    sm.scales_ready = 0;
    sm.task_next = 0;
    sm.task_done = 0;
    sm.codes_ready = 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the counters are set before barrier #1
  }

  // ---- phase 1: the control waves request row 0 of the input first, into LDS.
  int8_t* stage = lds + dg.acc_off;        // overlaps the accumulators (zeroed after it)
  int8_t* stage_g = stage + dg.stage_g;    // the RMSNorm gain
  __shared__ __align__(16) float pm_lds[kReq ? kPmWords : 4];
  uint32_t epoch = 0;
  // Given codes (rows quantized by an earlier kernel): copied as they are, with the row
  // scales; no prologue arithmetic.
  const bool codes_in = GC || p.prologue == PRO_CODES;   // (GC: always given codes)
  if (wave < kDcCtl) {
    if (codes_in) {
      if constexpr (!GC) stage_codes(p, act, dg.act_ld);
      // The row scales go straight into LDS like the codes: copied through a register,
      // their use would make the compiler wait for every load in flight, the leftover
      // quarter's weights included (measured on MI355X at 16 rows: the codes were
      // released 2 us after they had landed).
      if (tid < p.M)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(p.sa + tid),
                                         reinterpret_cast<__shared__ uint32_t*>(sm.row_scale),
                                         4, 0, 0);
    } else {
      if constexpr (kReq) {
        stage_pmax(p, pm_lds);
        stage_chunks<kF32Units>(p.hin, p.K * 4, stage);
      } else {
        stage_chunks<kBfUnits>(p.x, p.K * 2, stage);
        if (p.gamma) stage_chunks<kBfUnits>(p.gamma, p.K * 2, stage_g);
      }
    }
    epoch = *p.epoch_in;
  }
  // #1: every row request of the workgroup precedes every weight request.  A plain
  // barrier: a release fence here would also wait for the staged row to land.
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __asm__ __volatile__("" ::: "memory");

  // ---- the weight stream.  The workgroup's whole tiles are flattened into W = nt * St K
  // steps (tile-major); the stream waves take equal contiguous ranges of them.  (Measured
  // on MI355X at Qwen3-14B shapes: letting the control waves take a share once their
  // prologue work is done was slower at every size tried; the stream waves already keep
  // the CU's memory pipeline full.)  A wave keeps its INT32 sums in registers and adds them into the LDS accumulator of the
  // K segment (a tile, or a tile's K partition) when its range leaves that segment
  // (integer addition: exact in any order).  Loads run two batches of U steps ahead; they
  // are unconditional (past the range's end a wave re-reads its last step), so the
  // compiler's waits for one batch never cover the other.
  const int32_t W = nt * St;
  const int32_t ss = (W + kDcStream - 1) / kDcStream;
  int32_t r0 = 0, rn = 0;
  if (wave >= kDcCtl) {
    const int32_t sw = wave - kDcCtl;
    r0 = sw * ss < W ? sw * ss : W;
    rn = (r0 + ss < W ? r0 + ss : W) - r0;
  }
  const int32_t nb = (rn + U - 1) / U;
  const int32_t rlast = rn > 0 ? r0 + rn - 1 : 0;
  const bool aval = row16 < p.M;
  const int64_t aoff = (aval ? row16 : 0) * act_ld + kg * 16;
  const int64_t lane_off = (LAYOUT == LAYOUT_TILED) ? int64_t(lane) * 16
                                                    : int64_t(row16) * p.K + kg * 16;
  const int8_t* w0l = p.w0 + lane_off;
  const int8_t* w1l = (NMAT == 2) ? p.w1 + lane_off : nullptr;
  auto wofs = [&](int32_t f) -> int64_t {
    if constexpr (LAYOUT == LAYOUT_TILED) return (int64_t(tb0) * St + f) * 1024;
    const int32_t tl = f / St;
    return (int64_t(tb0) + tl) * 16 * p.K + int64_t(f - tl * St) * 64;
  };
  // GC: the codes of each step from global memory (tiled: 1 KB per K step, 16 bytes per
  // lane), K step from a load cursor (batches are requested in order); cached loads,
  // since every workgroup reads the same codes.
  const int8_t* cal = p.a + lane * 16;
  int32_t lk = r0 % St;
  auto load_batch = [&](i32x4 (&wv)[U][NB], int32_t i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t f = r0 + i * U + u;
      const int64_t o = wofs(f < rlast ? f : rlast);
      wv[u][0] = ld16_stream(w0l + o);
      if constexpr (NMAT == 2) wv[u][1] = ld16_stream(w1l + o);
      if constexpr (GC) {
        wv[u][NMAT] = *reinterpret_cast<const i32x4*>(cal + int64_t(lk) * 1024);
        if (++lk == St) lk = 0;
      }
    }
  };
  // Step cursor (wave-uniform): next step, its segment, the segment's end, its K step.
  int32_t cf = r0, csg = Ss > 0 ? r0 / Ss : 0, cend = (csg + 1) * Ss, ck = r0 % St;
  const int32_t rend = r0 + rn;
  i32x4 acc[NMAT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i) acc[i] = i32x4{0, 0, 0, 0};
  auto flush = [&]() {
    int32_t* dst = accum + csg * kPart + lane * 4;
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        __hip_atomic_fetch_add(dst + i * kWave * 4 + c, acc[i][c], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int i = 0; i < NMAT; ++i) acc[i] = i32x4{0, 0, 0, 0};
  };
  auto step = [&](const i32x4 (&wu)[NB]) {
    if (cf == cend) {
      flush();
      ++csg;
      cend += Ss;
    }
    if (ck == St) ck = 0;
    i32x4 v;
    if constexpr (GC) v = wu[NB - 1];
    else v = *reinterpret_cast<const i32x4*>(act + aoff + int64_t(ck) * 64);
    const i32x4 bv = aval ? v : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NMAT; ++i) acc[i] = mfma_i8(wu[i], bv, acc[i]);
    ++cf;
    ++ck;
  };
  // A batch that may run past the range's end (the last one).
  auto compute = [&](const i32x4 (&wv)[U][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cf < rend) step(wv[u]);
  };
  // A batch wholly inside the range (no range test).
  auto compute_full = [&](const i32x4 (&wv)[U][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(wv[u]);
  };
  // Batches 0 and 1 are requested by the caller; this streams the rest and flushes.
  auto stream_rest = [&](i32x4 (&wA)[U][NB], i32x4 (&wB)[U][NB]) {
    int32_t i = 0;
    for (; i + 3 < nb; i += 2) {   // batches i and i + 1 are whole
      compute_full(wA);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(wA, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_full(wB);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(wB, i + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nb - i == 3) {
      compute_full(wA);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(wA, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_full(wB);
      compute(wA);
    } else {
      compute_full(wA);
      compute(wB);
    }
    if (rn > 0) flush();
  };

  if (wave >= kDcCtl) {
    // ================================================================= stream waves
    // Down with one row: help with the codes once the first batch is requested.
    const bool help = kReq && p.M == 1 && !codes_in;
    auto help_codes = [&]() {
      if (help) {
        lds_wait_flag(&sm.scales_ready, 1);
        codes_tasks_f32(p, sm, act, lds + dg.acc_off, taps, sm.row_scale[0]);
      }
    };
    // A stream wave has no memory operation in flight before its first batch, so waiting
    // until at most that batch is outstanding costs nothing.  It tells the compiler that
    // the control waves' LDS-DMA requests (which it cannot tell apart from this wave's
    // own) are done; while it believes one is in flight, every wait for a weight it
    // emits waits for all loads, and the two batches no longer overlap.
    auto after_first_batch = [&]() {
      __asm__ __volatile__("" ::: "memory");
      constexpr int kB = U * NB;   // vmcnt(kB); expcnt and lgkmcnt unconstrained
      __builtin_amdgcn_s_waitcnt((kB & 0xF) | 0x0F70 | ((kB >> 4) << 14));
      __asm__ __volatile__("" ::: "memory");
    };
    if (nb <= 1) {
      // A range of one batch (O and single-tile QKV workgroups at Qwen3-14B shapes):
      // no second batch, whose loads would only re-read the last step.
      i32x4 wA[U][NB];
      load_batch(wA, 0);
      __builtin_amdgcn_sched_barrier(0);
      after_first_batch();
      help_codes();
      lds_wait_flag(&sm.codes_ready, 1);   // the codes are in LDS, the accumulators cleared
      __builtin_amdgcn_sched_barrier(0);
      compute(wA);
      if (rn > 0) flush();
    } else {
      i32x4 wA[U][NB], wB[U][NB];
      load_batch(wA, 0);
      __builtin_amdgcn_sched_barrier(0);
      after_first_batch();
      help_codes();
      load_batch(wB, 1);
      __builtin_amdgcn_sched_barrier(0);
      lds_wait_flag(&sm.codes_ready, 1);
      __builtin_amdgcn_sched_barrier(0);
      stream_rest(wA, wB);
    }
  } else {
    // ================================================================= control waves
    // The leftover quarter's weights are requested right behind the row: the control waves
    // are the oldest of the workgroup, so these loads are queued ahead of most of the
    // stream and have landed by the time the codes are ready.  Each control wave takes a
    // quarter of the quarter; the first V steps of it are requested here.
    constexpr int V = lo_steps(EPI);
    const int32_t Q = St / 4, qq = b & 3;
    const int32_t lt = dg.leftover ? dg.grid * dg.whole_q + b / 4 : -1;
    const int32_t ql = Q / kDcCtl, qr = Q % kDcCtl;
    const int32_t ls0 = qq * Q + wave * ql + (wave < qr ? wave : qr);
    const int32_t ls1 = ls0 + ql + (wave < qr ? 1 : 0);
    i32x4 lw[V][NMAT];
    // Down's share is longer than its register budget: the next VL steps go straight into
    // an LDS array of their own, requested with the rest.
    // With codes in global memory (GC) the codes of all V + VL steps are copied into LDS
    // too, behind the weights' copies.
    constexpr int VL = lo_lds_steps(EPI);
    constexpr int VC = GC ? V + VL : 0;
    constexpr int kLoLds = kDcCtl * VL * 1024;
    __shared__ __align__(16) int8_t lo_lds[VL + VC > 0 ? kLoLds + kDcCtl * VC * 1024 : 16];
    auto lo_code_lds = [&](int u) -> i32x4 {   // GC: codes of step ls0 + u
      return *reinterpret_cast<const i32x4*>(lo_lds + kLoLds + (wave * VC + u) * 1024 + lane * 16);
    };
    auto load_lo_lds = [&]() {
#pragma unroll
      for (int u = 0; u < VL; ++u) {
        const int32_t sv = ls0 + V + u;
        const int32_t sq = sv < ls1 ? sv : ls1 - 1;
        const int64_t o = (LAYOUT == LAYOUT_TILED) ? (int64_t(lt) * St + sq) * 1024
                                                   : int64_t(lt) * 16 * p.K + int64_t(sq) * 64;
        // Lane l's 16 bytes land at lo_lds + (wave * VL + u) * 1024 + 16 * l.
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(w0l + o),
                                         reinterpret_cast<__shared__ uint32_t*>(
                                             lo_lds + (wave * VL + u) * 1024),
                                         16, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < VC; ++u) {
        const int32_t sq = ls0 + u < ls1 ? ls0 + u : ls1 - 1;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(cal + int64_t(sq) * 1024),
                                         reinterpret_cast<__shared__ uint32_t*>(
                                             lo_lds + kLoLds + (wave * VC + u) * 1024),
                                         16, 0, 0);
      }
    };
    auto load_lo = [&](int32_t s0) {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int32_t sq = (s0 + u < ls1) ? s0 + u : ls1 - 1;
        const int64_t o = (LAYOUT == LAYOUT_TILED) ? (int64_t(lt) * St + sq) * 1024
                                                   : int64_t(lt) * 16 * p.K + int64_t(sq) * 64;
        lw[u][0] = ld16_stream(w0l + o);
        if constexpr (NMAT == 2) lw[u][1] = ld16_stream(w1l + o);
      }
    };

    if (dg.leftover) {
      // The LDS-bound steps first: this wave's last copy into LDS is then older than its
      // register loads, and the wait below covers it.  (While the compiler counts a copy
      // into LDS as possibly in flight, every wait it emits is for all loads: the row scales
      // would wait for the leftover's weights.)
      if constexpr (VL + VC > 0) load_lo_lds();
      load_lo(ls0);
      __builtin_amdgcn_sched_barrier(0);
      // The row, the partial maxima and the LDS-bound steps, requested before these V * NMAT
      // loads, which complete in order, have landed.
      __asm__ __volatile__("" ::: "memory");
      constexpr int kAfter = V * NMAT;   // vmcnt(kAfter); expcnt and lgkmcnt unconstrained
      __builtin_amdgcn_s_waitcnt((kAfter & 0xF) | 0x0F70 | ((kAfter >> 4) << 14));
      __asm__ __volatile__("" ::: "memory");
    } else {
      wait_memory_done();   // this wave's staged chunks (and the partial maxima) have landed
    }
    int gen = 0;
    ctl_sync(sm, gen);    // ... and every control wave's
    if (codes_in) {
      // The row scales are in LDS already.
    } else if constexpr (kReq) {
      if (p.M == 1) {
        // One row: every wave takes code tasks (the stream waves once their first batch
        // is requested); the row is dead when all tasks are done.
        const float s0 = ctl_requant_scale_one(p, sm, pm_lds, taps, gen);
        if (tid == 0) {
          lds_release_only();   // the row scale before the flag
          lds_set_flag(&sm.scales_ready, 1);
        }
        codes_tasks_f32(p, sm, act, stage, taps, s0);
        lds_wait_flag(&sm.task_done, code_tasks(p.K));
      } else {
        ctl_requant_scales(p, sm, pm_lds, taps, gen);
        __builtin_amdgcn_sched_barrier(0);
        ctl_row_f32(p, sm, act, 0, stage, taps);
      }
      for (int m = 1; m < p.M; ++m) {
        ctl_sync(sm, gen);  // row m - 1 read by every control wave
        stage_chunks<kF32Units>(p.hin + int64_t(m) * p.ldhin, p.K * 4, stage);
        wait_memory_done();
        ctl_sync(sm, gen);
        ctl_row_f32(p, sm, act + m * act_ld, m, stage, taps);
      }
    } else {
      ctl_row_bf16(p, sm, act, 0, stage, stage_g, taps, gen);
      for (int m = 1; m < p.M; ++m) {
        ctl_sync(sm, gen);
        stage_chunks<kBfUnits>(p.x + int64_t(m) * p.ldx, p.K * 2, stage);
        wait_memory_done();
        ctl_sync(sm, gen);
        ctl_row_bf16(p, sm, act + m * act_ld, m, stage, stage_g, taps, gen);
      }
    }
    // The staged row is dead once every control wave has read it: clear the accumulators,
    // then release the stream waves.
    ctl_sync(sm, gen);
    for (int e = tid; e < nt * P * kPart / 4; e += kDcCtlThreads)
      reinterpret_cast<i32x4*>(accum)[e] = i32x4{0, 0, 0, 0};
    ctl_sync(sm, gen);
    if (tid == 0) lds_set_flag(&sm.codes_ready, 1);

    // The leftover quarter's matrix work (its first V steps have landed by now).
    int prev = -1;
    if (dg.leftover) {
      // Codes of leftover step st past the early ones (clamped into the share).
      auto lo_code = [&](int32_t st) -> i32x4 {
        const int32_t sc = st < ls1 ? st : ls1 - 1;
        if constexpr (GC) return *reinterpret_cast<const i32x4*>(cal + int64_t(sc) * 1024);
        else return *reinterpret_cast<const i32x4*>(act + aoff + int64_t(sc) * 64);
      };
      i32x4 lacc[NMAT];
#pragma unroll
      for (int i = 0; i < NMAT; ++i) lacc[i] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if (ls0 + u < ls1) {
          i32x4 v;
          if constexpr (GC) v = lo_code_lds(u);
          else v = *reinterpret_cast<const i32x4*>(act + aoff + int64_t(ls0 + u) * 64);
          const i32x4 bv = aval ? v : i32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < NMAT; ++i) lacc[i] = mfma_i8(lw[u][i], bv, lacc[i]);
        }
      }
      if constexpr (VL > 0) {
#pragma unroll
        for (int u = 0; u < VL; ++u) {
          if (ls0 + V + u < ls1) {
            const i32x4 wv = *reinterpret_cast<const i32x4*>(lo_lds + (wave * VL + u) * 1024 + lane * 16);
            i32x4 v;
            if constexpr (GC) v = lo_code_lds(V + u);
            else v = *reinterpret_cast<const i32x4*>(act + aoff + int64_t(ls0 + V + u) * 64);
            const i32x4 bv = aval ? v : i32x4{0, 0, 0, 0};
            lacc[0] = mfma_i8(wv, bv, lacc[0]);
          }
        }
      }
      // Steps past those requested early (shapes with longer quarters) load now.
      for (int32_t s0 = ls0 + V + VL; s0 < ls1; s0 += V) {
        load_lo(s0);
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const i32x4 v = lo_code(s0 + u);
          if (s0 + u < ls1) {
            const i32x4 bv = aval ? v : i32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < NMAT; ++i) lacc[i] = mfma_i8(lw[u][i], bv, lacc[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
        *reinterpret_cast<i32x4*>(lred + wave * kPart + (i * kWave + lane) * 4) = lacc[i];
      lds_release_only();
      if (lane == 0)
        prev = __hip_atomic_fetch_add(&sm.lo_arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      prev = __builtin_amdgcn_readfirstlane(prev);
    }
    const bool last = prev == kDcCtl - 1;   // the last control wave to finish its part

    // Epilogue inputs of the workgroup's tiles (and of its leftover tile) into LDS: every
    // load is issued before the first store, so they cost one memory round trip.
    const int ct = tid;
    constexpr int kSwN = (kDcMaxTiles + 1) * 16 * NMAT;                  // <= 192
    constexpr int kResN = (kDcMaxTiles + 1) * kDcMaxRows * 16;           // 1536
    constexpr int kResIt = (kResN + kDcCtlThreads - 1) / kDcCtlThreads;  // 6
    float swv = 0.0f;
    int32_t sw_t = -1;
    int sw_slot = 0, sw_mat = 0, sw_c = 0;
    if (ct < kSwN) {
      sw_slot = ct / (16 * NMAT);
      const int rem = ct % (16 * NMAT);
      sw_mat = rem / 16;
      sw_c = rem % 16;
      sw_t = sw_slot < kDcMaxTiles ? (sw_slot < nt ? tb0 + sw_slot : -1) : lt;
      if (sw_t >= 0) swv = (sw_mat == 0 ? p.sw0 : p.sw1)[int64_t(sw_t) * 16 + sw_c];
    }
    uint16_t rv[kResIt];
    int32_t r_t[kResIt];
    int r_slot[kResIt], r_m[kResIt], r_c[kResIt];
#pragma unroll
    for (int it = 0; it < kResIt; ++it) {
      const int e = ct + it * kDcCtlThreads;
      r_slot[it] = e / (kDcMaxRows * 16);
      const int rem = e % (kDcMaxRows * 16);
      r_m[it] = rem / 16;
      r_c[it] = rem % 16;
      r_t[it] = -1;
      rv[it] = 0;
      if constexpr (EPI == EPI_BF16_RES || EPI == EPI_DOWN) {
        if (e < kResN && r_m[it] < p.M) {
          r_t[it] = r_slot[it] < kDcMaxTiles ? (r_slot[it] < nt ? tb0 + r_slot[it] : -1) : lt;
          if (r_t[it] >= 0) rv[it] = p.res[int64_t(r_m[it]) * p.ldr + int64_t(r_t[it]) * 16 + r_c[it]];
        }
      }
    }

    // The last control wave adds the four partials and publishes the quarter; the owner of
    // quarter 0 gathers the other three instead (they are published early in workgroups
    // b + 1 .. b + 3, so this usually succeeds within a few reads).  The wait is bounded;
    // past the bound the tile's output is left unwritten.
    const uint32_t tag32 = epoch ^ (uint32_t(EPI + 1) << 29);
    uint64_t* slots = reinterpret_cast<uint64_t*>(p.slots);
    i32x4 piece[NMAT], got[3][NMAT];
    bool ok = false;
    if (last) {
      __asm__ __volatile__("" ::: "memory");
#pragma unroll
      for (int i = 0; i < NMAT; ++i) {
        piece[i] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < kDcCtl; ++w)
          piece[i] += *reinterpret_cast<const i32x4*>(lred + w * kPart + (i * kWave + lane) * 4);
      }
      // Slot block layout: word c * 64 + lane holds component c of the lane's sums, so
      // each store instruction writes 512 contiguous bytes (whole lines).
      if (qq != 0) {
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
          store_tagged_lanes(slots + (int64_t(b) * NMAT + i) * kSlotWords, lane, piece[i], tag32);
      } else {
        // Poll one word per neighbour (lanes 0-2: word 0 of its first block, the first
        // one it writes) until each carries the call's tag, then read every word; a word
        // still missing sends the wave back to the full read.  (A full read as the first
        // attempt measured slower: when it fails, it costs a round trip under the weight
        // stream before the polling starts.)  Every wait is bounded.
        bool seen = false;
        for (int attempt = 0; attempt < (1 << 16) && !seen; ++attempt) {
          bool mine = true;
          if (lane < 3) {
            const uint64_t w0 = __hip_atomic_load(slots + int64_t(b + 1 + lane) * NMAT * kSlotWords,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            mine = uint32_t(w0 >> 32) == tag32;
          }
          seen = __builtin_amdgcn_ballot_w64(!mine) == 0;
          if (!seen) __builtin_amdgcn_s_sleep(8);
        }
        for (int attempt = 0; attempt < (1 << 12) && seen && !ok; ++attempt) {
          bool all = true;
#pragma unroll
          for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int i = 0; i < NMAT; ++i) {
              const TaggedX4 tw =
                  load_tagged_lanes(slots + (int64_t(b + 1 + j) * NMAT + i) * kSlotWords, lane);
              got[j][i] = i32x4{0, 0, 0, 0};
              add_tagged(got[j][i], tw, tag32, all);
            }
          ok = __builtin_amdgcn_ballot_w64(!all) == 0;
          if (!ok) __builtin_amdgcn_s_sleep(2);
        }
      }
    }

    // The epilogue inputs to LDS.
    if (sw_t >= 0) sm.sw[sw_slot][sw_mat][sw_c] = swv;
#pragma unroll
    for (int it = 0; it < kResIt; ++it)
      if (r_t[it] >= 0) sm.res[r_slot[it]][r_m[it]][r_c[it]] = rv[it];

    if (dg.leftover) {
      lds_release_only();
      if (lane == 0) lds_add_sync(&sm.pf_done, 1);
      if (last && qq == 0 && ok) {
        // The tile's sums per K partition into LDS (the partials just read are dead):
        // quarter j lies in partition j / qpp; quarter 0 is this workgroup's piece.
        const int32_t qpp = Ss / Q;   // quarters per K partition
        for (int q = 0; q < P; ++q)
#pragma unroll
          for (int i = 0; i < NMAT; ++i) {
            i32x4 a = q == 0 ? piece[i] : i32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 3; ++j) a += ((j + 1) / qpp == q) ? got[j][i] : i32x4{0, 0, 0, 0};
            *reinterpret_cast<i32x4*>(lred + q * kPart + (i * kWave + lane) * 4) = a;
          }
        lds_wait_flag(&sm.pf_done, kDcCtl);   // every control wave's epilogue inputs
        for (int32_t pq0 = 0; pq0 < p.M; pq0 += 4)
          dc_epilogue<EPI, NMAT>(
              p, sm, static_cast<int32_t>(p.M), pq0 + lane / 16, P,
              [&](int32_t, int q, int mat, int64_t m, int n) {
                return acc_elem(lred + q * kPart, mat, m, n);
              },
              [&](int32_t) { return lt; }, [&](int32_t) { return kDcMaxTiles; });
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // #3: every range is added into its segments' accumulators

  // ---- epilogue of the whole tiles, one (tile, row) pair per 16 lanes.
  {
    const int32_t npairs = nt * static_cast<int32_t>(p.M);
    for (int32_t pq0 = wave * 4; pq0 < npairs; pq0 += kDcWaves * 4)
      dc_epilogue<EPI, NMAT>(
          p, sm, npairs, pq0 + lane / 16, P,
          [&](int32_t j, int q, int mat, int64_t m, int n) {
            return acc_elem(accum + (j * P + q) * kPart, mat, m, n);
          },
          [&](int32_t j) { return tb0 + j; }, [&](int32_t j) { return static_cast<int>(j); });
  }
  if (b == 0 && tid == 0) *p.epoch_out = epoch + 1;
}

template <int EPI, int NMAT, int LAYOUT, bool GC = false>
hipError_t launch_t(const StreamKArgs& a, const DecodeGeom& g, hipStream_t s) {
  const auto kern = decode_kernel<EPI, NMAT, LAYOUT, GC>;
  if (g.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, g.lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(g.grid)), dim3(kDcThreads),
                     static_cast<size_t>(g.lds), s, a, g);
  return hipGetLastError();
}

template <int EPI, int NMAT, bool GC = false>
hipError_t launch_l(const StreamKArgs& a, const DecodeGeom& g, hipStream_t s) {
  if (a.layout == LAYOUT_TILED) return launch_t<EPI, NMAT, LAYOUT_TILED, GC>(a, g, s);
  return launch_t<EPI, NMAT, LAYOUT_ROWMAJOR, GC>(a, g, s);
}

}  // namespace

bool plan_decode(int epi, int64_t M, int64_t N, int64_t K, int parts, bool codes_in,
                 DecodeGeom& g) {
  g = DecodeGeom{};
  if (M < 1 || M > (codes_in ? kDcMaxRows : kFuseMaxRows) || N % 16 || K % 64 || N <= 0)
    return false;
  const int nmat = epi == EPI_SILU ? 2 : 1;
  const int P = epi == EPI_DOWN ? parts : 1;
  const int64_t T = N / 16, St = K / 64;
  if (St % P) return false;
  const int64_t Ss = St / P;
  if (P > 8) return false;
  // Prologue registers: the control waves hold a whole input row.
  if (!codes_in && (epi == EPI_DOWN ? K > kF32MaxK : K > kBfMaxK)) return false;
  if (T >= (int64_t(1) << 24) || St >= (int64_t(1) << 20)) return false;
  // Static LDS of the kernel beside the dynamic part.
  const size_t stat = sizeof(DcSmem) +
                      (epi == EPI_DOWN ? kPmWords * 4 + size_t(kDcCtl) * lo_lds_steps(EPI_DOWN) * 1024 : 32);
  // Given codes read from global memory beside the weights, in the tiled order (every
  // workgroup reads the same codes, which stay in L2), instead of copied into LDS first:
  // Down when the codes do not fit LDS (Qwen3-14B at 16 rows: 278 KB), and QKV and O at
  // more than 4 rows, whose copy of the codes (80 KB at 16 rows) holds back the stream
  // by about 3 us (measured on MI355X at 16 rows: QKV 12.0 -> 11.3 us, O 11.0 -> 10.8 us).
  // Gate/Up keeps the copy: three loads per step instead of two cost it 6 us.
  const size_t part = size_t(nmat) * 4 * kWave * 4;   // bytes of one segment's sums
  const bool gc =
      codes_in && ((M > 4 && (epi == EPI_BF16 || epi == EPI_BF16_RES)) ||
                   (epi == EPI_DOWN &&
                    size_t(M) * size_t(K + 16) + size_t(kDcCtl + 1) * P * part + stat > kDcLdsPerCu));
  int64_t G = T < kDcMaxGrid ? T : kDcMaxGrid;
  // QKV and O: equal whole tiles for every workgroup when a grid of at least 5/8 of the
  // largest one divides the tiles (Qwen3-14B: QKV 448 = 224 x 2, O 320 = 160 x 2).  Measured
  // on MI355X, a plain weight stream keeps its rate on 160 or more CUs, and O then needs no
  // leftover exchange (its span fell from 8.0 to 6.9 us).  For Down the longer stream per
  // workgroup cost more than the exchange it saves.
  if ((epi == EPI_BF16 || epi == EPI_BF16_RES) && T > kDcMaxGrid)
    for (int64_t gg = kDcMaxGrid; gg * 8 >= kDcMaxGrid * 5; --gg)
      if (T % gg == 0 && T / gg <= kDcMaxTiles) {
        G = gg;
        break;
      }
  const int64_t q = T / G, r = T % G;
  // Leftover quarters: the last G/4 tiles are split in K quarters, one per workgroup,
  // each inside one K partition.
  const bool left = r != 0 && G % 4 == 0 && 4 * r == G && St % 4 == 0 && (St / 4) % kDcCtl == 0 &&
                    Ss % (St / 4) == 0 && P <= kDcCtl;
  const int64_t ntmax = left ? q : q + (r ? 1 : 0);
  if (ntmax > kDcMaxTiles) return false;
  g.tiles = static_cast<int32_t>(T);
  g.steps_tile = static_cast<int32_t>(St);
  g.steps_seg = static_cast<int32_t>(Ss);
  g.grid = static_cast<int32_t>(G);
  g.whole_q = static_cast<int32_t>(q);
  g.whole_r = static_cast<int32_t>(left ? 0 : r);
  g.leftover = left ? 1 : 0;
  g.gcodes = gc ? 1 : 0;
  // Rows of codes 16 bytes apart in LDS banks: the 16 rows a step reads (one per lane
  // group) then fall in different banks.  (With K a multiple of 256 bytes and no padding
  // they all fall in the same four.)
  const bool pad = M > 1 && (K / 16) % kWave == 0;
  g.act_ld = static_cast<int32_t>(pad ? K + 16 : K);
  const size_t codes = gc ? 0 : (size_t(M) * size_t(g.act_ld) + 255) / 256 * 256;
  g.acc_off = static_cast<int32_t>(codes);
  g.lred_off = static_cast<int32_t>(codes + size_t(ntmax) * P * part);
  // Staging of the input row at acc_off: FP32 h (Down) or BF16 x followed by the gain.
  const size_t unit_bytes = size_t(kDcCtlThreads) * 16;
  const size_t stage = codes_in ? 0 : epi == EPI_DOWN ? kF32Units * unit_bytes : 2 * kBfUnits * unit_bytes;
  g.stage_g = static_cast<int32_t>(kBfUnits * unit_bytes);
  size_t lds = size_t(g.lred_off) + size_t(kDcCtl) * part;
  if (codes + stage > lds) lds = codes + stage;
  // Dynamic LDS plus the kernel's static LDS within the CU's 160 KB.
  // (GC: the kernel's leftover array also holds the codes of the leftover's early steps.)
  const size_t stat_k = stat + (gc ? size_t(kDcCtl) * (lo_steps(epi) + lo_lds_steps(epi)) * 1024 : 0);
  if (lds > kDcMaxLds || lds + stat_k > kDcLdsPerCu) return false;
  g.lds = static_cast<int32_t>(lds);
  return true;
}

size_t decode_slot_elems(const DecodeGeom& g, int nmat) {
  // One tagged 64-bit word (two INT32 elements) per partial sum of each published quarter.
  return g.leftover ? 2 * size_t(g.grid) * size_t(nmat) * kSlotWords : 0;
}

hipError_t launch_decode(const StreamKArgs& a, const DecodeGeom& g, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  switch (a.epi) {
    case EPI_BF16:
      if (g.gcodes) return launch_l<EPI_BF16, 1, true>(a, g, s);
      return launch_l<EPI_BF16, 1>(a, g, s);
    case EPI_BF16_RES:
      if (g.gcodes) return launch_l<EPI_BF16_RES, 1, true>(a, g, s);
      return launch_l<EPI_BF16_RES, 1>(a, g, s);
    case EPI_SILU: return launch_l<EPI_SILU, 2>(a, g, s);
    case EPI_DOWN:
      if (g.gcodes) return launch_l<EPI_DOWN, 1, true>(a, g, s);
      return launch_l<EPI_DOWN, 1>(a, g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace a8w8
