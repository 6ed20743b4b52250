// Stream-K INT8 x INT8 -> INT32 decode GEMM on gfx950 matrix cores, with fused
// activation quantization (prologue) and fused dequant / SiLU / residual / split-K
// epilogues.  It serves the MLP block and the layer chain.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path (Gate/Up as INT8 x INT8 products summed in
// INT32, the sums turned into FP32 with the row scale and the channel scale, the
// normalized activations after attention given one INT8 scale per row) and > Decode scheduling (Down
// split two ways along K into independent accumulators), plus the CodeRabbit
// walkthrough row "Split down projection accumulation" (FP32 partials summed and
// narrowed together with the residual).  QKV and O reuse the same pattern.
//
// At decode batch sizes the weights are the traffic: every weight byte is read from HBM
// once and the kernel is a weight stream.
//   * The unit of work is a 64-byte K step of a 16-channel tile: one
//     v_mfma_i32_16x16x64_i8 with the weights as A (lane l feeds channel l%16 with the
//     16 bytes at k-offset 16*(l/16)) and the activation codes as B (one column per
//     decode row, zeros for missing rows).  Lane l's result holds channels 4*(l/16)+r of
//     row l%16.
//   * All steps of the problem form one sequence ordered by K chunk, tile, step.  In the
//     tiled weight layout a (chunk, tile) segment is one contiguous run of bytes.  The
//     sequence is dealt out in order and evenly (to one step) to every wave of a grid
//     sized to the machine, so all waves stream the same number of bytes and finish
//     together.  A wave keeps two batches of weight loads in flight in two register sets.
//   * When its range is done a wave leaves the INT32 partial sums of the (at most two)
//     segments it touched in LDS; the workgroup then adds its waves' partials per
//     segment.  A tile held by one workgroup alone goes straight to the epilogue; for
//     the others each workgroup stores its piece to a slot of its own as 64-bit words
//     that pair each value with the call's tag, waits until they are visible, and reads
//     every piece of the tile; a wave that finds the call's tag in all of them adds the
//     slots and runs the epilogue (two memory round trips).  Integer addition is exact,
//     so the result does not depend on the split.  A word holding another call's tag
//     counts as missing, so nothing needs clearing between calls, and no address is
//     contended.
//   * Fused prologue: every workgroup re-derives the row statistics (RMSNorm sum of
//     squares and absolute maximum, or the maximum of per-tile partial maxima for the
//     requantized Down input) and writes the codes of the K chunks its waves consume to
//     LDS.  Its first batch of weight loads is issued before it.
//   * No wait in the streaming loop covers more than the batch being consumed: loads are
//     unconditional with clamped addresses, dead steps multiply a zero operand, and the
//     workgroup barriers order LDS only.
#include "device_common.h"
#include "internal.h"

namespace a8w8 {

// First step of wave w (w = W gives the total).
__host__ __device__ inline int32_t sk_wave_start(const StreamKGeom& g, int32_t w) {
  return w * g.q + (w < g.r ? w : g.r);
}

// Wave whose range holds step f.
__host__ __device__ inline int32_t sk_owner(const StreamKGeom& g, int32_t f) {
  const int32_t cut = g.r * (g.q + 1);
  return f < cut ? static_cast<int32_t>(g.by_q1.div(static_cast<uint32_t>(f)))
                 : g.r + static_cast<int32_t>(g.by_q.div(static_cast<uint32_t>(f - cut)));
}

// K chunks [c0, c1] of the steps dealt to workgroup b (waves b*NW .. b*NW+NW-1).
__host__ __device__ inline void sk_wg_chunks(const StreamKGeom& g, int32_t b, int32_t NW,
                                             int32_t& c0, int32_t& c1) {
  const int32_t wl = (b + 1) * NW < g.waves ? (b + 1) * NW : g.waves;
  const int32_t A = sk_wave_start(g, b * NW), B = sk_wave_start(g, wl);
  c0 = static_cast<int32_t>(g.by_tiles.div(g.by_seg.div(static_cast<uint32_t>(A))));
  c1 = B > A ? static_cast<int32_t>(g.by_tiles.div(g.by_seg.div(static_cast<uint32_t>(B - 1)))) : c0;
}

namespace {

constexpr int kSkWaves = 8;
constexpr int64_t kSkTargetWgs = 512;      // two 8-wave workgroups per CU
constexpr int64_t kSkSmallWgs = 256;       // one per CU for GEMMs under kSkSmallSteps
constexpr int64_t kSkSmallSteps = 65536;
constexpr int64_t kSkMinSteps = 4;         // at least 4 KB of weights per wave
constexpr int64_t kSkTileWgsMin = 256;     // fewest tiles for one tile per workgroup
constexpr int kPV = 2;                     // prologue vectors of 8 values per thread
constexpr int64_t kPrologueMax = int64_t(kPV) * 8 * kSkWaves * kWave;  // 8192 values
constexpr size_t kSkMaxLds = 64 * 1024;

template <int NW>
struct SkSmem {
  double sum_slots[kFuseMaxRows][NW];
  float max_slots[kFuseMaxRows][NW];
  float row_scale[kFuseMaxRows];
  int32_t seg_lo[NW], seg_hi[NW];  // segments of each wave's partial sums (-1: none)
};

// Row 0's BF16 prologue inputs, fetched before the first weight batch: a wait for them
// then never covers weight loads (the memory counter completes in order).  Raw 16-byte
// registers (8 BF16 of x and of the gain) loaded unconditionally from clamped
// addresses; elements past the row are discarded where they are used.
struct PrologueRegs {
  u32x4 a[kPV];  // x[k..k+8) as BF16
  u32x4 b[kPV];  // gain[k..k+8) as BF16
};

template <int NW, int PRO>
__device__ __forceinline__ void sk_prologue_fetch(const StreamKArgs& p, int64_t klo, int64_t len,
                                                  PrologueRegs& r) {
  static_assert(PRO == PRO_QUANT_BF16, "only the BF16 prologue prefetches");
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kPV; ++j) {
    const int64_t e = int64_t(j) * NT * 8 + tid * 8;
    const int64_t k = e < p.K ? e : p.K - 8;
    r.a[j] = *reinterpret_cast<const u32x4*>(p.x + k);
    r.b[j] = *reinterpret_cast<const u32x4*>((p.gamma ? p.gamma : p.x) + k);
  }
}

// BF16 prologue, one row: RMSNorm (when a gain is given), row scale into
// sm.row_scale[m], codes of K values [klo, klo + len) into act[m * act_ld + (k - klo)].
// The row is held in registers (K <= kPrologueMax, checked by the planner).  Row 0
// comes from the prefetched registers (FIRST, no load on its path); later rows are
// loaded here.
template <int NW, int PRO, bool FIRST, typename SM>
__device__ __forceinline__ void sk_prologue_row(const StreamKArgs& p, SM& sm, int8_t* act,
                                                int64_t act_ld, int64_t klo, int64_t len,
                                                bool taps, const PrologueRegs& pre, int m) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
  float v[kPV][8];
  float s;
  int64_t vbase;  // K index of element (j, i) is vbase + j * NT * 8 + tid * 8 + i
  static_assert(PRO == PRO_QUANT_BF16, "the BF16 row prologue");
  {
    // RMSNorm statistics over the whole row, then the absolute maximum.
    vbase = 0;
    float g[kPV][8];
    const uint16_t* xr = p.x + int64_t(m) * p.ldx;
#pragma unroll
    for (int j = 0; j < kPV; ++j) {
      const int64_t k = int64_t(j) * NT * 8 + tid * 8;
      const bool in = k < p.K;
      u32x4 xa = pre.a[j], ga = pre.b[j];
      if constexpr (!FIRST) {
        const int64_t kc = in ? k : p.K - 8;
        xa = *reinterpret_cast<const u32x4*>(xr + kc);
        ga = *reinterpret_cast<const u32x4*>((p.gamma ? p.gamma : xr) + kc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = in ? bf16_lo(xa[i]) : 0.0f;
        v[j][2 * i + 1] = in ? bf16_hi(xa[i]) : 0.0f;
        g[j][2 * i] = bf16_lo(ga[i]);
        g[j][2 * i + 1] = bf16_hi(ga[i]);
      }
    }
    if (p.gamma) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < kPV; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += double(v[j][i]) * double(v[j][i]);
      const double S = block_sum_f64<NW>(ss, sm.sum_slots[m]);
      const float ms = static_cast<float>(S / static_cast<double>(p.K));
      const float t = ms + p.eps;
      const float r = 1.0f / __builtin_sqrtf(t);
#pragma unroll
      for (int j = 0; j < kPV; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = (v[j][i] * r) * g[j][i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPV; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    amax = block_max_f32<NW>(amax, sm.max_slots[m]);
    s = amax / 127.0f;
  }
  if (tid == 0) {
    sm.row_scale[m] = s;
    if (taps && p.tap_s) p.tap_s[m] = s;
  }
#pragma unroll
  for (int j = 0; j < kPV; ++j) {
    const int64_t k = vbase + int64_t(j) * NT * 8 + tid * 8;
    if (k >= klo && k < klo + len) {
      const u32x2 c = codes8(v[j], s);
      *reinterpret_cast<u32x2*>(act + m * act_ld + (k - klo)) = c;
      if (taps && p.tap_q) *reinterpret_cast<u32x2*>(p.tap_q + int64_t(m) * p.K + k) = c;
      if (taps && p.tap_xn) {
        f32x4* tx = reinterpret_cast<f32x4*>(p.tap_xn + int64_t(m) * p.K + k);
        tx[0] = f32x4{v[j][0], v[j][1], v[j][2], v[j][3]};
        tx[1] = f32x4{v[j][4], v[j][5], v[j][6], v[j][7]};
      }
    } else if (taps && k < p.K) {
      // Taps cover the whole row; workgroup 0 writes them.
      const u32x2 c = codes8(v[j], s);
      if (p.tap_q) *reinterpret_cast<u32x2*>(p.tap_q + int64_t(m) * p.K + k) = c;
      if (p.tap_xn) {
        f32x4* tx = reinterpret_cast<f32x4*>(p.tap_xn + int64_t(m) * p.K + k);
        tx[0] = f32x4{v[j][0], v[j][1], v[j][2], v[j][3]};
        tx[1] = f32x4{v[j][4], v[j][5], v[j][6], v[j][7]};
      }
    }
  }
}

// Fused prologue for rows 0..M-1, then one barrier for the codes in LDS.
template <int NW, int PRO, typename SM>
__device__ void sk_prologue(const StreamKArgs& p, SM& sm, int8_t* act, int64_t act_ld,
                            int64_t klo, int64_t len, bool taps, const PrologueRegs& pre) {
  sk_prologue_row<NW, PRO, true>(p, sm, act, act_ld, klo, len, taps, pre, 0);
  for (int m = 1; m < p.M; ++m)
    sk_prologue_row<NW, PRO, false>(p, sm, act, act_ld, klo, len, taps, pre, m);
  lds_barrier();
}

// Requantization prologue (Down input): the row scale comes from the per-tile partial
// maxima, so the K values [klo, klo + len) are quantized straight into LDS in a loop.
// Row 0's first partial maxima and values are fetched before any weight load
// (RequantRegs), so the wait for them never covers weight loads; the rest is loaded here.
constexpr int kReqPm = 3;  // partial maxima of row 0 per thread fetched ahead
constexpr int kReqHv = 5;  // 8-value groups of row 0 per thread fetched ahead (17408 values)

struct RequantRegs {
  float pm[kReqPm];
  f32x4 hv[kReqHv][2];
};

template <int NW>
__device__ __forceinline__ void sk_requant_fetch(const StreamKArgs& p, int64_t klo, int64_t len,
                                                 RequantRegs& r) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kReqPm; ++j) {
    const int64_t k = tid + int64_t(j) * NT;
    r.pm[j] = p.pmax[(k < p.npmax ? k : 0) * p.M];
  }
#pragma unroll
  for (int i = 0; i < kReqHv; ++i) {
    const int64_t e = int64_t(tid) * 8 + int64_t(i) * NT * 8;
    const f32x4* q = reinterpret_cast<const f32x4*>(p.hin + klo + (e < len ? e : 0));
    r.hv[i][0] = q[0];
    r.hv[i][1] = q[1];
  }
}

template <int NW, typename SM>
__device__ void sk_requant_prologue(const StreamKArgs& p, SM& sm, int8_t* act, int64_t act_ld,
                                    int64_t klo, int64_t len, bool taps, const RequantRegs& r) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
  for (int m = 0; m < p.M; ++m) {
    float amax = 0.0f;
    int64_t k = tid;
    if (m == 0) {
#pragma unroll
      for (int j = 0; j < kReqPm; ++j, k += NT)
        if (k < p.npmax) amax = fmaxf(amax, r.pm[j]);
    }
    for (; k < p.npmax; k += NT) amax = fmaxf(amax, p.pmax[k * p.M + m]);
    amax = block_max_f32<NW>(amax, sm.max_slots[m]);
    const float s = amax / 127.0f;
    if (tid == 0) {
      sm.row_scale[m] = s;
      if (taps && p.tap_s) p.tap_s[m] = s;
    }
    const float* hr = p.hin + int64_t(m) * p.ldhin + klo;
    int64_t e = int64_t(tid) * 8;
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < kReqHv; ++i, e += int64_t(NT) * 8) {
        if (e < len) {
          const float v[8] = {r.hv[i][0][0], r.hv[i][0][1], r.hv[i][0][2], r.hv[i][0][3],
                              r.hv[i][1][0], r.hv[i][1][1], r.hv[i][1][2], r.hv[i][1][3]};
          *reinterpret_cast<u32x2*>(act + e) = codes8(v, s);
        }
      }
    }
    for (; e < len; e += int64_t(NT) * 8) {
      float v[8];
      load8_f32(hr + e, v);
      *reinterpret_cast<u32x2*>(act + m * act_ld + e) = codes8(v, s);
    }
  }
  lds_barrier();
}

// Codes taps of the requantized Down input cover the whole row; workgroup 0 writes them
// in a separate pass (a debugging path only).
template <int NW>
__device__ void sk_requant_taps(const StreamKArgs& p, const float* row_scale) {
  constexpr int NT = NW * kWave;
  for (int m = 0; m < p.M; ++m)
    for (int64_t k = int64_t(threadIdx.x) * 8; k < p.K; k += NT * 8) {
      float v[8];
      load8_f32(p.hin + int64_t(m) * p.ldhin + k, v);
      *reinterpret_cast<u32x2*>(p.tap_q + int64_t(m) * p.K + k) = codes8(v, row_scale[m]);
    }
}

// EPI: epilogue, NMAT: weights per tile (2 for Gate/Up), NW: waves per workgroup, MB:
// 16-row blocks (1 with a fused prologue), LAYOUT: weight layout, PRO: prologue.
template <int EPI, int NMAT, int NW, int MB, int LAYOUT, int PRO>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(4)))
void streamk_kernel(StreamKArgs p) {
  constexpr bool kFused = PRO != PRO_CODES;
  // QKV and O (BF16 prologue, one weight) issue both batches before the prologue: five
  // steps each cover a wave's ten steps of a 5120-deep tile split over eight waves.
  constexpr bool kEarlyB = PRO == PRO_QUANT_BF16 && NMAT == 1;
  constexpr int kU0 = kFused ? (NMAT == 2 ? 4 : (kEarlyB ? 5 : 6)) : 4 / (NMAT * MB);
  constexpr int U = kU0 > 0 ? kU0 : 1;         // k steps per load batch
  constexpr int kSlot = NMAT * MB * 4 * kWave;  // tagged 64-bit words per slot
  constexpr int kGroup = 4 / (NMAT * MB) > 0 ? 4 / (NMAT * MB) : 1;  // pieces per round trip
  __shared__ SkSmem<NW> sm;
  extern __shared__ __align__(16) int8_t act[];

  const int tid = threadIdx.x;
  // The wave index lives in a scalar register so that every branch around a matrix
  // instruction is wave-uniform (a matrix instruction ignores a partial lane mask).
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int row16 = lane & 15, kg = lane >> 4;
  // Workgroups past wgs1 run the second geometry over tiles toff2.. as its workgroup
  // b = blockIdx.x - wgs1; tile indices below are local to the geometry (t + toff
  // addresses weights, channels and per-tile words).
  const bool second = static_cast<int32_t>(blockIdx.x) >= p.wgs1;
  const StreamKGeom& G = second ? p.g2 : p.g;
  const int32_t b = second ? static_cast<int32_t>(blockIdx.x) - p.wgs1
                           : static_cast<int32_t>(blockIdx.x);
  const int32_t nwg = second ? static_cast<int32_t>(gridDim.x) - p.wgs1 : p.wgs1;
  const int32_t toff = second ? p.toff2 : 0;
  const int32_t T = G.tiles, St = G.steps_tile, Ss = G.steps_seg, C = G.chunks;
  const int32_t wv = b * NW + wave;
  const int32_t w0 = sk_wave_start(G, wv), w1 = sk_wave_start(G, wv + 1);
  const bool has = w1 > w0;
  // A wave without steps (only when there are fewer steps than waves) addresses step 0
  // and never has a live step, so every wave issues the same unconditional loads.
  const int32_t f0 = has ? w0 : 0, f1 = has ? w1 : 1;
  const int32_t flive = has ? w1 : 0;
  const int64_t m0 = int64_t(blockIdx.y) * MB * 16;

  // Activation operand rows; lanes of missing rows read row 0 and feed zeros.
  bool aval[MB];
  int64_t aoff[MB];
  int64_t klo = 0, act_ld = 0, alen = 0;
  if constexpr (kFused) {
    int32_t c0, c1;
    sk_wg_chunks(G, b, NW, c0, c1);
    klo = int64_t(c0) * Ss * 64;
    alen = int64_t(c1 - c0 + 1) * Ss * 64;
    act_ld = p.act_row;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + mb * 16 + row16;
    aval[mb] = m < p.M;
    aoff[mb] = kFused ? (aval[mb] ? row16 : 0) * act_ld - klo + kg * 16
                      : (aval[mb] ? m : 0) * p.lda + kg * 16;
  }

  // Segments sA..sB of this workgroup; after the streaming, wave w runs the epilogue of
  // sA + w (and of every NW-th one after it).  Its channel scales and residual are
  // fetched now, ahead of the weights, so the epilogue waits for no load.
  const int32_t wfirst = b * NW;
  const int32_t wend = (wfirst + NW < G.waves) ? wfirst + NW : G.waves;
  const int32_t A = sk_wave_start(G, wfirst), B = sk_wave_start(G, wend);
  const int32_t sA = static_cast<int32_t>(G.by_seg.div(static_cast<uint32_t>(A)));
  const int32_t sB = B > A ? static_cast<int32_t>(G.by_seg.div(static_cast<uint32_t>(B - 1))) : sA;
  const int32_t sg0 = sA + wave;
  f32x4 sw0p, sw1p;
  u32x2 resp[MB];
  auto fetch_epilogue_inputs = [&](int32_t sg) {
    const int32_t t = sg - static_cast<int32_t>(G.by_tiles.div(static_cast<uint32_t>(sg))) * T;
    const int64_t en = int64_t(t + toff) * 16 + 4 * kg;
    sw0p = *reinterpret_cast<const f32x4*>(p.sw0 + en);
    sw1p = (NMAT == 2) ? *reinterpret_cast<const f32x4*>(p.sw1 + en) : sw0p;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t em = m0 + mb * 16 + row16;
      resp[mb] = u32x2{0u, 0u};
      if constexpr (EPI == EPI_BF16_RES || EPI == EPI_DOWN)
        resp[mb] = *reinterpret_cast<const u32x2*>(p.res + (aval[mb] ? em : 0) * p.ldr + en);
    }
  };

  // The range [f0, f1) covers at most two segments (the planner deals at least one
  // wave per segment): steps f < fx belong to segment segA, the others to segA + 1.
  // Within a segment, steps are consecutive 1 KB blocks (tiled layout) or consecutive
  // 64-byte groups of 16 rows (row-major), so each operand address is a linear
  // function of f on either side of fx: a scalar select, no per-step branches.
  const int32_t segA = static_cast<int32_t>(G.by_seg.div(static_cast<uint32_t>(f0)));
  const int32_t segN = segA + 1;
  const int32_t fx = (segN * Ss < f1) ? segN * Ss : f1;
  const int32_t cA = static_cast<int32_t>(G.by_tiles.div(static_cast<uint32_t>(segA)));
  const int32_t tA = segA - cA * T;
  const int32_t cB = static_cast<int32_t>(G.by_tiles.div(static_cast<uint32_t>(segN)));
  const int32_t tB = segN - cB * T;
  const int64_t kA0 = int64_t(cA) * Ss + (f0 - segA * Ss);   // K step of f0
  const int64_t kB0 = int64_t(cB) * Ss;                      // K step of fx
  constexpr int64_t kStep = (LAYOUT == LAYOUT_TILED) ? 1024 : 64;
  const int64_t lane_off = (LAYOUT == LAYOUT_TILED) ? int64_t(lane) * 16
                                                    : int64_t(row16) * p.K + kg * 16;
  const int64_t wA0 = (LAYOUT == LAYOUT_TILED) ? (int64_t(tA + toff) * St + kA0) * 1024
                                                : int64_t(tA + toff) * 16 * p.K + kA0 * 64;
  const int64_t wB0 = (LAYOUT == LAYOUT_TILED) ? (int64_t(tB + toff) * St + kB0) * 1024
                                                : int64_t(tB + toff) * 16 * p.K + kB0 * 64;
  auto wofs = [&](int32_t f) -> int64_t {
    return (f < fx) ? wA0 + int64_t(f - f0) * kStep : wB0 + int64_t(f - fx) * kStep;
  };
  auto kstep = [&](int32_t f) -> int64_t { return (f < fx) ? kA0 + (f - f0) : kB0 + (f - fx); };
  const int8_t* w0l = p.w0 + lane_off;
  const int8_t* w1l = (NMAT == 2) ? p.w1 + lane_off : nullptr;

  // Load side: batches of U steps; past the end of the range the last step is re-read.
  int32_t lf = f0;
  auto load_batch = [&](i32x4 (&wv_)[U][NMAT], i32x4 (&bv)[U][MB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t f = (lf + u < f1) ? lf + u : f1 - 1;
      const int64_t o = wofs(f);
      wv_[u][0] = ld16_stream(w0l + o);
      if constexpr (NMAT == 2) wv_[u][1] = ld16_stream(w1l + o);
      if constexpr (!kFused) {
        const int64_t ks = kstep(f);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) bv[u][mb] = ld16(p.a + aoff[mb] + ks * 64);
      }
    }
    lf += U;
  };

  // Compute side: one matrix instruction per weight and row block per step; at fx the
  // first segment's sums move to acc0, so no store happens inside the loop.
  i32x4 acc[NMAT][MB], acc0[NMAT][MB];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[i][mb] = i32x4{0, 0, 0, 0};
      acc0[i][mb] = i32x4{0, 0, 0, 0};
    }
  int32_t cf = f0;
  auto compute = [&](const i32x4 (&wv_)[U][NMAT], const i32x4 (&bv)[U][MB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t f = cf + u;
      const bool live = f < flive;
      i32x4 b[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        i32x4 v;
        if constexpr (kFused)
          v = *reinterpret_cast<const i32x4*>(act + aoff[mb] + kstep(live ? f : f1 - 1) * 64);
        else
          v = bv[u][mb];
        b[mb] = (live && aval[mb]) ? v : i32x4{0, 0, 0, 0};
      }
      if (f == fx && live) {
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            acc0[i][mb] = acc[i][mb];
            acc[i][mb] = i32x4{0, 0, 0, 0};
          }
      }
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma_i8(wv_[u][i], b[mb], acc[i][mb]);
    }
    cf += U;
  };

  i32x4 wA[U][NMAT], bA[U][MB], wB[U][NMAT], bB[U][MB];
  const int32_t nb = (flive - f0 + U - 1) / U;
  // Issue order, all unconditional (a guard here would let the compiler assume the
  // loads may arrive out of order, and its waits would then cover later batches):
  //  1. row 0 of the prologue's input: requested before any weight, so the prologue's
  //     waits cover no weight load and the row is not queued behind the weight stream;
  //  2. the first weight batch (both batches for QKV and O, whose whole per-wave range
  //     then is in flight during the prologue);
  //  3. the call's tag and the epilogue inputs (channel scales, residual), which are
  //     used only after the stream;
  //  4. the prologue itself, then the second batch.
  const bool taps = blockIdx.x == 0;
  RequantRegs rq;
  PrologueRegs pre;
  if constexpr (PRO == PRO_REQUANT_F32) sk_requant_fetch<NW>(p, klo, alen, rq);
  if constexpr (PRO == PRO_QUANT_BF16) sk_prologue_fetch<NW, PRO>(p, klo, alen, pre);
  __builtin_amdgcn_sched_barrier(0);
  load_batch(wA, bA);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kEarlyB) {
    load_batch(wB, bB);
    __builtin_amdgcn_sched_barrier(0);
  }
  // This GEMM's tag; the next GEMM on the workspace reads the advanced value (written
  // after the stream by workgroup (0, 0)).
  const uint32_t epoch = *p.epoch_in;
  fetch_epilogue_inputs(sg0 <= sB ? sg0 : sA);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PRO == PRO_REQUANT_F32) {
    sk_requant_prologue<NW>(p, sm, act, act_ld, klo, alen, taps, rq);
    if (taps && p.tap_q) sk_requant_taps<NW>(p, sm.row_scale);
  }
  if constexpr (PRO == PRO_QUANT_BF16) sk_prologue<NW, PRO>(p, sm, act, act_ld, klo, alen, taps, pre);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kEarlyB) load_batch(wB, bB);
  __builtin_amdgcn_sched_barrier(0);
  // Pairs of batches with no branch inside the body (a branch would let the compiler
  // sink the next batch's loads behind the other batch's compute) and scheduling
  // barriers between the phases (so no instruction of one batch's compute is hoisted
  // above the other's).  The last one to three batches are peeled off so that no load
  // past the range is left in flight: the exchange's wait and the epilogue would
  // otherwise wait for it.
  int32_t bi = 0;
  for (; bi + 3 < nb; bi += 2) {
    compute(wA, bA);
    __builtin_amdgcn_sched_barrier(0);
    load_batch(wA, bA);
    __builtin_amdgcn_sched_barrier(0);
    compute(wB, bB);
    __builtin_amdgcn_sched_barrier(0);
    load_batch(wB, bB);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (bi + 2 < nb) {
    compute(wA, bA);
    __builtin_amdgcn_sched_barrier(0);
    load_batch(wA, bA);
    __builtin_amdgcn_sched_barrier(0);
    compute(wB, bB);
    __builtin_amdgcn_sched_barrier(0);
    compute(wA, bA);
  } else if (bi + 1 < nb) {
    compute(wA, bA);
    __builtin_amdgcn_sched_barrier(0);
    compute(wB, bB);
  } else if (bi < nb) {
    compute(wA, bA);
  }

  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *p.epoch_out = epoch + 1;

  // Workgroup combine.  Each wave leaves the partial sums of its (at most two) segments
  // in LDS; after one barrier the workgroup's segments are dealt to its waves, and a
  // wave sums the workgroup's partials of its segment.
  constexpr int kRed = NMAT * MB * 4 * kWave;  // INT32 per (wave, segment) partial
  int32_t* red = reinterpret_cast<int32_t*>(act + p.red_off);
  {
    const int32_t sb_w = has ? static_cast<int32_t>(G.by_seg.div(static_cast<uint32_t>(f1 - 1))) : segA;
    const bool crossed = sb_w > segA;
    if (lane == 0) {
      sm.seg_lo[wave] = has ? segA : -1;
      sm.seg_hi[wave] = crossed ? sb_w : -1;
    }
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int o = ((i * MB + mb) * kWave + lane) * 4;
        *reinterpret_cast<i32x4*>(red + (wave * 2) * kRed + o) = crossed ? acc0[i][mb] : acc[i][mb];
        *reinterpret_cast<i32x4*>(red + (wave * 2 + 1) * kRed + o) =
            crossed ? acc[i][mb] : i32x4{0, 0, 0, 0};
      }
  }
  lds_barrier();

  if (B <= A) return;
  // Slots per 64-row group: one per (chunk, tile) segment and one per workgroup of the
  // first geometry, then the same for the second.
  const int64_t slots1 = int64_t(p.g.tiles) * p.g.chunks + p.wgs1;
  const int64_t slots_group =
      slots1 + (static_cast<int32_t>(gridDim.x) > p.wgs1
                    ? int64_t(p.g2.tiles) * p.g2.chunks + (static_cast<int32_t>(gridDim.x) - p.wgs1)
                    : 0);
  uint64_t* slots = reinterpret_cast<uint64_t*>(p.slots) +
                    (int64_t(blockIdx.y) * slots_group + (second ? slots1 : 0)) * kSlot;
  uint64_t* dones = p.dones + int64_t(blockIdx.y) * (p.N / 16);
  const uint64_t want = (uint64_t(epoch) << 24) | uint64_t(EPI + 1);
  // The GEMM's tag with its epilogue number folded into the top bits (never zero, so a
  // cleared word never matches): every GEMM of every call on this workspace reads a
  // different tag word value, so a word left by another GEMM or call differs.
  const uint32_t tag32 = epoch ^ (uint32_t(EPI + 1) << 29);

  // The pieces of tile t in chunks [ca, cb) are the slots (c*T + t) + g for the
  // workgroups g touching segment c*T + t, a contiguous run per chunk.  `visit` walks
  // them in groups of kGroup: the slot indices first (scalar work), then all the group's
  // loads at once, then their use, so a group costs one memory round trip.
  auto wg_of = [&](int32_t f) { return sk_owner(G, f) / NW; };
  auto visit = [&](int32_t t, int32_t ca, int32_t cb, auto&& load, auto&& use) {
    int32_t n = 0;
    for (int32_t c = ca; c < cb; ++c) {
      const int32_t s0 = (c * T + t) * Ss;
      n += wg_of(s0 + Ss - 1) - wg_of(s0) + 1;
    }
    int32_t ic = ca;
    int32_t ig = wg_of((ca * T + t) * Ss);
    int32_t igb = wg_of((ca * T + t) * Ss + Ss - 1);
    for (int32_t i0 = 0; i0 < n; i0 += kGroup) {
      int32_t idx[kGroup], chk[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        idx[k] = ic * T + t + ig;
        chk[k] = ic;
        if (i0 + k + 1 < n) {
          if (ig < igb) {
            ++ig;
          } else {
            ++ic;
            const int32_t s0 = (ic * T + t) * Ss;
            ig = wg_of(s0);
            igb = wg_of(s0 + Ss - 1);
          }
        }
      }
      decltype(load(0)) v[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) v[k] = load(idx[k]);
#pragma unroll
      for (int k = 0; k < kGroup; ++k)
        if (i0 + k < n) use(v[k], chk[k]);
    }
  };

  for (int32_t sg = sA + wave; sg <= sB; sg += NW) {
    const int32_t t = sg - static_cast<int32_t>(G.by_tiles.div(static_cast<uint32_t>(sg))) * T;
    i32x4 part[NMAT][MB];
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) part[i][mb] = i32x4{0, 0, 0, 0};
    // Every wave's partial of segment sg (its first or second slot), read in one pass
    // with no branch, so the LDS reads are issued together and waited for once.
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int32_t lo = sm.seg_lo[j], hi = sm.seg_hi[j];
      const bool second_slot = hi == sg;
      const bool use = second_slot || lo == sg;
      const int32_t* rj = red + (j * 2 + (second_slot ? 1 : 0)) * kRed;
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(rj + ((i * MB + mb) * kWave + lane) * 4);
          part[i][mb] += use ? v : i32x4{0, 0, 0, 0};
        }
    }
    // Epilogue inputs: prefetched for the first segment; later ones (a workgroup with
    // more segments than waves) fetch theirs here, before the exchange.  Lane l owns
    // channels en..en+3 of row em.
    if (sg != sg0) fetch_epilogue_inputs(sg);
    const int64_t en = int64_t(t + toff) * 16 + 4 * kg;
    const f32x4 sw0v = sw0p, sw1v = sw1p;
    u32x2 resv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) resv[mb] = resp[mb];

    // A tile of one chunk held by this workgroup alone needs no exchange.
    // (Its steps [t * Ss, t * Ss + Ss) lie in the workgroup's range [A, B).)
    const bool interior = C == 1 && t * Ss >= A && t * Ss + Ss <= B;
    if (!interior) {
      // Publish the piece as tagged words and wait until they are visible.  Every
      // owner then reads all pieces of the tile: the owner whose words became visible
      // last finds every tag, so at least one wave runs the epilogue.
      uint64_t* sp = slots + int64_t(sg + b) * kSlot;
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (aval[mb]) store_tagged(sp + ((i * MB + mb) * kWave + lane) * 4, part[i][mb], tag32);
      wait_memory_done();
    }

    // Sums of the pieces of chunks [ca, cb) of tile t, per weight and row block, into s
    // for chunks below csplit and into s2 for the others (one round trip per group of
    // pieces for both); false (for the whole wave) when a piece is not yet visible.
    auto gather2 = [&](i32x4 (&s)[NMAT][MB], i32x4 (&s2)[NMAT][MB], int32_t ca, int32_t cb,
                       int32_t csplit) -> bool {
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          s[i][mb] = interior ? part[i][mb] : i32x4{0, 0, 0, 0};
          s2[i][mb] = i32x4{0, 0, 0, 0};
        }
      if (interior) return true;
      struct Piece {
        TaggedX4 v[NMAT][MB];
      };
      bool ok = true;
      visit(t, ca, cb,
            [&](int32_t i) {
              Piece pc;
              const uint64_t* q = slots + int64_t(i) * kSlot;
#pragma unroll
              for (int j = 0; j < NMAT; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                  pc.v[j][mb] = aval[mb] ? load_tagged(q + ((j * MB + mb) * kWave + lane) * 4)
                                         : TaggedX4{{uint64_t(tag32) << 32, uint64_t(tag32) << 32,
                                                     uint64_t(tag32) << 32, uint64_t(tag32) << 32}};
              return pc;
            },
            [&](const Piece& pc, int32_t c) {
              const bool lo = c < csplit;
#pragma unroll
              for (int j = 0; j < NMAT; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                  i32x4 v = {0, 0, 0, 0};
                  add_tagged(v, pc.v[j][mb], tag32, ok);
                  if (lo) s[j][mb] += v; else s2[j][mb] += v;
                }
            });
      return __builtin_amdgcn_ballot_w64(!ok) == 0;
    };
    auto gather = [&](i32x4 (&s)[NMAT][MB], int32_t ca, int32_t cb) -> bool {
      i32x4 unused[NMAT][MB];
      return gather2(s, unused, ca, cb, cb);
    };
    // When the output overwrites the residual it reads, exactly one of the waves that
    // found every piece (the first to swap the tile's done word to this call's tag)
    // runs the epilogue.  Otherwise a repeated epilogue writes the same values.
    auto claim = [&]() -> bool {
      if (interior || !p.once) return true;
      uint64_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_exchange(dones + toff + t, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t plo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(prev));
      const uint32_t phi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(prev >> 32));
      return ((uint64_t(phi) << 32) | plo) != want;
    };
    float sa[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t em = m0 + mb * 16 + row16;
      sa[mb] = aval[mb] ? (kFused ? sm.row_scale[em] : p.sa[em]) : 0.0f;
    }

    if constexpr (EPI == EPI_BF16 || EPI == EPI_BF16_RES) {
      i32x4 s[NMAT][MB];
      if (!gather(s, 0, C) || !claim()) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (!aval[mb]) continue;
        const int64_t em = m0 + mb * 16 + row16;
        if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = s[0][mb];
        float y[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) y[c] = dq(s[0][mb][c], sa[mb], sw0v[c]);
        if constexpr (EPI == EPI_BF16_RES) {
          const u32x2 rr = resv[mb];
          y[0] = y[0] + bf16_lo(rr[0]);
          y[1] = y[1] + bf16_hi(rr[0]);
          y[2] = y[2] + bf16_lo(rr[1]);
          y[3] = y[3] + bf16_hi(rr[1]);
        }
        u32x2 o;
        o[0] = uint32_t(f32_to_bf16_rne(y[0])) | (uint32_t(f32_to_bf16_rne(y[1])) << 16);
        o[1] = uint32_t(f32_to_bf16_rne(y[2])) | (uint32_t(f32_to_bf16_rne(y[3])) << 16);
        *reinterpret_cast<u32x2*>(p.out + em * p.ldo + en) = o;
      }
    } else if constexpr (EPI == EPI_SILU) {
      i32x4 s[NMAT][MB];
      if (!gather(s, 0, C) || !claim()) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int64_t em = m0 + mb * 16 + row16;
        f32x4 h = {0.f, 0.f, 0.f, 0.f};
        if (aval[mb]) {
          if (p.tap_acc0) *reinterpret_cast<i32x4*>(p.tap_acc0 + em * p.N + en) = s[0][mb];
          if (p.tap_acc1) *reinterpret_cast<i32x4*>(p.tap_acc1 + em * p.N + en) = s[NMAT - 1][mb];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float g = dq(s[0][mb][c], sa[mb], sw0v[c]);
            const float u = dq(s[NMAT - 1][mb][c], sa[mb], sw1v[c]);
            h[c] = silu_mul(g, u);
          }
          *reinterpret_cast<f32x4*>(p.h + em * p.ldh + en) = h;
          if (p.tap_h) *reinterpret_cast<f32x4*>(p.tap_h + em * p.N + en) = h;
        }
        // Absolute maximum of the tile's 16 channels of row em (the four lanes sharing
        // l % 16 hold them), for the requantization scale of the next GEMM.
        float mx = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (p.pmax_out && aval[mb] && kg == 0) p.pmax_out[(t + toff) * p.M + em] = mx;
      }
    } else {  // EPI_DOWN: partitions summed in order, then the residual
      const int64_t MN = p.M * p.N;
      const int32_t cpp = C / p.parts;  // chunks per partition
      float tot[MB][4];
      bool have = true;
      // Two partitions (the usual split) are gathered together in one pass.
      i32x4 s01[2][NMAT][MB];
      if (p.parts == 2) have = gather2(s01[0], s01[1], 0, C, cpp);
      for (int32_t part = 0; part < p.parts && have; ++part) {
        i32x4 s[NMAT][MB];
        if (p.parts == 2) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) s[0][mb] = part == 0 ? s01[0][0][mb] : s01[1][0][mb];
        } else {
          have = gather(s, part * cpp, (part + 1) * cpp);
          if (!have) break;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (!aval[mb]) continue;
          const int64_t em = m0 + mb * 16 + row16;
          if (p.tap_acc0)
            *reinterpret_cast<i32x4*>(p.tap_acc0 + part * MN + em * p.N + en) = s[0][mb];
          f32x4 pv;
#pragma unroll
          for (int c = 0; c < 4; ++c) pv[c] = dq(s[0][mb][c], sa[mb], sw0v[c]);
          if (p.tap_p) *reinterpret_cast<f32x4*>(p.tap_p + part * MN + em * p.N + en) = pv;
#pragma unroll
          for (int c = 0; c < 4; ++c) tot[mb][c] = (part == 0) ? pv[c] : tot[mb][c] + pv[c];
        }
      }
      if (!have || !claim()) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (!aval[mb]) continue;
        const int64_t em = m0 + mb * 16 + row16;
        const u32x2 rr = resv[mb];
        const float o0 = tot[mb][0] + bf16_lo(rr[0]);
        const float o1 = tot[mb][1] + bf16_hi(rr[0]);
        const float o2 = tot[mb][2] + bf16_lo(rr[1]);
        const float o3 = tot[mb][3] + bf16_hi(rr[1]);
        u32x2 o;
        o[0] = uint32_t(f32_to_bf16_rne(o0)) | (uint32_t(f32_to_bf16_rne(o1)) << 16);
        o[1] = uint32_t(f32_to_bf16_rne(o2)) | (uint32_t(f32_to_bf16_rne(o3)) << 16);
        *reinterpret_cast<u32x2*>(p.out + em * p.ldo + en) = o;
      }
    }
  }
}

template <int EPI, int NMAT, int MB, int LAYOUT, int PRO>
hipError_t launch_one(const StreamKArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const auto kern = streamk_kernel<EPI, NMAT, kSkWaves, MB, LAYOUT, PRO>;
  if (lds > 64 * 1024) {
    // Above the default dynamic LDS limit (only the wide row blocks need it).
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kSkWaves * kWave), lds, s, a);
  return hipGetLastError();
}

template <int EPI, int NMAT, int MB, int PRO>
hipError_t launch_layout(const StreamKArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  if (a.layout == LAYOUT_TILED) return launch_one<EPI, NMAT, MB, LAYOUT_TILED, PRO>(a, grid, lds, s);
  return launch_one<EPI, NMAT, MB, LAYOUT_ROWMAJOR, PRO>(a, grid, lds, s);
}

template <int EPI, int NMAT, int PROF>
hipError_t launch_epi(const StreamKArgs& a, const StreamKPlan& pl, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(pl.wgs), static_cast<unsigned>(pl.mgroups));
  if (a.prologue != PRO_CODES) return launch_layout<EPI, NMAT, 1, PROF>(a, grid, pl.lds, s);
  switch (pl.mb) {
    case 1: return launch_layout<EPI, NMAT, 1, PRO_CODES>(a, grid, pl.lds, s);
    case 2: return launch_layout<EPI, NMAT, 2, PRO_CODES>(a, grid, pl.lds, s);
    default: return launch_layout<EPI, NMAT, 4, PRO_CODES>(a, grid, pl.lds, s);
  }
}

}  // namespace

// Geometry of T tiles of St steps in C chunks dealt to W waves.
static void set_geom(StreamKGeom& g, int64_t T, int64_t St, int64_t C, int64_t W) {
  const int64_t Tot = T * St;
  g.tiles = static_cast<int32_t>(T);
  g.steps_tile = static_cast<int32_t>(St);
  g.steps_seg = static_cast<int32_t>(St / C);
  g.chunks = static_cast<int32_t>(C);
  g.total = static_cast<int32_t>(Tot);
  g.waves = static_cast<int32_t>(W);
  g.q = static_cast<int32_t>(Tot / W);
  g.r = static_cast<int32_t>(Tot % W);
  g.by_seg = FastDiv(static_cast<uint32_t>(St / C));
  g.by_tiles = FastDiv(static_cast<uint32_t>(T));
  g.by_q = FastDiv(static_cast<uint32_t>(g.q > 0 ? g.q : 1));
  g.by_q1 = FastDiv(static_cast<uint32_t>(g.q + 1));
}

StreamKPlan plan_streamk(int epi, int64_t M, int64_t N, int64_t K, int parts, bool fused) {
  StreamKPlan pl{};
  pl.waves = kSkWaves;
  const int P = (epi == EPI_DOWN) ? parts : 1;
  const int64_t T = N / 16, St = K / 64;
  // One chunk per K partition, so a tile inside one workgroup needs no exchange; more
  // for a fused requantized Down input while the codes of two chunks (a workgroup's
  // steps span at most two) would not fit LDS beside the combine area.
  int64_t cpp = 1;
  const int nmat = (epi == EPI_SILU) ? 2 : 1;
  if (epi == EPI_DOWN && fused) {
    const int64_t red = int64_t(kSkWaves) * 2 * nmat * 4 * kWave * 4;
    while ((St / P) % (2 * cpp) == 0 && M * 2 * (St / (P * cpp)) * 64 + red > int64_t(kSkMaxLds))
      cpp *= 2;
  }
  const int64_t C = P * cpp, Ss = St / C, Tot = T * St;
  // Smaller GEMMs stream a little faster with fewer, longer ranges (measured on the
  // 5120 x 5120 and 7168 x 5120 projections); the large ones with two per CU.
  int64_t wgs = Tot / (int64_t(kSkWaves) * kSkMinSteps);
  const int64_t target = Tot < kSkSmallSteps ? kSkSmallWgs : kSkTargetWgs;
  if (wgs > target) wgs = target;
  // At least one wave per segment: a wave's range (at most ceil(Tot / W) <= Ss + 1
  // steps) then spans at most two segments, which the kernel relies on.
  const int64_t per_seg = (T * C + kSkWaves - 1) / kSkWaves;
  if (wgs < per_seg) wgs = per_seg;
  if (wgs < 1) wgs = 1;
  // One tile per workgroup when the tiles fill the grid and split evenly over its
  // waves: every tile is then summed within its workgroup (LDS), with no exchange
  // between workgroups in the tail.
  if (C == 1 && T >= kSkTileWgsMin && T <= kSkTargetWgs && St % kSkWaves == 0) wgs = T;
  pl.wgs = static_cast<int>(wgs);
  pl.wgs1 = pl.wgs;
  pl.toff2 = 0;
  set_geom(pl.geom, T, St, C, wgs * kSkWaves);
  pl.geom2 = pl.geom;
  // Two per CU, the second workgroup on a CU (blockIdx >= wgs / 2) is dispatched last
  // and streams last.  When the tiles allow, those workgroups take k whole tiles each
  // (summed in LDS, no exchange) and the first half runs the stream-K split of the other
  // tiles, so the exchanges finish while the second half still streams and the kernel's
  // tail holds no exchange.
  if (C == 1 && wgs == kSkTargetWgs) {
    const int64_t half = wgs / 2, k = T / wgs;
    const int64_t T2 = half * k, T1 = T - T2;
    if (k >= 1 && (k * St) % kSkWaves == 0 && T1 >= 1 && T1 * C <= half * kSkWaves) {
      pl.wgs1 = static_cast<int>(half);
      pl.toff2 = static_cast<int>(T1);
      set_geom(pl.geom, T1, St, C, half * kSkWaves);
      set_geom(pl.geom2, T2, St, C, half * kSkWaves);
    }
  }
  if (fused) {
    pl.mgroups = 1;
    pl.mb = 1;
    int64_t row = 0;
    for (int32_t b = 0; b < pl.wgs; ++b) {
      const bool two = b >= pl.wgs1;
      const StreamKGeom& gb = two ? pl.geom2 : pl.geom;
      int32_t c0, c1;
      sk_wg_chunks(gb, two ? b - pl.wgs1 : b, kSkWaves, c0, c1);
      const int64_t bytes = int64_t(c1 - c0 + 1) * gb.steps_seg * 64;
      if (bytes > row) row = bytes;
    }
    pl.act_row = row;
    pl.red_off = (size_t(M) * size_t(row) + 15) / 16 * 16;
  } else {
    pl.mgroups = static_cast<int>((M + 63) / 64);
    const int64_t rows = M < 64 ? M : 64;
    const int64_t b16 = (rows + 15) / 16;
    pl.mb = b16 <= 1 ? 1 : (b16 <= 2 ? 2 : 4);
    pl.act_row = 0;
    pl.red_off = 0;
  }
  pl.lds = pl.red_off + size_t(kSkWaves) * 2 * nmat * pl.mb * 4 * kWave * sizeof(int32_t);
  // Tagged slots: one 64-bit word (two INT32 elements) per partial sum.
  pl.slot_elems = 2 * size_t(pl.mgroups) * size_t(T * C + wgs) * size_t(nmat) * pl.mb * 4 * kWave;
  pl.done_elems = size_t(pl.mgroups) * size_t(T);
  // Shapes the one-workgroup-per-CU kernel covers run on it: with the fused prologue, or
  // with the codes given by the row-quantization kernels.
  if (plan_decode(epi, M, N, K, P, !fused, pl.dec)) {
    pl.use_decode = 1;
    const size_t se = decode_slot_elems(pl.dec, nmat);
    if (se > pl.slot_elems) pl.slot_elems = se;
  }
  return pl;
}

bool streamk_fusable(const StreamKPlan& pl, int64_t M, int64_t K_in, bool bf16_rows) {
  if (M > kFuseMaxRows) return false;
  if (pl.use_decode) return true;
  if (pl.lds > kSkMaxLds) return false;
  // The BF16 prologue holds its rows in registers; the requantization one does not.
  return !bf16_rows || K_in <= kPrologueMax;
}

hipError_t launch_streamk(const StreamKArgs& a_in, const StreamKPlan& pl, hipStream_t stream) {
  if (a_in.M == 0) return hipSuccess;
  if (pl.use_decode) return launch_decode(a_in, pl.dec, stream);
  StreamKArgs a = a_in;
  a.red_off = static_cast<int64_t>(pl.red_off);
  switch (a.epi) {
    case EPI_BF16: return launch_epi<EPI_BF16, 1, PRO_QUANT_BF16>(a, pl, stream);
    case EPI_BF16_RES: return launch_epi<EPI_BF16_RES, 1, PRO_QUANT_BF16>(a, pl, stream);
    case EPI_SILU: return launch_epi<EPI_SILU, 2, PRO_QUANT_BF16>(a, pl, stream);
    case EPI_DOWN: return launch_epi<EPI_DOWN, 1, PRO_REQUANT_F32>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace a8w8
