// Prefill-shaped W8A16 GEMMs on gfx950 BF16 matrix cores, on the shared INT8 weights.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path: prefill keeps the INT8 checkpoint weights
// and turns every INT8 weight tile into BF16 values ahead of the matrix-core product.  Every weight
// element becomes W' = rne_bf16(fl32(w * s[n])), the activations are BF16, products
// accumulate in FP32 (v_mfma_f32_32x32x16_bf16).
//
// Work shape: tiles of 256 rows of M by 128 weight channels.
//   * Gate/Up tiles hold 64 Gate channels and the same 64 Up channels, so silu(g) * u is
//     formed from one workgroup's accumulators; Down tiles hold 128 channels of one
//     weight.  A unit of work is a 64-k step of a tile; steps are scheduled in quads.
//   * Schedule: with T tiles and G workgroups, each workgroup first runs T / G whole
//     tiles (tiles w, w + G, ...), then the leftover tiles' quads are dealt evenly, in
//     (tile, k) order, over all workgroups.  A workgroup runs its whole list as one
//     software pipeline.  A tile run whole by one workgroup is finished in the kernel;
//     the pieces of a split tile leave FP32 partial sums in workspace slots, and a
//     second kernel adds them in K order and applies the epilogue, so results do not
//     depend on timing.
//   * Weights: per step each of the 256 threads loads two 16-byte chunks of the tiled
//     INT8 tile, dequantizes them and stores the BF16 operands to an LDS double buffer
//     in the order of the matrix-core operand; every wave then reads the operands of
//     all 128 channels.  A weight element is fetched and dequantized once per
//     workgroup.  int8 -> FP32 uses the biased byte u = w + 128 (exact) and one fused
//     multiply-add u * s + (-128 * s), whose exact value is w * s, so its single rounding
//     gives fl32(w * s); FP32 -> BF16 is the RNE conversion.
//   * Activations: wave w owns rows 64w..64w+63 of the tile (two 32-row blocks) and
//     loads its BF16 operands from global memory straight into registers, three steps
//     ahead.  They are stored in the prefill operand layout (prefill_operand_index), so
//     each load instruction reads one contiguous 1 KB.
//   * Matrix-core operands (32x32x16): weights are A (lane l: channel l%32 of a 32-channel
//     block, k = 8*(l/32)..+7 of a 16-k substep), activations B (lane l: row l%32, the
//     same k); lane l of the result holds row l%32 and channels 8*(r/4) + 4*(l/32) + r%4
//     of register r.
//   * A step is 16 blocks of (substep, channel block), each one LDS operand (read 4
//     blocks ahead) and two MFMAs; an eighth of the next step's dequantization and the
//     step's loads for later steps are spread between them, so the vector ALU and the
//     address unit work while the matrix core runs.  Load addresses are wave-uniform
//     bases computed once per quad plus constant lane offsets.
//   * EPI_PF_SILU: h = rne_bf16(silu(g) * u) in the prefill operand layout for the Down
//     GEMM (+ FP32 taps of g and u, a row-major tap of h).
//     EPI_PF_RES: out = rne_bf16(d + res) row-major (+ FP32 tap of d); without a residual
//                 (res == nullptr) out = rne_bf16(d).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 4;
constexpr int kPfRb = 2;                          // 32-row blocks per wave
constexpr int kPfCb = 4;                          // 32-channel blocks per tile
constexpr int kPfSub = 4;                         // 16-k substeps per 64-k step
constexpr int kPfTileRows = kPfWaves * kPfRb * 32;
constexpr int kPfBufBytes = kPfCb * kPfSub * kWave * 16;  // dequantized step: 16 KB
constexpr int kPfGroups = kPfRb * kPfCb * 4;      // f32x4 accumulator groups per lane
constexpr int kPfSlotWave = kPfGroups * kWave * 4;  // floats per wave of one piece
constexpr int kLdsAhead = 4;                      // LDS operand reads in flight (blocks)

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ f32x4 group4(const f32x16& v, int g) {
  return f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

// Output of one accumulator group: row m, channels n0..n0+3 (g: the Gate or Down sums,
// u: the Up sums).
template <int EPI>
__device__ __forceinline__ void epilogue_group(const PrefillGemmArgs& p, int64_t m, int64_t n0,
                                               f32x4 g, f32x4 u) {
  if constexpr (EPI == EPI_PF_SILU) {
    if (p.tap_g) *reinterpret_cast<f32x4*>(p.tap_g + m * p.N + n0) = g;
    if (p.tap_u) *reinterpret_cast<f32x4*>(p.tap_u + m * p.N + n0) = u;
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(silu_mul(g[0], u[0]))) |
           (uint32_t(f32_to_bf16_rne(silu_mul(g[1], u[1]))) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(silu_mul(g[2], u[2]))) |
           (uint32_t(f32_to_bf16_rne(silu_mul(g[3], u[3]))) << 16);
    *reinterpret_cast<u32x2*>(p.out + prefill_operand_index(m, n0, p.N)) = o;
    if (p.tap_h) *reinterpret_cast<u32x2*>(p.tap_h + m * p.N + n0) = o;
  } else {
    if (p.tap_d) *reinterpret_cast<f32x4*>(p.tap_d + m * p.N + n0) = g;
    // Without a residual the accumulator is narrowed as it is (no add of +0, which
    // would turn a -0 result into +0).
    f32x4 y = g;
    if (p.res) {
      const u32x2 rr = *reinterpret_cast<const u32x2*>(p.res + m * p.ldr + n0);
      y[0] = g[0] + bf16_lo(rr[0]);
      y[1] = g[1] + bf16_hi(rr[0]);
      y[2] = g[2] + bf16_lo(rr[1]);
      y[3] = g[3] + bf16_hi(rr[1]);
    }
    u32x2 o;
    o[0] = uint32_t(f32_to_bf16_rne(y[0])) | (uint32_t(f32_to_bf16_rne(y[1])) << 16);
    o[1] = uint32_t(f32_to_bf16_rne(y[2])) | (uint32_t(f32_to_bf16_rne(y[3])) << 16);
    *reinterpret_cast<u32x2*>(p.out + m * p.ldo + n0) = o;
  }
}

// Leftover-tile bookkeeping shared by the GEMM and the reduction kernel.  Leftover
// quad x (of tiles_dp + x / quads) belongs to workgroup sk_owner(x); workgroup w owns
// leftover quads [sk_start(w), sk_start(w + 1)).
struct Sched {
  const PrefillGemmArgs& p;
  __device__ int32_t sk_start(int32_t w) const { return w * p.q + min(w, p.r); }
  __device__ int32_t sk_owner(int32_t x) const {
    const int32_t cut = p.r * (p.q + 1);
    return x < cut ? x / (p.q + 1) : p.r + (x - cut) / p.q;
  }
  // Slot of workgroup w's piece of leftover tile t: its first or its last leftover tile.
  __device__ int32_t slot(int32_t w, int32_t t) const {
    return 2 * w + (t != p.tiles_dp + sk_start(w) / p.quads ? 1 : 0);
  }
};

struct AStage {
  u32x4 a[kPfRb][kPfSub];
};
struct WStage {
  u32x4 w[2];
  float s[2];
};

template <int EPI, int NMAT, int LAYOUT>
__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_gemm_kernel(PrefillGemmArgs p) {
  constexpr int kBlkPerMat = 8 / NMAT;  // 16-channel weight blocks of one matrix per tile
  __shared__ __align__(16) uint8_t wsm[2][kPfBufBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int32_t wg = static_cast<int32_t>(blockIdx.x);
  const Sched sc{p};
  const int32_t SQ = p.quads;                 // quads per tile
  const int32_t ndpq = p.dp_per_wg * SQ;      // whole-tile quads of this workgroup
  const int32_t qa = sc.sk_start(wg), qb = sc.sk_start(wg + 1);
  const int32_t nq = ndpq + (qb - qa);
  if (nq <= 0) return;
  const int64_t K = p.K;
  const int64_t k_steps = K / 64;
  const int32_t row_blocks = static_cast<int32_t>((p.M + 31) / 32);

  // Tile and first step of this workgroup's quad v (v < nq).
  auto quad_at = [&](int32_t v, int32_t& t, int32_t& ks0) {
    if (v < ndpq) {
      const int32_t i = static_cast<int32_t>(p.by_quads.div(static_cast<uint32_t>(v)));
      t = wg + p.grid * i;
      ks0 = (v - i * SQ) * 4;
    } else {
      const int32_t x = qa + (v - ndpq);
      const int32_t i = static_cast<int32_t>(p.by_quads.div(static_cast<uint32_t>(x)));
      t = p.tiles_dp + i;
      ks0 = (x - i * SQ) * 4;
    }
  };
  // Wave-uniform bases of a quad's operands (step 0 of the quad).
  struct QuadBase {
    const uint8_t* act[kPfRb];
    const int8_t* w[2];
    const float* s[2];
  };
  auto quad_base = [&](int32_t t, int32_t ks0, QuadBase& b) {
    const int32_t nt = static_cast<int32_t>(p.by_mtiles.div(static_cast<uint32_t>(t)));
    const int32_t mt = t - nt * p.mtiles;
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      // rows past M re-read the last row block (their results are never stored)
      const int32_t R = min(mt * (kPfTileRows / 32) + wave * kPfRb + rb, row_blocks - 1);
      b.act[rb] = reinterpret_cast<const uint8_t*>(p.act) + (int64_t(R) * k_steps + ks0) * 4096;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int b16 = 4 * c + wave;
      const int mat = b16 / kBlkPerMat;
      const int64_t t16 = int64_t(nt) * kBlkPerMat + (b16 % kBlkPerMat);
      const int8_t* wb = (NMAT == 2 && mat == 1) ? p.w1 : p.w0;
      b.w[c] = wb + t16 * 16 * K + int64_t(ks0) * ((LAYOUT == LAYOUT_TILED) ? 1024 : 64);
      b.s[c] = ((NMAT == 2 && mat == 1) ? p.sw1 : p.sw0) + t16 * 16;
    }
  };
  const uint32_t a_lane = static_cast<uint32_t>(lane) * 16u;
  const uint32_t w_lane = (LAYOUT == LAYOUT_TILED)
                              ? static_cast<uint32_t>(lane) * 16u
                              : static_cast<uint32_t>((lane & 15) * K + (lane >> 4) * 16);
  constexpr int64_t kWStep = (LAYOUT == LAYOUT_TILED) ? 1024 : 64;
  auto load_act_one = [&](AStage& st, int rb, int s, const QuadBase& b, int j) {
    st.a[rb][s] = *reinterpret_cast<const u32x4*>(b.act[rb] + j * 4096 + s * 1024 + a_lane);
  };
  auto load_w_chunk = [&](WStage& st, int c, const QuadBase& b, int j) {
    // Weight bytes are read once; the activation operand is re-read by every workgroup
    // and must stay cached, so the weights are loaded non-temporally.
    st.w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b.w[c] + j * kWStep + w_lane));
    st.s[c] = b.s[c][lane & 15];
  };

  f32x16 acc[kPfRb][kPfCb];
#pragma unroll
  for (int rb = 0; rb < kPfRb; ++rb)
#pragma unroll
    for (int cb = 0; cb < kPfCb; ++cb) acc[rb][cb] = f32x16{};

  // ---- tile completion
  auto finish = [&](int32_t t) {
    const int32_t nt = static_cast<int32_t>(p.by_mtiles.div(static_cast<uint32_t>(t)));
    const int32_t mt = t - nt * p.mtiles;
    bool whole = t < p.tiles_dp;
    if (!whole) {
      const int32_t u = t - p.tiles_dp;
      whole = sc.sk_owner(u * SQ) == sc.sk_owner(u * SQ + SQ - 1);
    }
    if (!whole) {
      // a piece of a split tile: its partial sums go to this workgroup's slot
      float* dst = p.slots + (int64_t(sc.slot(wg, t)) * kPfWaves + wave) * kPfSlotWave;
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
#pragma unroll
        for (int cb = 0; cb < kPfCb; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int q = (rb * kPfCb + cb) * 4 + g;
            *reinterpret_cast<f32x4*>(dst + (q * kWave + lane) * 4) = group4(acc[rb][cb], g);
          }
      return;
    }
    constexpr int kOut = (EPI == EPI_PF_SILU) ? kPfCb / 2 : kPfCb;
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const int64_t m = int64_t(mt) * kPfTileRows + wave * 64 + rb * 32 + (lane & 31);
      if (m >= p.M) continue;
#pragma unroll
      for (int cb = 0; cb < kOut; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n0 = int64_t(nt) * (kOut * 32) + cb * 32 + g * 8 + (lane >> 5) * 4;
          const f32x4 x = group4(acc[rb][cb], g);
          const f32x4 y = (EPI == EPI_PF_SILU) ? group4(acc[rb][(cb + 2) % kPfCb], g) : x;
          epilogue_group<EPI>(p, m, n0, x, y);
        }
    }
  };

  // ---- the pipeline.  Invariant at the start of step g (stage j = g % 4): A[j] holds
  // (or is loading) the activations of step g, A[j+1], A[j+2] those of g+1, g+2;
  // R[j+1..j+3] the raw weights of steps g+1..g+3; LDS buffer g%2 the dequantized
  // weights of step g.  Loads past the last step re-read the last quad (never used).
  AStage A[4];
  WStage R[4];
  QuadBase cur, nxt;
  int32_t t_cur, ks_cur, t_nxt, ks_nxt;
  quad_at(0, t_cur, ks_cur);
  quad_base(t_cur, ks_cur, cur);
  // The prologue issues its loads in the steady state's order (the scheduling barriers
  // keep them there): the loop head's waits are derived from every path into it.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < 3) {
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
#pragma unroll
        for (int s = 0; s < kPfSub; ++s) load_act_one(A[j], rb, s, cur, j);
    }
    load_w_chunk(R[j], 0, cur, j);
    load_w_chunk(R[j], 1, cur, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Dequantization of dword d of chunk c of a weight stage into the operand halves.
  auto dq_piece = [&](const WStage& st, int c, int d, u32x4& lo, u32x4& hi) {
    const float s = st.s[c];
    const float bias = -128.0f * s;
    const uint32_t u = st.w[c][d] ^ 0x80808080u;  // biased bytes w + 128
    float f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      f[b] = __builtin_fmaf(static_cast<float>((u >> (8 * b)) & 0xFFu), s, bias);
    u32x4& dst = (d < 2) ? lo : hi;
    dst[(d & 1) * 2] = pack_bf16x2(f[0], f[1]);
    dst[(d & 1) * 2 + 1] = pack_bf16x2(f[2], f[3]);
  };
  // LDS position of chunk c's operand halves: operand (32-channel block, substep), lane
  // = channel within the block for the first 8 k, + 32 for the second 8 k.
  const int ch32 = (wave & 1) * 16 + (lane & 15);
  auto dq_store = [&](uint8_t* buf, int c, const u32x4& lo, const u32x4& hi) {
    const int b16 = 4 * c + wave;
    const int op = (b16 >> 1) * kPfSub + (lane >> 4);
    *reinterpret_cast<u32x4*>(buf + (op * kWave + ch32) * 16) = lo;
    *reinterpret_cast<u32x4*>(buf + (op * kWave + ch32 + 32) * 16) = hi;
  };
  {
    u32x4 lo, hi;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int d = 0; d < 4; ++d) dq_piece(R[0], c, d, lo, hi);
      dq_store(wsm[0], c, lo, hi);
    }
  }
  lds_barrier();

  auto step = [&](auto J) {
    constexpr int j = decltype(J)::value;
    const uint8_t* rbuf = wsm[j & 1];
    uint8_t* wbuf = wsm[(j + 1) & 1];
    const WStage& R1 = R[(j + 1) & 3];
    const AStage& Aj = A[j];
    AStage& An = A[(j + 3) & 3];
    // activations for step g+3: quad position 3 of this quad (j = 0) or j-1 of the next
    const QuadBase& ab = (j == 0) ? cur : nxt;
    constexpr int aj = (j == 0) ? 3 : j - 1;
    constexpr int kBlocks = kPfSub * kPfCb;
    auto read_op = [&](int b) {
      const int s1 = b / kPfCb, cb1 = b % kPfCb;
      return *reinterpret_cast<const u32x4*>(rbuf + ((cb1 * kPfSub + s1) * kWave + lane) * 16);
    };
    u32x4 wop[kLdsAhead];
#pragma unroll
    for (int b = 0; b < kLdsAhead; ++b) wop[b] = read_op(b);
    u32x4 lo, hi;
#pragma unroll
    for (int blk = 0; blk < kBlocks; ++blk) {
      const int s = blk / kPfCb, cb = blk % kPfCb;
      const u32x4 a = wop[blk % kLdsAhead];
      if (blk + kLdsAhead < kBlocks) wop[blk % kLdsAhead] = read_op(blk + kLdsAhead);
      if (blk < kPfRb * kPfSub) load_act_one(An, blk / kPfSub, blk % kPfSub, ab, aj);
      if (blk == 8 || blk == 9) load_w_chunk(R[j], blk - 8, nxt, j);
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
        acc[rb][cb] = mfma32(a, Aj.a[rb][s], acc[rb][cb]);
      if (blk & 1) {
        const int pc = blk >> 1, c = pc >> 2, d = pc & 3;
        dq_piece(R1, c, d, lo, hi);
        if (d == 3) dq_store(wbuf, c, lo, hi);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int32_t v = 0; v < nq; ++v) {
    if (v + 1 < nq) {
      quad_at(v + 1, t_nxt, ks_nxt);
    } else {
      t_nxt = t_cur;
      ks_nxt = ks_cur;
    }
    quad_base(t_nxt, ks_nxt, nxt);
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    if (v + 1 == nq || t_nxt != t_cur) {
      finish(t_cur);
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
#pragma unroll
        for (int cb = 0; cb < kPfCb; ++cb) acc[rb][cb] = f32x16{};
    }
    t_cur = t_nxt;
    ks_cur = ks_nxt;
    cur = nxt;
  }
}

// Completes the split leftover tiles: adds each tile's pieces in K order (workgroup
// order) and applies the epilogue.  One thread per accumulator group of a lane.
template <int EPI>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillGemmArgs p) {
  constexpr int kOut = (EPI == EPI_PF_SILU) ? kPfCb / 2 : kPfCb;
  constexpr int kItems = kPfWaves * kPfRb * kOut * 4 * kWave;  // per tile
  // Split-tile pieces fetched together (at 16 the Gate/Up copy spilled to scratch, and
  // after a spill-free rewrite it was still no faster than 8).
  constexpr int kReduceBatch = 8;
  const Sched sc{p};
  const int32_t SQ = p.quads;
  const int32_t u = static_cast<int32_t>(blockIdx.y);
  const int32_t t = p.tiles_dp + u;
  const int32_t wa = sc.sk_owner(u * SQ), wb = sc.sk_owner(u * SQ + SQ - 1);
  if (wa == wb) return;  // finished by its only workgroup
  const int32_t nt = t / p.mtiles, mt = t - nt * p.mtiles;
  for (int item = blockIdx.x * blockDim.x + threadIdx.x; item < kItems;
       item += gridDim.x * blockDim.x) {
    const int lane = item & (kWave - 1);
    int rest = item / kWave;
    const int g = rest & 3;
    rest >>= 2;
    const int cb = rest % kOut;
    rest /= kOut;
    const int rb = rest % kPfRb;
    const int wave = rest / kPfRb;
    const int64_t m = int64_t(mt) * kPfTileRows + wave * 64 + rb * 32 + (lane & 31);
    if (m >= p.M) continue;
    const int q0 = (rb * kPfCb + cb) * 4 + g;
    const int q1 = (rb * kPfCb + (cb + 2) % kPfCb) * 4 + g;  // the Up group (EPI_PF_SILU)
    // The pieces are fetched kReduceBatch at a time, all loads of a batch in flight
    // together (a piece past the last re-reads the last one and is not added), and
    // added one by one in K order.
    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
    for (int32_t w0 = wa; w0 <= wb; w0 += kReduceBatch) {
      f32x4 pa[kReduceBatch], pb[kReduceBatch];
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        const int32_t w = min(w0 + i, wb);
        const float* src = p.slots + (int64_t(sc.slot(w, t)) * kPfWaves + wave) * kPfSlotWave;
        pa[i] = *reinterpret_cast<const f32x4*>(src + (q0 * kWave + lane) * 4);
        if constexpr (EPI == EPI_PF_SILU)
          pb[i] = *reinterpret_cast<const f32x4*>(src + (q1 * kWave + lane) * 4);
      }
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        const int32_t w = w0 + i;
        if (w <= wb) {
          x = (w == wa) ? pa[i] : x + pa[i];
          if constexpr (EPI == EPI_PF_SILU) y = (w == wa) ? pb[i] : y + pb[i];
        }
      }
    }
    const int64_t n0 = int64_t(nt) * (kOut * 32) + cb * 32 + g * 8 + (lane >> 5) * 4;
    epilogue_group<EPI>(p, m, n0, x, (EPI == EPI_PF_SILU) ? y : x);
  }
}

template <int EPI, int NMAT>
hipError_t launch_epi(const PrefillGemmArgs& a, hipStream_t s) {
  const dim3 block(kPfWaves * kWave);
  if (a.layout == LAYOUT_TILED)
    hipLaunchKernelGGL((prefill_gemm_kernel<EPI, NMAT, LAYOUT_TILED>), dim3(a.grid), block, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<EPI, NMAT, LAYOUT_ROWMAJOR>), dim3(a.grid), block, 0,
                       s, a);
  if (hipError_t e = hipGetLastError()) return e;
  const int32_t left = a.tiles - a.tiles_dp;
  if (left > 0) {
    constexpr int kOut = (EPI == EPI_PF_SILU) ? kPfCb / 2 : kPfCb;
    constexpr int kItems = kPfWaves * kPfRb * kOut * 4 * kWave;
    hipLaunchKernelGGL((prefill_reduce_kernel<EPI>), dim3(kItems / 256, left), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

int prefill_tile_channels(int epi) { return epi == EPI_PF_SILU ? 64 : 128; }

PrefillPlan plan_prefill(int epi, int64_t M, int64_t N, int64_t K) {
  PrefillPlan pl{};
  pl.mtiles = static_cast<int32_t>((M + kPfTileRows - 1) / kPfTileRows);
  pl.ntiles = static_cast<int32_t>(N / prefill_tile_channels(epi));
  pl.quads = static_cast<int32_t>(K / 256);
  pl.tiles = pl.mtiles * pl.ntiles;
  const int64_t total = int64_t(pl.tiles) * pl.quads;
  pl.grid = static_cast<int32_t>(total < kPrefillGrid ? total : kPrefillGrid);
  if (pl.grid <= 0) return pl;
  pl.dp_per_wg = pl.tiles / pl.grid;
  pl.tiles_dp = pl.dp_per_wg * pl.grid;
  const int64_t left = int64_t(pl.tiles - pl.tiles_dp) * pl.quads;
  pl.q = static_cast<int32_t>(left / pl.grid);
  pl.r = static_cast<int32_t>(left % pl.grid);
  return pl;
}

size_t prefill_slot_floats() { return size_t(kPfWaves) * kPfSlotWave; }

hipError_t launch_prefill_gemm(const PrefillGemmArgs& in, hipStream_t stream) {
  if (in.M == 0) return hipSuccess;
  PrefillGemmArgs a = in;
  const PrefillPlan pl = plan_prefill(a.epi, a.M, a.N, a.K);
  if (pl.grid <= 0) return hipSuccess;
  a.mtiles = pl.mtiles;
  a.quads = pl.quads;
  a.tiles = pl.tiles;
  a.grid = pl.grid;
  a.dp_per_wg = pl.dp_per_wg;
  a.tiles_dp = pl.tiles_dp;
  a.q = pl.q;
  a.r = pl.r;
  a.by_quads = FastDiv(static_cast<uint32_t>(pl.quads));
  a.by_mtiles = FastDiv(static_cast<uint32_t>(pl.mtiles));
  if (a.epi == EPI_PF_SILU) return launch_epi<EPI_PF_SILU, 2>(a, stream);
  if (a.epi == EPI_PF_RES) return launch_epi<EPI_PF_RES, 1>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace a8w8
