// Prefill-shaped W8A16 GEMMs on gfx950 BF16 matrix cores, on the shared INT8 weights.
//
// Method: pypto-lib PR #810 "perf(qwen3-a8w8): optimize decode scheduling and data
// paths", What changed > Gate/Up INT8 path: prefill keeps the INT8 checkpoint weights
// and dequantizes each weight tile to BF16 before the matrix multiply.  Every weight
// element becomes W' = rne_bf16(fl32(w * s[n])), the activations are BF16, products
// accumulate in FP32 (v_mfma_f32_16x16x32_bf16).
//
// Work shape: stream-K over tiles of 256 rows of M by 16 * NCB weight channels.
//   * Gate/Up tiles hold NCB/2 16-channel blocks of Gate and the same channels of Up,
//     so silu(g) * u is formed from one workgroup's accumulators; Down tiles hold NCB
//     blocks of one weight.
//   * One unit of work is a 64-k step of one tile.  Units are ordered (tile, k) and
//     dealt to a fixed grid of workgroups in contiguous runs of whole quads (4 steps);
//     a workgroup runs its whole run as one software pipeline across tile boundaries.
//   * Weights: per step each of the 256 threads loads NCB/4 16-byte chunks of the INT8
//     tile (the chunk a matrix-core lane needs), dequantizes them and stores the BF16
//     operands to an LDS double buffer; every wave then reads the operands of all NCB
//     blocks from LDS.  A weight element is fetched and dequantized once per workgroup.
//     int8 -> FP32 uses the biased byte u = w + 128 (exact) and one fused multiply-add
//     u * s + (-128 * s), whose exact value is w * s, so its single rounding gives
//     fl32(w * s); FP32 -> BF16 is the RNE conversion.
//   * Activations: wave w owns rows 64w..64w+63 of the tile and loads its BF16 operands
//     straight from global memory into registers, three steps ahead of use.  They are
//     stored row-block tiled (rowblock_tiled_index), so each load instruction reads one
//     contiguous 1 KB (8 whole cache lines); the loads of a step are spread between its
//     matrix-core blocks so that none waits for the address unit in front of an MFMA.
//   * Matrix-core operands: the weights are A (lane l: channel l%16 of a block, 8
//     k-values), the activations B (lane l: row l%16, the same 8 k-values); the 16
//     bytes a lane holds of a tiled 64-k block (k-offsets 16*(l/16)..+15) feed two
//     MFMAs (their first and second 8 k), and the activation operands are gathered in
//     the same k order.  The result of lane l holds channels 4*(l/16)+r of row l%16.
//   * A tile whose steps span several workgroups is completed by exchange: each wave
//     leaves its FP32 partial sums in a slot of the workspace (agent-coherent) and sets
//     its flag to the call's tag; a wave that then finds every piece's flag set claims
//     the tile through its done word and adds the pieces in K order, so the sum does
//     not depend on which workgroup finishes last.
//   * EPI_PF_SILU: h = rne_bf16(silu(g) * u), row-block tiled for the Down GEMM (+ FP32
//     taps of g and u, a row-major tap of h).
//     EPI_PF_RES: out = rne_bf16(d + res) (+ FP32 tap of d).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPfWaves = 4;
constexpr int kPfRowBlocks = 4;     // 16-row blocks per wave
constexpr int kPfTileRows = kPfWaves * kPfRowBlocks * 16;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16 INT8 weights of one channel -> two BF16 operands of 8 (first and second 8 k).
__device__ __forceinline__ void dequant16(u32x4 raw, float s, u32x4& lo, u32x4& hi) {
  const float bias = -128.0f * s;
  float f[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = raw[d] ^ 0x80808080u;  // biased bytes w + 128
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float fu = static_cast<float>((u >> (8 * b)) & 0xFFu);
      f[4 * d + b] = __builtin_fmaf(fu, s, bias);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f[2 * e], f[2 * e + 1]}, bf16x2));
    hi[e] = __builtin_bit_cast(uint32_t,
                               __builtin_convertvector(f32x2{f[8 + 2 * e], f[9 + 2 * e]}, bf16x2));
  }
}

template <int NCB>
struct WStage {
  u32x4 w[NCB / 4];
  float s[NCB / 4];
};

struct AStage {
  u32x4 a[kPfRowBlocks][2];
};

template <int EPI, int NMAT, int NCB, int LAYOUT>
__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_sk_kernel(PrefillGemmArgs p) {
  static_assert(NCB % 4 == 0 && (NMAT == 1 || NCB % 8 == 0), "tile shape");
  constexpr int NCH = NCB / 4;                 // weight chunks per thread per step
  constexpr int kBlkPerMat = NCB / NMAT;       // 16-channel blocks of one weight per tile
  constexpr int kBufBytes = NCB * 2 * kWave * 16;
  constexpr int kSlotWave = kPfRowBlocks * NCB * kWave * 4;  // floats per wave and piece
  __shared__ __align__(16) uint8_t wsm[2][kBufBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int32_t wg = static_cast<int32_t>(blockIdx.x);
  const int32_t S = p.steps;                   // 64-k steps per tile
  const int32_t SQ = S / 4;                    // quads per tile
  const int32_t qa = wg * p.q + min(wg, p.r);
  const int32_t qb = qa + p.q + (wg < p.r ? 1 : 0);
  const int32_t glast = qb * 4 - 1;            // last step of this workgroup
  const int64_t K = p.K;

  // ---- operand fetch for global step g (tile g / S, step g % S), clamped by callers
  auto tile_of = [&](int32_t g, int32_t& ks, int32_t& mt, int32_t& nt) {
    const int32_t t = static_cast<int32_t>(p.by_steps.div(static_cast<uint32_t>(g)));
    ks = g - t * S;
    nt = static_cast<int32_t>(p.by_mtiles.div(static_cast<uint32_t>(t)));
    mt = t - nt * p.mtiles;
  };
  // Loads are a wave-uniform base plus a 32-bit per-lane byte offset (the global_load
  // saddr form), so a step's address arithmetic is almost all scalar.
  const int32_t row_blocks = static_cast<int32_t>((p.M + 15) / 16);
  const int64_t k_steps = K / 64;
  const uint32_t a_lane = static_cast<uint32_t>(lane) * 16u;
  const uint32_t w_lane = (LAYOUT == LAYOUT_TILED) ? static_cast<uint32_t>(lane) * 16u
                                                   : static_cast<uint32_t>(r16 * K + g4 * 16);
  // The two 1 KB operand halves of row block rb of step g (rows past M re-read the last
  // row block; their results are never stored).
  auto act_block = [&](int32_t g, int rb) {
    int32_t ks, mt, nt;
    tile_of(g, ks, mt, nt);
    const int32_t R = min(mt * (kPfTileRows / 16) + wave * kPfRowBlocks + rb, row_blocks - 1);
    return reinterpret_cast<const uint8_t*>(p.act) + (int64_t(R) * k_steps + ks) * 2048;
  };
  auto load_act_rb = [&](AStage& st, int rb, const uint8_t* blk) {
    st.a[rb][0] = *reinterpret_cast<const u32x4*>(blk + a_lane);
    st.a[rb][1] = *reinterpret_cast<const u32x4*>(blk + 1024 + a_lane);
  };
  auto load_act = [&](AStage& st, int32_t g) {
#pragma unroll
    for (int rb = 0; rb < kPfRowBlocks; ++rb) load_act_rb(st, rb, act_block(g, rb));
  };
  auto load_w_chunk = [&](WStage<NCB>& st, int c, int32_t g) {
    int32_t ks, mt, nt;
    tile_of(g, ks, mt, nt);
    const int cb = 4 * c + wave;
    const int mat = cb / kBlkPerMat;
    const int64_t t16 = int64_t(nt) * kBlkPerMat + (cb % kBlkPerMat);
    const int8_t* wbase = (NMAT == 2 && mat == 1) ? p.w1 : p.w0;
    const float* sc = (NMAT == 2 && mat == 1) ? p.sw1 : p.sw0;
    const int8_t* blk = wbase + t16 * 16 * K + int64_t(ks) * ((LAYOUT == LAYOUT_TILED) ? 1024 : 64);
    st.w[c] = *reinterpret_cast<const u32x4*>(blk + w_lane);
    st.s[c] = (sc + t16 * 16)[r16];
  };
  auto load_w = [&](WStage<NCB>& st, int32_t g) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) load_w_chunk(st, c, g);
  };
  auto dequant_store = [&](const WStage<NCB>& st, uint8_t* buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int cb = 4 * c + wave;
      u32x4 lo, hi;
      dequant16(st.w[c], st.s[c], lo, hi);
      *reinterpret_cast<u32x4*>(buf + ((cb * 2 + 0) * kWave + lane) * 16) = lo;
      *reinterpret_cast<u32x4*>(buf + ((cb * 2 + 1) * kWave + lane) * 16) = hi;
    }
  };

  f32x4 acc[kPfRowBlocks][NCB];
#pragma unroll
  for (int rb = 0; rb < kPfRowBlocks; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};



  // ---- tile completion
  const uint64_t want = p.tag | uint64_t(EPI + 1);
  auto start_of = [&](int32_t w) { return w * p.q + min(w, p.r); };
  auto owner_of = [&](int32_t quad) {
    const int32_t cut = p.r * (p.q + 1);
    return quad < cut ? quad / (p.q + 1) : p.r + (quad - cut) / p.q;
  };
  auto slot_of = [&](int32_t w, int32_t t) {
    return 2 * w + (t != start_of(w) / SQ ? 1 : 0);
  };
  auto finish = [&](int32_t t) {
    const int32_t nt = t / p.mtiles, mt = t - nt * p.mtiles;
    const int32_t wa = owner_of(t * SQ), wb = owner_of(t * SQ + SQ - 1);
    if (wa != wb) {
      // Publish this wave's piece, then its flag, each agent-coherent and waited for.
      float* mine = p.slots + (int64_t(slot_of(wg, t)) * kPfWaves + wave) * kSlotWave;
#pragma unroll
      for (int rb = 0; rb < kPfRowBlocks; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          store_coherent(reinterpret_cast<int32_t*>(mine + ((rb * NCB + cb) * kWave + lane) * 4),
                         __builtin_bit_cast(i32x4, acc[rb][cb]));
      wait_memory_done();
      uint64_t* myflag = p.flags + int64_t(slot_of(wg, t)) * kPfWaves + wave;
      if (lane == 0) __hip_atomic_store(myflag, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_memory_done();
      // Every wave whose flag became visible after all others finds them all set.
      bool all = true;
      for (int32_t w = wa; w <= wb; ++w) {
        const uint64_t f = __hip_atomic_load(p.flags + int64_t(slot_of(w, t)) * kPfWaves + wave,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        all = all && (f == want);
      }
      if (!__builtin_amdgcn_readfirstlane(all ? 1 : 0)) return;
      // Several waves can find them all set: the first to swap the done word to this
      // call's tag completes the tile (the output may overwrite the residual it reads).
      uint64_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_exchange(p.dones + int64_t(t) * kPfWaves + wave, want,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t plo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(prev));
      const uint32_t phi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(prev >> 32));
      if (((uint64_t(phi) << 32) | plo) == want) return;
      // Sum of the pieces in K order (workgroup order), all read back from the slots.
      for (int32_t w = wa; w <= wb; ++w) {
        const float* src = p.slots + (int64_t(slot_of(w, t)) * kPfWaves + wave) * kSlotWave;
        f32x4 v[kPfRowBlocks][NCB];
#pragma unroll
        for (int rb = 0; rb < kPfRowBlocks; ++rb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            v[rb][cb] = __builtin_bit_cast(
                f32x4, load_coherent(reinterpret_cast<const int32_t*>(
                           src + ((rb * NCB + cb) * kWave + lane) * 4)));
#pragma unroll
        for (int rb = 0; rb < kPfRowBlocks; ++rb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = (w == wa) ? v[rb][cb] : acc[rb][cb] + v[rb][cb];
      }
    }
#pragma unroll
    for (int rb = 0; rb < kPfRowBlocks; ++rb) {
      const int64_t m = int64_t(mt) * kPfTileRows + wave * 64 + rb * 16 + r16;
      if (m >= p.M) continue;
      if constexpr (EPI == EPI_PF_SILU) {
#pragma unroll
        for (int cb = 0; cb < kBlkPerMat; ++cb) {
          const int64_t n = (int64_t(nt) * kBlkPerMat + cb) * 16 + 4 * g4;
          const f32x4 g = acc[rb][cb], u = acc[rb][kBlkPerMat + cb];
          if (p.tap_g) *reinterpret_cast<f32x4*>(p.tap_g + m * p.N + n) = g;
          if (p.tap_u) *reinterpret_cast<f32x4*>(p.tap_u + m * p.N + n) = u;
          u32x2 o;
          o[0] = uint32_t(f32_to_bf16_rne(silu_mul(g[0], u[0]))) |
                 (uint32_t(f32_to_bf16_rne(silu_mul(g[1], u[1]))) << 16);
          o[1] = uint32_t(f32_to_bf16_rne(silu_mul(g[2], u[2]))) |
                 (uint32_t(f32_to_bf16_rne(silu_mul(g[3], u[3]))) << 16);
          *reinterpret_cast<u32x2*>(p.out + rowblock_tiled_index(m, n, p.N)) = o;
          if (p.tap_h) *reinterpret_cast<u32x2*>(p.tap_h + m * p.N + n) = o;
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int64_t n = (int64_t(nt) * NCB + cb) * 16 + 4 * g4;
          const f32x4 d = acc[rb][cb];
          if (p.tap_d) *reinterpret_cast<f32x4*>(p.tap_d + m * p.N + n) = d;
          const u32x2 rr = *reinterpret_cast<const u32x2*>(p.res + m * p.ldr + n);
          u32x2 o;
          o[0] = uint32_t(f32_to_bf16_rne(d[0] + bf16_lo(rr[0]))) |
                 (uint32_t(f32_to_bf16_rne(d[1] + bf16_hi(rr[0]))) << 16);
          o[1] = uint32_t(f32_to_bf16_rne(d[2] + bf16_lo(rr[1]))) |
                 (uint32_t(f32_to_bf16_rne(d[3] + bf16_hi(rr[1]))) << 16);
          *reinterpret_cast<u32x2*>(p.out + m * p.ldo + n) = o;
        }
      }
    }
  };

  // ---- the pipeline.  Invariant at the start of step g (stage j = g % 4): A[j] holds
  // (or is loading) the activations of step g, A[j+1], A[j+2] those of g+1, g+2;
  // R[j+1..j+3] the raw weights of steps g+1..g+3; LDS buffer g%2 the dequantized
  // weights of step g.  Loads past the last step re-read the last step (never used).
  AStage A[4];
  WStage<NCB> R[4];
  // The prologue issues its loads in the steady state's order (the scheduling barriers
  // keep them there): the loop head's waits are derived from every path into it, so a
  // load issued late here would make each iteration wait for nearly all of its loads.
  const int32_t g0 = qa * 4;
  load_act(A[0], g0);
  load_w(R[0], g0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(R[1], min(g0 + 1, glast));
  __builtin_amdgcn_sched_barrier(0);
  load_act(A[1], min(g0 + 1, glast));
  __builtin_amdgcn_sched_barrier(0);
  load_w(R[2], min(g0 + 2, glast));
  __builtin_amdgcn_sched_barrier(0);
  load_act(A[2], min(g0 + 2, glast));
  __builtin_amdgcn_sched_barrier(0);
  load_w(R[3], min(g0 + 3, glast));
  __builtin_amdgcn_sched_barrier(0);
  dequant_store(R[0], wsm[0]);
  lds_barrier();

  // One step: per 16-channel block its 8 MFMAs, an eighth of the next step's
  // dequantization (4 weights of one chunk) so the vector ALU works while the matrix
  // core runs, and a share of the loads for steps g+3 (activations) and g+4 (weights);
  // each block's weight operands are read from LDS one block ahead.  The scheduling
  // barriers keep this order.
  auto step = [&](auto J, int32_t g) {
    constexpr int j = decltype(J)::value;
    const uint8_t* rbuf = wsm[j & 1];
    uint8_t* wbuf = wsm[(j + 1) & 1];
    const WStage<NCB>& R1 = R[(j + 1) & 3];
    const AStage& Aj = A[j];
    const int32_t ga = min(g + 3, glast), gw = min(g + 4, glast);
    u32x4 wop[2][2];
    auto read_op = [&](int cb, u32x4 (&o)[2]) {
      o[0] = *reinterpret_cast<const u32x4*>(rbuf + ((cb * 2 + 0) * kWave + lane) * 16);
      o[1] = *reinterpret_cast<const u32x4*>(rbuf + ((cb * 2 + 1) * kWave + lane) * 16);
    };
    read_op(0, wop[0]);
    u32x4 dq_lo, dq_hi;
    constexpr int kPieces = 4 * NCH;  // dequantization pieces: one weight dword each
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb + 1 < NCB) read_op(cb + 1, wop[(cb + 1) & 1]);
      // this block's share of the loads for later steps
      if (cb < kPfRowBlocks) load_act_rb(A[(j + 3) & 3], cb, act_block(ga, cb));
      if (cb >= kPfRowBlocks && cb < kPfRowBlocks + NCH) load_w_chunk(R[j], cb - kPfRowBlocks, gw);
#pragma unroll
      for (int rb = 0; rb < kPfRowBlocks; ++rb)
        acc[rb][cb] = mfma_bf16(wop[cb & 1][0], Aj.a[rb][0], acc[rb][cb]);
#pragma unroll
      for (int rb = 0; rb < kPfRowBlocks; ++rb)
        acc[rb][cb] = mfma_bf16(wop[cb & 1][1], Aj.a[rb][1], acc[rb][cb]);
      // dequantization pieces spread evenly over the blocks
#pragma unroll
      for (int pc = cb * kPieces / NCB; pc < (cb + 1) * kPieces / NCB; ++pc) {
        const int c = pc / 4, d = pc % 4;
        const float sc = R1.s[c];
        const float bias = -128.0f * sc;
        const uint32_t u = R1.w[c][d] ^ 0x80808080u;  // biased bytes w + 128
        float f[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
          f[b] = __builtin_fmaf(static_cast<float>((u >> (8 * b)) & 0xFFu), sc, bias);
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f[0], f[1]}, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f[2], f[3]}, bf16x2));
        u32x4& dst = (d < 2) ? dq_lo : dq_hi;
        dst[(d & 1) * 2] = p0;
        dst[(d & 1) * 2 + 1] = p1;
        if (d == 3) {
          const int wcb = 4 * c + wave;
          *reinterpret_cast<u32x4*>(wbuf + ((wcb * 2 + 0) * kWave + lane) * 16) = dq_lo;
          *reinterpret_cast<u32x4*>(wbuf + ((wcb * 2 + 1) * kWave + lane) * 16) = dq_hi;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Segments: the run of quads of one tile; the pipeline runs on across segment ends.
  int32_t Q = qa;
  while (Q < qb) {
    const int32_t t = static_cast<int32_t>(p.by_steps.div(static_cast<uint32_t>(Q * 4)));
    const int32_t qe = min(qb, (t + 1) * SQ);
    for (; Q < qe; ++Q) {
      const int32_t g = Q * 4;
      step(std::integral_constant<int, 0>{}, g);
      step(std::integral_constant<int, 1>{}, g + 1);
      step(std::integral_constant<int, 2>{}, g + 2);
      step(std::integral_constant<int, 3>{}, g + 3);
    }
    finish(t);
#pragma unroll
    for (int rb = 0; rb < kPfRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int EPI, int NMAT, int NCB>
hipError_t launch_layout(const PrefillGemmArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.grid)), block(kPfWaves * kWave);
  if (a.layout == LAYOUT_TILED)
    hipLaunchKernelGGL((prefill_sk_kernel<EPI, NMAT, NCB, LAYOUT_TILED>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_sk_kernel<EPI, NMAT, NCB, LAYOUT_ROWMAJOR>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

int prefill_tile_channels(int epi) { return epi == EPI_PF_SILU ? 64 : 128; }

PrefillPlan plan_prefill(int epi, int64_t M, int64_t N, int64_t K) {
  PrefillPlan pl{};
  pl.mtiles = static_cast<int32_t>((M + kPfTileRows - 1) / kPfTileRows);
  pl.ntiles = static_cast<int32_t>(N / prefill_tile_channels(epi));
  pl.steps = static_cast<int32_t>(K / 64);
  const int64_t quads = int64_t(pl.mtiles) * pl.ntiles * (pl.steps / 4);
  pl.grid = static_cast<int32_t>(quads < kPrefillGrid ? quads : kPrefillGrid);
  if (pl.grid > 0) {
    pl.q = static_cast<int32_t>(quads / pl.grid);
    pl.r = static_cast<int32_t>(quads % pl.grid);
  }
  return pl;
}

size_t prefill_slot_floats() {
  return size_t(kPfWaves) * kPfRowBlocks * 8 * kWave * 4;  // one piece of an 8-block tile
}

hipError_t launch_prefill_gemm(const PrefillGemmArgs& in, hipStream_t stream) {
  if (in.M == 0) return hipSuccess;
  PrefillGemmArgs a = in;
  const PrefillPlan pl = plan_prefill(a.epi, a.M, a.N, a.K);
  if (pl.grid <= 0) return hipSuccess;
  a.mtiles = pl.mtiles;
  a.steps = pl.steps;
  a.q = pl.q;
  a.r = pl.r;
  a.grid = pl.grid;
  a.by_steps = FastDiv(static_cast<uint32_t>(pl.steps));
  a.by_mtiles = FastDiv(static_cast<uint32_t>(pl.mtiles));
  if (a.epi == EPI_PF_SILU) return launch_layout<EPI_PF_SILU, 2, 8>(a, stream);
  if (a.epi == EPI_PF_RES) return launch_layout<EPI_PF_RES, 1, 8>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace a8w8
