// Device-side helpers shared by the gfx950 kernels of liba8w8.
//
// Numerics: every FP32 step is a single IEEE binary32 operation rounded to nearest
// even.  The library is compiled with -ffp-contract=off so that a product followed
// by a sum is never fused; division and square root use the correctly rounded
// lowering (hipcc's default), denormals are kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace a8w8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// FP32 -> BF16 with round-to-nearest-even (the conversion instruction of gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Prefill operand layout of BF16 activations: for each block of 32 rows and 64-k step a
// 4 KB block of four 1 KB operands (one per 16-k substep), each in the order of the
// 32x32x16 matrix-core operand: lane l = row l%32 and k-half l/32, 8 values per lane.
// Rows are padded to a multiple of 32.  Element index of (m, k) for K columns:
__device__ __forceinline__ int64_t prefill_operand_index(int64_t m, int64_t k, int64_t K) {
  return ((m >> 5) * (K >> 6) + (k >> 6)) * 2048 + ((k >> 4) & 3) * 512 +
         ((m & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
}

// Decode codes in the weights' tiled operand order (one 16-row tile, rows past M unused):
// one 1 KB block per 64-byte k step, lane l = (m % 16) + 16 * ((k % 64) / 16) holding
// 16 bytes.  16 * K bytes for up to 16 rows.  Byte index of (m, k):
__device__ __forceinline__ int64_t tiled_code_index(int64_t m, int64_t k) {
  return (k >> 6) * 1024 + ((m & 15) + 16 * ((k >> 4) & 3)) * 16 + (k & 15);
}

// Low / high BF16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Symmetric INT8 code of one value: clamp(rint(v / s), -127, 127), s > 0.
__device__ __forceinline__ int quant_code(float v, float s) {
  float t = rintf(v / s);
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return static_cast<int>(t);
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Stores one value with device-scope atomic exchange semantics and returns the old one.
__device__ __forceinline__ int32_t atomic_take(int32_t* p) {
  return __hip_atomic_exchange(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int32_t atomic_add_dev(int32_t* p, int32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ INT8 matrix-core helpers
__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 ld16(const int8_t* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// Weight bytes are read once per call: a non-temporal load keeps the weight stream from
// displacing the kernel's code, the activation rows and the exchange words from the
// caches (each kernel's instruction fetches otherwise queue behind the stream).
__device__ __forceinline__ i32x4 ld16_stream(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// Dequantized value: fl32(fl32(f(acc) * sa) * sw).
__device__ __forceinline__ float dq(int32_t acc, float sa, float sw) {
  return (static_cast<float>(acc) * sa) * sw;
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)), exp evaluated in FP64 and rounded once.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = static_cast<float>(exp(-static_cast<double>(g)));
  const float den = 1.0f + e;
  return (g / den) * u;
}

__device__ __forceinline__ void load8_bf16(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ void load8_f32(const float* p, float (&v)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Eight INT8 codes of v under row scale s, packed little-endian (all zero when s == 0).
__device__ __forceinline__ u32x2 codes8(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t(quant_code(v[i], s)) & 0xFFu) << (8 * i);
      hi |= (uint32_t(quant_code(v[4 + i], s)) & 0xFFu) << (8 * i);
    }
  }
  return u32x2{lo, hi};
}

// Workgroup barrier that orders LDS only.  A full __syncthreads also waits for every
// outstanding global load of the wave, which would drain a weight stream's prefetch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup reductions over LDS slots: each wave reduces, lane 0 posts, and after one
// barrier every thread combines the slots in wave order (same bits in every thread).
template <int NW>
__device__ __forceinline__ double block_sum_f64(double v, double* slots) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = v;
  lds_barrier();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += slots[w];
  return s;
}

template <int NW>
__device__ __forceinline__ float block_max_f32(float v, float* slots) {
  v = wave_max_f32(v);
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = v;
  lds_barrier();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s = fmaxf(s, slots[w]);
  return s;
}

// Agent-coherent 16-byte store and load (two relaxed 64-bit device-scope atomics each):
// they go to the coherence point shared by all XCDs, so data passed between workgroups
// this way needs no L2 write-back or invalidation.
__device__ __forceinline__ void store_coherent(int32_t* p, i32x4 v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(p);
  const uint64_t lo = uint64_t(uint32_t(v[0])) | (uint64_t(uint32_t(v[1])) << 32);
  const uint64_t hi = uint64_t(uint32_t(v[2])) | (uint64_t(uint32_t(v[3])) << 32);
  __hip_atomic_store(d, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ i32x4 load_coherent(const int32_t* p) {
  const uint64_t* d = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(d + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return i32x4{int32_t(uint32_t(lo)), int32_t(uint32_t(lo >> 32)), int32_t(uint32_t(hi)),
               int32_t(uint32_t(hi >> 32))};
}

// Tagged 16-byte slot: four 64-bit words, each an INT32 value in its low half and the
// writer's 32-bit tag in its high half, stored and loaded as relaxed device-scope
// atomics.  A reader that finds the expected tag in every word has the writer's values
// (each word is written whole), so no separate ready flag is needed.
__device__ __forceinline__ void store_tagged(uint64_t* d, i32x4 v, uint32_t tag) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    __hip_atomic_store(d + c, (uint64_t(tag) << 32) | uint32_t(v[c]), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

struct TaggedX4 {
  uint64_t w[4];
};

__device__ __forceinline__ TaggedX4 load_tagged(const uint64_t* d) {
  TaggedX4 t;
#pragma unroll
  for (int c = 0; c < 4; ++c) t.w[c] = __hip_atomic_load(d + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return t;
}

// Adds the values of a tagged slot to `s`; clears `ok` unless every word carries `tag`.
__device__ __forceinline__ void add_tagged(i32x4& s, const TaggedX4& t, uint32_t tag, bool& ok) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    ok = ok && uint32_t(t.w[c] >> 32) == tag;
    s[c] += int32_t(uint32_t(t.w[c]));
  }
}

// Waits until every memory operation this wave has issued has completed (vmcnt = 0),
// with compiler barriers so that no memory access moves across it.
__device__ __forceinline__ void wait_memory_done() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
  __asm__ __volatile__("" ::: "memory");
}

}  // namespace a8w8
