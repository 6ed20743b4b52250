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

// Low / high BF16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
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

}  // namespace a8w8
