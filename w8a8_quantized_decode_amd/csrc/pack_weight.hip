// Conversion of [N, K] row-major INT8 weights to the tiled layout the decode kernels
// stream: 16-channel tiles, each 64-byte K step a contiguous 1 KB block in the operand
// order of v_mfma_i32_16x16x64_i8 (lane l = channel l%16, k-offset 16*(l/16)).
#include "device_common.h"
#include "internal.h"

namespace a8w8 {
namespace {

// One thread moves one 16-byte operand chunk.
__global__ __launch_bounds__(256) void pack_tiled_kernel(const int8_t* w, int64_t N, int64_t K,
                                                         int8_t* out) {
  const int64_t chunks = N * K / 16;
  const int64_t per_tile = K;  // 16 rows * K bytes / 16 bytes per chunk
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += int64_t(gridDim.x) * blockDim.x) {
    const int64_t tile = c / per_tile, rem = c % per_tile;
    const int64_t t = rem / 64, l = rem % 64;
    const int64_t row = tile * 16 + (l & 15);
    const int64_t k = t * 64 + (l >> 4) * 16;
    *reinterpret_cast<i32x4*>(out + c * 16) = ld16(w + row * K + k);
  }
}

}  // namespace

hipError_t launch_pack_tiled(const int8_t* w, int64_t N, int64_t K, int8_t* out,
                             hipStream_t stream) {
  const int64_t chunks = N * K / 16;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_tiled_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     w, N, K, out);
  return hipGetLastError();
}

}  // namespace a8w8
