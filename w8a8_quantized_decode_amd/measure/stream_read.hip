// Measurement aid, not part of the A8W8 boundary: a plain streaming read of a device
// buffer, the achievable-HBM-read ceiling that the decode GEMMs (pure weight streams at
// decode batch sizes) are compared against.  Built into libmeasure.so; only bench.py
// loads it.
//
// One 1024-thread workgroup per CU; each of its 16 waves reads one contiguous run of the
// buffer (the access pattern of the decode GEMMs' weight stream), 1 KB per load
// instruction, eight loads in flight, nontemporal.  Every load is bounds-checked.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
constexpr int kWaves = 16;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kWaves * 64) void stream_runs(const int4v* __restrict__ p, int64_t n16,
                                                           int64_t per_wave16, int* out) {
  const int lane = threadIdx.x & 63;
  const int64_t w = int64_t(blockIdx.x) * kWaves + threadIdx.x / 64;
  const int64_t b0 = w * per_wave16;
  const int64_t b1 = b0 + per_wave16 < n16 ? b0 + per_wave16 : n16;
  int4v acc = {0, 0, 0, 0};
  for (int64_t o = b0 + lane; o < b1; o += 64 * kInFlight) {
    int4v v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t j = o + int64_t(u) * 64;
      v[u] = j < b1 ? __builtin_nontemporal_load(p + j) : int4v{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  // A data-dependent store keeps every load live.
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5A5A5A5A) out[0] = 1;
}

}  // namespace

extern "C" {

// Reads nbytes (a multiple of 16) at buf, 16-byte aligned, on `stream`; out: one int of
// device memory.  Returns 0 or the HIP error code.
int a8w8m_stream_read(const void* buf, int64_t nbytes, int* out, int cus, void* stream) {
  if (!buf || !out || nbytes <= 0 || nbytes % 16 || cus <= 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u))
    return int(hipErrorInvalidValue);
  const int64_t n16 = nbytes / 16;
  const int64_t waves = int64_t(cus) * kWaves;
  const int64_t per_wave16 = (n16 + waves - 1) / waves;
  hipLaunchKernelGGL(stream_runs, dim3(static_cast<unsigned>(cus)), dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const int4v*>(buf), n16,
                     per_wave16, out);
  return int(hipGetLastError());
}

}  // extern "C"
