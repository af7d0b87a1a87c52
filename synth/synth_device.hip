// Device path of the seeded synthetic-input generator (see synth/__init__.py).
//
// Element i of a stream with key `key` is TABLE[mix64(key + (i + 1) * gamma) >> 44],
// where mix64 is the SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014)
// and TABLE is the 2^20-entry bfloat16 normal-quantile table built on the host.
// Integer arithmetic and a table lookup only, so the bits equal the host path's.
// This is input generation for tests and benchmarks, not part of the attention path.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) fill_kernel(uint16_t* __restrict__ out, int64_t n,
                                                   int64_t start, uint64_t key,
                                                   const uint16_t* __restrict__ table) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t u = mix64(key + (uint64_t)(start + i + 1) * kGamma);
    out[i] = table[u >> 44];
  }
}

}  // namespace

extern "C" int hca_synth_fill_bf16(void* out, int64_t n, int64_t start, uint64_t key,
                                   const void* table, void* stream) {
  if (n < 0 || start < 0 || (n > 0 && (!out || !table))) return 1;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)out, n, start, key, (const uint16_t*)table);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
