// copy_probe.hip - measurement support, not part of the attention path: the
// MFMA issue rate of one SIMD, and the rate at which one CU moves 1 KiB key
// rows from memory, by LDS DMA (the way
// the prefill, decode and gate kernels stage their tiles) or by 16-byte loads
// into VGPRs.  Built into its own library (libhca_probe.so) for bench.py's
// --copy-rate mode.
//
// Each workgroup owns `bytes_per_wg` bytes of `src` (a whole number of KiB).
// Wave w of nw takes rows w, w + nw, ... in groups of 16 per wave, waits for
// each group, and then issues the next.  `passes` passes run back to back;
// only the last is timed (the earlier ones bring the data into L2 / MALL when
// `warm`).  Per workgroup, clk[3 i .. 3 i + 2] = shader-clock cycles of the
// timed pass (s_memtime), constant-clock ticks of it (s_memrealtime, 100 MHz),
// and a checksum of the loaded words (register mode only, so the loads are
// not removed).
#include "hca_common.h"

namespace hca {
namespace {

template <bool kDma>
__global__ void __launch_bounds__(512) copy_probe_kernel(const uint8_t* src, int bytes_per_wg,
                                                         int passes, unsigned long long* clk) {
  // Per wave 16 rows of 1 KiB: the DMA destinations (8 waves at most).
  __shared__ __attribute__((aligned(1024))) uint8_t lds[8 * 16 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int rows = bytes_per_wg >> 10;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)blockIdx.x * bytes_per_wg, bytes_per_wg);
  uint8_t* const dst = lds + wave * 16 * 1024;
  unsigned sum = 0;
  unsigned long long c0 = 0, r0 = 0;
  for (int pass = 0; pass < passes; ++pass) {
    __syncthreads();
    if (pass == passes - 1) {
      c0 = __builtin_amdgcn_s_memtime();
      r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int g0 = wave; g0 < rows; g0 += 16 * nw) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int r = g0 + u * nw;
        if (r < rows) {
          if constexpr (kDma) {
            dma16_buf(rs, r * 1024 + 16 * lane, (lds_void*)(dst + u * 1024));
          } else {
            const u32x4 v = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, r * 1024 + 16 * lane, 0, 0));
            sum += v[0] ^ v[1] ^ v[2] ^ v[3];
          }
        }
      }
      wait_vmem();
    }
  }
  __syncthreads();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[3 * blockIdx.x] = c1 - c0;
    clk[3 * blockIdx.x + 1] = r1 - r0;
  }
  if (!kDma) atomicXor(reinterpret_cast<unsigned*>(&clk[3 * blockIdx.x + 2]), sum);
}

// MFMA issue rate: each wave runs `n` v_mfma_f32_32x32x16_bf16 in `chains`
// independent accumulator chains (1 or 4), timed with s_memtime; clk[2 i] =
// cycles of wave i, clk[2 i + 1] = a word of its result (so the chain is kept).
template <int kChains>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int n, unsigned long long* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  __syncthreads();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < n; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[u % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u % kChains], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) r += acc[c][0];
  asm volatile("" : "+v"(r));
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const int w = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (lane == 0) {
    clk[2 * w] = c1 - c0;
    clk[2 * w + 1] = (unsigned long long)__float_as_uint(r);
  }
}

}  // namespace
}  // namespace hca

// One workgroup of 4 waves (one per SIMD); n a multiple of 4; clk holds 8
// words.  Returns a hipError_t.
extern "C" int hca_probe_mfma_rate(int n, int chains, unsigned long long* clk, void* stream) {
  if (n < 4 || (n & 3) != 0 || (chains != 1 && chains != 4)) return (int)hipErrorInvalidValue;
  if (chains == 1)
    hipLaunchKernelGGL(hca::mfma_probe_kernel<1>, dim3(1), dim3(256), 0, (hipStream_t)stream, n, clk);
  else
    hipLaunchKernelGGL(hca::mfma_probe_kernel<4>, dim3(1), dim3(256), 0, (hipStream_t)stream, n, clk);
  return (int)hipGetLastError();
}

// grid workgroups of waves * 64 threads; src must hold grid * bytes_per_wg
// bytes; clk must hold 3 * grid zeroed words.  Returns a hipError_t.
extern "C" int hca_probe_copy_rate(const void* src, int grid, int waves, int bytes_per_wg,
                                   int passes, int dma, unsigned long long* clk, void* stream) {
  if (grid < 1 || waves < 1 || waves > 8 || bytes_per_wg < 1024 || (bytes_per_wg & 1023) != 0 ||
      passes < 1)
    return (int)hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b((unsigned)(64 * waves));
  const uint8_t* s = static_cast<const uint8_t*>(src);
  if (dma)
    hipLaunchKernelGGL(hca::copy_probe_kernel<true>, g, b, 0, (hipStream_t)stream, s, bytes_per_wg,
                       passes, clk);
  else
    hipLaunchKernelGGL(hca::copy_probe_kernel<false>, g, b, 0, (hipStream_t)stream, s,
                       bytes_per_wg, passes, clk);
  return (int)hipGetLastError();
}
