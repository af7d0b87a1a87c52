// compress.hip - block compression: one cache entry per completed block of 128 rows.
//
// The pages say HCA caches one entry for every 128 tokens (aitest123.com,
// "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B", section 模型结构; lininn.cn,
// section 43 层里，37 层只读摘要) without saying how the entry is formed.  This
// library takes the plainest reading: entry = arithmetic mean of the block's
// rows, for K and V separately, stored as bfloat16.
//
// Arithmetic: each column is summed in binary64, one row after another in
// row order (the same operations, in the same order, as a plain sequential
// binary64 sum; for bfloat16 inputs the sum is exact unless the exponents of
// the block span more than ~45 binades).  The sum is scaled by 1/128 (exact)
// and rounded once to nearest-even bfloat16.
//
// HBM bound: 2 * 128 rows * 1 KiB read per entry pair, 2 KiB written.  One
// wave per (block, tensor); lane i owns columns 8i..8i+7 (one 16-byte load per
// row), so each row is read as one coalesced 1 KiB transaction per wave.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

// binary64 -> bfloat16 bits, round to nearest, ties to even.  A bfloat16 has
// 8 significant bits and the binary32 exponent range, so a value with
// 2^(e-1) <= |x| < 2^e is quantised to multiples of 2^(e-8) (2^-133 below the
// normal range).  Scaling by powers of two and rint are exact.
__device__ inline uint32_t f64_to_bf16_rne(double x) {
  if (__builtin_isnan(x)) return 0x7FC0u;
  if (x == 0.0 || __builtin_isinf(x)) return __float_as_uint((float)x) >> 16;
  int e;
  (void)frexp(x, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  const double r = ldexp(__builtin_rint(ldexp(x, -q)), q);
  return __float_as_uint((float)r) >> 16;  // exact, or +-inf past the bf16 range
}

__global__ void __launch_bounds__(64) compress_kernel(const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int64_t ld,
                                                      uint16_t* __restrict__ ck,
                                                      uint16_t* __restrict__ cv) {
  const int64_t b = blockIdx.x;
  const uint16_t* src = blockIdx.y ? v : k;
  uint16_t* dst = blockIdx.y ? cv : ck;
  if (src == nullptr) return;
  const int lane = threadIdx.x;
  const uint16_t* p = src + b * kBlock * ld + 8 * lane;

  double acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0;

  for (int i0 = 0; i0 < kBlock; i0 += 16) {
    uint4 rows[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) rows[u] = *reinterpret_cast<const uint4*>(p + (i0 + u) * ld);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t w[4] = {rows[u].x, rows[u].y, rows[u].z, rows[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] += (double)bf16_bits_to_f32(w[c] & 0xFFFFu);
        acc[2 * c + 1] += (double)bf16_bits_to_f32(w[c] >> 16);
      }
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    o[c] = f64_to_bf16_rne(acc[2 * c] * (1.0 / kBlock)) |
           (f64_to_bf16_rne(acc[2 * c + 1] * (1.0 / kBlock)) << 16);
  *reinterpret_cast<uint4*>(dst + b * kD + 8 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_compress(const uint16_t* k, const uint16_t* v, int64_t T, int64_t ld,
                           uint16_t* ck, uint16_t* cv, hipStream_t stream) {
  const int64_t nb = T / kBlock;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)nb, 2), dim3(64), 0, stream, k, v, ld, ck,
                     cv);
  return hipGetLastError();
}

}  // namespace hca
