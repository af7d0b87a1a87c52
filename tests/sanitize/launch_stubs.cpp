// Host stand-ins for the kernel launchers, for the sanitizer build of the C ABI's
// argument checks: they record the call and launch nothing (no GPU is used).
#include <hip/hip_runtime.h>

#include "../../long_context_compressed_hca_amd/csrc/hca_kernels.h"

int g_launches = 0;

namespace hca {
hipError_t launch_compress(const uint16_t*, const uint16_t*, int64_t, int64_t, uint16_t*,
                           uint16_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill(const PrefillProblem&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeProblem&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_multi(const DecodeProblem&, const uint16_t*, const uint16_t*, int,
                               hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_sk(const DecodeProblem&, const uint16_t*, const uint16_t*, int, void*,
                            hipStream_t) { ++g_launches; return hipSuccess; }
int decode_splits(int B, int H, int64_t nc_cap) {
  if (B <= 0) return 1;
  const int64_t wgs = (int64_t)B * ((H + 15) / 16);
  if (wgs >= 128) return 1;
  int n = (int)(256 / wgs);
  const int64_t tiles = (nc_cap + 15) / 16 + 8;
  const int64_t cap = tiles / 8 > 1 ? tiles / 8 : 1;
  if (n > cap) n = (int)cap;
  if (n > 16) n = 16;
  return n < 1 ? 1 : n;
}
hipError_t launch_gate(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, int,
                       hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_backward(const BackwardProblem&, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t backward_workspace_bytes(int64_t T, int H) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t rows = T * H, Nc = T / kBlock;
  return up(rows * 4) * 2 + up(rows * kD * 2) + up(Nc * kD * 4) * 2 + 256;
}
size_t decode_workspace_bytes(int B, int H, int64_t nc_cap) {
  const int n = decode_splits(B, H, nc_cap);
  return n <= 1 ? 0 : (size_t)B * ((H + 15) / 16) * n * (32 + 16 * kD) * sizeof(float);
}
}  // namespace hca
