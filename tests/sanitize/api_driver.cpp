// Host driver for the sanitizer build of the C ABI (api.cpp linked with launch
// stubs): every entry point with valid arguments (reaching the stub launcher),
// with each kind of invalid argument, and the no-op sizes.  Fake device
// pointers are never dereferenced.  Exit status 0 when every status is as
// expected; AddressSanitizer and UndefinedBehaviorSanitizer abort on errors.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hca.h"

extern int g_launches;
static int failures = 0;
#define EXPECT(call, want)                                                                     \
  do {                                                                                        \
    const hca_status_t st_ = (call);                                                          \
    if (st_ != (want)) {                                                                      \
      std::fprintf(stderr, "line %d: got %d want %d (%s)\n", __LINE__, (int)st_, (int)(want), \
                   hca_last_error());                                                         \
      ++failures;                                                                             \
    }                                                                                         \
    (void)std::strlen(hca_last_error());                                                      \
    (void)std::strlen(hca_status_string(st_));                                                \
  } while (0)

int main() {
  void* P = reinterpret_cast<void*>(0x10000);
  void* MIS = reinterpret_cast<void*>(0x10008);
  const int64_t* pos = reinterpret_cast<const int64_t*>(0x20000);
  const float sc = 0.044194173f;
  // compress
  EXPECT(hca_compress(P, P, 256, 512, 512, 128, P, P, nullptr), HCA_OK);
  EXPECT(hca_compress(P, P, 100, 512, 512, 128, nullptr, nullptr, nullptr), HCA_OK);
  EXPECT(hca_compress(P, P, 256, 500, 512, 128, P, P, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_compress(MIS, P, 256, 512, 512, 128, P, P, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_compress(P, P, 256, 512, 256, 128, P, P, nullptr), HCA_ERR_UNSUPPORTED);
  // prefill
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, 256, 0, 256, 0, 2, 64, 512, 128, 128, sc, P, HCA_BF16,
                          nullptr), HCA_OK);
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, 0, 0, 0, 0, 0, 64, 512, 128, 128, sc, P, HCA_BF16,
                          nullptr), HCA_OK);
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, 256, 300, 256, 0, 2, 64, 512, 128, 128, sc, P,
                          HCA_BF16, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, 256, 0, 256, 0, 1, 64, 512, 128, 128, sc, P, HCA_F32,
                          nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, 256, 0, 256, 0, 2, 65, 512, 128, 128, sc, P, HCA_F32,
                          nullptr), HCA_ERR_UNSUPPORTED);
  EXPECT(hca_attn_prefill(P, P, P, P, P, P, (int64_t)1 << 40, 0, (int64_t)1 << 40, 0,
                          (int64_t)1 << 33, 64, 512, 128, 128, sc, P, HCA_F32, nullptr),
         HCA_ERR_UNSUPPORTED);
  EXPECT(hca_attn_prefill_vha(P, P, P, P, P, P, 256, 0, 256, 0, 2, 64, 512, 128, 128, sc, P, P, 16,
                              P, HCA_BF16, nullptr), HCA_OK);
  EXPECT(hca_attn_prefill_vha(P, P, P, P, P, P, 256, 0, 256, 0, 2, 64, 512, 128, 128, sc, P, P, 6,
                              P, HCA_BF16, nullptr), HCA_ERR_UNSUPPORTED);
  // decode: a full batch (no workspace) and a split one (workspace checked)
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 64, 64, 512, 128, 128, sc, P, HCA_BF16,
                         nullptr, 0, nullptr), HCA_OK);
  const size_t need = hca_decode_workspace_size(8, 64, 512, 256);
  if (need == 0) ++failures;
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 8, 64, 512, 128, 128, sc, P, HCA_BF16, P,
                         need, nullptr), HCA_OK);
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 8, 64, 512, 128, 128, sc, P, HCA_BF16, P,
                         need - 1, nullptr), HCA_ERR_WORKSPACE);
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 8, 8, 512, 128, 128, sc, P, HCA_F32, nullptr,
                         0, nullptr), HCA_ERR_WORKSPACE);
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 0, 64, 512, 128, 128, sc, P, HCA_BF16,
                         nullptr, 0, nullptr), HCA_OK);
  EXPECT(hca_attn_decode(P, P, P, P, -1, P, P, pos, 8, 64, 512, 128, 128, sc, P, HCA_BF16,
                         nullptr, 0, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_decode(P, P, P, P, 256, P, P, pos, 8, 0, 512, 128, 128, sc, P, HCA_BF16,
                         nullptr, 0, nullptr), HCA_ERR_UNSUPPORTED);
  // the no-allocation form: full batches launch; split ones look up the scratch
  // on the current device, which a host without a GPU does not have
  EXPECT(hca_attn_decode_noalloc(P, P, P, P, 256, P, P, pos, 64, 64, 512, 128, 128, sc, P,
                                 HCA_BF16, nullptr), HCA_OK);
  const hca_status_t st = hca_attn_decode_noalloc(P, P, P, P, 256, P, P, pos, 8, 64, 512, 128,
                                                  128, sc, P, HCA_BF16, nullptr);
  if (st != HCA_OK && st != HCA_ERR_HIP) ++failures;
  // multi-token decode
  EXPECT(hca_attn_decode_multi(P, P, P, P, 256, P, P, P, P, pos, 64, 3, 64, 512, 128, 128, sc, P,
                               HCA_BF16, nullptr), HCA_OK);
  EXPECT(hca_attn_decode_multi(P, P, P, P, 256, P, P, P, P, pos, 64, 3, 8, 512, 128, 128, sc, P,
                               HCA_BF16, nullptr), HCA_OK);
  EXPECT(hca_attn_decode_multi(P, P, P, P, 256, P, P, P, P, pos, 64, 17, 64, 512, 128, 128, sc, P,
                               HCA_BF16, nullptr), HCA_ERR_UNSUPPORTED);
  EXPECT(hca_attn_decode_multi(P, P, P, P, 256, P, P, nullptr, P, pos, 64, 3, 64, 512, 128, 128,
                               sc, P, HCA_BF16, nullptr), HCA_ERR_INVALID_ARG);
  // gate logits
  EXPECT(hca_gate_logits(P, P, 1000, 1024, 32768, P, nullptr), HCA_OK);
  EXPECT(hca_gate_logits(P, P, 0, 1024, 32768, P, nullptr), HCA_OK);
  EXPECT(hca_gate_logits(P, P, 1000, 1000, 32768, P, nullptr), HCA_ERR_UNSUPPORTED);
  EXPECT(hca_gate_logits(P, P, 1000, 1024, 1000, P, nullptr), HCA_ERR_UNSUPPORTED);
  EXPECT(hca_gate_logits(MIS, P, 1000, 1024, 32768, P, nullptr), HCA_ERR_INVALID_ARG);
  // backward
  const size_t bneed = hca_backward_workspace_size(1000, 64, 512);
  if (bneed == 0) ++failures;
  EXPECT(hca_attn_backward(P, P, P, P, P, P, P, 1000, 64, 512, 128, 128, sc, P, P, P, P, P, bneed,
                           nullptr), HCA_OK);
  EXPECT(hca_attn_backward(P, P, P, P, P, P, P, 1000, 64, 512, 128, 128, sc, P, P, P, P, P,
                           bneed - 1, nullptr), HCA_ERR_WORKSPACE);
  EXPECT(hca_attn_backward(P, P, P, P, nullptr, nullptr, P, 100, 8, 512, 128, 128, sc, P, P, P, P,
                           P, hca_backward_workspace_size(100, 8, 512), nullptr), HCA_OK);
  EXPECT(hca_attn_backward(P, P, P, P, P, P, P, 1000, 0, 512, 128, 128, sc, P, P, P, P, P, bneed,
                           nullptr), HCA_ERR_UNSUPPORTED);
  EXPECT(hca_attn_backward(P, P, P, P, P, P, MIS, 1000, 64, 512, 128, 128, sc, P, P, P, P, P,
                           bneed, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_backward(nullptr, P, P, P, P, P, P, 0, 64, 512, 128, 128, sc, nullptr, P, P, P,
                           nullptr, 0, nullptr), HCA_OK);
  // saved-state training pair: prefill with the row log-sum-exp, backward from it
  float* L = reinterpret_cast<float*>(0x30000);
  EXPECT(hca_attn_prefill_lse(P, P, P, P, P, P, 256, 0, 256, 0, 2, 64, 512, 128, 128, sc, P,
                              HCA_BF16, L, nullptr), HCA_OK);
  EXPECT(hca_attn_prefill_lse(P, P, P, P, P, P, 256, 0, 256, 0, 2, 64, 512, 128, 128, sc, P,
                              HCA_BF16, nullptr, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_prefill_lse(P, P, P, P, P, P, 0, 0, 0, 0, 0, 64, 512, 128, 128, sc, nullptr,
                              HCA_BF16, nullptr, nullptr), HCA_OK);
  EXPECT(hca_attn_backward_saved(P, P, P, P, P, P, P, HCA_F32, L, P, 1000, 64, 512, 128, 128, sc,
                                 P, P, P, P, P, bneed, nullptr), HCA_OK);
  EXPECT(hca_attn_backward_saved(P, P, P, P, P, P, nullptr, HCA_BF16, L, P, 1000, 64, 512, 128,
                                 128, sc, P, P, P, P, P, bneed, nullptr), HCA_ERR_INVALID_ARG);
  EXPECT(hca_attn_backward_saved(P, P, P, P, P, P, P, HCA_BF16, L, P, 1000, 64, 512, 128, 128, sc,
                                 P, P, P, P, P, 16, nullptr), HCA_ERR_WORKSPACE);
  if (g_launches < 13) ++failures;
  if (hca_version() < 100) ++failures;
  std::printf("api sanitizer run: %d failures, %d stub launches\n", failures, g_launches);
  return failures == 0 ? 0 : 1;
}
