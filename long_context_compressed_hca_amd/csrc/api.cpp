// api.cpp - the C ABI declared in include/hca.h: argument checks, then launches.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect on the device.  Messages for the last failure are kept per thread.
#include "../../include/hca.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "hca_kernels.h"

namespace {

thread_local char g_msg[512] = "";

hca_status_t fail(hca_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return st;
}

hca_status_t ok() {
  g_msg[0] = '\0';
  return HCA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hca_status_t check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(HCA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(HCA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return HCA_OK;
}

hca_status_t check_shape(int D, int block, int window) {
  if (D != hca::kD) return fail(HCA_ERR_UNSUPPORTED, "D = %d (only 512 is supported)", D);
  if (block != hca::kBlock)
    return fail(HCA_ERR_UNSUPPORTED, "block = %d (only 128 is supported)", block);
  if (window != hca::kWindow)
    return fail(HCA_ERR_UNSUPPORTED, "window = %d (only 128 is supported)", window);
  return HCA_OK;
}

hca_status_t check_scale(float scale) {
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(HCA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  return HCA_OK;
}

hca_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(HCA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ok();
}

#define TRY(expr)                          \
  do {                                     \
    const hca_status_t st_ = (expr);       \
    if (st_ != HCA_OK) return st_;         \
  } while (0)

}  // namespace

extern "C" {

const char* hca_status_string(hca_status_t status) {
  switch (status) {
    case HCA_OK: return "ok";
    case HCA_ERR_INVALID_ARG: return "invalid argument";
    case HCA_ERR_UNSUPPORTED: return "unsupported shape";
    case HCA_ERR_WORKSPACE: return "workspace missing or too small";
    case HCA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* hca_last_error(void) { return g_msg; }

int hca_version(void) { return 100; }

hca_status_t hca_compress(const void* k, const void* v, int64_t T, int64_t ld, int D, int block,
                          void* ck, void* cv, void* stream) {
  TRY(check_shape(D, block, hca::kWindow));
  if (T < 0) return fail(HCA_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
  if (ld < D || ld % 8 != 0)
    return fail(HCA_ERR_INVALID_ARG, "ld = %lld (need ld >= D and ld %% 8 == 0)", (long long)ld);
  if (T / block == 0) return ok();  // no complete block: nothing to write
  if ((k == nullptr) != (ck == nullptr))
    return fail(HCA_ERR_INVALID_ARG, "k and ck must be both given or both NULL");
  if ((v == nullptr) != (cv == nullptr))
    return fail(HCA_ERR_INVALID_ARG, "v and cv must be both given or both NULL");
  if (k == nullptr && v == nullptr)
    return fail(HCA_ERR_INVALID_ARG, "nothing to compress (k and v are NULL)");
  if (k) {
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(ck, "ck"));
  }
  if (v) {
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(cv, "cv"));
  }
  return hip_status(hca::launch_compress(static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), T, ld,
                                         static_cast<uint16_t*>(ck), static_cast<uint16_t*>(cv),
                                         static_cast<hipStream_t>(stream)),
                    "hca_compress launch");
}

// Prefill with an optional VHA head mix (vha_rank 0: none).
static hca_status_t prefill_impl(const void* q, const void* g, const void* k, const void* v,
                                 const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                 int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                 int block, int window, float scale, const void* vha_up,
                                 const void* vha_down, int vha_rank, void* out,
                                 hca_dtype_t out_dtype, void* stream, const char* what) {
  TRY(check_shape(D, block, window));
  if (H < 1 || H > 64) return fail(HCA_ERR_UNSUPPORTED, "H = %d (need 1 <= H <= 64)", H);
  if (vha_rank != 0) {
    if (H != 64) return fail(HCA_ERR_UNSUPPORTED, "VHA needs H = 64 (got %d)", H);
    if (vha_rank < 4 || vha_rank > 32 || vha_rank % 4 != 0)
      return fail(HCA_ERR_UNSUPPORTED, "VHA rank %d (need a multiple of 4, 4 .. 32)", vha_rank);
  }
  if (Tq < 0 || q_start < 0 || Tkv < 0 || kv_start < 0 || Nc < 0)
    return fail(HCA_ERR_INVALID_ARG, "negative size or position");
  if (out_dtype != HCA_BF16 && out_dtype != HCA_F32)
    return fail(HCA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
  TRY(check_scale(scale));
  if (Tq == 0) return ok();
  constexpr int64_t kMax = 0x7fffffff;  // positions and row counts are 32-bit in the kernel
  if (q_start > kMax - Tq || kv_start > kMax - Tkv || Tq > kMax / H || Nc > kMax)
    return fail(HCA_ERR_UNSUPPORTED, "positions, rows or entries beyond 2^31 - 1");
  const int64_t first_needed = q_start - (window - 1) > 0 ? q_start - (window - 1) : 0;
  if (kv_start > first_needed)
    return fail(HCA_ERR_INVALID_ARG,
                "kv_start = %lld but the first query (position %lld) needs raw rows from %lld",
                (long long)kv_start, (long long)q_start, (long long)first_needed);
  if (kv_start + Tkv < q_start + Tq)
    return fail(HCA_ERR_INVALID_ARG, "raw rows end at %lld but the last query is at %lld",
                (long long)(kv_start + Tkv - 1), (long long)(q_start + Tq - 1));
  const int64_t needed_entries = (q_start + Tq) / block;
  if (Nc < needed_entries)
    return fail(HCA_ERR_INVALID_ARG, "Nc = %lld but the last query sees %lld entries",
                (long long)Nc, (long long)needed_entries);
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(g, "g"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(out, "out"));
  if (needed_entries > 0) {
    TRY(check_ptr(ck, "ck"));
    TRY(check_ptr(cv, "cv"));
  }
  if (vha_rank != 0) {
    TRY(check_ptr(vha_up, "vha_up"));
    TRY(check_ptr(vha_down, "vha_down"));
  }
  hca::PrefillProblem p;
  p.q = static_cast<const uint16_t*>(q);
  p.g = static_cast<const uint16_t*>(g);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.ck = static_cast<const uint16_t*>(ck);
  p.cv = static_cast<const uint16_t*>(cv);
  p.out = out;
  p.Tq = Tq;
  p.q_start = q_start;
  p.Tkv = Tkv;
  p.kv_start = kv_start;
  p.Nc = needed_entries;  // entries past the last query's range are never visible
  p.H = H;
  p.scale = scale;
  p.out_f32 = out_dtype == HCA_F32;
  p.vha_up = static_cast<const uint16_t*>(vha_up);
  p.vha_down = static_cast<const uint16_t*>(vha_down);
  p.vha_rank = vha_rank;
  return hip_status(hca::launch_prefill(p, static_cast<hipStream_t>(stream)), what);
}

hca_status_t hca_attn_prefill(const void* q, const void* g, const void* k, const void* v,
                              const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                              int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D, int block,
                              int window, float scale, void* out, hca_dtype_t out_dtype,
                              void* stream) {
  return prefill_impl(q, g, k, v, ck, cv, Tq, q_start, Tkv, kv_start, Nc, H, D, block, window,
                      scale, nullptr, nullptr, 0, out, out_dtype, stream,
                      "hca_attn_prefill launch");
}

hca_status_t hca_attn_prefill_vha(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                  int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                  int block, int window, float scale, const void* vha_up,
                                  const void* vha_down, int vha_rank, void* out,
                                  hca_dtype_t out_dtype, void* stream) {
  if (vha_rank == 0) return fail(HCA_ERR_UNSUPPORTED, "VHA rank 0 (use hca_attn_prefill)");
  return prefill_impl(q, g, k, v, ck, cv, Tq, q_start, Tkv, kv_start, Nc, H, D, block, window,
                      scale, vha_up, vha_down, vha_rank, out, out_dtype, stream,
                      "hca_attn_prefill_vha launch");
}

hca_status_t hca_attn_decode(const void* q, const void* g, const void* ck, const void* cv,
                             int64_t nc_cap, const void* wk, const void* wv, const int64_t* pos,
                             int B, int H, int D, int block, int window, float scale, void* out,
                             hca_dtype_t out_dtype, void* stream) {
  TRY(check_shape(D, block, window));
  if (B < 0) return fail(HCA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (H < 16 || H > 64 || H % 16 != 0)
    return fail(HCA_ERR_UNSUPPORTED, "H = %d (need a multiple of 16, at most 64)", H);
  if (nc_cap < 0) return fail(HCA_ERR_INVALID_ARG, "nc_cap = %lld < 0", (long long)nc_cap);
  if (out_dtype != HCA_BF16 && out_dtype != HCA_F32)
    return fail(HCA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
  TRY(check_scale(scale));
  if (B == 0) return ok();
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(g, "g"));
  TRY(check_ptr(wk, "wk"));
  TRY(check_ptr(wv, "wv"));
  TRY(check_ptr(out, "out"));
  if (pos == nullptr) return fail(HCA_ERR_INVALID_ARG, "pos is NULL");
  if (reinterpret_cast<uintptr_t>(pos) % 8 != 0)
    return fail(HCA_ERR_INVALID_ARG, "pos is not 8-byte aligned");
  if (nc_cap > 0) {
    TRY(check_ptr(ck, "ck"));
    TRY(check_ptr(cv, "cv"));
  }
  hca::DecodeProblem p;
  p.q = static_cast<const uint16_t*>(q);
  p.g = static_cast<const uint16_t*>(g);
  p.ck = static_cast<const uint16_t*>(ck);
  p.cv = static_cast<const uint16_t*>(cv);
  p.wk = static_cast<const uint16_t*>(wk);
  p.wv = static_cast<const uint16_t*>(wv);
  p.pos = pos;
  p.out = out;
  p.nc_cap = nc_cap;
  p.B = B;
  p.H = H;
  p.scale = scale;
  p.out_f32 = out_dtype == HCA_F32;
  return hip_status(hca::launch_decode(p, static_cast<hipStream_t>(stream)),
                    "hca_attn_decode launch");
}

hca_status_t hca_attn_decode_multi(const void* q, const void* g, const void* ck, const void* cv,
                                   int64_t nc_cap, const void* wk, const void* wv,
                                   const void* nk, const void* nv, const int64_t* pos, int B,
                                   int M, int H, int D, int block, int window, float scale,
                                   void* out, hca_dtype_t out_dtype, void* stream) {
  TRY(check_shape(D, block, window));
  if (B < 0) return fail(HCA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (M < 1 || M > 16) return fail(HCA_ERR_UNSUPPORTED, "M = %d (need 1 .. 16)", M);
  if (H < 16 || H % 16 != 0 || M * H > 1024)
    return fail(HCA_ERR_UNSUPPORTED, "H = %d, M = %d (need H a multiple of 16, M*H <= 1024)", H,
                M);
  if (nc_cap < 0) return fail(HCA_ERR_INVALID_ARG, "nc_cap = %lld < 0", (long long)nc_cap);
  if (out_dtype != HCA_BF16 && out_dtype != HCA_F32)
    return fail(HCA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
  TRY(check_scale(scale));
  if (B == 0) return ok();
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(g, "g"));
  TRY(check_ptr(wk, "wk"));
  TRY(check_ptr(wv, "wv"));
  TRY(check_ptr(nk, "nk"));
  TRY(check_ptr(nv, "nv"));
  TRY(check_ptr(out, "out"));
  if (pos == nullptr) return fail(HCA_ERR_INVALID_ARG, "pos is NULL");
  if (reinterpret_cast<uintptr_t>(pos) % 8 != 0)
    return fail(HCA_ERR_INVALID_ARG, "pos is not 8-byte aligned");
  if (nc_cap > 0) {
    TRY(check_ptr(ck, "ck"));
    TRY(check_ptr(cv, "cv"));
  }
  hca::DecodeProblem p;
  p.q = static_cast<const uint16_t*>(q);
  p.g = static_cast<const uint16_t*>(g);
  p.ck = static_cast<const uint16_t*>(ck);
  p.cv = static_cast<const uint16_t*>(cv);
  p.wk = static_cast<const uint16_t*>(wk);
  p.wv = static_cast<const uint16_t*>(wv);
  p.pos = pos;
  p.out = out;
  p.nc_cap = nc_cap;
  p.B = B;
  p.H = H;
  p.scale = scale;
  p.out_f32 = out_dtype == HCA_F32;
  return hip_status(hca::launch_decode_multi(p, static_cast<const uint16_t*>(nk),
                                             static_cast<const uint16_t*>(nv), M,
                                             static_cast<hipStream_t>(stream)),
                    "hca_attn_decode_multi launch");
}

}  // extern "C"
