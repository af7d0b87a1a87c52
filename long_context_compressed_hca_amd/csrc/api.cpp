// api.cpp - the C ABI declared in include/hca.h: argument checks, then launches.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect on the device.  Messages for the last failure are kept per thread.
#include "../../include/hca.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

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

// Query rows (T * H) and positions stay below 2^31: the kernels index them in 32 bits.
constexpr int64_t kMaxRows = 0x7FFFFFFF;

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

// Device scratch of hca_attn_decode_noalloc: room for the largest decode
// workspace, one copy per GPU, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol): it uses the device address looked up once per device.
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[hca::kDecodeWorkspaceMax];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

#define TRY(expr)                          \
  do {                                     \
    const hca_status_t st_ = (expr);       \
    if (st_ != HCA_OK) return st_;         \
  } while (0)

// Device address of this GPU's scratch (the current device), looked up on the
// first call for that device.
hca_status_t scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(HCA_ERR_HIP, "hipGetDevice: %s (%d)", hipGetErrorString(e), (int)e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HCA_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || p == nullptr)
      return fail(HCA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s (%d)", dev,
                  hipGetErrorString(es), (int)es);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HCA_OK;
}

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
                                 hca_dtype_t out_dtype, float* lse, void* stream,
                                 const char* what) {
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
  if (lse != nullptr) TRY(check_ptr(lse, "lse"));
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
  p.lse = lse;
  return hip_status(hca::launch_prefill(p, static_cast<hipStream_t>(stream)), what);
}

hca_status_t hca_attn_prefill(const void* q, const void* g, const void* k, const void* v,
                              const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                              int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D, int block,
                              int window, float scale, void* out, hca_dtype_t out_dtype,
                              void* stream) {
  return prefill_impl(q, g, k, v, ck, cv, Tq, q_start, Tkv, kv_start, Nc, H, D, block, window,
                      scale, nullptr, nullptr, 0, out, out_dtype, nullptr, stream,
                      "hca_attn_prefill launch");
}

hca_status_t hca_attn_prefill_lse(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                  int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                  int block, int window, float scale, void* out,
                                  hca_dtype_t out_dtype, float* lse, void* stream) {
  if (lse == nullptr && Tq > 0) return fail(HCA_ERR_INVALID_ARG, "lse is NULL");
  return prefill_impl(q, g, k, v, ck, cv, Tq, q_start, Tkv, kv_start, Nc, H, D, block, window,
                      scale, nullptr, nullptr, 0, out, out_dtype, lse, stream,
                      "hca_attn_prefill_lse launch");
}

hca_status_t hca_attn_prefill_vha(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                  int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                  int block, int window, float scale, const void* vha_up,
                                  const void* vha_down, int vha_rank, void* out,
                                  hca_dtype_t out_dtype, void* stream) {
  if (vha_rank == 0) return fail(HCA_ERR_UNSUPPORTED, "VHA rank 0 (use hca_attn_prefill)");
  return prefill_impl(q, g, k, v, ck, cv, Tq, q_start, Tkv, kv_start, Nc, H, D, block, window,
                      scale, vha_up, vha_down, vha_rank, out, out_dtype, nullptr, stream,
                      "hca_attn_prefill_vha launch");
}

size_t hca_decode_workspace_size(int B, int H, int D, int64_t nc_cap) {
  if (B <= 0 || H < 1 || H > 64 || D != hca::kD || nc_cap < 0) return 0;
  return hca::decode_workspace_bytes(B, H, nc_cap);
}

// decode.hip's kernels take whole head blocks of 16 and address a sequence's
// entries through one buffer descriptor, whose 32-bit size holds fewer than 2^21
// entries of 1 KiB; decode_sk.hip's (per-tile descriptors) take the rest.
static bool whole_tile_kernel(int H, int64_t nc_cap) {
  return H % 16 == 0 && nc_cap < ((int64_t)1 << 21);
}

// Checks shared by the decode entry points; fills p.
static hca_status_t decode_check(const void* q, const void* g, const void* ck, const void* cv,
                                 int64_t nc_cap, const void* wk, const void* wv,
                                 const int64_t* pos, int B, int M, int H, int D, int block,
                                 int window, float scale, void* out, hca_dtype_t out_dtype,
                                 hca::DecodeProblem& p) {
  TRY(check_shape(D, block, window));
  if (B < 0) return fail(HCA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (M < 1 || M > 16) return fail(HCA_ERR_UNSUPPORTED, "M = %d (need 1 .. 16)", M);
  if (H < 1 || H > 64) return fail(HCA_ERR_UNSUPPORTED, "H = %d (need 1 <= H <= 64)", H);
  if (nc_cap < 0) return fail(HCA_ERR_INVALID_ARG, "nc_cap = %lld < 0", (long long)nc_cap);
  if (nc_cap > (int64_t)1 << 24)
    return fail(HCA_ERR_UNSUPPORTED, "nc_cap = %lld (at most 2^24 entries per sequence)",
                (long long)nc_cap);
  if (out_dtype != HCA_BF16 && out_dtype != HCA_F32)
    return fail(HCA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
  TRY(check_scale(scale));
  if (B == 0) return HCA_OK;
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
  return HCA_OK;
}

hca_status_t hca_attn_decode(const void* q, const void* g, const void* ck, const void* cv,
                             int64_t nc_cap, const void* wk, const void* wv, const int64_t* pos,
                             int B, int H, int D, int block, int window, float scale, void* out,
                             hca_dtype_t out_dtype, void* workspace, size_t ws_bytes,
                             void* stream) {
  hca::DecodeProblem p;
  TRY(decode_check(q, g, ck, cv, nc_cap, wk, wv, pos, B, 1, H, D, block, window, scale, out,
                   out_dtype, p));
  if (B == 0) return ok();
  const size_t need = hca::decode_workspace_bytes(B, H, nc_cap);
  if (need == 0 && whole_tile_kernel(H, nc_cap))
    // A batch that fills the GPU with one workgroup per 16 heads: the kernel
    // whose four waves walk each tile together (decode.hip) streams the keys
    // faster there.
    return hip_status(hca::launch_decode(p, static_cast<hipStream_t>(stream)),
                      "hca_attn_decode launch");
  if (need > 0) {
    if (workspace == nullptr || ws_bytes < need)
      return fail(HCA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (%s)",
                  workspace ? ws_bytes : (size_t)0, need, "hca_decode_workspace_size");
    if (!aligned16(workspace))
      return fail(HCA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  }
  return hip_status(hca::launch_decode_sk(p, nullptr, nullptr, 1, workspace,
                                          static_cast<hipStream_t>(stream)),
                    "hca_attn_decode launch");
}

hca_status_t hca_attn_decode_noalloc(const void* q, const void* g, const void* ck, const void* cv,
                                     int64_t nc_cap, const void* wk, const void* wv,
                                     const int64_t* pos, int B, int H, int D, int block,
                                     int window, float scale, void* out, hca_dtype_t out_dtype,
                                     void* stream) {
  hca::DecodeProblem p;
  TRY(decode_check(q, g, ck, cv, nc_cap, wk, wv, pos, B, 1, H, D, block, window, scale, out,
                   out_dtype, p));
  if (B == 0) return ok();
  const size_t need = hca::decode_workspace_bytes(B, H, nc_cap);
  if (need > hca::kDecodeWorkspaceMax)
    return fail(HCA_ERR_WORKSPACE, "needs %zu bytes of workspace, the built-in scratch holds %zu",
                need, hca::kDecodeWorkspaceMax);
  if (need == 0 && whole_tile_kernel(H, nc_cap))
    return hip_status(hca::launch_decode(p, static_cast<hipStream_t>(stream)),
                      "hca_attn_decode_noalloc launch");
  void* ws = nullptr;
  if (need > 0) TRY(scratch_address(&ws));
  return hip_status(hca::launch_decode_sk(p, nullptr, nullptr, 1, ws,
                                          static_cast<hipStream_t>(stream)),
                    "hca_attn_decode_noalloc launch");
}

hca_status_t hca_gate_logits(const void* latent, const void* w_g, int64_t T, int R, int N,
                             void* g, void* stream) {
  if (T < 0) return fail(HCA_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
  if (R < 64 || R > 16384 || R % 64 != 0)
    return fail(HCA_ERR_UNSUPPORTED, "R = %d (need a multiple of 64, 64 .. 16384)", R);
  if (N < 2048 || N > 65536 || N % 2048 != 0)
    return fail(HCA_ERR_UNSUPPORTED, "N = %d (need a multiple of 2048, at most 65536)", N);
  if (T > ((int64_t)1 << 40)) return fail(HCA_ERR_UNSUPPORTED, "T beyond 2^40");
  if (T == 0) return ok();
  TRY(check_ptr(latent, "latent"));
  TRY(check_ptr(w_g, "w_g"));
  TRY(check_ptr(g, "g"));
  return hip_status(hca::launch_gate(static_cast<const uint16_t*>(latent),
                                     static_cast<const uint16_t*>(w_g), static_cast<uint16_t*>(g),
                                     T, R, N, static_cast<hipStream_t>(stream)),
                    "hca_gate_logits launch");
}

hca_status_t hca_attn_decode_multi(const void* q, const void* g, const void* ck, const void* cv,
                                   int64_t nc_cap, const void* wk, const void* wv,
                                   const void* nk, const void* nv, const int64_t* pos, int B,
                                   int M, int H, int D, int block, int window, float scale,
                                   void* out, hca_dtype_t out_dtype, void* stream) {
  hca::DecodeProblem p;
  TRY(decode_check(q, g, ck, cv, nc_cap, wk, wv, pos, B, M, H, D, block, window, scale, out,
                   out_dtype, p));
  if (B == 0) return ok();
  TRY(check_ptr(nk, "nk"));
  TRY(check_ptr(nv, "nv"));
  if (whole_tile_kernel(H, nc_cap))
    // Head blocks of 16 rows: the kernel that gives one workgroup up to 4 blocks
    // of a sequence (decode.hip) reads each sequence's keys into fewer CUs.
    return hip_status(hca::launch_decode_multi(p, static_cast<const uint16_t*>(nk),
                                               static_cast<const uint16_t*>(nv), M,
                                               static_cast<hipStream_t>(stream)),
                      "hca_attn_decode_multi launch");
  return hip_status(hca::launch_decode_sk(p, static_cast<const uint16_t*>(nk),
                                          static_cast<const uint16_t*>(nv), M, nullptr,
                                          static_cast<hipStream_t>(stream)),
                    "hca_attn_decode_multi launch");
}

size_t hca_backward_workspace_size(int64_t T, int H, int D) {
  if (T <= 0 || H < 1 || H > 64 || D != hca::kD || T * H > kMaxRows) return 0;
  return hca::backward_workspace_bytes(T, H);
}

static hca_status_t backward_impl(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, const void* out,
                                  hca_dtype_t out_dtype, const float* lse, const void* dout,
                                  int64_t T, int H, int D, int block, int window, float scale,
                                  void* dq, void* dk, void* dv, void* dg, void* workspace,
                                  size_t ws_bytes, void* stream, bool saved, const char* what) {
  TRY(check_shape(D, block, window));
  if (T < 0) return fail(HCA_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
  if (H < 1 || H > 64) return fail(HCA_ERR_UNSUPPORTED, "H = %d (need 1 <= H <= 64)", H);
  if (T * H > kMaxRows)
    return fail(HCA_ERR_UNSUPPORTED, "T * H = %lld query rows (at most 2^31 - 1)",
                (long long)(T * H));
  TRY(check_scale(scale));
  if (saved && out_dtype != HCA_BF16 && out_dtype != HCA_F32)
    return fail(HCA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
  if (T == 0) return ok();
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(g, "g"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(dout, "dout"));
  if (saved) {
    TRY(check_ptr(out, "out"));
    TRY(check_ptr(lse, "lse"));
  }
  TRY(check_ptr(dq, "dq"));
  TRY(check_ptr(dk, "dk"));
  TRY(check_ptr(dv, "dv"));
  TRY(check_ptr(dg, "dg"));
  if (T >= hca::kBlock) {
    TRY(check_ptr(ck, "ck"));
    TRY(check_ptr(cv, "cv"));
  }
  const size_t need = hca::backward_workspace_bytes(T, H);
  if (workspace == nullptr || ws_bytes < need)
    return fail(HCA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
  TRY(check_ptr(workspace, "workspace"));
  hca::BackwardProblem p;
  p.q = static_cast<const uint16_t*>(q);
  p.g = static_cast<const uint16_t*>(g);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.ck = static_cast<const uint16_t*>(ck);
  p.cv = static_cast<const uint16_t*>(cv);
  p.dout = static_cast<const uint16_t*>(dout);
  p.dq = static_cast<float*>(dq);
  p.dk = static_cast<float*>(dk);
  p.dv = static_cast<float*>(dv);
  p.dg = static_cast<float*>(dg);
  p.T = T;
  p.H = H;
  p.scale = scale;
  if (saved) {
    p.out = out;
    p.lse = lse;
    p.out_f32 = out_dtype == HCA_F32;
  }
  return hip_status(hca::launch_backward(p, workspace, static_cast<hipStream_t>(stream)), what);
}

hca_status_t hca_attn_backward(const void* q, const void* g, const void* k, const void* v,
                               const void* ck, const void* cv, const void* dout, int64_t T, int H,
                               int D, int block, int window, float scale, void* dq, void* dk,
                               void* dv, void* dg, void* workspace, size_t ws_bytes,
                               void* stream) {
  return backward_impl(q, g, k, v, ck, cv, nullptr, HCA_BF16, nullptr, dout, T, H, D, block,
                       window, scale, dq, dk, dv, dg, workspace, ws_bytes, stream, false,
                       "hca_attn_backward launch");
}

hca_status_t hca_attn_backward_saved(const void* q, const void* g, const void* k, const void* v,
                                     const void* ck, const void* cv, const void* out,
                                     hca_dtype_t out_dtype, const float* lse, const void* dout,
                                     int64_t T, int H, int D, int block, int window, float scale,
                                     void* dq, void* dk, void* dv, void* dg, void* workspace,
                                     size_t ws_bytes, void* stream) {
  return backward_impl(q, g, k, v, ck, cv, out, out_dtype, lse, dout, T, H, D, block, window,
                       scale, dq, dk, dv, dg, workspace, ws_bytes, stream, true,
                       "hca_attn_backward_saved launch");
}

}  // extern "C"
