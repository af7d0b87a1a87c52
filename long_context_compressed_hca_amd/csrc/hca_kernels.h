// hca_kernels.h - launchers of the HIP kernels, called by the C ABI layer after
// it has validated every argument.  All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace hca {

// Problem constants of the HCA layer: 512-wide heads, one entry per 128 tokens,
// a 128-token raw window.
constexpr int kD = 512;
constexpr int kBlock = 128;
constexpr int kWindow = 128;

// ck/cv[b] = bf16(mean of rows 128b .. 128b+127 of k/v); k/v rows have stride ld.
hipError_t launch_compress(const uint16_t* k, const uint16_t* v, int64_t T, int64_t ld,
                           uint16_t* ck, uint16_t* cv, hipStream_t stream);

struct PrefillProblem {
  const uint16_t* q;   // [Tq, H, 512]
  const uint16_t* g;   // [Tq, H, 512]
  const uint16_t* k;   // [Tkv, 512], positions kv_start ..
  const uint16_t* v;
  const uint16_t* ck;  // [Nc, 512]
  const uint16_t* cv;
  void* out;           // [Tq, H, 512], bf16 or f32
  int64_t Tq, q_start, Tkv, kv_start, Nc;
  int H;
  float scale;
  bool out_f32;
  // VHA head mix after the gate (vha_rank 0: none): up [H, rank], down [rank, H].
  const uint16_t* vha_up = nullptr;
  const uint16_t* vha_down = nullptr;
  int vha_rank = 0;
};
hipError_t launch_prefill(const PrefillProblem& p, hipStream_t stream);

struct DecodeProblem {
  const uint16_t* q;   // [B, H, 512]
  const uint16_t* g;
  const uint16_t* ck;  // [B, nc_cap, 512]
  const uint16_t* cv;
  const uint16_t* wk;  // [B, 128, 512] ring, slot = position % 128
  const uint16_t* wv;
  const int64_t* pos;  // [B]
  void* out;           // [B, H, 512]
  int64_t nc_cap;
  int B, H;
  float scale;
  bool out_f32;
};
hipError_t launch_decode(const DecodeProblem& p, hipStream_t stream);
// M new tokens per sequence: q, g, out [B, M, H, 512]; the ring holds positions
// below pos; nk, nv [B, M, 512] hold the new tokens' rows.
hipError_t launch_decode_multi(const DecodeProblem& p, const uint16_t* nk, const uint16_t* nv,
                               int M, hipStream_t stream);

}  // namespace hca
