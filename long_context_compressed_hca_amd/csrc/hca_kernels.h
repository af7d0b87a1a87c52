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
  // Optional [Tq, H] fp32: each row's log-sum-exp ln sum_j exp(scale <q, k_j>).
  float* lse = nullptr;
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

// Split-K decode: keys split across the four waves of a workgroup and, for
// batches too small to fill the chip, across decode_splits() workgroups whose
// partial results go through a workspace of decode_workspace_bytes() bytes.
// nk == nullptr: one new token per sequence (its row in the ring slot).
// Otherwise M new tokens whose rows are in nk, nv [B, M, 512], q, g and out
// [B, M, H, 512], no split across workgroups and no workspace.
int decode_splits(int B, int H, int64_t nc_cap);
size_t decode_workspace_bytes(int B, int H, int64_t nc_cap);
// Largest workspace decode_workspace_bytes() returns: a split batch has at most
// 256 partials (B * head blocks * splits <= 256) of (32 + 16 * 512) floats.
constexpr size_t kDecodeWorkspaceMax = (size_t)256 * (32 + 16 * kD) * sizeof(float);
hipError_t launch_decode_sk(const DecodeProblem& p, const uint16_t* nk, const uint16_t* nv, int M,
                            void* ws, hipStream_t stream);

// Gate logits of the low-rank gate: g [T, N] = bf16(latent [T, R] * w [N, R]^T);
// R a multiple of 64, N a multiple of 2048.
hipError_t launch_gate(const uint16_t* latent, const uint16_t* w, uint16_t* g, int64_t T, int R,
                       int N, hipStream_t stream);

// Backward pass of a whole-sequence prefill (queries and raw rows at positions
// 0 .. T-1, Nc = floor(T / 128) entries): fp32 gradients of q, g, k, v for the
// upstream gradient dout of the gated output; an entry's gradient reaches the
// raw rows of its block divided by 128.  Workspace: backward_workspace_bytes().
struct BackwardProblem {
  const uint16_t *q, *g, *k, *v, *ck, *cv, *dout;  // q, g, dout [T, H, 512]; k, v [T, 512]
  float *dq, *dk, *dv, *dg;                         // dq, dg [T, H, 512]; dk, dv [T, 512]
  int64_t T;
  int H;
  float scale;
  // Optional saved state of the forward: its gated output [T, H, 512] (bf16, or
  // f32 if out_f32) and row log-sum-exp [T, H] (natural log).  Given, the row
  // statistics come from them instead of a recomputed forward.
  const void* out = nullptr;
  const float* lse = nullptr;
  bool out_f32 = false;
};
size_t backward_workspace_bytes(int64_t T, int H);
hipError_t launch_backward(const BackwardProblem& p, void* ws, hipStream_t stream);

}  // namespace hca
