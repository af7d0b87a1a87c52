/*
 * hca.h - C ABI of the HCA (Heavily Compressed Attention) library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  In 37 of the 43 layers of the model these pages describe,
 * attention reads two kinds of keys (aitest123.com, "ERNIE-5.5-Flash-Base开源：
 * 280B总参数，激活仅14B", section 模型结构; yilup.net, section 架構設計：稀疏 MoE
 * 與混合注意力機制; blog.derekhsu.net, section 潛在閘控稀疏注意力):
 *   (a) one cached entry per completed block of 128 tokens, and
 *   (b) the most recent 128 raw tokens (lininn.cn, "2800 亿参数的模型，每次只叫醒
 *       140 亿", section 43 层里，37 层只读摘要).
 * Heads are 512 wide and there are 64 query heads (blog.derekhsu.net,
 * section 潛在閘控稀疏注意力, the head-width paragraph; knowflowhub.com, table
 * 关键信息).  The attention output is multiplied elementwise by a learned
 * sigmoid gate (blog.derekhsu.net, section 低秩閘控注意力).
 *
 * Choices this library makes where the pages are silent:
 *   - entry b = arithmetic mean of the block's 128 K rows (and of its 128 V
 *     rows), rounded to bfloat16;
 *   - one K/V head shared by every query head;
 *   - entry b is visible to the query at position t iff 128*b + 127 <= t;
 *   - the window is positions max(0, t-127) .. t, inclusive;
 *   - one softmax over entries and window together, scores scale*<q,k>;
 *   - out[t,h,:] = attn[t,h,:] * sigmoid(G[t,h,:]) with G supplied.
 *
 * Conventions.
 *   - bf16 = IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *   - All tensors are dense, row major, with the innermost dimension listed
 *     last; device pointers must be 16-byte aligned.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronizes; all work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) and returns before it completes.
 *   - Inputs are read only; outputs are fully overwritten.
 *   - Argument checking happens on the host before any HIP call; a rejected
 *     call returns a non-zero status and enqueues nothing.  A launch failure
 *     returns HCA_ERR_HIP.  Faults during execution surface at the caller's
 *     next synchronization, as usual in HIP.
 *   - hca_last_error() gives a human-readable reason for the last non-OK
 *     status returned on the calling thread.
 *   - Supported shapes: D = 512, block = 128, window = 128, 1 <= H <= 64.
 */
#ifndef HCA_H
#define HCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HCA_OK = 0,
  HCA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, inconsistent ranges */
  HCA_ERR_UNSUPPORTED = 2, /* a shape the library has no kernel for (D, block, window, H) */
  HCA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  HCA_ERR_HIP = 4          /* the HIP runtime refused a launch */
} hca_status_t;

typedef enum { HCA_BF16 = 0, HCA_F32 = 1 } hca_dtype_t;

/* Static description of a status code. */
const char* hca_status_string(hca_status_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* hca_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int hca_version(void);

/*
 * Block compression (the cache entry of each completed block).
 *   k, v     device, bf16 [T, ld]: rows 0..T-1, the first D columns are used (ld >= D)
 *   ck, cv   device, bf16 [floor(T/block), D]: ck[b][d] = bf16(mean_{i<block} k[b*block+i][d]),
 *            likewise cv from v.  The sum is formed exactly (in binary64, in row
 *            order) and rounded once to nearest-even bfloat16.  A trailing partial
 *            block produces no entry.
 *   T >= 0.  Either of (k, ck) or (v, cv) may be NULL to compress only the other.
 *   T < block is a no-op (no pointer is checked).
 * For decode the caller compresses its 128-slot ring (T = 128) whenever a block
 * completes and appends the entry before the next decode call.
 */
hca_status_t hca_compress(const void* k, const void* v, int64_t T, int64_t ld, int D, int block,
                          void* ck, void* cv, void* stream);

/*
 * Prefill attention for Tq consecutive queries at positions q_start .. q_start+Tq-1.
 *   q, g     device, bf16 [Tq, H, D]     queries and pre-sigmoid gate logits
 *   k, v     device, bf16 [Tkv, D]       raw rows of positions kv_start .. kv_start+Tkv-1
 *   ck, cv   device, bf16 [Nc, D]        entries of blocks 0 .. Nc-1 (may be NULL if Nc = 0)
 *   out      device, [Tq, H, D]          bf16 (rounded to nearest-even) or f32
 *   scale    score scale (1/sqrt(512) for the model's layer)
 * Query at position t attends to entries b < Nc with 128*b+127 <= t and to the raw
 * rows of positions max(0, t-127) .. t.
 * Requirements when Tq > 0 (else HCA_ERR_INVALID_ARG):
 *   Tq, Tkv, Nc, q_start, kv_start >= 0 and scale finite and > 0;
 *   kv_start <= max(0, q_start-127)       (the first query's window is present);
 *   kv_start + Tkv >= q_start + Tq        (the last query's own row is present);
 *   Nc >= floor((q_start+Tq)/128)         (every entry a query can see is present;
 *                                          entries past that are never read).
 * Positions, Tq*H and Nc must stay below 2^31 (else HCA_ERR_UNSUPPORTED).
 * K and V must be finite: a key hidden from one row but visible to another row
 * of the same tile is multiplied by a zero weight.  Tq = 0 is a no-op.
 */
hca_status_t hca_attn_prefill(const void* q, const void* g, const void* k, const void* v,
                              const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                              int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D, int block,
                              int window, float scale, void* out, hca_dtype_t out_dtype,
                              void* stream);

/*
 * Prefill attention that also keeps, for the training pass, each query row's
 * log-sum-exp of its scores (the state hca_attn_backward_saved takes):
 *   lse[t, h] = ln sum_j exp(scale <q[t, h], key_j>)   over the keys row (t, h) sees,
 * as the kernel forms it: the weights exp(x_j - m) rounded to bfloat16 (the ones
 * the value product uses) summed in fp32, then m + ln(sum); so lse is within
 * ln(1 + 2^-8) of the exact value.
 *   lse    device, f32 [Tq, H] (overwritten); not NULL when Tq > 0 (else
 *          HCA_ERR_INVALID_ARG)
 * Other arguments, requirements and the output out exactly as hca_attn_prefill
 * (out is bitwise the same as hca_attn_prefill's).
 */
hca_status_t hca_attn_prefill_lse(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                  int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                  int block, int window, float scale, void* out,
                                  hca_dtype_t out_dtype, float* lse, void* stream);

/*
 * Prefill attention followed by the VHA head mix (virtual head attention:
 * blog.derekhsu.net, section 潛在閘控稀疏注意力, the VHA item: after attention a
 * light low-rank mix across heads with an identity skip, fused into the attention
 * kernel at inference).  With x[t, h, :] the gated output of hca_attn_prefill,
 *   out[t, h, :] = x[t, h, :] + sum_k up[h, k] * sum_h' down[k, h'] * x[t, h', :]
 * i.e. out = (I + up @ down) x over the heads of each query, the same for every dim.
 *   vha_up    device, bf16 [H, vha_rank]
 *   vha_down  device, bf16 [vha_rank, H]
 * Other arguments and requirements as for hca_attn_prefill, and: H = 64, vha_rank a
 * multiple of 4 from 4 to 32 (else HCA_ERR_UNSUPPORTED).  In the kernel the mix
 * takes x rounded to bf16, and sum_h' down x rounded to bf16, as its operands,
 * with fp32 accumulation and the identity term kept in fp32.
 */
hca_status_t hca_attn_prefill_vha(const void* q, const void* g, const void* k, const void* v,
                                  const void* ck, const void* cv, int64_t Tq, int64_t q_start,
                                  int64_t Tkv, int64_t kv_start, int64_t Nc, int H, int D,
                                  int block, int window, float scale, const void* vha_up,
                                  const void* vha_down, int vha_rank, void* out,
                                  hca_dtype_t out_dtype, void* stream);

/*
 * Bytes of device workspace hca_attn_decode needs for B sequences of H query heads
 * with nc_cap cached entries each (0: none).  Batches too small to fill the GPU
 * with one workgroup per 16 query heads split each sequence's keys across
 * workgroups (split-K); their partial softmax states (row maximum, row sum and
 * unnormalised output, fp32) go through the workspace and a second kernel merges
 * them.  Returns 0 for an unsupported shape (hca_attn_decode then reports it).
 */
size_t hca_decode_workspace_size(int B, int H, int D, int64_t nc_cap);

/*
 * Decode attention: one new query per sequence, for B sequences at once.
 *   q, g       device, bf16 [B, H, D]          the new token's queries and gate logits
 *   ck, cv     device, bf16 [B, nc_cap, D]     per-sequence entries (only the first
 *                                              floor((pos+1)/128) are read); may be NULL
 *                                              if nc_cap = 0
 *   wk, wv     device, bf16 [B, window, D]     per-sequence ring of raw rows; position p
 *                                              lives in slot p % window, and slots of
 *                                              positions max(0,pos-127)..pos must be valid
 *   pos        device, int64 [B]               position of the new token (already written
 *                                              into its ring slot)
 *   out        device, [B, H, D]               bf16 or f32
 *   workspace  device, at least hca_decode_workspace_size(B, H, D, nc_cap) bytes,
 *              16-byte aligned, owned by the caller; may be NULL when that size is 0
 *              (else HCA_ERR_WORKSPACE).  Its contents on entry do not matter and are
 *              undefined afterwards; calls that share a workspace must not overlap.
 * Supported: 1 <= H <= 64, nc_cap <= 2^24.
 * Entry counts come from device memory, so the host cannot check them: a pos with
 * floor((pos+1)/128) > nc_cap or pos < 0 is clamped on the device (never read out
 * of bounds) and its output is then unspecified.
 * B = 0 is a no-op.
 */
hca_status_t hca_attn_decode(const void* q, const void* g, const void* ck, const void* cv,
                             int64_t nc_cap, const void* wk, const void* wv, const int64_t* pos,
                             int B, int H, int D, int block, int window, float scale, void* out,
                             hca_dtype_t out_dtype, void* workspace, size_t ws_bytes,
                             void* stream);

/*
 * hca_attn_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, which comes from a scratch array built into the
 * library instead, one per GPU (8,421,376 bytes: the largest workspace
 * hca_decode_workspace_size returns), held until the process ends.  The call
 * allocates and frees nothing; a shape needing more scratch than that returns
 * HCA_ERR_WORKSPACE.  Every call on a GPU shares that GPU's scratch, so calls that
 * overlap on one GPU (concurrent streams, other threads) race and must be
 * serialised by the caller.  The first call on each device looks up the scratch's
 * device address (hipGetSymbolAddress); the stream must belong to the current device.
 */
hca_status_t hca_attn_decode_noalloc(const void* q, const void* g, const void* ck, const void* cv,
                                     int64_t nc_cap, const void* wk, const void* wv,
                                     const int64_t* pos, int B, int H, int D, int block,
                                     int window, float scale, void* out, hca_dtype_t out_dtype,
                                     void* stream);

/*
 * Multi-token decode: M new tokens per sequence at positions pos .. pos+M-1, for B
 * sequences at once, as when the tokens of a drafter are verified in one pass (the
 * ECHO layer doubles as a speculative-decoding drafter: blog.derekhsu.net, section
 * "ECHO：取代 MTP 模組"; two-step drafts in low-latency serving: lininn.cn, section
 * "把 MTP 模块删了").  Each new token is an ordinary query at its own position
 * (the prefill rule), so it sees the earlier new tokens but not the later ones.
 *   q, g     device, bf16 [B, M, H, D]       queries and gate logits of the new tokens
 *   ck, cv   device, bf16 [B, nc_cap, D]     per-sequence entries (only the first
 *                                            floor((pos+M)/128) are read: a block
 *                                            completed by a new token must already
 *                                            have its entry)
 *   wk, wv   device, bf16 [B, window, D]     ring of committed raw rows; position p lives
 *                                            in slot p % window, and slots of positions
 *                                            max(0,pos-127)..pos-1 must be valid
 *   nk, nv   device, bf16 [B, M, D]          raw rows of the new tokens
 *   pos      device, int64 [B]               position of the first new token
 *   out      device, [B, M, H, D]            bf16 or f32
 * 1 <= M <= 16 and 1 <= H <= 64 (else HCA_ERR_UNSUPPORTED).  With M = 1 this is
 * hca_attn_decode with the new row passed in nk, nv instead of its ring slot.  No
 * workspace: the M * H query rows of a batch fill the GPU without a key split.
 * As for hca_attn_decode, a pos with floor((pos+M)/128) > nc_cap or pos < 0 is
 * clamped on the device and its output is then unspecified.  B = 0 is a no-op.
 */
hca_status_t hca_attn_decode_multi(const void* q, const void* g, const void* ck, const void* cv,
                                   int64_t nc_cap, const void* wk, const void* wv,
                                   const void* nk, const void* nv, const int64_t* pos, int B,
                                   int M, int H, int D, int block, int window, float scale,
                                   void* out, hca_dtype_t out_dtype, void* stream);

/*
 * Gate logits of the low-rank gate (blog.derekhsu.net, section 潛在閘控稀疏注意力, the
 * 低秩閘控注意力 item: the gate comes from the query's low-rank latent, several times
 * narrower than the hidden state; yilup.net, section 架構設計):
 *   g[t, n] = sum_r latent[t, r] * w_g[n, r]      (g = latent w_g^T)
 * accumulated in fp32 and rounded to nearest-even bf16.  With n = h * D + d, g is the
 * [T, H, D] gate-logit tensor hca_attn_prefill takes, so the low-rank gated prefill is
 * this call followed by hca_attn_prefill on g.
 *   latent  device, bf16 [T, R]
 *   w_g     device, bf16 [N, R]    (out x in, like a linear layer's weight)
 *   g       device, bf16 [T, N]    (overwritten)
 * R a multiple of 64 from 64 to 16384, N a multiple of 2048 up to 65536 (H * 512 with
 * H a multiple of 4), else HCA_ERR_UNSUPPORTED.  T = 0 is a no-op.
 */
hca_status_t hca_gate_logits(const void* latent, const void* w_g, int64_t T, int R, int N,
                             void* g, void* stream);

/*
 * Bytes of device workspace hca_attn_backward needs for T positions and H query heads:
 * per query row its log-sum-exp and <dA, A> (fp32) and dA = dout * sigmoid(g) (bf16),
 * plus the fp32 gradients of the floor(T/128) entries.  0 for T <= 0 or an unsupported
 * shape.
 */
size_t hca_backward_workspace_size(int64_t T, int H, int D);

/*
 * Backward pass of a whole-sequence prefill (the training pass; the pages measure
 * the attention kernel on both passes: blog.derekhsu.net, section 訓練基礎設施):
 * queries and raw rows at positions 0 .. T-1, entries ck, cv of the Nc = floor(T/128)
 * completed blocks as hca_compress writes them, output o = softmax-attention(q) *
 * sigmoid(g) as hca_attn_prefill computes it (q_start = kv_start = 0).  For the
 * upstream gradient dout = dL/do:
 *   dg = dout * a * s * (1 - s),   a = ungated attention output, s = sigmoid(g)
 *   dq = scale * sum_j p_j (<da, v_j> - <da, a>) k_j,   da = dout * s
 *   dk[j], dv[j]: the same terms gathered per key; an entry's gradient is then
 *   added to each raw row of its block divided by 128 (the derivative of the mean;
 *   the bf16 rounding of the entry is passed through as the identity).
 *   q, g, dout  device, bf16 [T, H, D]
 *   k, v        device, bf16 [T, D]
 *   ck, cv      device, bf16 [floor(T/128), D] (may be NULL if T < 128)
 *   dq, dg      device, f32 [T, H, D]   (overwritten)
 *   dk, dv      device, f32 [T, D]      (overwritten)
 *   workspace   device, at least hca_backward_workspace_size(T, H, D) bytes, owned by
 *               the caller (else HCA_ERR_WORKSPACE); contents on entry do not matter.
 * 1 <= H <= 64 and T * H < 2^31 (else HCA_ERR_UNSUPPORTED).  The kernels recompute
 * the forward's softmax with its rounding (weights rounded to bf16 for the value
 * product); products take bf16 operands (weights, dA and the score gradients rounded
 * to nearest even) with fp32 accumulation.  Entry gradients are summed with fp32
 * atomics, so dk and dv are not bitwise reproducible from run to run.  T = 0 is a no-op.
 */
hca_status_t hca_attn_backward(const void* q, const void* g, const void* k, const void* v,
                               const void* ck, const void* cv, const void* dout, int64_t T, int H,
                               int D, int block, int window, float scale, void* dq, void* dk,
                               void* dv, void* dg, void* workspace, size_t ws_bytes,
                               void* stream);

/*
 * The same backward pass from the forward's saved state, as training frameworks
 * run it: the forward's gated output out and row log-sum-exp lse (as
 * hca_attn_prefill_lse writes them) replace the recomputed forward, so the row
 * pass walks the keys once instead of twice.  For row (t, h):
 *   p_j = exp(scale <q, k_j> - lse[t, h]),   Dt = <dout, out>  (= <da, a>),
 *   dg = dout * out * (1 - s),   dq = scale * sum_j p_j (<da, v_j> - Dt) k_j,
 * dk, dv and the entries' share as for hca_attn_backward.  With the exact out and
 * lse these are the exact gradients; with a bf16 out, Dt carries its rounding
 * (relative 2^-9 per element), the usual trade of a saved-state backward.
 *   out       device, [T, H, D] bf16 or f32 (out_dtype)
 *   lse       device, f32 [T, H]
 * Other arguments, the workspace and the requirements as hca_attn_backward; out and
 * lse must not be NULL when T > 0 (else HCA_ERR_INVALID_ARG).
 */
hca_status_t hca_attn_backward_saved(const void* q, const void* g, const void* k, const void* v,
                                     const void* ck, const void* cv, const void* out,
                                     hca_dtype_t out_dtype, const float* lse, const void* dout,
                                     int64_t T, int H, int D, int block, int window, float scale,
                                     void* dq, void* dk, void* dv, void* dg, void* workspace,
                                     size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H */
