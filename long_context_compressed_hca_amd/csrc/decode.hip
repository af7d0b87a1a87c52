// decode.hip - HCA decode attention on gfx950: one new query per sequence.
//
// For sequence b with its new token at position t (already written into its
// ring slot t % 128), the keys are the floor((t+1)/128) cached entries and the
// raw rows of positions max(0, t-127) .. t, read from the ring (aitest123.com,
// "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B", section 模型结构; lininn.cn,
// section 43 层里，37 层只读摘要).  The output is gated by sigmoid(G)
// (blog.derekhsu.net, section 低秩閘控注意力).
//
// Decomposition.  One workgroup per (sequence, 16 * NHB of its heads), NHB = 1
// or 2, chosen so that the batch fills the chip; the head groups of a sequence
// run on one XCD and share its K/V bytes in that XCD's L2.  The keys are walked
// in 16-key tiles: first the entries (the last entry tile masked past the last
// entry), then the window, so every tile comes from one buffer.  The four
// waves copy each tile into LDS together by DMA (four stages of K and of V).
// Each step runs three tiles at once:
//   scores  tile s+2: wave w computes the partial scores S^T[key][head] over
//           its dims 128w .. 128w+127 for every head (4 MFMA 16x16x32 per
//           16 heads, K from LDS, Q^T in VGPRs) and writes them to LDS;
//   softmax tile s+1: wave hb < NHB sums the four partial score tiles of head
//           block hb, masks, weighs, rounds to bf16 and writes P^T to LDS;
//   values  tile s: wave w adds O^T[dv][head] += V^T P^T for its 128 dims of
//           every head (8 MFMA 16x16x16 per 16 heads, V^T by LDS transpose
//           reads, P^T of every head block from LDS).
// The three parts of a step are independent, so their latencies overlap; one
// barrier per step publishes the partial scores and the weights.
//
// Softmax (as in prefill): scores in the exp2 domain; each head's reference m
// is the maximum of its first tile, and every key is weighed by 2^(x - m), so O
// is never rescaled.  If a score rises more than 2^64 above it, the sequence is
// run again with the exact maximum.  Memory bound: per sequence (nc + window)
// * 2 KiB of K/V plus 3 * H KiB of q, g and out.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kTile = 16;
constexpr int kKRow = 1024 + 16;  // LDS bytes between K rows (conflict-free b128 reads)
constexpr int kVRow = 1024 + 64;  // between V rows (conflict-free transpose reads)
constexpr int kKBytes = kTile * kKRow;
constexpr int kVBytes = kTile * kVRow;
constexpr float kHeadroom = 64.0f;

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

struct Args {
  const uint16_t* q;
  const uint16_t* g;
  const uint16_t* ck;
  const uint16_t* cv;
  const uint16_t* wk;
  const uint16_t* wv;
  const int64_t* pos;
  void* out;
  int64_t nc_cap;
  int B, H, n_hg;  // n_hg workgroups per sequence, 16 * NHB heads each
  float c;  // scale * log2(e)
  int out_f32;
};

// The keys of one sequence: n_et entry tiles (entries 0 .. nc-1), then the
// window tiles (positions lo .. t, ring slot = position % 128).
struct Keys {
  const uint16_t *ek, *ev, *wk, *wv;  // this sequence's entries and ring
  int nc, lo, nw, n_et, n_tiles;
};

// Tile j: entry or window tile, its first entry / window index, and its
// number of valid keys.  Wave-uniform.
struct TileRef {
  bool ent;
  int first, valid;
};
__device__ __forceinline__ TileRef tile_ref(const Keys& ks, int j) {
  TileRef r;
  r.ent = j < ks.n_et;
  r.first = kTile * (r.ent ? j : j - ks.n_et);
  const int v = (r.ent ? ks.nc : ks.nw) - r.first;
  r.valid = v < kTile ? v : kTile;
  return r;
}

// Copy rows 4w .. 4w+3 of tile j of one tensor (entries `ent`, ring `win`)
// into LDS rows `stride` bytes apart.  Entry rows past the last entry arrive as
// zeros (buffer range check); window rows past the last valid position repeat
// it (finite data under a zero weight, whatever the unused ring slots hold).
// Past the last tile the copies are still issued, through an empty buffer, so
// every step issues the same number of copies; they read no memory and write
// zeros into a stage no later step reads.
__device__ __forceinline__ void copy_rows(const Keys& ks, int j, const uint16_t* ent,
                                          const uint16_t* win, uint8_t* dst, int stride, int wave,
                                          int lane16) {
  asm volatile("" : "+s"(wave), "+s"(j));  // addresses computed here, not kept in registers
  const TileRef tr = tile_ref(ks, j);
  const int bytes = j < ks.n_tiles ? (tr.ent ? ks.nc : kWindow) * 1024 : 0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(tr.ent ? ent : win, bytes);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * wave + u;
    const int k = tr.first + r;
    const int row = tr.ent ? k : ((ks.lo + (k < ks.nw ? k : ks.nw - 1)) & (kWindow - 1));
    dma16_buf(rs, lane16 + row * 1024, (lds_void*)(dst + r * stride));
  }
}

// max / sum of x over lanes l and l ^ 16, and over l and l ^ 32.
__device__ __forceinline__ float xmax16(float x) {
  const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
__device__ __forceinline__ float xsum16(float x) {
  const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// s_waitcnt vmcnt(4n): at most n groups of 4 copies (one tensor's rows of one
// tile for this wave) still in flight.
__device__ __forceinline__ void wait_4_groups() { __builtin_amdgcn_s_waitcnt(0x4F70); }
__device__ __forceinline__ void wait_5_groups() { __builtin_amdgcn_s_waitcnt(0x4F74); }

// Partial scores of one tile over this wave's dims for one head block: lane
// (head l16, g4) gets keys 4g4 .. 4g4+3.  koff addresses K row l16, dims
// 128w + 8g4; fragment ss holds dims 128w + 32ss + 8g4 .. +7, like the Q
// fragments.
__device__ __forceinline__ void k_frags(const uint8_t* sK, int koff, bf16x8 (&kf)[4]) {
#pragma unroll
  for (int ss = 0; ss < 4; ++ss) kf[ss] = *reinterpret_cast<const bf16x8*>(sK + koff + 64 * ss);
}
__device__ __forceinline__ f32x4 partial_scores(const bf16x8 (&kf)[4], const bf16x8 (&qf)[4]) {
  f32x4 s0 = {}, s1 = {};
  s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qf[0], s0, 0, 0, 0);
  s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1], qf[1], s1, 0, 0, 0);
  s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2], qf[2], s0, 0, 0, 0);
  s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[3], qf[3], s1, 0, 0, 0);
  return s0 + s1;
}

// O^T block += V^T P^T.  Written as asm to keep the accumulator in AGPRs for
// the whole kernel (the compiler otherwise moves the accumulator registers
// between AGPRs and VGPRs at loop exits).  Hazards: the V^T and P^T operands
// come from LDS reads (the compiler inserts their lgkmcnt waits); the
// accumulators are zeroed by v_accvgpr_write long before the first MFMA and
// read back long after the last one.
__device__ __forceinline__ void pv_mfma(f32x4& acc, i16x4 v, i16x4 p) {
  asm("v_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}

template <int NHB>
__global__ void __launch_bounds__(256, 1) decode_kernel(Args a) {
  // Array sAi holds K stage i and V stage i+2 (mod 4): K(j) is in sA(j%4) and
  // V(j) in sA((j+2)%4).  Step s copies K(s+5) and V(s+3), both into
  // sA((s+1)%4), and reads K(s+2) and V(s), both in sA((s+2)%4); with the
  // arrays separate the compiler can tell every copy in flight from the reads
  // that follow.  Two buffers each of weights (P^T of every head block) and
  // of partial scores (every wave's, for every head block), the row sums and
  // the repeat flags.
  __shared__ __attribute__((aligned(256))) uint8_t sA0[kKBytes + kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sA1[kKBytes + kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sA2[kKBytes + kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sA3[kKBytes + kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sP0[NHB * 512];
  __shared__ __attribute__((aligned(256))) uint8_t sP1[NHB * 512];
  __shared__ __attribute__((aligned(256))) uint8_t sQ0[4 * NHB * 1024];
  __shared__ __attribute__((aligned(256))) uint8_t sQ1[4 * NHB * 1024];
  __shared__ float sL[16 * NHB];
  __shared__ int sFlag[4];

  // blockIdx -> (sequence, head group): XCD x = blockIdx % 8 takes sequences
  // x, x + 8, ... with all their head groups, which share K/V in its L2.
  const int L = blockIdx.x;
  const int k8 = L >> 3;
  const int hg = k8 % a.n_hg;
  const int b = (k8 / a.n_hg) * 8 + (L & 7);
  if (b >= a.B) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const bool owner = wave < NHB;  // this wave takes the softmax of head block `wave`

  // The position first: the copies wait for it.  The loads of the gate
  // logits follow; they overlap the first copies (the copies' waits below
  // cover them: loads complete in order).
  const int64_t t_raw = a.pos[b];
  const int64_t head0 = (int64_t)b * a.H + hg * 16 * NHB;
  // Gate logits of this lane's outputs: head 16hb + l16, dims 128w + 16db + 4g4 .. +3.
  const int64_t rowo = (head0 + l16) * kD + 128 * wave + 4 * g4;
  uint2 gw[NHB][8];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db)
      gw[hb][db] = *reinterpret_cast<const uint2*>(a.g + rowo + (int64_t)16 * hb * kD + 16 * db);
  // Q^T fragments (B operand of the partial scores): head 16hb + l16, dims
  // 128w + 32ss + 8g4 .. +7; loaded at the start of each pass (a value loaded
  // before the pass loop and used in it would make the compiler wait for every
  // load first).
  bf16x8 qf[NHB][4];
  const uint16_t* const qrow = a.q + (head0 + l16) * kD + 128 * wave + 8 * g4;

  // Positions below 2^31 (negative ones read as 0); wave-uniform.
  int64_t t64 = t_raw;
  t64 = t64 < 0 ? 0 : (t64 > 0x7FFFFFFF ? 0x7FFFFFFF : t64);
  const int t = __builtin_amdgcn_readfirstlane((int)t64);
  Keys ks;
  ks.nc = (int)(((int64_t)t + 1) / kBlock);
  if ((int64_t)ks.nc > a.nc_cap) ks.nc = (int)a.nc_cap;  // out-of-contract: never read past the cache
  ks.lo = t - (kWindow - 1) > 0 ? t - (kWindow - 1) : 0;
  ks.nw = t - ks.lo + 1;
  ks.n_et = (ks.nc + kTile - 1) / kTile;
  ks.n_tiles = ks.n_et + (ks.nw + kTile - 1) / kTile;
  ks.ek = a.ck + (int64_t)b * a.nc_cap * kD;
  ks.ev = a.cv + (int64_t)b * a.nc_cap * kD;
  ks.wk = a.wk + (int64_t)b * kWindow * kD;
  ks.wv = a.wv + (int64_t)b * kWindow * kD;
  const int n = ks.n_tiles;  // >= 1: the new token itself is always a key

  // Lane offsets: K fragment source (row l16, dims 128w + 8g4); V^T transpose
  // read source (key row 4g4 + l16/4, dims 128w + 4(l16&3)); the lane's slot
  // of a weight buffer (8 bytes) and of a partial-score buffer (16 bytes).
  const int koff = l16 * kKRow + 256 * wave + 16 * g4;
  const int voff = (4 * g4 + (l16 >> 2)) * kVRow + 256 * wave + 8 * (l16 & 3);
  const int lane8 = lane * 8, lane16 = lane * 16;

  // O^T blocks: o[hb][db] lane (head 16hb + l16, g4), reg r -> dim 128w + 16db + 4g4 + r
  f32x4 o[NHB][8];
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f;
  bool over = false, fixed_m = false;

  // This wave's partial scores of the tile whose K is in sK, for every head
  // block, into its slots of sQn.
  auto scores = [&](const uint8_t* sK, uint8_t* sQn) {
    bf16x8 kf[4];
    k_frags(sK, koff, kf);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      *reinterpret_cast<f32x4*>(sQn + (wave * NHB + hb) * 1024 + lane16) = partial_scores(kf, qf[hb]);
  };
  // The four waves' partial scores of head block `wave` from sQc.
  auto read_partials = [&](const uint8_t* sQc, f32x4 (&sp)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      sp[u] = *reinterpret_cast<const f32x4*>(sQc + (u * NHB + wave) * 1024 + lane16);
  };
  // Weights of tile j for head block `wave` (owner waves) from its four
  // partial score tiles: mask, reference, exp2, bf16, row sum; P^T fragment
  // stored at this wave's slot of sPn.  Past the last tile every key is masked
  // and nothing is added.
  auto weights = [&](int j, const f32x4 (&sp)[4], uint8_t* sPn) {
    f32x4 s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    const TileRef tr = tile_ref(ks, j);
    const int valid = j < n ? tr.valid : 0;
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = 4 * g4 + r < valid ? s[r] * a.c : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    if (j == 0 && !fixed_m) m = xmax32(xmax16(mt));  // the reference: max of the first tile
    mseen = fmaxf(mseen, mt);
    over |= mt > m + kHeadroom;
    const f32x4 e = {__builtin_amdgcn_exp2f(s[0] - m), __builtin_amdgcn_exp2f(s[1] - m),
                     __builtin_amdgcn_exp2f(s[2] - m), __builtin_amdgcn_exp2f(s[3] - m)};
    const bf16x4 pb = __builtin_convertvector(e, bf16x4);  // nearest even
    // l adds the rounded weights: dot products with ones.
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[0], pb[1]}, ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[2], pb[3]}, ones, l, false);
    *reinterpret_cast<i16x4*>(sPn + wave * 512 + lane8) = __builtin_bit_cast(i16x4, pb);
  };

  // Step s: K(s+2) and V(s) in sAr, the partial scores of tile s+1 in sQc, the
  // weights of tile s in sPc.  Adds the value product of tile s, writes the
  // weights of tile s+1 into sPn and the partial scores of tile s+2 into sQn,
  // and copies K(s+5) and V(s+3) into sAd.
  auto step = [&](int s, const uint8_t* sAr, const uint8_t* sQc, uint8_t* sQn, const uint8_t* sPc,
                  uint8_t* sPn, uint8_t* sAd) {
    int w = wave;
    asm volatile("" : "+s"(w), "+s"(s));  // per-step values computed here, not kept in registers
    // LDS reads first (a read issued after a copy would wait for it).
    bf16x8 kf[4];
    k_frags(sAr, koff, kf);
    f32x4 sp[4];
    if (owner) read_partials(sQc, sp);
    i16x4 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) pf[hb] = *reinterpret_cast<const i16x4*>(sPc + hb * 512 + lane8);
    i16x4 vf[8];
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vf[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sAr + kKBytes + voff + 32 * db));
    __builtin_amdgcn_sched_barrier(0);
    copy_rows(ks, s + 5, ks.ek, ks.wk, sAd, kKRow, w, lane16);
    copy_rows(ks, s + 3, ks.ev, ks.wv, sAd + kKBytes, kVRow, w, lane16);
    // scores of tile s+2
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      *reinterpret_cast<f32x4*>(sQn + (w * NHB + hb) * 1024 + lane16) = partial_scores(kf, qf[hb]);
    // weights of tile s+1 (its partial scores were read above)
    if (owner) weights(s + 1, sp, sPn);
    // values of tile s
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) pv_mfma(o[hb][db], vf[db], pf[hb]);
    // K(s+3) and V(s+1) are in for this wave (the copies issued after them,
    // by steps s-1 and s, may be in flight), the LDS writes done; then for
    // every wave.
    wait_4_groups();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_no_fence();
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) o[hb][db] = f32x4{};
    l = 0.0f;
    over = false;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
        qf[hb][ss] = *reinterpret_cast<const bf16x8*>(qrow + (int64_t)16 * hb * kD + 32 * ss);
    // Prologue.  Copies in the order of the steps that would issue them
    // (step c copies K(c+5), V(c+3)): K(0); K(1); K(2), V(0); K(3), V(1).
    copy_rows(ks, 0, ks.ek, ks.wk, sA0, kKRow, wave, lane16);
    copy_rows(ks, 1, ks.ek, ks.wk, sA1, kKRow, wave, lane16);
    copy_rows(ks, 2, ks.ek, ks.wk, sA2, kKRow, wave, lane16);
    copy_rows(ks, 0, ks.ev, ks.wv, sA2 + kKBytes, kVRow, wave, lane16);
    copy_rows(ks, 3, ks.ek, ks.wk, sA3, kKRow, wave, lane16);
    copy_rows(ks, 1, ks.ev, ks.wv, sA3 + kKBytes, kVRow, wave, lane16);
    wait_5_groups();  // K(0) in (and Q, G: loads complete in order)
    barrier_no_fence();
    scores(sA0, sQ0);
    wait_4_groups();  // K(1) in
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier_no_fence();  // partial scores of tile 0 written, K(0) read by every wave
    scores(sA1, sQ1);
    if (owner) {
      f32x4 sp[4];
      read_partials(sQ0, sp);
      weights(0, sp, sP0);
    }
    copy_rows(ks, 4, ks.ek, ks.wk, sA0, kKRow, wave, lane16);
    copy_rows(ks, 2, ks.ev, ks.wv, sA0 + kKBytes, kVRow, wave, lane16);
    wait_4_groups();  // K(2), V(0) in
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier_no_fence();
    // Whole groups of four steps, then the rest (nested, so the compiler
    // sees the same copies in flight on every path into a step).
    int s = 0;
    for (; s + 4 <= n; s += 4) {
      step(s, sA2, sQ1, sQ0, sP0, sP1, sA1);
      step(s + 1, sA3, sQ0, sQ1, sP1, sP0, sA2);
      step(s + 2, sA0, sQ1, sQ0, sP0, sP1, sA3);
      step(s + 3, sA1, sQ0, sQ1, sP1, sP0, sA0);
    }
    if (s < n) {
      step(s, sA2, sQ1, sQ0, sP0, sP1, sA1);
      if (s + 1 < n) {
        step(s + 1, sA3, sQ0, sQ1, sP1, sP0, sA2);
        if (s + 2 < n) step(s + 2, sA0, sQ1, sQ0, sP0, sP1, sA3);
      }
    }
    // Row sums and the repeat decision of every head block, through LDS.
    if (owner) {
      const float lh = xsum32(xsum16(l));
      if (lane < 16) sL[16 * wave + lane] = lh;
      const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
      if (lane == 0) sFlag[wave] = wover ? 1 : 0;
    } else if (lane == 0) {
      sFlag[wave] = 0;
    }
    __syncthreads();
    const bool redo = (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) != 0;
    // A score more than 2^kHeadroom above its reference (extreme score ranges
    // only): run again with the exact maximum of each head as reference.
    if (pass == 1 || !redo) break;
    m = xmax32(xmax16(mseen));
    fixed_m = true;
    __syncthreads();  // every wave has read the flags before they are rewritten
  }

  // out = O / l * sigmoid(G) for this wave's 128 dims of every head.
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float inv = 1.0f / sL[16 * hb + l16];
    const int64_t rowh = rowo + (int64_t)16 * hb * kD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint2 gv2 = gw[hb][db];
      const float gv[4] = {bf16_bits_to_f32(gv2.x & 0xFFFFu), bf16_bits_to_f32(gv2.x >> 16),
                           bf16_bits_to_f32(gv2.y & 0xFFFFu), bf16_bits_to_f32(gv2.y >> 16)};
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
        r[e] = o[hb][db][e] * inv * sig;
      }
      if (a.out_f32)
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + rowh + 16 * db) =
            make_float4(r[0], r[1], r[2], r[3]);
      else
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + rowh + 16 * db) =
            make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeProblem& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  Args a;
  a.q = p.q;
  a.g = p.g;
  a.ck = p.ck;
  a.cv = p.cv;
  a.wk = p.wk;
  a.wv = p.wv;
  a.pos = p.pos;
  a.out = p.out;
  a.nc_cap = p.nc_cap;
  a.B = p.B;
  a.H = p.H;
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  // Heads per workgroup: 32 when the batch still fills the chip with them,
  // else 16.
  const int nhb = (p.H % 32 == 0 && (int64_t)p.B * (p.H / 32) >= 256) ? 2 : 1;
  a.n_hg = p.H / 16 / nhb;
  const dim3 grid((unsigned)(((p.B + 7) / 8) * 8 * a.n_hg)), block(256);
  if (nhb == 2)
    hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
