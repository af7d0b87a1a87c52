// decode.hip - HCA decode attention on gfx950: one new query per sequence.
//
// For sequence b with its new token at position t (already written into its
// ring slot t % 128), the keys are the floor((t+1)/128) cached entries and the
// raw rows of positions max(0, t-127) .. t, read from the ring (aitest123.com,
// "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B", section 模型结构; lininn.cn,
// section 43 层里，37 层只读摘要).  The output is gated by sigmoid(G)
// (blog.derekhsu.net, section 低秩閘控注意力).
//
// Decomposition.  One workgroup per (sequence, 16 * NHB of its heads), NHB = 1,
// 2 or 4, chosen so that the batch fills the chip; the head groups of a sequence
// run on one XCD and share its K/V bytes in that XCD's L2.  The keys are walked
// in 16-key tiles: first the entries (the last entry tile masked past the last
// entry), then the window, so every tile comes from one buffer.  Each wave
// loads the K fragments of its dims straight into registers (a ring of six
// tiles); the four waves copy each V tile into LDS together by DMA (six
// stages).  Both run four or more steps ahead of their use.
// Each step runs three tiles at once:
//   scores  tile s+2: wave w computes the partial scores S^T[key][head] over
//           its dims 128w .. 128w+127 for every head (4 MFMA 16x16x32 per
//           16 heads, K and Q^T in VGPRs) and writes them to LDS;
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
constexpr int kVRow = 1024 + 64;  // between V rows (conflict-free transpose reads)
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
  int B, H, n_hg;  // H query rows per sequence; n_hg workgroups per sequence, 16 * NHB rows each
  float c;  // scale * log2(e)
  int out_f32;
  // Several new tokens per sequence (MT): rows of token j are j * hpt * 16 ..
  // (j+1) * hpt * 16 - 1; their keys and values are rows j of nk, nv [B, M, 512].
  const uint16_t* nk;
  const uint16_t* nv;
  int M, hpt;
};

// The keys of one sequence: n_et entry tiles (entries 0 .. nc-1), then the
// window tiles (positions lo .. lo+nw-1, ring slot = position % 128).  One new
// token: the window ends at its position t.  M new tokens (MT): the window ends
// at t-1 (n_rt ring tiles, possibly none), and one last tile holds the M new
// rows.
struct Keys {
  const uint16_t *ek, *ev, *wk, *wv;  // this sequence's entries and ring
  const uint16_t *nk, *nv;            // MT: this sequence's new rows
  int nc, lo, nw, n_et, n_tiles;
  int n_rt, M;                        // MT
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

// MT tile j: 0 entry, 1 ring, 2 new rows; its first index in that segment.
struct TileRefMT {
  int kind, first;
};
__device__ __forceinline__ TileRefMT tile_ref_mt(const Keys& ks, int j) {
  TileRefMT r;
  r.kind = j < ks.n_et ? 0 : (j < ks.n_et + ks.n_rt ? 1 : 2);
  r.first = kTile * (r.kind == 0 ? j : (r.kind == 1 ? j - ks.n_et : 0));
  return r;
}

// Tile j of one tensor: its buffer (bytes = 0 past the last tile: every load
// through it reads zeros and touches no memory) and the byte offset of key k of
// the tile.  Entry rows past the last entry and new rows past the last read as
// zeros (range check); ring rows past the last valid position repeat it (finite
// data under a zero weight, whatever the unused ring slots hold).
template <bool MT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Keys& ks, int j,
                                                            const uint16_t* ent,
                                                            const uint16_t* win,
                                                            const uint16_t* nrw) {
  if constexpr (!MT) {
    const TileRef tr = tile_ref(ks, j);
    const int bytes = j < ks.n_tiles ? (tr.ent ? ks.nc : kWindow) * 1024 : 0;
    return make_rsrc(tr.ent ? ent : win, bytes);
  } else {
    const TileRefMT tr = tile_ref_mt(ks, j);
    const int rows = tr.kind == 0 ? ks.nc : (tr.kind == 1 ? kWindow : ks.M);
    return make_rsrc(tr.kind == 0 ? ent : (tr.kind == 1 ? win : nrw),
                     j < ks.n_tiles ? rows * 1024 : 0);
  }
}
template <bool MT>
__device__ __forceinline__ int tile_row(const Keys& ks, int j, int k) {
  if constexpr (!MT) {
    const TileRef tr = tile_ref(ks, j);
    k += tr.first;
    return tr.ent ? k : ((ks.lo + (k < ks.nw ? k : ks.nw - 1)) & (kWindow - 1));
  } else {
    const TileRefMT tr = tile_ref_mt(ks, j);
    k += tr.first;
    return tr.kind != 1 ? k : ((ks.lo + (k < ks.nw ? k : ks.nw - 1)) & (kWindow - 1));
  }
}

// Copy rows 4w .. 4w+3 of tile j of one tensor (entries `ent`, ring `win`,
// new rows `nrw`) into LDS rows `stride` bytes apart.  Entry rows past the last entry arrive as
// zeros (buffer range check); window rows past the last valid position repeat
// it (finite data under a zero weight, whatever the unused ring slots hold).
// Past the last tile the copies are still issued, through an empty buffer, so
// every step issues the same number of copies; they read no memory and write
// zeros into a stage no later step reads.
template <bool MT>
__device__ __forceinline__ void copy_rows(const Keys& ks, int j, const uint16_t* ent,
                                          const uint16_t* win, const uint16_t* nrw, uint8_t* dst,
                                          int stride, int wave, int lane16) {
  asm volatile("" : "+s"(wave), "+s"(j));  // addresses computed here, not kept in registers
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc<MT>(ks, j, ent, win, nrw);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * wave + u;
    dma16_buf(rs, lane16 + tile_row<MT>(ks, j, r) * 1024, (lds_void*)(dst + r * stride));
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

// s_waitcnt vmcnt(8n): at most n steps' worth of this wave's loads (4 K
// fragment loads and 4 V row copies each) still in flight.
__device__ __forceinline__ void wait_4_steps() { __builtin_amdgcn_s_waitcnt(0x8F70); }  // vmcnt(32)

// K fragments of tile j for this wave's dims, loaded into registers: lane
// (key l16, g4) gets dims 128w + 32ss + 8g4 .. +7 of the tile's key l16
// (ss = 0..3).  Through a buffer descriptor: entry rows past the last entry,
// and every row of a tile past the last, read as zeros; window rows past the
// last valid position repeat it.
template <bool MT>
__device__ __forceinline__ void load_k(const Keys& ks, int j, int wave, int l16, int g4,
                                       bf16x8 (&kf)[4]) {
  asm volatile("" : "+s"(wave), "+s"(j));  // addresses computed here, not kept in registers
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc<MT>(ks, j, ks.ek, ks.wk, ks.nk);
  const int off = tile_row<MT>(ks, j, l16) * 1024 + 256 * wave + 16 * g4;
#pragma unroll
  for (int ss = 0; ss < 4; ++ss)
    kf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * ss, 0, 0));
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

// CW: four more waves (waves 4 .. 7) that only copy the V tiles, so the four
// compute waves issue only their K loads.  A wave issues its vector-memory
// instructions at a limited rate, so the step, whose copies and loads took
// about as long to issue as its arithmetic, gets shorter.  It needs the
// compute waves to fit two per SIMD (one head block, one token).
template <int NHB, bool MT, bool CW = false>
__global__ void __launch_bounds__(CW ? 512 : 256, 1) decode_kernel(Args a) {
  // Six V stages (V(j) in stage j % 6), two buffers each of weights (P^T of
  // every head block) and of partial scores (every wave's, for every head
  // block), the row sums and the repeat flags.  Separate arrays, so the
  // compiler can tell a copy into one stage from reads of another.
  __shared__ __attribute__((aligned(256))) uint8_t sV0[kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sV1[kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sV2[kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sV3[kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sV4[kVBytes];
  __shared__ __attribute__((aligned(256))) uint8_t sV5[kVBytes];
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
  const bool owner = NHB == 4 || wave < NHB;  // this wave takes the softmax of head block `wave`

  // The position first: the copies wait for it.  The loads of the gate
  // logits follow; they overlap the first copies.
  bf16x8 kr[6][4];  // K fragments in registers, tile j in slot j % 6
  auto prologue_loads = [&](const Keys& kk) {
    const int lane16 = lane * 16;
    load_k<MT>(kk, 0, wave, l16, g4, kr[0]);
    load_k<MT>(kk, 1, wave, l16, g4, kr[1]);
    if (!CW) copy_rows<MT>(kk, 0, kk.ev, kk.wv, kk.nv, sV0, kVRow, wave, lane16);
    load_k<MT>(kk, 2, wave, l16, g4, kr[2]);
    if (!CW) copy_rows<MT>(kk, 1, kk.ev, kk.wv, kk.nv, sV1, kVRow, wave, lane16);
    load_k<MT>(kk, 3, wave, l16, g4, kr[3]);
    if (!CW) copy_rows<MT>(kk, 2, kk.ev, kk.wv, kk.nv, sV2, kVRow, wave, lane16);
    load_k<MT>(kk, 4, wave, l16, g4, kr[4]);
    if (!CW) copy_rows<MT>(kk, 3, kk.ev, kk.wv, kk.nv, sV3, kVRow, wave, lane16);
    load_k<MT>(kk, 5, wave, l16, g4, kr[5]);
    if (!CW) copy_rows<MT>(kk, 4, kk.ev, kk.wv, kk.nv, sV4, kVRow, wave, lane16);
  };
  const int64_t t_raw = a.pos[b];
  const int64_t head0 = (int64_t)b * a.H + hg * 16 * NHB;
  // Gate logits of this lane's outputs: head 16hb + l16, dims 128w + 16db + 4g4 .. +3.
  const int64_t rowo = (head0 + l16) * kD + 128 * wave + 4 * g4;
  uint2 gw[NHB][8];
  if (!CW || wave < 4) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db)
        gw[hb][db] = *reinterpret_cast<const uint2*>(a.g + rowo + (int64_t)16 * hb * kD + 16 * db);
  }
  // Q^T fragments (B operand of the partial scores): head 16hb + l16, dims
  // 128w + 32ss + 8g4 .. +7; loaded at the start of each pass (a value loaded
  // before the pass loop and used in it would make the compiler wait for every
  // load first).
  bf16x8 qf[NHB][4];
  const uint16_t* const qrow = a.q + (head0 + l16) * kD + 128 * wave + 8 * g4;

  // Positions below 2^31 (below 2^31 - 16 for MT; negative ones read as 0);
  // wave-uniform.
  constexpr int64_t kTMax = MT ? 0x7FFFFFEF : 0x7FFFFFFF;
  int64_t t64 = t_raw;
  t64 = t64 < 0 ? 0 : (t64 > kTMax ? kTMax : t64);
  const int t = __builtin_amdgcn_readfirstlane((int)t64);
  Keys ks;
  ks.nc = (int)(((int64_t)t + (MT ? a.M : 1)) / kBlock);
  if ((int64_t)ks.nc > a.nc_cap) ks.nc = (int)a.nc_cap;  // out-of-contract: never read past the cache
  ks.lo = t - (kWindow - 1) > 0 ? t - (kWindow - 1) : 0;
  ks.nw = MT ? t - ks.lo : t - ks.lo + 1;
  ks.n_et = (ks.nc + kTile - 1) / kTile;
  ks.n_rt = (ks.nw + kTile - 1) / kTile;
  ks.n_tiles = ks.n_et + ks.n_rt + (MT ? 1 : 0);
  ks.M = a.M;
  ks.ek = a.ck + (int64_t)b * a.nc_cap * kD;
  ks.ev = a.cv + (int64_t)b * a.nc_cap * kD;
  ks.wk = a.wk + (int64_t)b * kWindow * kD;
  ks.wv = a.wv + (int64_t)b * kWindow * kD;
  ks.nk = MT ? a.nk + (int64_t)b * a.M * kD : nullptr;
  ks.nv = MT ? a.nv + (int64_t)b * a.M * kD : nullptr;
  const int n = ks.n_tiles;  // >= 1: the new token itself is always a key
  if constexpr (CW) {
    if (wave >= 4) {
      // Copy waves: V(j) into stage j % 6, rows 4 (wave - 4) .. +3, five tiles
      // ahead, meeting every barrier of the compute waves' passes (two before
      // the steps, one per step, two after).
      const int cw = wave - 4, lane16 = lane * 16;
      auto stage = [&](int j) -> uint8_t* {
        switch (j % 6) {
          case 0: return sV0;
          case 1: return sV1;
          case 2: return sV2;
          case 3: return sV3;
          case 4: return sV4;
          default: return sV5;
        }
      };
      for (int pass = 0;; ++pass) {
        for (int j = 0; j < 5; ++j) copy_rows<MT>(ks, j, ks.ev, ks.wv, ks.nv, stage(j), kVRow, cw, lane16);
        barrier_no_fence();  // the compute waves' partial scores of tiles 0, 1
        __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): V(0) is in (V(1) .. V(4) may be in flight)
        barrier_no_fence();
        for (int s = 0; s < n; ++s) {
          copy_rows<MT>(ks, s + 5, ks.ev, ks.wv, ks.nv, stage(s + 5), kVRow, cw, lane16);
          __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): V(s+1) is in
          barrier_no_fence();
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        const bool redo = (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) != 0;
        if (pass == 1 || !redo) return;
        __syncthreads();
      }
    }
  }
  // MT: the keys visible to the rows of head block `wave` (owner waves), whose
  // token j sits at position t + j: entries below ncj, ring rows from rlo on,
  // new rows up to j.
  int tok = 0, ncj = 0, rlo = 0;
  if constexpr (MT) {
    tok = (hg * NHB + wave) / a.hpt;
    tok = tok < a.M - 1 ? tok : a.M - 1;
    ncj = (t + tok + 1) / kBlock;
    ncj = ncj < ks.nc ? ncj : ks.nc;
    rlo = t + tok - (kWindow - 1) - ks.lo;
    rlo = rlo > 0 ? rlo : 0;
  }

  // Lane offsets: V^T transpose read source (key row 4g4 + l16/4, dims 128w +
  // 4(l16&3)); the lane's slot of a weight buffer (8 bytes) and of a
  // partial-score buffer (16 bytes).
  const int voff = (4 * g4 + (l16 >> 2)) * kVRow + 256 * wave + 8 * (l16 & 3);
  const int lane8 = lane * 8, lane16 = lane * 16;

  // O^T blocks: o[hb][db] lane (head 16hb + l16, g4), reg r -> dim 128w + 16db + 4g4 + r
  f32x4 o[NHB][8];
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f;
  bool over = false, fixed_m = false;

  // This wave's partial scores of a tile for every head block, from its K
  // fragments, into its slots of sQn.
  auto scores = [&](const bf16x8 (&kf)[4], uint8_t* sQn) {
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
    float mt = -INFINITY;
    float mx = m;  // exponent reference
    if constexpr (!MT) {
      const TileRef tr = tile_ref(ks, j);
      const int valid = j < n ? tr.valid : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = 4 * g4 + r < valid ? s[r] * a.c : -INFINITY;
        mt = fmaxf(mt, s[r]);
      }
      if (j == 0 && !fixed_m) m = xmax32(xmax16(mt));  // the reference: max of the first tile
      mx = m;
    } else {
      // Visible keys of the tile for this block's token: indexes lo_v .. hi_v-1.
      const TileRefMT tr = tile_ref_mt(ks, j);
      const int lo_v = tr.kind == 1 ? rlo - tr.first : 0;
      const int hi_v = j >= n ? 0 : (tr.kind == 0 ? ncj : (tr.kind == 1 ? ks.nw : tok + 1)) - tr.first;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 4 * g4 + r;
        s[r] = kk >= lo_v && kk < hi_v ? s[r] * a.c : -INFINITY;
        mt = fmaxf(mt, s[r]);
      }
      // The reference: the maximum of the first tile with a visible key (a
      // block's first tiles may hold none: entries of blocks completed by a
      // later new token, ring rows left of its window).
      if (!fixed_m && m == -INFINITY) m = xmax32(xmax16(mt));
      mx = m == -INFINITY ? 0.0f : m;  // nothing visible yet: every weight 0
    }
    mseen = fmaxf(mseen, mt);
    over |= mt > m + kHeadroom;
    const f32x4 e = {__builtin_amdgcn_exp2f(s[0] - mx), __builtin_amdgcn_exp2f(s[1] - mx),
                     __builtin_amdgcn_exp2f(s[2] - mx), __builtin_amdgcn_exp2f(s[3] - mx)};
    const bf16x4 pb = __builtin_convertvector(e, bf16x4);  // nearest even
    // l adds the rounded weights: dot products with ones.
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[0], pb[1]}, ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[2], pb[3]}, ones, l, false);
    *reinterpret_cast<i16x4*>(sPn + wave * 512 + lane8) = __builtin_bit_cast(i16x4, pb);
  };

  // Step s: K(s+2) in registers kc, V(s) in sVc, the partial scores of tile s+1
  // in sQc, the weights of tile s in sPc.  Writes the partial scores of tile
  // s+2 into sQn and the weights of tile s+1 into sPn, adds the value product
  // of tile s, and loads K(s+6) into kn (the slot of K(s)) and V(s+5) into sVd
  // (the stage of V(s-1)).
  auto step = [&](int s, const bf16x8 (&kc)[4], bf16x8 (&kn)[4], const uint8_t* sVc, uint8_t* sVd,
                  const uint8_t* sQc, uint8_t* sQn, const uint8_t* sPc, uint8_t* sPn) {
    int w = wave;
    asm volatile("" : "+s"(w), "+s"(s));  // per-step values computed here, not kept in registers
    // LDS reads first (a read issued after a copy would wait for it).
    f32x4 sp[4];
    if (owner) read_partials(sQc, sp);
    i16x4 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) pf[hb] = *reinterpret_cast<const i16x4*>(sPc + hb * 512 + lane8);
    i16x4 vf[8];
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vf[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sVc + voff + 32 * db));
    __builtin_amdgcn_sched_barrier(0);
    // The weights first: their chain (partial-score reads, exp2, the weight
    // write) ends the step for the owner waves, and issuing the copies takes
    // several hundred cycles.
    if (owner) weights(s + 1, sp, sPn);  // tile s+1
    scores(kc, sQn);  // tile s+2
    load_k<MT>(ks, s + 6, w, l16, g4, kn);
    if (!CW) copy_rows<MT>(ks, s + 5, ks.ev, ks.wv, ks.nv, sVd, kVRow, w, lane16);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) pv_mfma(o[hb][db], vf[db], pf[hb]);  // tile s
    // V(s+1) is in for this wave (the loads and copies of steps s-3 .. s may
    // be in flight; with copy waves, they wait for it), the LDS writes done;
    // then for every wave.
    if (!CW) wait_4_steps();
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
    // Prologue: the loads that steps -6 .. -1 would issue (step c loads
    // K(c+6) and V(c+5)), the partial scores of tiles 0 and 1, the weights of
    // tile 0.
    prologue_loads(ks);
    scores(kr[0], sQ0);
    scores(kr[1], sQ1);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_no_fence();  // every wave's partial scores of tiles 0, 1
    if (owner) {
      f32x4 sp[4];
      read_partials(sQ0, sp);
      weights(0, sp, sP0);
    }
    if (!CW) wait_4_steps();  // V(0) in
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier_no_fence();
    // Whole groups of six steps, then the rest (nested, so the compiler sees
    // the same loads in flight on every path into a step).
    int s = 0;
    for (; s + 6 <= n; s += 6) {
      step(s, kr[2], kr[0], sV0, sV5, sQ1, sQ0, sP0, sP1);
      step(s + 1, kr[3], kr[1], sV1, sV0, sQ0, sQ1, sP1, sP0);
      step(s + 2, kr[4], kr[2], sV2, sV1, sQ1, sQ0, sP0, sP1);
      step(s + 3, kr[5], kr[3], sV3, sV2, sQ0, sQ1, sP1, sP0);
      step(s + 4, kr[0], kr[4], sV4, sV3, sQ1, sQ0, sP0, sP1);
      step(s + 5, kr[1], kr[5], sV5, sV4, sQ0, sQ1, sP1, sP0);
    }
    if (s < n) {
      step(s, kr[2], kr[0], sV0, sV5, sQ1, sQ0, sP0, sP1);
      if (s + 1 < n) {
        step(s + 1, kr[3], kr[1], sV1, sV0, sQ0, sQ1, sP1, sP0);
        if (s + 2 < n) {
          step(s + 2, kr[4], kr[2], sV2, sV1, sQ1, sQ0, sP0, sP1);
          if (s + 3 < n) {
            step(s + 3, kr[5], kr[3], sV3, sV2, sQ0, sQ1, sP1, sP0);
            if (s + 4 < n) step(s + 4, kr[0], kr[4], sV4, sV3, sQ1, sQ0, sP0, sP1);
          }
        }
      }
    }
    // Loads past the last tile may still be in flight into registers.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
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
  // Heads per workgroup: the most (16, 32 or 64) that still give at least
  // 256 workgroups, so each K/V byte is copied into as few CUs as the batch
  // allows while the chip stays full.
  a.nk = nullptr;
  a.nv = nullptr;
  a.M = 1;
  a.hpt = p.H / 16;
  int nhb = 4;
  while (nhb > 1 && ((int64_t)p.B * (p.H / 16 / nhb) < 256 || (p.H / 16) % nhb != 0)) nhb >>= 1;
  a.n_hg = p.H / 16 / nhb;
  const dim3 grid((unsigned)(((p.B + 7) / 8) * 8 * a.n_hg)), block(256);
  switch (nhb) {
    case 4: hipLaunchKernelGGL((decode_kernel<4, false>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<2, false>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<1, false, true>), grid, dim3(512), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_multi(const DecodeProblem& p, const uint16_t* nk, const uint16_t* nv,
                               int M, hipStream_t stream) {
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
  a.H = M * p.H;  // rows per sequence, token-major
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  a.nk = nk;
  a.nv = nv;
  a.M = M;
  a.hpt = p.H / 16;
  // Blocks of 16 rows per workgroup (1 .. 4, dividing the M * H / 16 blocks of a
  // sequence).  A workgroup's time grows as about 4 + its block count (the key
  // walk, plus the MFMA and softmax work of each block), and workgroups past
  // one per CU run in further rounds: take the count with the least
  // rounds * (4 + blocks), the larger count on a tie (fewer copies of K/V).
  const int blocks = M * p.H / 16;
  int nhb = 1;
  int64_t best = -1;
  for (int c = 1; c <= 4; ++c) {
    if (blocks % c != 0) continue;
    const int64_t rounds = ((int64_t)p.B * (blocks / c) + 255) / 256;
    const int64_t cost = rounds * (4 + c);
    if (best < 0 || cost <= best) {
      best = cost;
      nhb = c;
    }
  }
  a.n_hg = blocks / nhb;
  const dim3 grid((unsigned)(((p.B + 7) / 8) * 8 * a.n_hg)), block(256);
  switch (nhb) {
    case 4: hipLaunchKernelGGL((decode_kernel<4, true>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<3, true>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<2, true>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<1, true>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace hca
