// decode.hip - HCA decode attention on gfx950: one new query per sequence.
//
// For sequence b with its new token at position t (already written into its
// ring slot t % 128), the keys are the floor((t+1)/128) cached entries and the
// raw rows of positions max(0, t-127) .. t, read from the ring (aitest123.com,
// "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B", section 模型结构; lininn.cn,
// section 43 层里，37 层只读摘要).  The output is gated by sigmoid(G)
// (blog.derekhsu.net, section 低秩閘控注意力).
//
// Decomposition.  One workgroup per (sequence, group of 16 heads); the head
// groups of a sequence run on the same XCD, so its K/V bytes come from HBM once
// and from that XCD's L2 for the other groups.  The keys are walked in 16-key
// tiles: first the entries (the last entry tile masked past the last entry),
// then the window, so every tile comes from one buffer.  The four waves copy
// each tile into LDS together by DMA, three tiles ahead of the one whose value
// product is computed (four LDS stages of K + V).  Wave w owns head dims
// 128w .. 128w+127:
//   scores  partial S^T[key][head] over the wave's dims (4 MFMA 16x16x32, K
//           from LDS, Q of the 16 heads in VGPRs), summed across the waves
//           through LDS, so each wave holds the full scores of the tile;
//   values  O^T[dv][head] for the wave's dims (8 MFMA 16x16x16, V^T by one
//           LDS transpose read each, P^T straight from the score registers).
// Step i sums the scores of tile i, takes its weights and adds its value
// product, while computing the partial scores of tile i+1.
//
// Softmax (as in prefill): scores in the exp2 domain; each head's reference m
// is the maximum of its first tile, and every key is weighed by 2^(x - m).  If
// a score rises more than 2^64 above it, the sequence is run again with the
// exact maximum.  Memory bound: per sequence (nc + window) * 2 KiB of K/V plus
// 3 * H KiB of q, g and out.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kHeads = 16;  // heads per workgroup
constexpr int kTile = 16;
constexpr int kKRow = 1024 + 16;  // LDS bytes between K rows (conflict-free b128 reads)
constexpr int kVRow = 1024 + 64;  // between V rows (conflict-free transpose reads)
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
  int B, H, n_hg;
  float c;  // scale * log2(e)
  int out_f32;
};

// The keys of one sequence: n_et entry tiles (entries 0 .. nc-1), then the
// window tiles (positions lo .. t, ring slot = position % 128).
struct Keys {
  const uint16_t *ek, *ev, *wk, *wv;  // this sequence's entries and ring
  int nc, lo, nw, n_et, n_tiles;
};

// Tile i: entry or window tile, its first entry / window index, and its
// number of valid keys.  Wave-uniform.
struct TileRef {
  bool ent;
  int first, valid;
};
__device__ __forceinline__ TileRef tile_ref(const Keys& ks, int i) {
  TileRef r;
  r.ent = i < ks.n_et;
  r.first = kTile * (r.ent ? i : i - ks.n_et);
  const int v = (r.ent ? ks.nc : ks.nw) - r.first;
  r.valid = v < kTile ? v : kTile;
  return r;
}

// Copy rows 4w .. 4w+3 of tile i into (sK, sV).  Entry rows past the last
// entry arrive as zeros (buffer range check); window rows wrap round the ring.
__device__ __forceinline__ void copy_tile(const Keys& ks, int i, uint8_t* sK, uint8_t* sV,
                                          int wave, int lane16) {
  asm volatile("" : "+s"(wave), "+s"(i));  // addresses computed here, not kept in registers
  const TileRef tr = tile_ref(ks, i);
  const int bytes = (tr.ent ? ks.nc : kWindow) * 1024;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(tr.ent ? ks.ek : ks.wk, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(tr.ent ? ks.ev : ks.wv, bytes);
  const int base = tr.ent ? tr.first : ks.lo + tr.first;
  const int mask = tr.ent ? 0x7FFFFFFF : kWindow - 1;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * wave + u;
    const int row = (base + r) & mask;
    dma16_buf(rk, lane16 + row * 1024, (lds_void*)(sK + r * kKRow));
    dma16_buf(rv, lane16 + row * 1024, (lds_void*)(sV + r * kVRow));
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

// s_waitcnt vmcnt(n) for the copies of n tiles (8 DMA instructions each).
__device__ __forceinline__ void wait_tiles_pending(int n) {
  if (n >= 2)
    __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Partial scores of a tile over this wave's dims: lane (head l16, g4) gets
// keys 4g4 .. 4g4+3.  koff addresses K row l16, dims 128w + 8g4; fragment ss
// holds dims 128w + 32ss + 8g4 .. +7.
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

__global__ void __launch_bounds__(256, 1) decode_kernel(Args a) {
  // Four stages of (K, V) tiles and two buffers of partial scores, separate
  // arrays so the compiler can tell a copy into one from reads of another.
  __shared__ __attribute__((aligned(256))) uint8_t sK0[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sK1[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sK2[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sK3[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV0[kTile * kVRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV1[kTile * kVRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV2[kTile * kVRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV3[kTile * kVRow];
  __shared__ __attribute__((aligned(1024))) uint8_t sS0[4 * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sS1[4 * 1024];

  // blockIdx -> (sequence, head group): XCD x = blockIdx % 8 takes sequences
  // x, x + 8, ... with all their head groups.
  const int L = blockIdx.x;
  const int k8 = L >> 3;
  const int hg = k8 % a.n_hg;
  const int b = (k8 / a.n_hg) * 8 + (L & 7);
  if (b >= a.B) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;

  // Q and the gate logits do not depend on the position: their loads go out
  // first, so their latency overlaps the position's and the first copies'.
  const int64_t head0 = (int64_t)b * a.H + hg * kHeads;
  // Q fragments (B operand of the partial scores): head l16, dims 128w +
  // 32ss + 8g4 .. +8.
  bf16x8 qf[4];
  {
    const uint16_t* qrow = a.q + (head0 + l16) * kD + 128 * wave + 8 * g4;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) qf[ss] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ss);
  }
  // Gate logits of this lane's output dims (see the epilogue).
  const int64_t rowo = (head0 + l16) * kD + 128 * wave + 4 * g4;
  uint2 gw[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) gw[db] = *reinterpret_cast<const uint2*>(a.g + rowo + 16 * db);

  // Positions below 2^31 (negative ones read as 0); wave-uniform.
  int64_t t64 = a.pos[b];
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
  const int n_tiles = ks.n_tiles;

  // Lane offsets: K fragment source (row l16, dims 128w + 8g4); V^T
  // transpose read source (key row 4g4 + l16/4, dims 128w + 4(l16&3)); the
  // lane's 16-byte slot of a partial-score buffer.
  const int koff = l16 * kKRow + 256 * wave + 16 * g4;
  const int voff = (4 * g4 + (l16 >> 2)) * kVRow + 256 * wave + 8 * (l16 & 3);
  const int lane16 = lane * 16;

  __builtin_amdgcn_s_waitcnt(0x0F70);  // Q and G in (the copies below are counted from here)

  // O^T blocks: o[db] lane (head l16, g4), reg r -> dim 128w + 16db + 4g4 + r
  f32x4 o[8];
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f;
  bool over = false, fixed_m = false;

  // Step i: tile i's partial scores are in sS (all waves'), its V in sV;
  // tile i+1's K in sKn.  Writes tile i+1's partial scores into sSn and
  // copies tile i+3 into (dK, dV), the stage of tile i-1.
  auto step = [&](int i, const uint8_t* sV, const uint8_t* sKn, const uint8_t* sS,
                  uint8_t* sSn, uint8_t* dK, uint8_t* dV) {
    int w = wave;
    asm volatile("" : "+s"(w), "+s"(i));  // per-step values computed here, not kept in registers
    // All LDS reads first (a read after a copy would wait for it), the K
    // fragments of the next tile's scores ahead of the rest so its MFMAs can
    // start while the others are in flight.  Past the last tile, K and
    // scores are of a stale stage and unused.
    bf16x8 kf[4];
    k_frags(sKn, koff, kf);
    f32x4 sp[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sp[u] = *reinterpret_cast<const f32x4*>(sS + u * 1024 + lane16);
    i16x4 vf[8];
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vf[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + voff + 32 * db));
    __builtin_amdgcn_sched_barrier(0);
    const bool next = i + 1 < n_tiles;
    const f32x4 sn = partial_scores(kf, qf);
    if (i + 3 < n_tiles) copy_tile(ks, i + 3, dK, dV, w, lane16);
    // Scores of tile i (exp2 domain), masked past its valid keys.
    const TileRef tr = tile_ref(ks, i);
    f32x4 s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = 4 * g4 + r < tr.valid ? s[r] * a.c : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    if (i == 0 && !fixed_m) m = xmax32(xmax16(mt));  // the reference: max of the first tile
    mseen = fmaxf(mseen, mt);
    over |= mt > m + kHeadroom;
    const f32x4 e = {__builtin_amdgcn_exp2f(s[0] - m), __builtin_amdgcn_exp2f(s[1] - m),
                     __builtin_amdgcn_exp2f(s[2] - m), __builtin_amdgcn_exp2f(s[3] - m)};
    const bf16x4 pb = __builtin_convertvector(e, bf16x4);  // nearest even
    // l adds the rounded weights: dot products with ones.
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[0], pb[1]}, ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[2], pb[3]}, ones, l, false);
    // P^T (B operand): lane (head l16, g4) holds keys 4g4 .. 4g4+3, the same
    // keys as the V^T fragments' k-slots.
    const i16x4 pf = __builtin_bit_cast(i16x4, pb);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[db], pf, o[db], 0, 0, 0);
    if (next) *reinterpret_cast<f32x4*>(sSn + wave * 1024 + lane16) = sn;
    // This wave's copies of tile i+2 and its partial scores of tile i+1 are
    // done (only the copies of tile i+3 may be in flight), then every wave's.
    wait_tiles_pending(i + 3 < n_tiles ? 1 : 0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_no_fence();
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{};
    l = 0.0f;
    over = false;
    // Prologue: tiles 0, 1, 2 copied; partial scores of tile 0.
    copy_tile(ks, 0, sK0, sV0, wave, lane16);
    if (n_tiles > 1) copy_tile(ks, 1, sK1, sV1, wave, lane16);
    if (n_tiles > 2) copy_tile(ks, 2, sK2, sV2, wave, lane16);
    wait_tiles_pending(n_tiles - 1 < 2 ? n_tiles - 1 : 2);  // tile 0 in
    barrier_no_fence();
    {
      bf16x8 kf[4];
      k_frags(sK0, koff, kf);
      const f32x4 s0 = partial_scores(kf, qf);
      *reinterpret_cast<f32x4*>(sS0 + wave * 1024 + lane16) = s0;
    }
    wait_tiles_pending(n_tiles > 2 ? 1 : 0);  // tile 1 in
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier_no_fence();
    for (int i = 0; i < n_tiles; i += 4) {
      step(i, sV0, sK1, sS0, sS1, sK3, sV3);
      if (i + 1 >= n_tiles) break;
      step(i + 1, sV1, sK2, sS1, sS0, sK0, sV0);
      if (i + 2 >= n_tiles) break;
      step(i + 2, sV2, sK3, sS0, sS1, sK1, sV1);
      if (i + 3 >= n_tiles) break;
      step(i + 3, sV3, sK0, sS1, sS0, sK2, sV2);
    }
    // A score more than 2^kHeadroom above its reference (extreme score ranges
    // only): run again with the exact maximum of each head as reference.
    const bool redo = __builtin_amdgcn_ballot_w64(over) != 0;
    if (pass == 1 || !redo) break;
    m = xmax32(xmax16(mseen));
    fixed_m = true;
  }

  // out = O / l * sigmoid(G) for this wave's 128 dims.
  l = xsum32(xsum16(l));
  const float inv = 1.0f / l;
  constexpr float kLog2e = 1.4426950408889634f;
  float r[8][4];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const float gv[4] = {bf16_bits_to_f32(gw[db].x & 0xFFFFu), bf16_bits_to_f32(gw[db].x >> 16),
                         bf16_bits_to_f32(gw[db].y & 0xFFFFu), bf16_bits_to_f32(gw[db].y >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
      r[db][e] = o[db][e] * inv * sig;
    }
  }
  if (a.out_f32) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + rowo + 16 * db) =
          make_float4(r[db][0], r[db][1], r[db][2], r[db][3]);
  } else {
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + rowo + 16 * db) =
          make_uint2(pack_bf16x2(r[db][0], r[db][1]), pack_bf16x2(r[db][2], r[db][3]));
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
  a.n_hg = p.H / kHeads;
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  const unsigned blocks = (unsigned)(((p.B + 7) / 8) * 8 * a.n_hg);
  hipLaunchKernelGGL(decode_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
