// prefill.hip - HCA prefill attention on gfx950 (MI355X).
//
// What is computed (aitest123.com, "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B",
// section 模型结构; blog.derekhsu.net, sections 潛在閘控稀疏注意力 and
// 低秩閘控注意力; lininn.cn, section 43 层里，37 层只读摘要): for the query at
// position t and head h,
//   keys  = { entry b : b < Nc, 128b+127 <= t }  U  { raw row p : max(0,t-127) <= p <= t }
//   out   = softmax_j(scale * <q, key_j>) . value_j  *  sigmoid(G[t,h,:])
// with one 512-wide K/V head shared by every query head.
//
// Work decomposition.  The query tensor is a flat list of Tq*H rows (row =
// query*H + head).  A work item is 128 consecutive rows (for H = 64: two
// queries, all heads).  It walks, in one softmax, the 32-key tiles of the
// compressed entries its rows can see and then of their raw window.  Each K/V
// tile is copied once into LDS and shared by the 4 waves:
//   scores   wave w owns rows 32w .. 32w+31 (Q of those rows in VGPRs):
//            S^T[key][row] = K . Q^T, 32 MFMA 32x32x16; mask and softmax with
//            one row per lane; the weights P go to LDS.
//   values   wave w owns output dims 128w .. 128w+127 for all 128 rows:
//            O^T[dv][row] += V^T . P^T, 32 MFMA 32x32x16 (V^T by LDS
//            transpose reads of the wave's quarter of the V tile, P^T from LDS).
// Splitting the value product by output dims makes each wave read a quarter
// of the V tile instead of all of it; the score product, whose B operand is
// Q, stays split by rows.  O (256 accumulator registers) and Q (128 VGPRs)
// stay in registers for the whole item.
//
// Pipeline.  K runs one tile ahead of V: step i computes O += V(i) P(i) and,
// in the same straight-line block, the scores and weights P(i+1) of the next
// tile, so the softmax arithmetic fills the gaps between MFMAs.  Meanwhile
// DMA brings K(i+2) and V(i+1) into the stages freed by step i-1.  LDS:
// 2 K stages + 2 V stages (32 keys x 1 KiB each) + 2 P buffers (8 KiB).
// Tiles are copied global -> LDS by DMA (buffer_load_dwordx4 ... lds, no
// VGPRs), one 1 KiB key row per wave instruction, with an XOR swizzle of the
// 16-byte chunks chosen so the read patterns are bank-conflict free:
//   K: chunk c of key r stored at c ^ (r & 15)   (b128 reads, 16 keys x 1 chunk)
//   V: chunk c of key r stored at c ^ 4(r & 3)   (b64 transpose reads, 4 keys x 4 chunks)
//
// Persistent schedule.  The kernel runs one workgroup per CU; each workgroup
// loops over items.  Items are dealt so that the workgroups of one XCD take
// runs of adjacent items, whose raw windows overlap in that XCD's L2.
//
// Softmax: scores are kept in the exp2 domain (x = s * scale * log2 e).  Each
// row fixes its reference m at its first tile with a visible key and weighs
// every key by p = 2^(x - m); O is never rescaled in the loop (a rescale of
// 256 accumulator registers per lane would cost more than a tile's MFMAs).
// If any score rises more than 2^64 above its reference, the item's tiles are
// run again with the exact row maximum as reference.  P is rounded to bf16
// for the MFMA and the row sum l adds the rounded values, so O/l is a
// weighted mean of V rows up to fp32 accumulation.
//
// Epilogue: out = O / l * sigmoid(G), sigmoid(x) = 1/(1 + 2^(-x log2 e)),
// which is exactly 0 at G = -inf and 1 at G = +inf.  bf16 (nearest even) or
// f32 output.  Q, G and bf16 output move between HBM and registers through
// LDS so that global traffic is whole rows (or 256-byte row quarters).
//
// Roofline: 4*512 flop per (row, visible key); at 128K context the kernel is
// MFMA bound (about 420 flop per HBM byte).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kRowsPerItem = 128;
constexpr int kTile = 32;
constexpr float kHeadroom = 64.0f;  // p = 2^(x - m) stays below 2^64 in a pass

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

struct Args {
  const uint16_t* q;
  const uint16_t* g;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  void* out;
  int rows;                   // Tq * H
  int q_start, kv_start, Nc;  // positions and counts fit in 31 bits (checked on the host)
  int n_items;
  int per_xcd;                // workgroups per XCD (grid = 8 * per_xcd)
  int H;
  float c;  // scale * log2(e)
  int out_f32;
};

__device__ __forceinline__ int n_entries(int t, int Nc) {
  const int n = (t + 1) / kBlock;
  return n < Nc ? n : Nc;
}

// One work item as seen by one lane.
struct Item {
  int row0, last;      // rows of the item (last clamped to the final row)
  int my_row;          // this lane's score row (wave rows), clamped to `last`
  int t;               // its query position
  int t_max;           // last position of the item
  int tw_min, tw_max;  // positions of the wave's first and last score rows
  int nc_wg;           // entries visible to the last row of the item
  int w_lo;            // first raw position of the item's window union
  int n_ct;            // compressed tiles
  int n_tiles;
};

__device__ __forceinline__ Item make_item(const Args& a, int idx, int wave, int l32) {
  Item it;
  it.row0 = idx * kRowsPerItem;
  it.last = (it.row0 + kRowsPerItem < a.rows ? it.row0 + kRowsPerItem : a.rows) - 1;
  const int r = it.row0 + wave * 32 + l32;
  it.my_row = r < it.last ? r : it.last;
  it.t = a.q_start + it.my_row / a.H;
  const int wr0 = it.row0 + wave * 32, wr1 = wr0 + 31;
  it.tw_min = a.q_start + (wr0 < it.last ? wr0 : it.last) / a.H;
  it.tw_max = a.q_start + (wr1 < it.last ? wr1 : it.last) / a.H;
  const int t_min = a.q_start + it.row0 / a.H;
  it.t_max = a.q_start + it.last / a.H;
  it.nc_wg = n_entries(it.t_max, a.Nc);
  it.w_lo = t_min - (kWindow - 1) > 0 ? t_min - (kWindow - 1) : 0;
  it.n_ct = (it.nc_wg + kTile - 1) / kTile;
  it.n_tiles = it.n_ct + (it.t_max - it.w_lo + 1 + kTile - 1) / kTile;
  return it;
}

// Source of one 32-key tile of K or V: a buffer descriptor that covers exactly
// the tile's valid rows.  Reads past its end return zeros (hardware range
// check), so rows past the tile's last key arrive as zeros: those keys are
// masked (their weights are 0), and every LDS row of the tile is written.  A
// tile index past the item's last tile gets an empty descriptor, so the
// pipeline can issue copies without branches.
struct TileSrc {
  __amdgpu_buffer_rsrc_t rs;
};

__device__ __forceinline__ TileSrc tile_src(const Args& a, const Item& it, int i, bool v) {
  const uint16_t* base;
  int first, last;
  if (i < it.n_ct) {
    base = v ? a.cv : a.ck;
    first = i * kTile;
    last = it.nc_wg - 1;
  } else {
    base = v ? a.v : a.k;
    first = it.w_lo + (i - it.n_ct) * kTile - a.kv_start;
    last = it.t_max - a.kv_start;
  }
  TileSrc s;
  const int nrows = last - first + 1 < kTile ? last - first + 1 : kTile;
  const int bytes = i < it.n_tiles ? nrows * kD * 2 : 0;
  s.rs = make_rsrc(i < it.n_tiles ? base + (size_t)first * kD : base, bytes);
  return s;
}

// Copy key row u (0..7) of this wave's quarter of a K tile / a V tile.
__device__ __forceinline__ void dma_k_row(const TileSrc& s, uint8_t* sK, int u, int wave,
                                          int lane) {
  const int r = wave * (kTile / 4) + u;
  dma16_buf(s.rs, r * 1024 + ((lane ^ (r & 15)) << 4), (lds_void*)(sK + r * 1024));
}
__device__ __forceinline__ void dma_v_row(const TileSrc& s, uint8_t* sV, int u, int wave,
                                          int lane) {
  const int r = wave * (kTile / 4) + u;
  dma16_buf(s.rs, r * 1024 + ((lane ^ ((r & 3) << 2)) << 4), (lds_void*)(sV + r * 1024));
}

// Copy dims 128w .. 128w+127 (256 bytes) of the item's 128 rows of a
// [rows, 512] bf16 tensor into a 32 KiB LDS region: row r at r*256, chunk c of
// the quarter stored at c ^ (r & 15).  One instruction moves 4 rows.
__device__ __forceinline__ void dma_quarter(const uint16_t* base, int row0, int last, int wave,
                                            uint8_t* region, int lane) {
  asm volatile("" : "+v"(lane));
  const int nrows = last - row0 + 1;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (size_t)row0 * kD, nrows * kD * 2);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int r = 4 * j + (lane >> 4);
    const int src = (r < nrows ? r : nrows - 1) * 1024 + 256 * wave;
    dma16_buf(rs, src + (((lane & 15) ^ (r & 15)) << 4), (lds_void*)(region + j * 1024));
    if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

// Q fragments of the wave's score rows (B operand of S^T), loaded from global
// memory straight into registers: lane (row l%32, half g) holds dims 16ss +
// 8g .. +8 of its row for ss = 0..31, so one load instruction covers 32 B of
// each of 32 rows.  Rows past the item's last repeat the last one.
__device__ __forceinline__ const uint16_t* q_row(const Args& a, const Item& it, int wave,
                                                 int lane) {
  const int r = it.row0 + wave * 32 + (lane & 31);
  return a.q + (size_t)(r < it.last ? r : it.last) * kD + 8 * (lane >> 5);
}
// Fragments ss0 .. ss0+n-1.
__device__ __forceinline__ void load_q(const uint16_t* row, int ss0, int n, bf16x8 (&qf)[32]) {
#pragma unroll
  for (int ss = ss0; ss < ss0 + n; ++ss) qf[ss] = *reinterpret_cast<const bf16x8*>(row + 16 * ss);
}

struct WaveState {
  f32x16 o[16];  // O^T accumulators: block 4bb+rb = dims 128w+32bb.., rows 32rb + lane%32
  float m;       // score row reference max (exp2 domain), -inf before the first visible key
  float mseen;   // largest score of the row seen so far
  float l;       // this lane's partial row sum (its 16 keys of every tile)
  bool over;     // a score exceeded m + kHeadroom in this pass
};

// The lane's visible keys within tile i's key space: [lo, lo + width).
struct ScoreTile {
  int first, lo, width;
};

__device__ __forceinline__ ScoreTile score_tile(const Args& a, const Item& it, int i) {
  ScoreTile s;
  if (i >= it.n_tiles) {  // past the last tile: nothing visible
    s.first = 0;
    s.lo = 0;
    s.width = 0;
  } else if (i < it.n_ct) {
    s.first = i * kTile;
    s.lo = 0;
    s.width = n_entries(it.t, a.Nc);
  } else {
    s.first = it.w_lo + (i - it.n_ct) * kTile;
    s.lo = it.t - (kWindow - 1);
    s.width = kWindow;
  }
  return s;
}

// Whether every score row of the wave sees every key of tile i (no masking
// needed).  Wave-uniform.
__device__ __forceinline__ bool tile_full(const Args& a, const Item& it, int i) {
  if (i >= it.n_tiles) return false;
  if (i < it.n_ct) return i * kTile + kTile <= n_entries(it.tw_min, a.Nc);
  const int first = it.w_lo + (i - it.n_ct) * kTile;
  return first >= it.tw_max - (kWindow - 1) && first + kTile - 1 <= it.tw_min;
}

// The score accumulator S^T is kept in VGPRs: the 256 accumulator registers
// hold O, and the MFMA builtins leave the accumulator's register file to the
// allocator, which then puts S^T in accumulator registers and moves O blocks
// out and back around every tile.  So the score MFMAs are written out with
// VGPR operands.  The compiler inserts no wait states around inline asm: the
// last MFMA of a chain carries the 20 that a VALU read of its result needs
// (the compiler itself emits 12 for this opcode), and no VALU instruction may
// write an operand within 2 wait states before one of these MFMAs (their
// operands come from LDS reads; a test checks the generated code for this).
// A chain accumulating into the same registers issues back to back.
// The first MFMA of a chain accumulates into the score bias, written by VALU
// instructions just before: it waits the 2 wait states that needs.
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 3"
               : "+v"(d)
               : "v"(a), "v"(b));
}

// S^T (32 keys x the wave's 32 rows) = K . Q^T for the K tile in sK, with K
// fragments read kAhead MFMAs ahead; `copy(ss)` is called after MFMA ss
// (copies of later tiles, spread over the chain).  The order of MFMAs, reads
// and copies is fixed with scheduling barriers.
template <int kAhead, typename Copy>
__device__ __forceinline__ f32x16 qk_chain(const bf16x8 (&qf)[32], const uint8_t* sK,
                                           const f32x16& bias, int lane, Copy copy) {
  const int l32 = lane & 31, g = lane >> 5;
  // Step ss reads chunk 2ss+g of key row l32, stored at (2ss+g) ^ (l32&15);
  // with ss = 8j + i that is 16j + ((2i + g) ^ (l32&15)), so 8 lane offsets
  // serve all steps (j becomes an immediate offset).
  const uint8_t* krow = sK + l32 * 1024;
  int koff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) koff[i] = ((2 * i + g) ^ (l32 & 15)) << 4;
  bf16x8 kf[kAhead];
#pragma unroll
  for (int ss = 0; ss < kAhead; ++ss)
    kf[ss] = *reinterpret_cast<const bf16x8*>(krow + koff[ss & 7] + 256 * (ss >> 3));
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s = bias;
#pragma unroll
  for (int ss = 0; ss < 32; ++ss) {
    if (ss == 0)
      mfma_s_first(s, kf[0], qf[0]);
    else if (ss == 31)
      mfma_s_last(s, kf[ss % kAhead], qf[ss]);
    else
      mfma_s_acc(s, kf[ss % kAhead], qf[ss]);
    if (ss + kAhead < 32) {
      const int n = ss + kAhead;
      kf[ss % kAhead] = *reinterpret_cast<const bf16x8*>(krow + koff[n & 7] + 256 * (n >> 3));
    }
    copy(ss);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// Softmax of one tile's scores for the wave's rows, in slices that a pipeline
// step spreads over its MFMAs: mask (one score per slice), row max, weights
// (two per slice), and the weights to LDS as PV B-operand fragments of row
// block `wave`.  Keys outside the lane's visible interval get weight 0 (as
// does every key of a tile the lane's row cannot see).
struct SoftmaxTile {
  f32x16 s;   // scores (-inf where the key is not visible)
  float mt;   // running max of the scores, then the row max (exp2 domain)
  float msub;
  bf16x2 pk[8];
};

__device__ __forceinline__ void sm_init(SoftmaxTile& x, const f32x16& s) {
  x.s = s;
  x.mt = -INFINITY;
}

// The mask of tile i as an additive score bias: 0 for the lane's visible keys,
// -inf for the others (score register r holds key 8(r/4) + 4(lane/32) + r%4 of
// the tile).  It is the initial accumulator of the tile's score MFMAs, so the
// masked scores come out of the MFMAs.  Tiles every score row of the wave sees
// in full get zeros without the per-key tests.
__device__ __forceinline__ f32x16 score_bias(const Args& a, const Item& it, int i, int lane) {
  f32x16 b;
  if (tile_full(a, it, i)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) b[r] = 0.0f;
  } else {
    const ScoreTile sc = score_tile(a, it, i);
    const unsigned width = (unsigned)sc.width;
    const int d0 = sc.first - sc.lo + 4 * (lane >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      b[r] = (unsigned)(d0 + 8 * (r >> 2) + (r & 3)) < width ? 0.0f : -INFINITY;
  }
  return b;
}

// Row max over both wave halves (lanes l and l^32 hold the same row), and the
// reference update: fixed at the row's first tile with a visible key.
__device__ __forceinline__ void sm_reduce(const Args& a, WaveState& st, SoftmaxTile& x) {
  float mt = x.mt * a.c;
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                   false, false);
  mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  st.mseen = fmaxf(st.mseen, mt);
  st.m = st.m == -INFINITY ? mt : st.m;
  st.over |= mt > st.m + kHeadroom;
  x.msub = st.m == -INFINITY ? 0.0f : st.m;
}

__device__ __forceinline__ void sm_exp(const Args& a, WaveState& st, SoftmaxTile& x, int j) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x2 pr = {__builtin_amdgcn_exp2f(__builtin_fmaf(x.s[2 * j], a.c, -x.msub)),
                    __builtin_amdgcn_exp2f(__builtin_fmaf(x.s[2 * j + 1], a.c, -x.msub))};
  x.pk[j] = __builtin_convertvector(pr, bf16x2);
  st.l = __builtin_amdgcn_fdot2_f32_bf16(x.pk[j], ones, st.l, false);
}

// B operand of O^T += V^T P^T for 16-key half c2: lane (row n, half g) holds
// k-slots 8g..8g+7 = keys 16c2 + {4g..4g+3, 8+4g..8+4g+3}, which are exactly
// this lane's score registers 8c2 .. 8c2+7.
__device__ __forceinline__ void sm_write(const SoftmaxTile& x, uint8_t* sP, int c2, int lane,
                                         int wave) {
  bf16x8 pf;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pf[2 * e] = x.pk[4 * c2 + e][0];
    pf[2 * e + 1] = x.pk[4 * c2 + e][1];
  }
  *reinterpret_cast<bf16x8*>(sP + (wave * 2 + c2) * 1024 + lane * 16) = pf;
}

// Slice k (0..31) of the softmax.
__device__ __forceinline__ void sm_slice(const Args& a, WaveState& st, SoftmaxTile& x,
                                         uint8_t* sP, int k, int lane, int wave) {
  if (k < 16)
    x.mt = fmaxf(x.mt, x.s[k]);
  else if (k == 16)
    sm_reduce(a, st, x);
  else if (k < 25)
    sm_exp(a, st, x, k - 17);
  else if (k < 27)
    sm_write(x, sP, k - 25, lane, wave);
}

// V^T fragment of PV block n = 4 c2 + bb (keys 16c2.., dims 128w + 32bb..)
// from the V tile in sV.  Transpose reads: in each 16-lane group, source lane
// s16 addresses key row 4(lane/32) + s16/4 (+16 c2 + 8 r) and dims 32b +
// 16((lane/16)&1) + 4(s16&3); the result lane holds 4 keys of one dim.  Dim
// block b = 4w + bb sits at chunk (4b + cbase) ^ 4sw = 16w + 4(bb ^ sw) + cbase.
__device__ __forceinline__ bf16x8 v_frag(const uint8_t* sV, int n, int lane, int wave) {
  const int s16 = lane & 15, q4 = lane >> 4;
  const int sw = (s16 >> 2) & 3;
  const int cbase = 2 * (q4 & 1) + ((s16 & 3) >> 1);
  const int half = (s16 & 1) << 3;
  const int c2 = n >> 2, bb = n & 3;
  const uint8_t* p = sV + (4 * (q4 >> 1) + (s16 >> 2)) * 1024 + 256 * wave + 16384 * c2 +
                     ((4 * (bb ^ sw) + cbase) << 4) + half;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8192));
  const i16x8 w8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w8);
}

// P^T fragment of row block rb, key half c2.
__device__ __forceinline__ bf16x8 p_frag(const uint8_t* sP, int rb, int c2, int lane) {
  return *reinterpret_cast<const bf16x8*>(sP + (rb * 2 + c2) * 1024 + lane * 16);
}

// One step of the three-stage tile pipeline.  With tile i's weights P(i) in
// sP, V(i) in sV, K(i+2) in sK and the scores of tile i+1 in `carry`:
//   O += V(i) P(i)                         32 MFMAs (accumulator registers)
//   softmax of tile i+1 -> P(i+1) in sPn    VALU, in slices
//   carry = scores of tile i+2              32 MFMAs (one VGPR chain)
//   copies of K(i+3) into sKd, V(i+1) into sVd (empty past the last tile).
// The three parts are independent; group k issues score MFMA k, PV MFMA k,
// softmax slice k, the K read three MFMAs ahead, and groups 5..20 one copy
// row each.  Scheduling barriers keep that
// order, so the softmax arithmetic and the score chain's latency hide behind
// the MFMAs.
__device__ __forceinline__ void step(const Args& a, WaveState& st, const bf16x8 (&qf)[32],
                                     f32x16& carry, const Item& it, int i, const uint8_t* sV,
                                     const uint8_t* sP, const uint8_t* sK, uint8_t* sPn,
                                     uint8_t* sKd, uint8_t* sVd, int lane, int wave) {
  asm volatile("" : "+v"(lane));
  asm volatile("" : "+s"(wave));  // per-row LDS addresses recomputed, not kept in registers
  const int l32 = lane & 31, g = lane >> 5;
  const TileSrc ks = tile_src(a, it, i + 3, false);
  const TileSrc vs = tile_src(a, it, i + 1, true);
  SoftmaxTile x;
  sm_init(x, carry);
  f32x16 s = score_bias(a, it, i + 2, lane);  // scores of tile i+2 accumulate onto its mask

  // K fragment for score MFMA ss: chunk 2ss+g of key row l32, stored at
  // (2ss+g) ^ (l32&15) = 16j + ((2i + g) ^ (l32&15)) for ss = 8j + i.
  const uint8_t* krow = sK + l32 * 1024;
  const int kx = (g ^ (l32 & 15)) << 4;  // chunk offset of step 0; step ss: ^ (32 (ss & 7))
  auto kread = [&](int ss) {
    return *reinterpret_cast<const bf16x8*>(krow + (kx ^ (32 * (ss & 7))) + 256 * (ss >> 3));
  };
  // The V^T fragments of key half 0 are read first, those of half 1 in
  // groups 1..4, and the copies issued from group 5 on: the compiler cannot
  // tell transpose reads from the copies' LDS writes and would make every
  // transpose read after a copy wait for all copies.
  constexpr int kAhead = 3;
  bf16x8 kf[kAhead], vf[8], pf[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) vf[n] = v_frag(sV, n, lane, wave);
#pragma unroll
  for (int ss = 0; ss < kAhead; ++ss) kf[ss] = kread(ss);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) pf[rb] = p_frag(sP, rb, 0, lane);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k == 0)
      mfma_s_first(s, kf[0], qf[0]);
    else if (k == 31)
      mfma_s_last(s, kf[k % kAhead], qf[k]);
    else
      mfma_s_acc(s, kf[k % kAhead], qf[k]);
    // PV MFMA k: block n = k/4 (key half n/4, dim block n%4), row block k%4
    const int n = k >> 2, rb = k & 3;
    st.o[4 * (n & 3) + rb] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n], pf[rb], st.o[4 * (n & 3) + rb], 0, 0, 0);
    if (k + kAhead < 32) kf[k % kAhead] = kread(k + kAhead);
    if (k >= 1 && k < 5) vf[k + 3] = v_frag(sV, k + 3, lane, wave);
    if (k >= 12 && k < 16) pf[rb] = p_frag(sP, rb, 1, lane);  // last use of half 0 was MFMA k
    if (k >= 5 && k < 13) dma_k_row(ks, sKd, k - 5, wave, lane);
    if (k >= 13 && k < 21) dma_v_row(vs, sVd, k - 13, wave, lane);
    sm_slice(a, st, x, sPn, k, lane, wave);
    __builtin_amdgcn_sched_barrier(0);
  }
  carry = s;
}

// Gate and normalise the wave's output block (dims 128w.., all 128 rows), with
// the gate logits staged in `region` by dma_quarter.  bf16 output is written
// back over the logits (same size, same place) and stored later as row
// quarters; f32 output is stored from registers.  The 16 logit pieces of a
// row block are read before any result of that block is written back, so the
// reads are not ordered behind the writes.  If next_q is set, a quarter of
// the next item's Q fragments is loaded before each row block.
template <bool kF32>
__device__ __forceinline__ void gate_block(const Args& a, const WaveState& st, const Item& it,
                                           uint8_t* region, const float* sL, int lane, int wave,
                                           const uint16_t* next_q, bf16x8 (&qf)[32]) {
  asm volatile("" : "+v"(lane));
  constexpr float kLog2e = 1.4426950408889634f;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (next_q) load_q(next_q, 8 * rb, 8, qf);
    const int r = 32 * rb + l32;  // item row
    const float l = sL[r];
    uint8_t* row = region + r * 256 + 8 * g;
    uint2 gw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)  // j = 4 bb + q: dims 32bb + 8q + 4g .. +3
      gw[j] = *reinterpret_cast<const uint2*>(row + ((j ^ (r & 15)) << 4));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int bb = j >> 2, q = j & 3;
      const float gv[4] = {bf16_bits_to_f32(gw[j].x & 0xFFFFu), bf16_bits_to_f32(gw[j].x >> 16),
                           bf16_bits_to_f32(gw[j].y & 0xFFFFu), bf16_bits_to_f32(gw[j].y >> 16)};
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // O / l * sigmoid(g) = O / (l + l * 2^(-g log2 e))
        const float den = __builtin_fmaf(l, __builtin_amdgcn_exp2f(-gv[e] * kLog2e), l);
        o[e] = st.o[4 * bb + rb][4 * q + e] * __builtin_amdgcn_rcpf(den);
      }
      if (kF32) {
        if (it.row0 + r <= it.last)
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)(it.row0 + r) * kD +
                                     128 * wave + 32 * bb + 8 * q + 4 * g) =
              make_float4(o[0], o[1], o[2], o[3]);
      } else {
        const bf16x2 lo = __builtin_convertvector((f32x2){o[0], o[1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){o[2], o[3]}, bf16x2);
        *reinterpret_cast<uint2*>(row + ((j ^ (r & 15)) << 4)) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Store the wave's bf16 output block (dims 128w.., 128 rows) from its region,
// 4 row quarters (256 bytes each) per instruction.  The descriptor covers the
// item's rows only, so stores of rows past the last one are dropped.
__device__ __forceinline__ void store_block(const Args& a, const Item& it, const uint8_t* region,
                                            int lane, int wave) {
  asm volatile("" : "+v"(lane));
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(static_cast<uint16_t*>(a.out) + (size_t)it.row0 * kD, (it.last - it.row0 + 1) * 1024);
  const int c = lane & 15;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int r = 4 * j + (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + r * 256 + ((c ^ (r & 15)) << 4));
    store16_buf(rs, r * 1024 + 256 * wave + 16 * c, v);
    if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool kF32>
__global__ void __launch_bounds__(256, 1) prefill_kernel(Args a) {
  // Separate arrays per stage: the compiler then knows a copy into one stage
  // cannot alias reads of another and inserts no wait between them.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sP0[8 * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sP1[8 * 1024];
  __shared__ float sL[kRowsPerItem];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31;

  // Items sorted heaviest first, p = 0, 1, ... being item n_items-1-p, are
  // dealt in rounds of G: round r covers p in [r*G, (r+1)*G), and within a
  // round XCD x (the workgroups with blockIdx % 8 == x) takes the run of
  // per_xcd adjacent items starting at x*per_xcd.  XCD x walks the rounds
  // starting at round x*R/8 and wrapping around: every workgroup does the same
  // items as in plain round order, but the XCDs are out of phase, so their
  // HBM-heavy item boundaries (gate and Q in, output out) do not coincide.
  const int G = gridDim.x;
  const int slot = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
  const int R = (a.n_items + G - 1) / G;
  const int r0 = ((blockIdx.x & 7) * R) >> 3;
  int j = 0;  // rounds visited
  auto next_p = [&]() -> int {  // next item of this workgroup, -1 when done
    while (j < R) {
      const int r = j + r0 < R ? j + r0 : j + r0 - R;
      ++j;
      const int q = r * G + slot;
      if (q < a.n_items) return q;
    }
    return -1;
  };
  int p = next_p();
  if (p < 0) return;
  Item it = make_item(a, a.n_items - 1 - p, wave, l32);

  // The wave's 32 KiB staging region for Q, gate and output (the tile stages
  // are free between items).
  uint8_t* const region = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;

  bf16x8 qf[32];
  load_q(q_row(a, it, wave, lane), 0, 32, qf);

  for (;;) {
    WaveState st;
    st.m = -INFINITY;
    st.mseen = -INFINITY;
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int b = 0; b < 16; ++b) st.o[b] = f32x16{};
      st.l = 0.0f;
      st.over = false;
      // Prologue: K(0), V(0), K(1) in; scores of tiles 0 and 1; K(2) in;
      // weights of tile 0.
      f32x16 carry;
      {
        int ln = lane;  // recomputed lane-dependent offsets rather than kept across the loop
        asm volatile("" : "+v"(ln));
        const TileSrc k0 = tile_src(a, it, 0, false), v0 = tile_src(a, it, 0, true);
        const TileSrc k1 = tile_src(a, it, 1, false);
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_k_row(k0, sK0, u, wave, ln);
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_v_row(v0, sV0, u, wave, ln);
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_k_row(k1, sK1, u, wave, ln);
        wait_vmem();
        __syncthreads();
        const f32x16 s0 = qk_chain<4>(qf, sK0, score_bias(a, it, 0, ln), ln, [](int) {});
        carry = qk_chain<4>(qf, sK1, score_bias(a, it, 1, ln), ln, [](int) {});
        __syncthreads();
        const TileSrc k2 = tile_src(a, it, 2, false);
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_k_row(k2, sK0, u, wave, ln);
        SoftmaxTile x;
        sm_init(x, s0);
#pragma unroll
        for (int k = 0; k < 27; ++k) sm_slice(a, st, x, sP0, k, ln, wave);
        wait_vmem();
        __syncthreads();
      }
      // Step i: V(i) in sV[i&1], P(i) in sP[i&1], K(i+2) in sK[i&1]; it
      // writes P(i+1) into sP[(i+1)&1] and copies K(i+3) and V(i+1) into the
      // other stages.  Steps past the last tile only add zeros.
      for (int i = 0; i < it.n_tiles; i += 2) {
        step(a, st, qf, carry, it, i, sV0, sP0, sK0, sP1, sK1, sV1, lane, wave);
        wait_vmem();
        __syncthreads();
        step(a, st, qf, carry, it, i + 1, sV1, sP1, sK1, sP0, sK0, sV0, lane, wave);
        wait_vmem();
        __syncthreads();
      }
      // Only if some score rose more than 2^kHeadroom above its row reference
      // (possible only for extreme score ranges) is the pass repeated, with the
      // exact row maximum of the first pass as reference; that cannot overflow.
      if (pass == 1 || !__syncthreads_or(st.over)) break;
      st.m = st.mseen;
    }

    // Epilogue.  Row sums to every wave, gate logits in through LDS, output out
    // through LDS (bf16).  The regions alias the tile stages, which are idle
    // here.
    {
      const float l_tot = st.l + __shfl_xor(st.l, 32);
      if (lane < 32) sL[wave * 32 + lane] = l_tot;
    }
    dma_quarter(a.g, it.row0, it.last, wave, region, lane);
    __syncthreads();  // sL complete
    wait_vmem();
    // The next item's Q is loaded while the gate is computed (a quarter of it
    // before each row block).
    p = next_p();
    const bool more = p >= 0;
    const Item nx = more ? make_item(a, a.n_items - 1 - p, wave, l32) : it;
    gate_block<kF32>(a, st, it, region, sL, lane, wave, more ? q_row(a, nx, wave, lane) : nullptr,
                     qf);
    if (!kF32) store_block(a, it, region, lane, wave);
    __syncthreads();  // every wave is done with its region and with sL
    if (!more) break;
    it = nx;
  }
}

int g_cus[64];  // CUs per device, looked up once

}  // namespace

hipError_t launch_prefill(const PrefillProblem& p, hipStream_t stream) {
  Args a;
  a.q = p.q;
  a.g = p.g;
  a.k = p.k;
  a.v = p.v;
  a.ck = p.ck;
  a.cv = p.cv;
  a.out = p.out;
  a.rows = (int)(p.Tq * p.H);
  a.q_start = (int)p.q_start;
  a.kv_start = (int)p.kv_start;
  a.Nc = (int)p.Nc;
  a.H = p.H;
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  a.n_items = (a.rows + kRowsPerItem - 1) / kRowsPerItem;
  if (a.n_items == 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (g_cus[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus[dev] = cus > 0 ? cus : 256;
  }
  // One workgroup per CU (LDS and registers allow no more), a multiple of the
  // 8 XCDs, and no more workgroups than items.
  int per_xcd = g_cus[dev] / 8;
  if (per_xcd < 1) per_xcd = 1;
  const int need = (a.n_items + 7) / 8;
  if (per_xcd > need) per_xcd = need;
  a.per_xcd = per_xcd;
  if (a.out_f32)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(8 * per_xcd), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(8 * per_xcd), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
