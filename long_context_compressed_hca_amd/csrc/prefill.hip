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
// Pipeline.  Step i computes O += V(i) P(i), the softmax of tile i+1 (its
// scores carried in registers from the step before) and the scores of tile
// i+2; meanwhile DMA brings K(i+3) and V(i+1) into the stages freed by step
// i-1.  LDS: 2 K stages + 2 V stages (32 keys each) + 2 P buffers (8 KiB).
// Tiles are copied global -> LDS by DMA (buffer_load_dwordx4 ... lds, no
// VGPRs), one 1 KiB key row per wave instruction, into padded rows (K:
// 1040 bytes apart, V: 1088) that keep the operand reads bank-conflict free
// with immediate offsets.  The last two steps of an item compute no scores;
// they stage the next item's Q and the first gate logits through the stages
// they leave idle.
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
// f32 output.  Q, G and bf16 output move between HBM and LDS as 256-byte row
// quarters (LDS copies move several times more bytes per CU than loads into
// registers), gated one 32-row block at a time as their logits arrive.
//
// Roofline: 4*512 flop per (row, visible key); at 128K context the kernel is
// MFMA bound (about 420 flop per HBM byte).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kRowsPerItem = 128;
constexpr int kTile = 32;
// Bytes between key rows in the LDS stages.  The padding (16 bytes for K, 64
// for V) spreads the rows over the LDS banks so the MFMA operand reads are
// conflict free, and every read address is a per-lane base plus an immediate:
//   K: b128 reads of one 16-byte chunk by 16 consecutive key rows land in 16
//      different bank groups (row r starts 16 r bytes further round the banks);
//   V: transpose reads of 64 bytes from each of 4 consecutive key rows cover
//      all banks once (row r starts 64 r bytes further round).
constexpr int kKRow = 1024 + 16;
constexpr int kVRow = 1024 + 64;
constexpr float kHeadroom = 64.0f;  // p = 2^(x - m) stays below 2^64 in a pass

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

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
  int h_shift;                // log2(H) when H is a power of two, else -1
  float c;  // scale * log2(e)
  int out_f32;
  // VHA head mix (H = 64): up [64, rank], down [rank, 64], rank a multiple of 4 <= 32.
  const uint16_t* vha_up;
  const uint16_t* vha_down;
  int vha_rank;
  // Optional [Tq * H]: each row's log-sum-exp of its scores (natural log), the
  // statistic a training pass keeps for the backward.
  float* lse;
};

// Row -> query index (row / H), a shift when H is a power of two.
__device__ __forceinline__ int row_query(const Args& a, int row) {
  return a.h_shift >= 0 ? row >> a.h_shift : row / a.H;
}

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
  int wlen;            // raw positions in the window union
  int n_ct;            // compressed tiles
  int n_tiles;
  int e_full;          // tiles 0 .. e_full-1 and wf_lo .. wf_hi are seen in full
  int wf_lo, wf_hi;    // by every score row of the wave
};

__device__ __forceinline__ Item make_item(const Args& a, int idx, int wave, int l32) {
  Item it;
  it.row0 = idx * kRowsPerItem;
  it.last = (it.row0 + kRowsPerItem < a.rows ? it.row0 + kRowsPerItem : a.rows) - 1;
  const int r = it.row0 + wave * 32 + l32;
  it.my_row = r < it.last ? r : it.last;
  it.t = a.q_start + row_query(a, it.my_row);
  const int wr0 = it.row0 + wave * 32, wr1 = wr0 + 31;
  it.tw_min = a.q_start + row_query(a, wr0 < it.last ? wr0 : it.last);
  it.tw_max = a.q_start + row_query(a, wr1 < it.last ? wr1 : it.last);
  const int t_min = a.q_start + row_query(a, it.row0);
  it.t_max = a.q_start + row_query(a, it.last);
  it.nc_wg = n_entries(it.t_max, a.Nc);
  it.w_lo = t_min - (kWindow - 1) > 0 ? t_min - (kWindow - 1) : 0;
  it.wlen = it.t_max - it.w_lo + 1;
  it.n_ct = (it.nc_wg + kTile - 1) / kTile;
  it.n_tiles = it.n_ct + (it.wlen + kTile - 1) / kTile;
  // Entry tile i is full if its last entry is visible to the wave's first
  // row; window tile j (keys w_lo + 32j ..) if its keys lie within the
  // windows of both the wave's first and last rows.
  it.e_full = n_entries(it.tw_min, a.Nc) / kTile;
  const int x = it.tw_max - (kWindow - 1) - it.w_lo;  // first full: 32j >= x
  const int y = it.tw_min - (kTile - 1) - it.w_lo;    // last full: 32j <= y
  it.wf_lo = it.n_ct + (x <= 0 ? 0 : (x + kTile - 1) / kTile);
  it.wf_hi = it.n_ct + (y < 0 ? -1 : y / kTile);
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
  // Tile i is tile rel of the entries (rows 0 .. nc_wg-1) or of the window
  // (rows w_lo .. t_max); past the last tile it has no rows.
  const bool ent = i < it.n_ct;
  const int rel = ent ? i : i - it.n_ct;
  int n = (ent ? it.nc_wg : it.wlen) - rel * kTile;
  n = n < 0 ? 0 : n > kTile ? kTile : n;
  const uint16_t* base = ent ? (v ? a.cv : a.ck) : (v ? a.v : a.k);
  const int r0 = (ent ? 0 : it.w_lo - a.kv_start) + rel * kTile;
  TileSrc s;  // uniform values, kept in scalar registers so the descriptor is scalar
  s.rs = make_rsrc(base + (size_t)__builtin_amdgcn_readfirstlane(r0) * kD,
                   __builtin_amdgcn_readfirstlane(n * kD * 2));
  return s;
}

// Copy key row u (0..7) of this wave's quarter of a tile into a stage whose
// rows are kRow bytes apart; lane16 = 16 * lane.
template <int kRow>
__device__ __forceinline__ void dma_row(const TileSrc& s, uint8_t* stage, int u, int wave,
                                        int lane16) {
  const int r = wave * (kTile / 4) + u;
  dma16_buf(s.rs, lane16 + r * 1024, (lds_void*)(stage + r * kRow));
}

// 256-byte column slices of 32-row blocks move between HBM and 8 KiB LDS
// regions (row r at r*256, 16-byte chunk c stored at c ^ (r & 15)): the gate
// logits of row block rb, dims 128w .. 128w+127, for wave w; and quarter qq
// of the next item's Q (dims 128qq ..) of wave w's 32 score rows.
// Instruction j (0..7) moves rows 4j .. 4j+3.  The descriptor covers the
// item's rows of the block only, so rows past the last arrive as zeros (and
// stores there are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, const Item& it,
                                                             int rb) {
  const int r0 = it.row0 + 32 * rb;
  int n = it.last - r0 + 1;
  n = n < 0 ? 0 : n > 32 ? 32 : n;
  // Uniform values, kept in scalar registers so the descriptor is scalar.
  return make_rsrc(static_cast<const uint8_t*>(base) +
                       (size_t)__builtin_amdgcn_readfirstlane(r0) * (kD * 2),
                   __builtin_amdgcn_readfirstlane(n * (kD * 2)));
}
__device__ __forceinline__ void dma_rows(const __amdgpu_buffer_rsrc_t& rs, int j, int col,
                                         uint8_t* region, int lane) {
  const int r = 4 * j + (lane >> 4);
  dma16_buf(rs, r * 1024 + col + (((lane & 15) ^ (r & 15)) << 4), (lds_void*)(region + j * 1024));
}
// Q fragments qf[8qq .. 8qq+7] of the lane's score row from quarter qq staged
// by dma_rows: dims 128qq + 16j + 8(lane/32) .. +7 = chunk 2j + lane/32.
__device__ __forceinline__ void read_q_quarter(const uint8_t* region, int qq, int lane,
                                               bf16x8 (&qf)[32]) {
  asm volatile("" : "+v"(lane));  // addresses recomputed here, not kept across the loop
  const int l32 = lane & 31;
  const uint8_t* row = region + l32 * 256;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    qf[8 * qq + j] =
        *reinterpret_cast<const bf16x8*>(row + (((2 * j + (lane >> 5)) ^ (l32 & 15)) << 4));
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
  return i < it.e_full || (i >= it.wf_lo && i <= it.wf_hi);
}

// The score accumulator S^T is kept in VGPRs: the 256 accumulator registers
// hold O, and the MFMA builtins leave the accumulator's register file to the
// allocator, which then puts S^T in accumulator registers and moves O blocks
// out and back around every tile.  So the score MFMAs are written out with
// VGPR operands.  The compiler inserts no wait states around inline asm: the
// last MFMA of a chain carries the 20 that a VALU read of its result needs
// (the compiler itself emits 12 for this opcode), and no VALU instruction may
// write an operand within 2 wait states before one of these MFMAs (their
// operands come from LDS and global reads; a test checks the generated code
// for this).  A chain accumulating into the same registers issues back to
// back.  The first MFMA of a chain starts from the inline constant 0.
__device__ __forceinline__ void mfma_s_zero(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 3"
               : "+v"(d)
               : "v"(a), "v"(b));
}

// Lane-dependent byte offsets of the operand reads, computed once per kernel
// (the step adds the stage base, and for V the wave's 256-byte column):
//   k: K row lane%32, chunk lane/32 (k_row)
//   v: V^T transpose-read source of the lane (v_base)
//   p: 16 * lane (weights, copies)
struct LaneOff {
  int k, v, p;
};
__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int s16 = lane & 15, q4 = lane >> 4;
  LaneOff o;
  o.k = (lane & 31) * kKRow + 16 * (lane >> 5);
  o.v = (4 * (q4 >> 1) + (s16 >> 2)) * kVRow + 32 * (q4 & 1) + 8 * (s16 & 3);
  o.p = lane * 16;
  return o;
}

// K fragment of score MFMA ss for this lane (key row lane%32, k-slots
// 16ss + 8(lane/32) ..): krow = sK + LaneOff::k, fragment at krow + 32 ss.
__device__ __forceinline__ bf16x8 k_frag(const uint8_t* krow, int ss) {
  return *reinterpret_cast<const bf16x8*>(krow + 32 * ss);
}

// S^T (32 keys x the wave's 32 rows) = K . Q^T for the K tile in sK, with K
// fragments read kAhead MFMAs ahead; after_mfma(ss) places other work after
// MFMA ss.  The order of MFMAs and reads is fixed with scheduling barriers.
template <int kAhead, typename F>
__device__ __forceinline__ f32x16 qk_chain(const bf16x8 (&qf)[32], const uint8_t* sK, int koff,
                                           F&& after_mfma) {
  const uint8_t* krow = sK + koff;
  bf16x8 kf[kAhead];
#pragma unroll
  for (int ss = 0; ss < kAhead; ++ss) kf[ss] = k_frag(krow, ss);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s;
#pragma unroll
  for (int ss = 0; ss < 32; ++ss) {
    if (ss == 0)
      mfma_s_zero(s, kf[0], qf[0]);
    else if (ss == 31)
      mfma_s_last(s, kf[ss % kAhead], qf[ss]);
    else
      mfma_s_acc(s, kf[ss % kAhead], qf[ss]);
    if (ss + kAhead < 32) kf[ss % kAhead] = k_frag(krow, ss + kAhead);
    after_mfma(ss);
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
  f32x16 s;        // scores (-inf where the key is not visible)
  float mt;        // running max of the scores, then the row max (exp2 domain)
  float r0, r1;    // the row max of both wave halves
  float msub;      // the reference subtracted in the exponent
  f32x2 f[2];      // exponents of score pairs j (in f[j & 1])
  f32x2 e[2];      // their weights in fp32
  bf16x2 pk[8];    // the weights in bf16
};

__device__ __forceinline__ void sm_init(SoftmaxTile& x, const f32x16& s) {
  x.s = s;
  x.mt = -INFINITY;
}

// Mask tile i's scores: keys the lane's row does not see get -inf (score
// register r holds key 8(r/4) + 4(lane/32) + r%4 of the tile).  Tiles that
// every score row of the wave sees in full are left as they are (a
// wave-uniform branch), so only the few partial tiles of an item pay for it.
__device__ __forceinline__ void mask_scores(const Args& a, const Item& it, int i, int lane,
                                            f32x16& s) {
  if (tile_full(a, it, i)) return;
  const ScoreTile sc = score_tile(a, it, i);
  const unsigned width = (unsigned)sc.width;
  const int d0 = sc.first - sc.lo + 4 * (lane >> 5);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    s[r] = (unsigned)(d0 + 8 * (r >> 2) + (r & 3)) < width ? s[r] : -INFINITY;
}

// Parts of the softmax that a pipeline step places between its MFMAs:
//   max j (0..7)       running max over scores 2j, 2j+1
//   reduce 0..6        row max over both wave halves (lanes l and l^32 hold
//                      the same row) and the reference update: fixed at the
//                      row's first tile with a visible key
//   fma, exp, cvt, sum j (0..7)  weights of scores 2j, 2j+1: exponent,
//                      weight, bf16, added to the row sum
//   write c2 (0, 1)    the weights of key half c2 to LDS
__device__ __forceinline__ void sm_max(SoftmaxTile& x, int j) {
  x.mt = fmaxf(fmaxf(x.mt, x.s[2 * j]), x.s[2 * j + 1]);
}
// The row max reduction in single dependent operations (r = 0..6).
__device__ __forceinline__ void sm_reduce(const Args& a, WaveState& st, SoftmaxTile& x, int r) {
  switch (r) {
    case 0:
      x.mt *= a.c;
      break;
    case 1: {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.mt),
                                                       __float_as_uint(x.mt), false, false);
      x.r0 = __uint_as_float(sw[0]);
      x.r1 = __uint_as_float(sw[1]);
      break;
    }
    case 2:
      x.mt = fmaxf(x.r0, x.r1);
      break;
    case 3:
      st.mseen = fmaxf(st.mseen, x.mt);
      break;
    case 4:
      st.m = st.m == -INFINITY ? x.mt : st.m;
      break;
    case 5:
      st.over |= x.mt > st.m + kHeadroom;
      break;
    default:
      x.msub = st.m == -INFINITY ? 0.0f : st.m;
      break;
  }
}
// Weights of score pair j in four dependent stages, each placed a part
// (an MFMA) or more after the one before it.
__device__ __forceinline__ void sm_fma(const Args& a, SoftmaxTile& x, int j) {
  x.f[j & 1] = (f32x2){__builtin_fmaf(x.s[2 * j], a.c, -x.msub),
                       __builtin_fmaf(x.s[2 * j + 1], a.c, -x.msub)};
}
__device__ __forceinline__ void sm_exp(SoftmaxTile& x, int j) {
  x.e[j & 1] = (f32x2){__builtin_amdgcn_exp2f(x.f[j & 1][0]), __builtin_amdgcn_exp2f(x.f[j & 1][1])};
}
__device__ __forceinline__ void sm_cvt(SoftmaxTile& x, int j) {
  x.pk[j] = __builtin_convertvector(x.e[j & 1], bf16x2);
}
__device__ __forceinline__ void sm_sum(WaveState& st, const SoftmaxTile& x, int j) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
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

// The softmax parts of pipeline group k: part A goes between the group's
// score MFMA and its value MFMA, parts B and C after the value MFMA.
// Dependent instructions sit in different parts, an MFMA apart, and the
// exponentials are spread one pair per two groups.
//   group          part A              part B           part C
//   0..7           -                   max k            -
//   8..10          reduce 0, 2, 4      reduce 1, 3, 5   -
//   11             reduce 6            -                -
//   12, 14 .. 26   fma (k-12)/2        exp (k-12)/2     -
//   13, 15 .. 27   cvt (k-13)/2        -                sum (k-13)/2
//   21, 29         write 0, 1          -                -
__device__ __forceinline__ void sm_part_a(const Args& a, WaveState& st, SoftmaxTile& x,
                                          uint8_t* sP, int k, int lane, int wave) {
  if (k >= 8 && k < 11) sm_reduce(a, st, x, 2 * (k - 8));
  if (k == 11) sm_reduce(a, st, x, 6);
  if (k >= 12 && k < 28 && (k & 1) == 0) sm_fma(a, x, (k - 12) >> 1);
  if (k >= 13 && k < 29 && (k & 1) == 1) sm_cvt(x, (k - 13) >> 1);
  if (k == 21) sm_write(x, sP, 0, lane, wave);
  if (k == 29) sm_write(x, sP, 1, lane, wave);
}
__device__ __forceinline__ void sm_part_b(const Args& a, WaveState& st, SoftmaxTile& x, int k) {
  if (k < 8) sm_max(x, k);
  if (k >= 8 && k < 11) sm_reduce(a, st, x, 2 * (k - 8) + 1);
  if (k >= 12 && k < 28 && (k & 1) == 0) sm_exp(x, (k - 12) >> 1);
}
__device__ __forceinline__ void sm_part_c(WaveState& st, const SoftmaxTile& x, int k) {
  if (k >= 13 && k < 29 && (k & 1) == 1) sm_sum(st, x, (k - 13) >> 1);
}

// V^T fragments of PV block n = 4 c2 + bb (keys 16c2.., dims 128w + 32bb..)
// from the V tile in sV, by transpose reads: in each 16-lane group, source
// lane s16 addresses key row 4(lane/32) + s16/4 (+ 16 c2, + 8 for the second
// read) and dims 128w + 32bb + 16((lane/16)&1) + 4(s16&3); the result lane
// holds 4 keys of one dim.  vb = sV + LaneOff::v + 256 * wave.
__device__ __forceinline__ bf16x8 v_frag(const uint8_t* vb, int n) {
  const uint8_t* p = vb + 16 * kVRow * (n >> 2) + 64 * (n & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * kVRow));
  const i16x8 w8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w8);
}

// P^T fragment of row block rb, key half c2 (poff = 16 * lane).
__device__ __forceinline__ bf16x8 p_frag(const uint8_t* sP, int rb, int c2, int poff) {
  return *reinterpret_cast<const bf16x8*>(sP + poff + (rb * 2 + c2) * 1024);
}

// Step kinds.  A full step is the one described below.  The last two steps of
// an item have no scores left to compute (their score tiles lie past the last
// tile), so they compute none and leave the Q registers free: the next item's
// Q comes in through the stages they leave idle (each quarter of it in one
// stage, each wave's 32 rows x 256 bytes in its own 8 KiB of it), as do the
// gate logits of row block 2.  Tail steps run with stage parities 0, 1.
//   kFull:  O += V(i) P(i); softmax of tile i+1; scores of tile i+2; copies
//   kTailA: O += V(i) P(i); softmax of tile i+1; copy of V(i+1); next Q
//           quarters 0, 1 into K stages 0, 1
//   kTailB: O += V(i) P(i); next Q quarters 0, 1 into registers; quarters
//           2, 3 into the K stages; gate logits of row block 2 into V stage 0
enum StepKind { kFull, kTailA, kTailB };

// One step of the three-stage tile pipeline.  With tile i's weights P(i) in
// sP, V(i) in sV, K(i+2) in sK and the scores of tile i+1 in `carry`:
//   O += V(i) P(i)                         32 MFMAs (accumulator registers)
//   softmax of tile i+1 -> P(i+1) in sPn    VALU, in parts
//   carry = scores of tile i+2              32 MFMAs (one VGPR chain)
//   copies of K(i+3) into sKd, V(i+1) into sVd (empty past the last tile).
// The three parts are independent.  Group k issues score MFMA k, the K read
// three MFMAs ahead, softmax part A, then value MFMA k, one copy row (groups
// 5..20) and softmax part B; scheduling barriers keep that order, so the
// other instructions fill the MFMAs' issue gaps.  The V^T fragments are all
// read before the first copy: the compiler cannot tell transpose reads from
// the copies' LDS writes and would make a transpose read after a copy wait
// for every copy.
template <int kKind>
__device__ __forceinline__ void step(const Args& a, WaveState& st, bf16x8 (&qf)[32],
                                     f32x16& carry, const Item& it, int i, const uint8_t* sV,
                                     const uint8_t* sP, const uint8_t* sK, uint8_t* sPn,
                                     uint8_t* sKd, uint8_t* sVd, int lane, int wave,
                                     const __amdgpu_buffer_rsrc_t& qs, LaneOff lo, TileSrc& ks,
                                     TileSrc& vs) {
  asm volatile("" : "+v"(lane));
  asm volatile("" : "+s"(wave));  // per-row LDS addresses recomputed, not kept in registers
  asm volatile("" : "+v"(lo.k), "+v"(lo.v), "+v"(lo.p));  // one register each
  constexpr bool kScores = kKind == kFull;
  constexpr bool kSoftmax = kKind != kTailB;
  SoftmaxTile x;
  if (kSoftmax) sm_init(x, carry);
  constexpr int kAhead = 3;
  const uint8_t* krow = sK + lo.k;
  const uint8_t* vb = sV + lo.v + 256 * wave;
  bf16x8 kf[kAhead], vf[8], pf[4];
  // The operands of the first two MFMAs are read first.
  if (kScores) kf[0] = k_frag(krow, 0);
  vf[0] = v_frag(vb, 0);
  pf[0] = p_frag(sP, 0, 0, lo.p);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 1; n < (kScores ? 4 : 8); ++n) vf[n] = v_frag(vb, n);
  if (kScores) {
#pragma unroll
    for (int ss = 1; ss < kAhead; ++ss) kf[ss] = k_frag(krow, ss);
  }
#pragma unroll
  for (int rb = 1; rb < 4; ++rb) pf[rb] = p_frag(sP, rb, 0, lo.p);
  const int greg = wave * 8192;
  if (kKind == kTailB) {  // K stages: parity 1 has sKd = K stage 0
    read_q_quarter(sKd + greg, 0, lane, qf);
    read_q_quarter(sK + greg, 1, lane, qf);
  }
  if (kSoftmax) mask_scores(a, it, i + 1, lane, x.s);
  __builtin_amdgcn_sched_barrier(0);

  const int lane16 = lo.p;
  __amdgpu_buffer_rsrc_t gs;
  if (kKind == kTailB) gs = block_rsrc(a.g, it, 2);
  f32x16 s;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (kScores) {
      if (k == 0)
        mfma_s_zero(s, kf[0], qf[0]);
      else if (k == 31)
        mfma_s_last(s, kf[k % kAhead], qf[k]);
      else
        mfma_s_acc(s, kf[k % kAhead], qf[k]);
      if (k + kAhead < 32) kf[k % kAhead] = k_frag(krow, k + kAhead);
      if (k >= 1 && k < 5) vf[k + 3] = v_frag(vb, k + 3);
    }
    if (kSoftmax) sm_part_a(a, st, x, sPn, k, lane, wave);
    __builtin_amdgcn_sched_barrier(0);
    // value MFMA k: block n = k/4 (key half n/4, dim block n%4), row block k%4
    const int n = k >> 2, rb = k & 3;
    st.o[4 * (n & 3) + rb] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n], pf[rb], st.o[4 * (n & 3) + rb], 0, 0, 0);
    if (k >= 12 && k < 16) pf[rb] = p_frag(sP, rb, 1, lo.p);  // last use of half 0 was MFMA k
    // The copies use descriptors made by the previous step (ks: K(i+3), vs:
    // V(i+1)); this step makes the next step's in its MFMA-bound last groups.
    if (kScores) {
      if (k >= 5 && k < 13) dma_row<kKRow>(ks, sKd, k - 5, wave, lane16);
      if (k == 25) ks = tile_src(a, it, i + 4, false);
    }
    if (kSoftmax && k >= 13 && k < 21) dma_row<kVRow>(vs, sVd, k - 13, wave, lane16);
    if (kScores && k == 28) vs = tile_src(a, it, i + 2, true);
    // Tail A (parity 0): K stage 0 = sK, 1 = sKd.  Tail B (parity 1): K
    // stage 0 = sKd, 1 = sK; the quarters it copies overwrite the ones it
    // read into registers, so it waits for those reads first.
    if (kKind == kTailA && k < 8) dma_rows(qs, k, 0, const_cast<uint8_t*>(sK) + greg, lane);
    if (kKind == kTailA && k >= 8 && k < 16) dma_rows(qs, k - 8, 256, sKd + greg, lane);
    if (kKind == kTailB && k < 8) dma_rows(gs, k, 256 * wave, sVd + greg, lane);
    if (kKind == kTailB && k == 8) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (kKind == kTailB && k >= 8 && k < 16) dma_rows(qs, k - 8, 512, sKd + greg, lane);
    if (kKind == kTailB && k >= 16 && k < 24) dma_rows(qs, k - 16, 768, const_cast<uint8_t*>(sK) + greg, lane);
    if (kSoftmax) sm_part_b(a, st, x, k);
    if (kSoftmax) sm_part_c(st, x, k);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kScores) carry = s;
}

// Gate and normalise row block rb of the wave's output block (dims 128w..,
// rows 32rb + lane%32), with the gate logits of those rows staged in the
// wave's region by dma_g_rows.  bf16 output is written back over the logits
// (same size, same place) and stored by store_rb; f32 output is stored from
// registers.  The 16 logit pieces are read before any result is written back,
// so the reads are not ordered behind the writes.
//   out = O / l * sigmoid(G) = O / (l + l * 2^(-G log2 e))
// issue(j) runs at the start of output piece j: copies whose issue is spread
// over the gating, so that they leave the memory path room as they go.
template <bool kF32, typename F>
__device__ __forceinline__ void gate_rb(const Args& a, const WaveState& st, const Item& it, int rb,
                                        uint8_t* region, const float* sL, int lane, int wave,
                                        F&& issue) {
  asm volatile("" : "+v"(lane));
  constexpr float kLog2e = 1.4426950408889634f;
  const int l32 = lane & 31, g = lane >> 5;
  const float l = sL[32 * rb + l32];
  uint8_t* row = region + l32 * 256 + 8 * g;
  uint2 gw[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)  // j = 4 bb + q: dims 32bb + 8q + 4g .. +3
    gw[j] = *reinterpret_cast<const uint2*>(row + ((j ^ (l32 & 15)) << 4));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    issue(j);
    const int bb = j >> 2, q = j & 3;
    const float gv[4] = {bf16_bits_to_f32(gw[j].x & 0xFFFFu), bf16_bits_to_f32(gw[j].x >> 16),
                         bf16_bits_to_f32(gw[j].y & 0xFFFFu), bf16_bits_to_f32(gw[j].y >> 16)};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float den = __builtin_fmaf(l, __builtin_amdgcn_exp2f(-gv[e] * kLog2e), l);
      o[e] = st.o[4 * bb + rb][4 * q + e] * __builtin_amdgcn_rcpf(den);
    }
    if (kF32) {
      if (it.row0 + 32 * rb + l32 <= it.last)
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) +
                                   (size_t)(it.row0 + 32 * rb + l32) * kD + 128 * wave + 32 * bb +
                                   8 * q + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      const bf16x2 lo = __builtin_convertvector((f32x2){o[0], o[1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector((f32x2){o[2], o[3]}, bf16x2);
      // Written with inline asm: the compiler cannot tell this region from
      // the one the gate logits of row block 3 are being copied into, and
      // would make an ordinary LDS store wait for that copy.  The asm's
      // memory clobber keeps later LDS reads behind it.
      const u32x2 w2 = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      const uint32_t addr = (uint32_t)(uintptr_t)(row + ((j ^ (l32 & 15)) << 4));
      asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(w2) : "memory");
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Store row block rb of the wave's bf16 output block from its region, 4 row
// quarters (256 bytes each) per instruction.  The descriptor covers the
// item's rows of the block only, so stores of rows past the last are dropped.
__device__ __forceinline__ void store_rb(const Args& a, const Item& it, int rb,
                                         const uint8_t* region, int lane, int wave) {
  asm volatile("" : "+v"(lane));
  const __amdgpu_buffer_rsrc_t rs = block_rsrc(a.out, it, rb);
  const int c = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + r * 256 + ((c ^ (r & 15)) << 4));
    store16_buf(rs, r * 1024 + 256 * wave + 16 * c, v);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- VHA epilogue
// With the head mix (H = 64, so an item is two whole queries: row blocks 0, 1
// are the 64 heads of its first query, 2, 3 those of its second), every wave
// holds all heads of both queries for its 128 dims, and the mix of a query is
// two small products per 32-dim block bb:
//   Z^T[r][dim]  = Down[r][heads] . X[heads][dim]      (M = r padded to 32, K = 64 heads)
//   Y^T[dim][h] += Z[dim][r] . Up^T[r][h]              (M = 32 dims, K = 32, into O^T)
// X is the gated output, rounded to bf16, read back transposed from the rows
// gate_rb_vha wrote into the row blocks' regions; O^T holds the gated output
// in fp32 and takes the product as its accumulator (the identity skip).
// The k index of both products runs in the order the registers give:
// k-slot 8g + j (lane half g = lane / 32) is head / rank index
// 16s + 4g + j for j < 4 and 16s + 8 + 4g + (j - 4) for j >= 4, in K-step s.

// Gate row block rb as gate_rb does, keep the gated values in O^T (fp32)
// and write them, rounded to bf16, over the logits in the region.
__device__ __forceinline__ void gate_rb_vha(WaveState& st, int rb, uint8_t* region,
                                            const float* sL, int lane) {
  asm volatile("" : "+v"(lane));
  constexpr float kLog2e = 1.4426950408889634f;
  const int l32 = lane & 31, g = lane >> 5;
  const float l = sL[32 * rb + l32];
  uint8_t* row = region + l32 * 256 + 8 * g;
  uint2 gw[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)  // j = 4 bb + q: dims 32bb + 8q + 4g .. +3
    gw[j] = *reinterpret_cast<const uint2*>(row + ((j ^ (l32 & 15)) << 4));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bb = j >> 2, q = j & 3;
    const float gv[4] = {bf16_bits_to_f32(gw[j].x & 0xFFFFu), bf16_bits_to_f32(gw[j].x >> 16),
                         bf16_bits_to_f32(gw[j].y & 0xFFFFu), bf16_bits_to_f32(gw[j].y >> 16)};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float den = __builtin_fmaf(l, __builtin_amdgcn_exp2f(-gv[e] * kLog2e), l);
      o[e] = st.o[4 * bb + rb][4 * q + e] * __builtin_amdgcn_rcpf(den);
      st.o[4 * bb + rb][4 * q + e] = o[e];
    }
    const bf16x2 lo = __builtin_convertvector((f32x2){o[0], o[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){o[2], o[3]}, bf16x2);
    const u32x2 w2 = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    const uint32_t addr = (uint32_t)(uintptr_t)(row + ((j ^ (l32 & 15)) << 4));
    asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(w2) : "memory");
  }
  __builtin_amdgcn_sched_barrier(0);
}

// X fragment (B operand of Z^T = Down X) of K-step s for dim block bb, from
// the region of heads 32(s/2) ..: transpose reads, in each 16-lane group source
// lane s16 addressing region row 16(s&1) + 4(lane/32) + s16/4 (+ 8 for the
// second read) at dims 32bb + 16((lane/16)&1) + 4(s16&3), through the
// region's 16-byte chunk swizzle (chunk ^ (row & 15)).  Result lane: dim
// 32bb + lane%32, heads of k-slots 8g .. 8g+7.
__device__ __forceinline__ bf16x8 vha_x_frag(const uint8_t* region, int s, int bb, int lane) {
  const int s16 = lane & 15;
  const int d = 32 * bb + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  const int r0 = 16 * (s & 1) + 4 * (lane >> 5) + (s16 >> 2);
  const int r1 = r0 + 8;
  const uint8_t* p0 = region + r0 * 256 + (((d >> 3) ^ (r0 & 15)) << 4) + 2 * (d & 7);
  const uint8_t* p1 = region + r1 * 256 + (((d >> 3) ^ (r1 & 15)) << 4) + 2 * (d & 7);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  const i16x8 w8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w8);
}

// The down product's MFMAs: the score chain's VGPR-accumulator forms with
// the 2 wait states a VALU write of an operand needs in front (the compiler
// may pass a fragment through accumulator registers right before the MFMA).
__device__ __forceinline__ void mfma_z_zero(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_z_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_z_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 3"
               : "+v"(d)
               : "v"(a), "v"(b));
}

// 16 bytes at two 8-byte halves of a buffer (offsets past its size read 0).
__device__ __forceinline__ bf16x8 load_2x8(__amdgpu_buffer_rsrc_t rs, int off_lo, int off_hi) {
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_lo, 0, 0));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off_hi, 0, 0));
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// The factor fragments of the mix (the same for every query and wave):
//   dn[s]      A operand of Z^T: lane (r = l32, g), the heads of K-step s;
//   up[p][s2]  B operand of the mix: lane (head 32p + l32, g), the r of K-step s2.
struct VhaFrags {
  bf16x8 dn[4];
  bf16x8 up[2][2];
};
__device__ __forceinline__ void load_vha_frags(const Args& a, VhaFrags& f, int lane) {
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, g = lane >> 5;
  const int rank = a.vha_rank;
  // Down rows r >= rank lie past the buffer and read as zeros.
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.vha_down, rank * 64 * 2);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.vha_up, 64 * rank * 2);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int off = (l32 * 64 + 16 * s + 4 * g) * 2;
    f.dn[s] = load_2x8(rd, off, off + 16);
  }
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int r0 = 16 * s2 + 4 * g, r1 = r0 + 8;  // rank is a multiple of 4
      const int base = (32 * p + l32) * rank;
      f.up[p][s2] = load_2x8(ru, r0 < rank ? (base + r0) * 2 : 0x40000000,
                             r1 < rank ? (base + r1) * 2 : 0x40000000);
    }
}

// The head mix of query qq of the item (row blocks 2qq, 2qq+1, gated by
// gate_rb_vha into regions rlo, rhi).  The result replaces the gated output in
// O^T; bf16 output is written back into the regions for store_rb, f32 output
// is stored from registers.
// The caller loads the factor fragments one row block's gating ahead: kept
// live across the gating of the item's other query, they take registers the
// allocator then finds by moving O blocks to scratch.
template <bool kF32>
__device__ __forceinline__ void vha_query(const Args& a, WaveState& st, const Item& it, int qq,
                                          const VhaFrags& f, uint8_t* rlo, uint8_t* rhi, int lane,
                                          int wave) {
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, g = lane >> 5;
  const bf16x8 (&dn)[4] = f.dn;
  const bf16x8 (&up)[2][2] = f.up;
  // Z^T of one 32-dim block in VGPRs (with the builtin the allocator takes
  // accumulator registers for it and moves O blocks out of them); the last
  // MFMA carries the wait states of the VALU reads of the result.
  auto down_product = [&](int bb, f32x16& z) {
    mfma_z_zero(z, dn[0], vha_x_frag(rlo, 0, bb, lane));
    mfma_z_acc(z, dn[1], vha_x_frag(rlo, 1, bb, lane));
    mfma_z_acc(z, dn[2], vha_x_frag(rhi, 2, bb, lane));
    mfma_z_last(z, dn[3], vha_x_frag(rhi, 3, bb, lane));
  };
  // Block bb's up product follows block bb+1's down product, so the MFMAs of
  // one overlap the conversion of the other.
  f32x16 z;
  down_product(0, z);
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    // z: lane (dim 32bb + l32, g), register i = r 8(i/4) + 4g + i%4, so
    // registers 8s2 .. 8s2+7 are the k-slots of K-step s2 in the order above.
    bf16x8 za[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) za[s2][j] = (__bf16)z[8 * s2 + j];
    if (bb < 3) down_product(bb + 1, z);
    // Into the O^T block in its accumulator registers.  The s_nop gives the 2
    // wait states a VALU write of za (and of the block, in gate_rb_vha) needs
    // before an MFMA reads it.
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(st.o[4 * bb + 2 * qq + p])
                     : "v"(za[s2]), "v"(up[p][s2]));
  }
  // The wait states a VALU read of the last blocks written needs.
  asm volatile("s_nop 15\n\ts_nop 3");
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rb = 2 * qq + p;
    uint8_t* row = (p ? rhi : rlo) + l32 * 256 + 8 * g;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int bb = j >> 2, q = j & 3;
      const f32x4 o = {st.o[4 * bb + rb][4 * q], st.o[4 * bb + rb][4 * q + 1],
                       st.o[4 * bb + rb][4 * q + 2], st.o[4 * bb + rb][4 * q + 3]};
      if (kF32) {
        if (it.row0 + 32 * rb + l32 <= it.last)
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) +
                                     (size_t)(it.row0 + 32 * rb + l32) * kD + 128 * wave +
                                     32 * bb + 8 * q + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        const bf16x2 lo = __builtin_convertvector((f32x2){o[0], o[1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){o[2], o[3]}, bf16x2);
        const u32x2 w2 = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        const uint32_t addr = (uint32_t)(uintptr_t)(row + ((j ^ (l32 & 15)) << 4));
        asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(w2) : "memory");
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <bool kF32, bool kVha, bool kLse>
__global__ void __launch_bounds__(256, 1) prefill_kernel(Args a) {
  // Separate arrays per stage: the compiler then knows a copy into one stage
  // cannot alias reads of another and inserts no wait between them.
  __shared__ __attribute__((aligned(256))) uint8_t sK0[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sK1[kTile * kKRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV0[kTile * kVRow];
  __shared__ __attribute__((aligned(256))) uint8_t sV1[kTile * kVRow];
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

  // K(0) and K(1) of an item are copied ahead: for the first item here, for
  // the next item during the epilogue.
  auto first_k_copies = [&](const Item& x) {
    int ln = lane;  // recomputed lane-dependent offsets rather than kept across the loop
    asm volatile("" : "+v"(ln));
    const int ln16 = ln << 4;
    const TileSrc k0 = tile_src(a, x, 0, false), k1 = tile_src(a, x, 1, false);
#pragma unroll
    for (int u = 0; u < 8; ++u) dma_row<kKRow>(k0, sK0, u, wave, ln16);
#pragma unroll
    for (int u = 0; u < 8; ++u) dma_row<kKRow>(k1, sK1, u, wave, ln16);
  };
  // The wave's 8 KiB slice of an LDS stage for staged Q quarters and gate
  // logits (and bf16 output).
  const int greg = wave * 8192;

  const LaneOff lo = lane_offsets(lane);
  bf16x8 qf[32];
  load_q(q_row(a, it, wave, lane), 0, 32, qf);
  first_k_copies(it);

  for (;;) {
    WaveState st;
    st.m = -INFINITY;
    st.mseen = -INFINITY;
    p = next_p();
    const bool more = p >= 0;
    const Item nx = more ? make_item(a, a.n_items - 1 - p, wave, l32) : it;
    // The next item's Q rows of this wave (none past the last item).
    const __amdgpu_buffer_rsrc_t next_qs = make_rsrc(
        a.q + (size_t)__builtin_amdgcn_readfirstlane(nx.row0 + 32 * wave) * kD,
        more ? __builtin_amdgcn_readfirstlane(
                   (nx.last - nx.row0 - 32 * wave + 1 < 0    ? 0
                    : nx.last - nx.row0 - 32 * wave + 1 > 32 ? 32
                                                             : nx.last - nx.row0 - 32 * wave + 1) *
                   (kD * 2))
             : 0);
    for (int pass = 0;; ++pass) {
      st.l = 0.0f;
      st.over = false;
      // Steps: N = max(n_tiles, 2) of them (an item with a single tile runs a
      // second on a tile past its last, which adds zeros); the last two are
      // tail steps, the M = N - 2 before them full steps.  Step i reads V(i),
      // P(i) and K(i+2) from the stages of parity (i + M) & 1, so the tail
      // steps always use parities 0 and 1.
      const int M = (it.n_tiles > 2 ? it.n_tiles : 2) - 2;
      const bool odd = M & 1;
      // Prologue: scores of tiles 0 and 1; K(2) and V(0) in; weights of tile 0.
      f32x16 carry;
      TileSrc ks, vs;
      {
        if (pass) {
          load_q(q_row(a, it, wave, lane), 0, 32, qf);
          first_k_copies(it);
        }
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int ln16 = ln << 4;
        // This wave's copies of K(0), K(1) and its Q done, then everyone's.
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        barrier_no_fence();
        // The O accumulators are zeroed between the score MFMAs of tiles 0
        // and 1 (four registers after each), where the VALU is idle.
        auto zero4 = [&](int k) {
#pragma unroll
          for (int e = 0; e < 4; ++e) st.o[k >> 2][4 * (k & 3) + e] = 0.0f;
        };
        f32x16 s0 = qk_chain<4>(qf, sK0, (ln & 31) * kKRow + 16 * (ln >> 5),
                                [&](int ss) { zero4(ss); });
        carry = qk_chain<4>(qf, sK1, (ln & 31) * kKRow + 16 * (ln >> 5),
                            [&](int ss) { zero4(32 + ss); });
        barrier_no_fence();  // every wave's reads of K(0) are done
        const TileSrc k2 = tile_src(a, it, 2, false), v0 = tile_src(a, it, 0, true);
        uint8_t* const sK2 = odd ? sK1 : sK0;
        uint8_t* const sVs = odd ? sV1 : sV0;
        uint8_t* const sPs = odd ? sP1 : sP0;
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_row<kKRow>(k2, sK2, u, wave, ln16);
#pragma unroll
        for (int u = 0; u < 8; ++u) dma_row<kVRow>(v0, sVs, u, wave, ln16);
        ks = tile_src(a, it, 3, false);  // copies of the first step
        vs = tile_src(a, it, 1, true);
        mask_scores(a, it, 0, ln, s0);
        SoftmaxTile x;
        sm_init(x, s0);
#pragma unroll
        for (int k = 0; k < 30; ++k) {
          sm_part_a(a, st, x, sPs, k, ln, wave);
          sm_part_b(a, st, x, k);
          sm_part_c(st, x, k);
        }
        wait_vmem();
        __syncthreads();
      }
      // Full step i (parity p): V(i) in sV[p], P(i) in sP[p], K(i+2) in sK[p];
      // it writes P(i+1) into sP[1-p] and copies K(i+3) and V(i+1) into the
      // other stages.  With M odd, the first step runs in the parity-1 slot.
      int i = 0;
      bool slot0 = !odd;
      for (;;) {
        if (slot0) {
          if (i >= M) break;
          step<kFull>(a, st, qf, carry, it, i, sV0, sP0, sK0, sP1, sK1, sV1, lane, wave, next_qs, lo, ks, vs);
          wait_vmem();
          __syncthreads();
          ++i;
        }
        slot0 = true;
        if (i >= M) break;
        step<kFull>(a, st, qf, carry, it, i, sV1, sP1, sK1, sP0, sK0, sV0, lane, wave, next_qs, lo, ks, vs);
        wait_vmem();
        __syncthreads();
        ++i;
      }
      step<kTailA>(a, st, qf, carry, it, M, sV0, sP0, sK0, sP1, sK1, sV1, lane, wave, next_qs, lo, ks, vs);
      wait_vmem();
      __syncthreads();
      step<kTailB>(a, st, qf, carry, it, M + 1, sV1, sP1, sK1, sP0, sK0, sV0, lane, wave, next_qs, lo, ks, vs);
      wait_vmem();
      __syncthreads();
      // Only if some score rose more than 2^kHeadroom above its row reference
      // (possible only for extreme score ranges) is the pass repeated, with the
      // exact row maximum of the first pass as reference; that cannot overflow.
      // The tail steps have started on the next item's Q: the repeat loads
      // this item's again.
      if (pass == 1 || !__syncthreads_or(st.over)) break;
      st.m = st.mseen;
    }

    // Epilogue.  Row sums to every wave through LDS.  The next item's Q
    // quarters 2, 3 are read from the K stages, which then take the gate
    // logits of row blocks 0, 1; those of block 2 arrived during the last
    // step, those of block 3 are copied into V stage 1 now.  Blocks 2, 3 are
    // gated while the logits of 0, 1 arrive.
    read_q_quarter(sK0 + greg, 2, lane, qf);
    read_q_quarter(sK1 + greg, 3, lane, qf);
    {
      const float l_tot = st.l + __shfl_xor(st.l, 32);
      if (lane < 32) sL[wave * 32 + lane] = l_tot;
      // log-sum-exp of row 32 wave + lane: the weights are 2^(x - m), x the
      // scores in base-2 units, so ln sum = (m + log2 l) ln 2
      if (kLse && lane < 32 && it.row0 + wave * 32 + lane <= it.last)
        a.lse[it.row0 + wave * 32 + lane] =
            (st.m + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const __amdgpu_buffer_rsrc_t gs = block_rsrc(a.g, it, 3);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) dma_rows(gs, jj, 256 * wave, sV1 + greg, ln);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): row sums written, Q read
    barrier_no_fence();                  // everyone's
    // The gate logits of row blocks 0, 1 into the K stages (each wave its own
    // region): with the plain epilogue one row per output piece of block 2.
    const __amdgpu_buffer_rsrc_t g0 = block_rsrc(a.g, it, 0), g1 = block_rsrc(a.g, it, 1);
    auto copy_g01 = [&](int jj) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if (jj < 8)
        dma_rows(g0, jj, 256 * wave, sK0 + greg, ln);
      else
        dma_rows(g1, jj - 8, 256 * wave, sK1 + greg, ln);
    };
    if constexpr (!kVha) {
      auto none = [](int) {};
      gate_rb<kF32>(a, st, it, 2, sV0 + greg, sL, lane, wave, copy_g01);
      if (!kF32) store_rb(a, it, 2, sV0 + greg, lane, wave);
      gate_rb<kF32>(a, st, it, 3, sV1 + greg, sL, lane, wave, none);
      if (!kF32) store_rb(a, it, 3, sV1 + greg, lane, wave);
      gate_rb<kF32>(a, st, it, 0, sK0 + greg, sL, lane, wave, none);
      if (!kF32) store_rb(a, it, 0, sK0 + greg, lane, wave);
      gate_rb<kF32>(a, st, it, 1, sK1 + greg, sL, lane, wave, none);
      if (!kF32) store_rb(a, it, 1, sK1 + greg, lane, wave);
    } else {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) copy_g01(jj);
      // The item's second query (row blocks 2, 3) first: its logits are in.
      gate_rb_vha(st, 2, sV0 + greg, sL, lane);
      VhaFrags vf;
      load_vha_frags(a, vf, lane);  // in flight during the next gating
      gate_rb_vha(st, 3, sV1 + greg, sL, lane);
      vha_query<kF32>(a, st, it, 1, vf, sV0 + greg, sV1 + greg, lane, wave);
      if (!kF32) store_rb(a, it, 2, sV0 + greg, lane, wave);
      if (!kF32) store_rb(a, it, 3, sV1 + greg, lane, wave);
      gate_rb_vha(st, 0, sK0 + greg, sL, lane);
      load_vha_frags(a, vf, lane);
      gate_rb_vha(st, 1, sK1 + greg, sL, lane);
      vha_query<kF32>(a, st, it, 0, vf, sK0 + greg, sK1 + greg, lane, wave);
      if (!kF32) store_rb(a, it, 0, sK0 + greg, lane, wave);
      if (!kF32) store_rb(a, it, 1, sK1 + greg, lane, wave);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the K stages are done
    barrier_no_fence();                  // everyone's
    if (more) first_k_copies(nx);
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
  a.h_shift = (p.H & (p.H - 1)) == 0 ? __builtin_ctz((unsigned)p.H) : -1;
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  a.vha_up = p.vha_up;
  a.vha_down = p.vha_down;
  a.vha_rank = p.vha_rank;
  a.lse = p.lse;
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
  // The head mix needs whole queries per item: H = 64 (checked on the host).
  const bool vha = p.vha_rank > 0;
  if (vha && p.H != 64) return hipErrorInvalidValue;
  const dim3 grid(8 * per_xcd), block(256);
  // The row log-sum-exp is written by its own variants (not with the mix).
  if (a.lse != nullptr && vha) return hipErrorInvalidValue;
  if (a.lse != nullptr && a.out_f32)
    hipLaunchKernelGGL((prefill_kernel<true, false, true>), grid, block, 0, stream, a);
  else if (a.lse != nullptr)
    hipLaunchKernelGGL((prefill_kernel<false, false, true>), grid, block, 0, stream, a);
  else if (a.out_f32 && vha)
    hipLaunchKernelGGL((prefill_kernel<true, true, false>), grid, block, 0, stream, a);
  else if (a.out_f32)
    hipLaunchKernelGGL((prefill_kernel<true, false, false>), grid, block, 0, stream, a);
  else if (vha)
    hipLaunchKernelGGL((prefill_kernel<false, true, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<false, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
