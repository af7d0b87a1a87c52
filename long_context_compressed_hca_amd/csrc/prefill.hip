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
// tile is copied once into LDS and read by the 4 waves; wave w owns rows
// 32w .. 32w+31 of the item with all 512 dims:
//   S^T[key][row] = K . Q^T      32 MFMA 32x32x16 (A = K from LDS, B = Q in VGPRs)
//   mask, softmax                each lane owns one row and 16 of the 32 keys
//   O^T[dv][row] += V^T . P^T    32 MFMA 32x32x16 (A = V^T via LDS transpose reads)
// Q (128 VGPRs) and O (256 accumulator registers) stay in registers for the
// whole item.  Computing the transposes keeps a row in one lane and makes P^T
// the B operand straight from the S^T accumulator layout.
//
// Persistent schedule.  The kernel runs one workgroup per CU; each workgroup
// loops over items, heaviest (latest positions, most entries) first.  Items
// are dealt so that the workgroups of one XCD take runs of adjacent items,
// whose raw windows overlap in that XCD's L2.
//
// Q, G and out move between HBM and registers through LDS (each wave stages
// its 32 rows in a 32 KiB region that aliases the idle tile stages between
// items): global traffic is whole 1 KiB rows, while the MFMA layouts spread
// a wave's registers over 32 rows.
//
// LDS: two stages x (K tile + V tile) x 32 rows x 1 KiB = 128 KiB.  Tiles are
// copied global -> LDS by DMA (buffer_load_dwordx4 ... lds, no VGPRs), one
// 1 KiB row per wave instruction, with an XOR swizzle of the 16-byte chunks
// chosen so the two read patterns are bank-conflict free:
//   K: chunk c of key r stored at c ^ (r & 15)   (b128 reads, 16 keys x 1 chunk)
//   V: chunk c of key r stored at c ^ 4(r & 3)   (b64 transpose reads, 4 keys x 4 chunks)
// The copy of tile i+1 is issued spread over tile i's MFMAs and is in flight
// while tile i is computed.  LDS fragments are read a few MFMAs ahead of use.
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
// f32 output.
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
typedef __attribute__((ext_vector_type(8))) short i16x8;

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
  int my_row_raw;      // this lane's row (may be past `last` in the final item)
  int my_row;          // clamped to `last`
  int t;               // this lane's query position
  int tw_min, tw_max;  // positions of this wave's first and last row
  int t_max;           // last position of the item
  int nc_wg;           // entries visible to the last row of the item
  int w_lo;            // first raw position of the item's window union
  int n_ct;            // compressed tiles
  int n_tiles;
};

__device__ __forceinline__ Item make_item(const Args& a, int idx, int wave, int l32) {
  Item it;
  it.row0 = idx * kRowsPerItem;
  it.last = (it.row0 + kRowsPerItem < a.rows ? it.row0 + kRowsPerItem : a.rows) - 1;
  const int wr0 = it.row0 + wave * 32 < it.last ? it.row0 + wave * 32 : it.last;
  const int wr1 = it.row0 + wave * 32 + 31 < it.last ? it.row0 + wave * 32 + 31 : it.last;
  it.my_row_raw = it.row0 + wave * 32 + l32;
  it.my_row = it.my_row_raw < it.last ? it.my_row_raw : it.last;
  it.t = a.q_start + it.my_row / a.H;
  it.tw_min = a.q_start + wr0 / a.H;
  it.tw_max = a.q_start + wr1 / a.H;
  const int t_min = a.q_start + it.row0 / a.H;
  it.t_max = a.q_start + it.last / a.H;
  it.nc_wg = n_entries(it.t_max, a.Nc);
  it.w_lo = t_min - (kWindow - 1) > 0 ? t_min - (kWindow - 1) : 0;
  it.n_ct = (it.nc_wg + kTile - 1) / kTile;
  it.n_tiles = it.n_ct + (it.t_max - it.w_lo + 1 + kTile - 1) / kTile;
  return it;
}

// First key (entry index or raw position) of tile `i`; kind 0 = entries, 1 = window.
__device__ __forceinline__ int tile_first(const Item& it, int i, int& kind) {
  if (i < it.n_ct) {
    kind = 0;
    return i * kTile;
  }
  kind = 1;
  return it.w_lo + (i - it.n_ct) * kTile;
}

// The copy of one 32-key tile into (sK, sV): buffer descriptors that cover
// exactly the tile's valid rows.  Each wave copies 8 of the 32 key rows of K and
// of V (dma_row); rows past the end repeat the last valid row (finite data;
// those keys are masked), so every LDS row of the tile is written.
struct TileCopy {
  __amdgpu_buffer_rsrc_t rk, rv;
  int nrows;
  uint8_t* sK;
  uint8_t* sV;
};

__device__ __forceinline__ TileCopy tile_copy(const Args& a, const Item& it, int i, uint8_t* sK,
                                              uint8_t* sV) {
  const uint8_t* kb;
  const uint8_t* vb;
  int first, last;
  if (i < it.n_ct) {
    kb = reinterpret_cast<const uint8_t*>(a.ck);
    vb = reinterpret_cast<const uint8_t*>(a.cv);
    first = i * kTile;
    last = it.nc_wg - 1;
  } else {
    kb = reinterpret_cast<const uint8_t*>(a.k);
    vb = reinterpret_cast<const uint8_t*>(a.v);
    first = it.w_lo + (i - it.n_ct) * kTile - a.kv_start;
    last = it.t_max - a.kv_start;
  }
  TileCopy c;
  c.nrows = last - first + 1 < kTile ? last - first + 1 : kTile;
  c.rk = make_rsrc(kb + (size_t)first * (kD * 2), c.nrows * kD * 2);
  c.rv = make_rsrc(vb + (size_t)first * (kD * 2), c.nrows * kD * 2);
  c.sK = sK;
  c.sV = sV;
  return c;
}

// Copy key row u (0..7) of this wave's share of a tile (two DMA instructions).
__device__ __forceinline__ void dma_row(const TileCopy& c, int u, int wave, int lane) {
  const int r = wave * (kTile / 4) + u;  // key row within the tile
  const int src = (r < c.nrows ? r : c.nrows - 1) * 1024;
  dma16_buf(c.rk, src + ((lane ^ (r & 15)) << 4), (lds_void*)(c.sK + r * 1024));
  dma16_buf(c.rv, src + ((lane ^ ((r & 3) << 2)) << 4), (lds_void*)(c.sV + r * 1024));
}

__device__ __forceinline__ void issue_tile(const Args& a, const Item& it, int i, uint8_t* sK,
                                           uint8_t* sV, int wave, int lane) {
  const TileCopy c = tile_copy(a, it, i, sK, sV);
#pragma unroll
  for (int u = 0; u < kTile / 4; ++u) dma_row(c, u, wave, lane);
}

// Copy this wave's 32 rows of a [rows, 512] bf16 tensor (rows row0w .. row0w+31)
// into the wave's 32 KiB LDS region, one 1 KiB row per instruction (coalesced),
// chunk c of row r stored at c ^ (r & 15).  Rows past `last` repeat `last`.
__device__ __forceinline__ void dma_rows(const uint16_t* base, int row0w, int last,
                                         uint8_t* region, int lane) {
  const int first = row0w < last ? row0w : last;
  const int nrows = last - first + 1 < 32 ? last - first + 1 : 32;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const uint8_t*>(base) + (size_t)first * (kD * 2), nrows * kD * 2);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int src = (r < nrows ? r : nrows - 1) * 1024;
    dma16_buf(rs, src + ((lane ^ (r & 15)) << 4), (lds_void*)(region + r * 1024));
  }
}

// Q fragments (B operand of S^T) from the wave's region: lane holds row l%32,
// dims 16ss + 8g .. +8, i.e. chunk 2ss+g of its row (same swizzle as K).
__device__ __forceinline__ void read_q(const uint8_t* region, int lane, bf16x8 (&qf)[32]) {
  const int l32 = lane & 31, g = lane >> 5;
  const uint8_t* row = region + l32 * 1024;
#pragma unroll
  for (int ss = 0; ss < 32; ++ss)
    qf[ss] = *reinterpret_cast<const bf16x8*>(
        row + 256 * (ss >> 3) + (((2 * (ss & 7) + g) ^ (l32 & 15)) << 4));
}

struct WaveState {
  f32x16 o[16];  // O^T accumulators: dv block b, lane row l%32
  float m;       // row reference max (exp2 domain), -inf before the first visible key
  float mseen;   // largest score of the row seen so far
  float l;       // this lane's partial row sum (its 16 keys of every tile)
  bool over;     // a score exceeded m + kHeadroom in this pass
};

// Process one 32-key tile.  kind 0: entries first .. first+31; kind 1: raw positions.
// If `copy_next`, the copy of the next tile (`nc`) is issued spread over this
// tile's MFMAs (one K and one V row every 4 MFMAs), so the vector memory path
// works in the background instead of stalling the wave's instruction issue.
__device__ __forceinline__ void compute_tile(const Args& a, WaveState& st, const bf16x8 (&qf)[32],
                                             const uint8_t* sK, const uint8_t* sV, int kind,
                                             int first, const Item& it, int lane, int wave,
                                             bool copy_next, const TileCopy& nc) {
  const int l32 = lane & 31, g = lane >> 5;
  bool need, full;
  if (kind == 0) {
    need = first < n_entries(it.tw_max, a.Nc);
    full = first + kTile <= n_entries(it.tw_min, a.Nc);
  } else {
    need = first <= it.tw_max && first + kTile - 1 >= it.tw_min - (kWindow - 1);
    full = first >= it.tw_max - (kWindow - 1) && first + kTile - 1 <= it.tw_min;
  }
  if (!need) {
    if (copy_next)
#pragma unroll
      for (int u = 0; u < kTile / 4; ++u) dma_row(nc, u, wave, lane);
    return;
  }

  // ---- S^T = K . Q^T.  Step ss reads chunk 2ss+g of key row l32, stored at
  // (2ss+g) ^ (l32&15); with ss = 8j + i that is 16j + ((2i + g) ^ (l32&15)),
  // so 8 lane offsets serve all steps (j becomes an immediate offset).
  f32x16 s = {};
  const uint8_t* krow = sK + l32 * 1024;
  int koff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) koff[i] = ((2 * i + g) ^ (l32 & 15)) << 4;
  constexpr int kAhead = 4;  // K fragments read this many MFMAs ahead
  bf16x8 kf[kAhead];
#pragma unroll
  for (int ss = 0; ss < kAhead; ++ss)
    kf[ss] = *reinterpret_cast<const bf16x8*>(krow + koff[ss & 7] + 256 * (ss >> 3));
#pragma unroll
  for (int ss = 0; ss < 32; ++ss) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ss % kAhead], qf[ss], s, 0, 0, 0);
    if (ss + kAhead < 32) {
      const int n = ss + kAhead;
      kf[ss % kAhead] = *reinterpret_cast<const bf16x8*>(krow + koff[n & 7] + 256 * (n >> 3));
    }
    if ((ss & 7) == 7 && copy_next) dma_row(nc, ss >> 3, wave, lane);
  }
#pragma unroll
  for (int ss = 0; ss < kAhead; ++ss) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int ss = 0; ss < 32; ++ss) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (ss + kAhead < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if ((ss & 7) == 7) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
  }

  // ---- mask, on tiles that some row of this wave sees only in part.  The
  // lane's visible keys form one interval [lo, hi] of this tile's key space.
  if (!full) {
    const int lo = kind == 0 ? 0 : it.t - (kWindow - 1);
    const int hi = kind == 0 ? n_entries(it.t, a.Nc) - 1 : it.t;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = first + 8 * (r >> 2) + 4 * g + (r & 3);
      s[r] = (key >= lo && key <= hi) ? s[r] : -INFINITY;
    }
  }

  // ---- softmax weights against the row's reference max (exp2 domain)
  float mt = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
  mt *= a.c;
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  st.mseen = fmaxf(st.mseen, mt);
  st.m = st.m == -INFINITY ? mt : st.m;  // fixed at the row's first visible key
  st.over |= mt > st.m + kHeadroom;
  const float msub = st.m == -INFINITY ? 0.0f : st.m;
  bf16x2 pk[8];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const f32x2 pr = {__builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -msub)),
                      __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], a.c, -msub))};
    pk[r >> 1] = __builtin_convertvector(pr, bf16x2);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(pk[r >> 1], ones, st.l, false);
  }

  // ---- O^T += V^T . P^T.  Transpose reads: in each 16-lane group, source lane
  // s16 addresses key row 4(lane/32) + s16/4 (+16 c2 + 8 r) and dims
  // 32b + 16((lane/16)&1) + 4(s16&3); the result lane holds 4 keys of one dim.
  const int s16 = lane & 15, q4 = lane >> 4;
  const int sw = (s16 >> 2) & 3;                      // V swizzle of those rows (4-chunk units)
  const int cbase = 2 * (q4 & 1) + ((s16 & 3) >> 1);  // + 4b
  const int half = (s16 & 1) << 3;
  // dv block b = 4j + i reads chunk (4b + cbase) ^ 4sw = 16j + 4(i ^ sw) + cbase
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = ((4 * (i ^ sw) + cbase) << 4) + half;
  bf16x8 pf[2];  // P^T for keys 0..15 and 16..31 of the tile (lane's row, slot order)
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pf[c2][2 * e] = pk[4 * c2 + e][0];
      pf[c2][2 * e + 1] = pk[4 * c2 + e][1];
    }
  const uint8_t* vbase = sV + (4 * (q4 >> 1) + (s16 >> 2)) * 1024;
  auto vread = [&](int n) -> bf16x8 {  // step n = 16 c2 + b
    const int c2 = n >> 4, b = n & 15;
    const uint8_t* p = vbase + 16384 * c2 + voff[b & 3] + 256 * (b >> 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8192));
    const i16x8 w8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w8);
  };
  constexpr int kV = 3;  // V fragments read this many MFMAs ahead
  bf16x8 vf[kV];
#pragma unroll
  for (int n = 0; n < kV; ++n) vf[n] = vread(n);
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    const int b = n & 15;
    st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n % kV], pf[n >> 4], st.o[b], 0, 0, 0);
    if (n + kV < 32) vf[n % kV] = vread(n + kV);
    if ((n & 7) == 7 && copy_next) dma_row(nc, 4 + (n >> 3), wave, lane);
  }
#pragma unroll
  for (int n = 0; n < kV; ++n) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    if (n + kV < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    if ((n & 7) == 7) __builtin_amdgcn_sched_group_barrier(0x020, 2, 1);
  }
}

// Epilogue for this lane's row, with the row's gate logits in the wave's LDS
// region: out = O / l * sigmoid(G).  Lane (row n, half g) owns dims
// 32b + 8i + 4g .. +3, i.e. bytes 8g.. of chunk 4b+i of row n.  bf16 output is
// written back over the logits it replaces (same size) and stored later as
// whole rows; f32 output is stored from registers.
template <bool kF32>
__device__ __forceinline__ void gate_rows(const Args& a, const WaveState& st, const Item& it,
                                          uint8_t* region, int lane, float inv) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int l32 = lane & 31, g = lane >> 5;
  uint8_t* row = region + l32 * 1024 + 8 * g;
#pragma unroll
  for (int b = 0; b < 16; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint8_t* p = row + 256 * (b >> 2) + (((4 * (b & 3) + i) ^ (l32 & 15)) << 4);
      const uint2 gw = *reinterpret_cast<const uint2*>(p);
      const float gv[4] = {bf16_bits_to_f32(gw.x & 0xFFFFu), bf16_bits_to_f32(gw.x >> 16),
                           bf16_bits_to_f32(gw.y & 0xFFFFu), bf16_bits_to_f32(gw.y >> 16)};
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
        r[e] = st.o[b][4 * i + e] * inv * sig;
      }
      if (kF32) {
        if (it.my_row_raw <= it.last)
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)it.my_row * kD +
                                     32 * b + 8 * i + 4 * g) = make_float4(r[0], r[1], r[2], r[3]);
      } else {
        const bf16x2 lo = __builtin_convertvector((f32x2){r[0], r[1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){r[2], r[3]}, bf16x2);
        *reinterpret_cast<uint2*>(p) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    }
  }
}

// Store the wave's bf16 output rows from its LDS region, one 1 KiB row per
// instruction (lane i writes chunk i of the row).
__device__ __forceinline__ void store_rows(const Args& a, int row0w, int last,
                                           const uint8_t* region, int lane) {
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if (row0w + r > last) break;  // wave-uniform
    const uint4 v = *reinterpret_cast<const uint4*>(region + r * 1024 + ((lane ^ (r & 15)) << 4));
    *reinterpret_cast<uint4*>(out + (size_t)(row0w + r) * kD + 8 * lane) = v;
  }
}

template <bool kF32>
__global__ void __launch_bounds__(256, 1) prefill_kernel(Args a) {
  // Separate arrays per stage: the compiler then knows a tile copy into one
  // stage cannot alias reads of the other and inserts no wait between them.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTile * 1024];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31;

  // Items in processing order p = 0, 1, ... are item n_items-1-p (heaviest
  // first).  Round r covers p in [r*G, (r+1)*G); within a round, XCD x (the
  // workgroups with blockIdx % 8 == x) takes the run of per_xcd adjacent items
  // starting at x*per_xcd.
  const int G = gridDim.x;
  int p = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
  if (p >= a.n_items) return;
  Item it = make_item(a, a.n_items - 1 - p, wave, l32);

  // The wave's 32 KiB staging region for its Q, gate and output rows (the
  // tile stages are free between items).
  uint8_t* const region = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;

  bf16x8 qf[32];
  dma_rows(a.q, it.row0 + wave * 32, it.last, region, lane);
  wait_vmem();
  read_q(region, lane, qf);
  __syncthreads();
  issue_tile(a, it, 0, sK0, sV0, wave, lane);

  for (;;) {
    WaveState st;
    st.m = -INFINITY;
    st.mseen = -INFINITY;
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int b = 0; b < 16; ++b) st.o[b] = f32x16{};
      st.l = 0.0f;
      st.over = false;
      if (pass > 0) issue_tile(a, it, 0, sK0, sV0, wave, lane);
      wait_vmem();
      __syncthreads();
      for (int i = 0; i < it.n_tiles; i += 2) {
        int kind, first;
        first = tile_first(it, i, kind);
        compute_tile(a, st, qf, sK0, sV0, kind, first, it, lane, wave, i + 1 < it.n_tiles,
                     tile_copy(a, it, i + 1, sK1, sV1));
        wait_vmem();
        __syncthreads();
        if (i + 1 >= it.n_tiles) break;
        first = tile_first(it, i + 1, kind);
        compute_tile(a, st, qf, sK1, sV1, kind, first, it, lane, wave, i + 2 < it.n_tiles,
                     tile_copy(a, it, i + 2, sK0, sV0));
        wait_vmem();
        __syncthreads();
      }
      // Only if some score rose more than 2^kHeadroom above its row reference
      // (possible only for extreme score ranges) is the pass repeated, with the
      // exact row maximum of the first pass as reference; that cannot overflow.
      if (pass == 1 || !__syncthreads_or(st.over)) break;
      st.m = st.mseen;
    }

    // Epilogue: gate logits in through LDS, output out through LDS (bf16),
    // then the next item's Q rows in through LDS; all transfers move whole
    // 1 KiB rows.  The regions alias the tile stages, which are idle here.
    const float l_tot = st.l + __shfl_xor(st.l, 32);
    const float inv = 1.0f / l_tot;
    dma_rows(a.g, it.row0 + wave * 32, it.last, region, lane);
    wait_vmem();
    gate_rows<kF32>(a, st, it, region, lane, inv);
    if (!kF32) store_rows(a, it.row0 + wave * 32, it.last, region, lane);
    p += G;
    const bool more = p < a.n_items;
    Item nx = it;
    if (more) {
      nx = make_item(a, a.n_items - 1 - p, wave, l32);
      dma_rows(a.q, nx.row0 + wave * 32, nx.last, region, lane);
      wait_vmem();
      read_q(region, lane, qf);
    }
    __syncthreads();  // every wave is done with its region
    if (more) issue_tile(a, nx, 0, sK0, sV0, wave, lane);
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
