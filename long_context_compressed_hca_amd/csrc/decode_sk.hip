// decode_sk.hip - HCA decode attention on gfx950 with the keys split across
// waves and, for small batches, across workgroups (split-K), the partial
// softmax states combined by an LDS reduction inside the workgroup and by a
// second kernel across workgroups.
//
// What is computed (aitest123.com, "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B",
// section 模型结构; lininn.cn, section 43 层里，37 层只读摘要; blog.derekhsu.net,
// section 低秩閘控注意力): for sequence b with new token(s) from position t, a
// query row of token j (position t + j) attends to the floor((t+j+1)/128)
// cached entries and to the raw rows of positions max(0, t+j-127) .. t+j; the
// output is gated by sigmoid(G).  One new token: its row is in the ring slot
// t % 128.  M new tokens (MT): the ring holds committed rows below t and the
// new rows come in nk, nv [B, M, 512].
//
// Decomposition.  A workgroup takes one sequence, one block of 16 query rows
// (rows 16hb .. 16hb+15 of the sequence's M*H rows; rows past M*H are padding)
// and one key split ks of n_ks.  The key list of the sequence is cut into
// 16-key tiles (entries, then ring rows, then for MT the new rows), and tile j
// belongs to stream j % S, S = 4 n_ks; stream 4 ks + w is walked by wave w of
// split ks.  Each wave runs its own online softmax over its tiles, with no
// barrier in the key loop:
//   scores  S^T[key][row] = K Q^T: 16 MFMA 16x16x32, K fragments loaded
//           straight into registers (two tiles in flight), Q^T in registers;
//   softmax mask, tile maximum per row, weights 2^(x - m) rounded to bf16,
//           row sums of the rounded weights; the score layout is the value
//           product's B operand, so P never leaves the registers;
//   values  O^T[dim][row] += V^T P^T: 32 MFMA 16x16x16, V^T by transposing
//           LDS reads from the wave's own two V stages (LDS DMA).
// Softmax reference (as in prefill): each row's reference m is the maximum of
// the first tile of the stream with a visible key, and every key is weighed
// by 2^(x - m), so O is never rescaled.  If a score rises more than 2^64 above
// m (extreme score ranges only), the wave walks its stream a second time with
// the exact maximum of each row as reference.  At the end the four waves' (m, l, O) are combined: m* = max m_w,
// O = sum 2^(m_w - m*) O_w, l likewise, wave w finishing dims 128w..128w+127
// from the other waves' scaled partials exchanged through LDS.  With n_ks = 1
// the gate is applied and the output stored; otherwise the workgroup's
// (m*, l*, O) go to the workspace and combine_kernel merges the splits.
//
// Memory bound: per sequence (entries + window) * 2 KiB of K and V plus 3 KiB
// per query row of q, g and out.  The head blocks of a sequence run on one
// XCD, so each K/V byte comes from HBM once and from that XCD's L2 after.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kTile = 16;
constexpr int kVRow = 1024 + 64;            // V rows in LDS (conflict-free transpose reads)
constexpr int kStage = kTile * kVRow;        // one V stage: 17408 bytes
constexpr float kHeadroom = 64.0f;           // weights 2^(x - m) stay below 2^64 in a pass
constexpr int kPart = 32 + 16 * kD;          // floats per partial: m[16], l[16], O[16][512]

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

struct SkArgs {
  const uint16_t *q, *g, *ck, *cv, *wk, *wv, *nk, *nv;
  const int64_t* pos;
  void* out;
  float* ws;       // partials, n_ks > 1 only
  int64_t nc_cap;
  int B, H, M, R;  // R = M * H query rows per sequence
  int n_hb, n_ks;
  float c;         // scale * log2(e)
  int out_f32;
};

// The keys of one sequence, wave-uniform.
struct Seq {
  const uint16_t *ek, *ev, *wk, *wv, *nk, *nv;
  int nc;       // entries in the list
  int lo, nw;   // ring rows: positions lo .. lo+nw-1
  int n_et, n_rt, n_tiles, M;
};

// Tile j of the list: its kind (0 entries, 1 ring, 2 new rows), its first
// index in that segment and buffer descriptors of its K and V rows.  Entry
// rows past the last entry and new rows past the last read as zeros (range
// check); a tile past the list has empty descriptors (no memory is read).
struct Tile {
  __amdgpu_buffer_rsrc_t rk, rv;
  int kind, first;
};

__device__ __forceinline__ Tile tile_at(const Seq& s, int j) {
  Tile t;
  if (j < s.n_et) {
    t.kind = 0;
    t.first = kTile * j;
    const int rows = s.nc - t.first < kTile ? s.nc - t.first : kTile;
    t.rk = make_rsrc(s.ek + (int64_t)t.first * kD, rows * 1024);
    t.rv = make_rsrc(s.ev + (int64_t)t.first * kD, rows * 1024);
  } else if (j < s.n_et + s.n_rt) {
    t.kind = 1;
    t.first = kTile * (j - s.n_et);
    t.rk = make_rsrc(s.wk, kWindow * 1024);
    t.rv = make_rsrc(s.wv, kWindow * 1024);
  } else if (j < s.n_tiles) {
    t.kind = 2;
    t.first = 0;
    t.rk = make_rsrc(s.nk, s.M * 1024);
    t.rv = make_rsrc(s.nv, s.M * 1024);
  } else {
    t.kind = 0;
    t.first = 0;
    t.rk = make_rsrc(s.wk, 0);
    t.rv = make_rsrc(s.wv, 0);
  }
  return t;
}

// Row (within the tile's descriptor) of key kk of the tile.  Ring rows past
// the last valid position repeat it: finite data under a zero weight,
// whatever the unused ring slots hold.
__device__ __forceinline__ int key_row(const Seq& s, const Tile& t, int kk) {
  if (t.kind != 1) return kk;
  int w = t.first + kk;
  w = w < s.nw ? w : s.nw - 1;
  return (s.lo + w) & (kWindow - 1);
}

// K fragments of tile j into registers: lane (key l16, g4) gets dims
// 32ss + 8g4 .. +7 of the tile's key l16, ss = 0..15.
__device__ __forceinline__ void load_k(const Seq& s, int j, int l16, int g4, bf16x8 (&kf)[16]) {
  const Tile t = tile_at(s, j);
  const int off = key_row(s, t, l16) * 1024 + 16 * g4;
#pragma unroll
  for (int ss = 0; ss < 16; ++ss)
    kf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(t.rk, off + 64 * ss, 0, 0));
}

// V rows of tile j into an LDS stage by DMA: key row r at st + r * kVRow.
__device__ __forceinline__ void copy_v(const Seq& s, int j, int lane16, uint8_t* st) {
  const Tile t = tile_at(s, j);
#pragma unroll
  for (int r = 0; r < kTile; ++r)
    dma16_buf(t.rv, lane16 + key_row(s, t, r) * 1024, (lds_void*)(st + r * kVRow));
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

__device__ __forceinline__ float sigmoid(float g) {
  constexpr float kLog2e = 1.4426950408889634f;
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
}

// The MFMAs are inline asm so that the register files stay put: O^T and the
// two K tiles in the accumulator registers (K read as the A operand), Q^T,
// the score chain and the V^T fragments in VGPRs.  The compiler
// inserts no wait states around inline asm, so each MFMA carries the 2 that a
// VALU write of an operand needs in front (P is converted by VALU right
// before the value product; the compiler may also copy a fragment), and the
// last MFMA of the score chain the 16 that a VALU read of its result needs.
// Back-to-back MFMAs accumulating into the same registers need none.
__device__ __forceinline__ void mfma_s_first(f32x4& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "a"(k), "v"(q));
}
__device__ __forceinline__ void mfma_s(f32x4& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "a"(k), "v"(q));
}
__device__ __forceinline__ void mfma_s_last(f32x4& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 15"
               : "+v"(d)
               : "a"(k), "v"(q));
}
// O^T += V^T P^T for the 32 dim blocks of a tile, the V^T fragments read
// from the stage with transposing LDS reads.  One asm block: the reads, the
// waits for them and the MFMAs are ordered by hand (a group of 8 reads in
// flight while the previous group's MFMAs issue), and the compiler, which
// cannot see these LDS reads, inserts no wait for the stage's copies (the
// caller has waited for V(i) with vmcnt).  P is written by VALU well before
// (32 reads and a wait in between).  Every fragment has its own registers,
// so no read overwrites an operand of an MFMA still in flight.
__device__ __forceinline__ void pv_tile(f32x4 (&o)[32], uint32_t ad, const i16x4& p) {
  i16x4 t[32];
  asm volatile(
      "ds_read_b64_tr_b16 %[t0], %[ad] offset:0\n\t"
      "ds_read_b64_tr_b16 %[t1], %[ad] offset:32\n\t"
      "ds_read_b64_tr_b16 %[t2], %[ad] offset:64\n\t"
      "ds_read_b64_tr_b16 %[t3], %[ad] offset:96\n\t"
      "ds_read_b64_tr_b16 %[t4], %[ad] offset:128\n\t"
      "ds_read_b64_tr_b16 %[t5], %[ad] offset:160\n\t"
      "ds_read_b64_tr_b16 %[t6], %[ad] offset:192\n\t"
      "ds_read_b64_tr_b16 %[t7], %[ad] offset:224\n\t"
      "ds_read_b64_tr_b16 %[t8], %[ad] offset:256\n\t"
      "ds_read_b64_tr_b16 %[t9], %[ad] offset:288\n\t"
      "ds_read_b64_tr_b16 %[t10], %[ad] offset:320\n\t"
      "ds_read_b64_tr_b16 %[t11], %[ad] offset:352\n\t"
      "ds_read_b64_tr_b16 %[t12], %[ad] offset:384\n\t"
      "ds_read_b64_tr_b16 %[t13], %[ad] offset:416\n\t"
      "ds_read_b64_tr_b16 %[t14], %[ad] offset:448\n\t"
      "ds_read_b64_tr_b16 %[t15], %[ad] offset:480\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o0], %[t0], %[p], %[o0]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o1], %[t1], %[p], %[o1]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o2], %[t2], %[p], %[o2]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o3], %[t3], %[p], %[o3]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o4], %[t4], %[p], %[o4]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o5], %[t5], %[p], %[o5]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o6], %[t6], %[p], %[o6]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o7], %[t7], %[p], %[o7]\n\t"
      "ds_read_b64_tr_b16 %[t16], %[ad] offset:512\n\t"
      "ds_read_b64_tr_b16 %[t17], %[ad] offset:544\n\t"
      "ds_read_b64_tr_b16 %[t18], %[ad] offset:576\n\t"
      "ds_read_b64_tr_b16 %[t19], %[ad] offset:608\n\t"
      "ds_read_b64_tr_b16 %[t20], %[ad] offset:640\n\t"
      "ds_read_b64_tr_b16 %[t21], %[ad] offset:672\n\t"
      "ds_read_b64_tr_b16 %[t22], %[ad] offset:704\n\t"
      "ds_read_b64_tr_b16 %[t23], %[ad] offset:736\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o8], %[t8], %[p], %[o8]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o9], %[t9], %[p], %[o9]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o10], %[t10], %[p], %[o10]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o11], %[t11], %[p], %[o11]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o12], %[t12], %[p], %[o12]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o13], %[t13], %[p], %[o13]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o14], %[t14], %[p], %[o14]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o15], %[t15], %[p], %[o15]\n\t"
      "ds_read_b64_tr_b16 %[t24], %[ad] offset:768\n\t"
      "ds_read_b64_tr_b16 %[t25], %[ad] offset:800\n\t"
      "ds_read_b64_tr_b16 %[t26], %[ad] offset:832\n\t"
      "ds_read_b64_tr_b16 %[t27], %[ad] offset:864\n\t"
      "ds_read_b64_tr_b16 %[t28], %[ad] offset:896\n\t"
      "ds_read_b64_tr_b16 %[t29], %[ad] offset:928\n\t"
      "ds_read_b64_tr_b16 %[t30], %[ad] offset:960\n\t"
      "ds_read_b64_tr_b16 %[t31], %[ad] offset:992\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o16], %[t16], %[p], %[o16]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o17], %[t17], %[p], %[o17]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o18], %[t18], %[p], %[o18]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o19], %[t19], %[p], %[o19]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o20], %[t20], %[p], %[o20]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o21], %[t21], %[p], %[o21]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o22], %[t22], %[p], %[o22]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o23], %[t23], %[p], %[o23]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o24], %[t24], %[p], %[o24]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o25], %[t25], %[p], %[o25]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o26], %[t26], %[p], %[o26]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o27], %[t27], %[p], %[o27]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o28], %[t28], %[p], %[o28]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o29], %[t29], %[p], %[o29]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o30], %[t30], %[p], %[o30]\n\t"
      "v_mfma_f32_16x16x16_bf16 %[o31], %[t31], %[p], %[o31]"
      : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]),
        [o4] "+a"(o[4]), [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]),
        [o8] "+a"(o[8]), [o9] "+a"(o[9]), [o10] "+a"(o[10]), [o11] "+a"(o[11]),
        [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]), [o15] "+a"(o[15]),
        [o16] "+a"(o[16]), [o17] "+a"(o[17]), [o18] "+a"(o[18]), [o19] "+a"(o[19]),
        [o20] "+a"(o[20]), [o21] "+a"(o[21]), [o22] "+a"(o[22]), [o23] "+a"(o[23]),
        [o24] "+a"(o[24]), [o25] "+a"(o[25]), [o26] "+a"(o[26]), [o27] "+a"(o[27]),
        [o28] "+a"(o[28]), [o29] "+a"(o[29]), [o30] "+a"(o[30]), [o31] "+a"(o[31]),
        [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]),
        [t4] "=&v"(t[4]), [t5] "=&v"(t[5]), [t6] "=&v"(t[6]), [t7] "=&v"(t[7]),
        [t8] "=&v"(t[8]), [t9] "=&v"(t[9]), [t10] "=&v"(t[10]), [t11] "=&v"(t[11]),
        [t12] "=&v"(t[12]), [t13] "=&v"(t[13]), [t14] "=&v"(t[14]), [t15] "=&v"(t[15]),
        [t16] "=&v"(t[16]), [t17] "=&v"(t[17]), [t18] "=&v"(t[18]), [t19] "=&v"(t[19]),
        [t20] "=&v"(t[20]), [t21] "=&v"(t[21]), [t22] "=&v"(t[22]), [t23] "=&v"(t[23]),
        [t24] "=&v"(t[24]), [t25] "=&v"(t[25]), [t26] "=&v"(t[26]), [t27] "=&v"(t[27]),
        [t28] "=&v"(t[28]), [t29] "=&v"(t[29]), [t30] "=&v"(t[30]), [t31] "=&v"(t[31])
      : [ad] "v"(ad), [p] "v"(p)
      : "memory");
}
// Wait states for a VALU read of accumulators written by the MFMAs above.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15"); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// s_waitcnt vmcnt(48): at most three tiles' worth of this wave's 16-load
// groups (K(i+1), V(i+1), K(i+2)) in flight, so V(i) has landed.
__device__ __forceinline__ void wait_v() { __builtin_amdgcn_s_waitcnt(0xCF70); }

// LDS of a workgroup: two V stages per wave, the gate logits of its 16 rows
// (1040-byte rows: conflict-free reads), the waves' (m, l).
constexpr int kGRow = 1024 + 16;
constexpr int kLdsG = 8 * kStage;
constexpr int kLdsML = kLdsG + 16 * kGRow;
constexpr int kLdsBytes = kLdsML + 4 * 32 * 4;

template <bool MT>
__global__ void __launch_bounds__(256, 1) decode_sk_kernel(SkArgs a) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kLdsBytes];

  // blockIdx -> (sequence, key split, head block): XCD x = blockIdx % 8 takes
  // the (sequence, split) pairs x, x + 8, ... with all their head blocks, which
  // walk the same tiles at the same time and share them through that XCD's
  // L2.  The splits of one sequence go to different XCDs, so a small batch
  // still spreads over the whole GPU.
  const int L = blockIdx.x;
  const int k8 = L >> 3;
  const int pair = (k8 / a.n_hb) * 8 + (L & 7);
  const int hb = k8 % a.n_hb;
  const int b = pair / a.n_ks, ks = pair % a.n_ks;
  if (b >= a.B) return;
  const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4, lane16 = lane * 16;
  uint8_t* const st0 = lds + (2 * W) * kStage;
  uint8_t* const st1 = lds + (2 * W + 1) * kStage;
  uint8_t* const sG = lds + kLdsG;
  float* const sML = reinterpret_cast<float*>(lds + kLdsML);

  // Position of the first new token, clamped so that every index stays in
  // range (an out-of-contract position gives unspecified output, never an
  // out-of-bounds access).
  constexpr int64_t kTMax = 0x7FFFFFEF;
  int64_t t64 = a.pos[b];
  t64 = t64 < 0 ? 0 : (t64 > kTMax ? kTMax : t64);
  const int t = __builtin_amdgcn_readfirstlane((int)t64);
  Seq s;
  s.M = MT ? a.M : 1;
  s.nc = (int)(((int64_t)t + s.M) / kBlock);
  if ((int64_t)s.nc > a.nc_cap) s.nc = (int)a.nc_cap;
  s.lo = t - (kWindow - 1) > 0 ? t - (kWindow - 1) : 0;
  s.nw = MT ? t - s.lo : t - s.lo + 1;
  s.n_et = (s.nc + kTile - 1) / kTile;
  s.n_rt = (s.nw + kTile - 1) / kTile;
  s.n_tiles = s.n_et + s.n_rt + (MT ? 1 : 0);
  s.ek = a.ck + (int64_t)b * a.nc_cap * kD;
  s.ev = a.cv + (int64_t)b * a.nc_cap * kD;
  s.wk = a.wk + (int64_t)b * kWindow * kD;
  s.wv = a.wv + (int64_t)b * kWindow * kD;
  s.nk = MT ? a.nk + (int64_t)b * a.M * kD : nullptr;
  s.nv = MT ? a.nv + (int64_t)b * a.M * kD : nullptr;

  // This lane's query row (head block hb, row l16) and its visible keys:
  // entries below nc_row, ring rows from index rlo_row on, new rows up to tok.
  const int row = 16 * hb + l16;
  int tok = 0;
  if constexpr (MT) {
    tok = row / a.H;
    tok = tok < a.M - 1 ? tok : a.M - 1;
  }
  int nc_row = (t + tok + 1) / kBlock;
  nc_row = nc_row < s.nc ? nc_row : s.nc;
  int rlo_row = t + tok - (kWindow - 1) - s.lo;
  rlo_row = rlo_row > 0 ? rlo_row : 0;

  // In order: Q^T fragments (rows past R read as zeros), the gate logits of
  // rows 4W .. 4W+3 of the block into LDS, then the stream's first two tiles.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)b * a.R * kD, a.R * 1024);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + (int64_t)b * a.R * kD, a.R * 1024);
  bf16x8 qf[16];
#pragma unroll
  for (int ss = 0; ss < 16; ++ss)
    qf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, row * 1024 + 64 * ss + 16 * g4, 0, 0));
  sched_fence();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    dma16_buf(rg, (16 * hb + 4 * W + r) * 1024 + lane16, (lds_void*)(sG + (4 * W + r) * kGRow));
  sched_fence();

  // This wave's stream: tiles sid, sid + Sn, ...
  const int Sn = 4 * a.n_ks;
  const int sid = 4 * ks + W;
  const int n_my = s.n_tiles > sid ? (s.n_tiles - sid + Sn - 1) / Sn : 0;

  bf16x8 ka[16], kb[16];
  // The stream's first two tiles (issued again for a second pass).
  auto first_loads = [&]() {
    load_k(s, sid, l16, g4, ka);
    sched_fence();
    copy_v(s, sid, lane16, st0);
    sched_fence();
    load_k(s, sid + Sn, l16, g4, kb);
    sched_fence();
    copy_v(s, sid + Sn, lane16, st1);
    sched_fence();
  };
  first_loads();

  f32x4 o[32];
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f;
  bool fixed_m = false, over = false;
  // Lane's V^T transpose-read offset: key row 4g4 + l16/4, dims 4(l16 & 3) (+ 16 db).
  const int voff = (4 * g4 + (l16 >> 2)) * kVRow + 8 * (l16 & 3);

  // Tile i of the stream (tile j = sid + i * Sn of the list), K in kf and V in
  // stage st; loads tile i + 2 into the same places.  Issue order of this
  // wave's loads: ... K(i) V(i) K(i+1) V(i+1) [K(i+2) here, after the scores]
  // [V(i+2) here, after the value product].
  auto tile = [&](int i, bf16x8 (&kf)[16], uint8_t* st) {
    const int j = sid + i * Sn;
    f32x4 sc;
    mfma_s_first(sc, kf[0], qf[0]);
#pragma unroll
    for (int ss = 1; ss < 15; ++ss) mfma_s(sc, kf[ss], qf[ss]);
    mfma_s_last(sc, kf[15], qf[15]);
    sched_fence();
    load_k(s, j + 2 * Sn, l16, g4, kf);
    sched_fence();
    // Mask: key kk = 4g4 + r of the tile is visible to this lane's row iff
    // lo_v <= kk < hi_v.
    const Tile tm = tile_at(s, j);
    int lo_v = 0, hi_v;
    if (j >= s.n_tiles) {
      hi_v = 0;
    } else if (tm.kind == 0) {
      hi_v = nc_row - tm.first;
    } else if (tm.kind == 1) {
      lo_v = rlo_row - tm.first;
      hi_v = s.nw - tm.first;
    } else {
      hi_v = tok + 1;
    }
    float x[4], mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 4 * g4 + r;
      x[r] = kk >= lo_v && kk < hi_v ? sc[r] * a.c : -INFINITY;
      mt = fmaxf(mt, x[r]);
    }
    mt = xmax32(xmax16(mt));
    // Reference: the maximum of the row's first tile with a visible key.
    if (!fixed_m && m == -INFINITY) m = mt;
    mseen = fmaxf(mseen, mt);
    over |= mt > m + kHeadroom;
    const float mx = m == -INFINITY ? 0.0f : m;  // nothing visible yet: every weight 0
    const f32x4 e = {__builtin_amdgcn_exp2f(x[0] - mx), __builtin_amdgcn_exp2f(x[1] - mx),
                     __builtin_amdgcn_exp2f(x[2] - mx), __builtin_amdgcn_exp2f(x[3] - mx)};
    const bf16x4 pb = __builtin_convertvector(e, bf16x4);  // nearest even
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[0], pb[1]}, ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[2], pb[3]}, ones, l, false);
    const i16x4 pf = __builtin_bit_cast(i16x4, pb);
    // V(i) has landed once at most K(i+1), V(i+1), K(i+2) are in flight.
    sched_fence();
    wait_v();
    sched_fence();
    pv_tile(o, (uint32_t)(uintptr_t)(st + voff), pf);
    sched_fence();  // pv_tile has waited for its reads: the stage is free
    copy_v(s, j + 2 * Sn, lane16, st);
    sched_fence();
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < 32; ++db) o[db] = f32x4{};
    l = 0.0f;
    over = false;
    // Tiles in pairs (a past-the-end tile of an odd count has no visible key).
    for (int i = 0; i < n_my; i += 2) {
      tile(i, ka, st0);
      tile(i + 1, kb, st1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every load and copy of this wave has landed
    // A score more than 2^kHeadroom above its reference (extreme score
    // ranges only): walk the stream again with the exact maximum of each row.
    if (pass == 1 || __builtin_amdgcn_ballot_w64(over) == 0) break;
    m = mseen;
    fixed_m = true;
    first_loads();
  }
  mfma_drain();

  // ---- combine the four waves' states
  const float lsum = xsum32(xsum16(l));
  if (lane < 16) {
    sML[32 * W + lane] = m;
    sML[32 * W + 16 + lane] = lsum;
  }
  __syncthreads();
  float mw[4], lw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = sML[32 * w + l16];
    lw[w] = sML[32 * w + 16 + l16];
  }
  const float mstar = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
  float lstar = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    lstar += mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - mstar) * lw[w];
  const float fown = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mstar);
  // Wave W's scaled partials of the other waves' dims, into its own stages:
  // the block for wave w2 (its k-th other wave) at k * 8 KiB of st0 (k < 2)
  // or at st1.
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    if (w2 == W) continue;
    const int k = w2 < W ? w2 : w2 - 1;
    uint8_t* dst = k < 2 ? st0 + k * 8192 : st1;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<f32x4*>(dst + d * 1024 + lane16) = o[8 * w2 + d] * fown;
  }
  __syncthreads();
  f32x4 acc[8];
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    if (w2 != W) continue;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = o[8 * w2 + d] * fown;
  }
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    if (w2 == W) continue;
    const int k = W < w2 ? W : W - 1;  // W's index among w2's other waves
    const uint8_t* src = lds + (k < 2 ? (2 * w2) * kStage + k * 8192 : (2 * w2 + 1) * kStage);
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] += *reinterpret_cast<const f32x4*>(src + d * 1024 + lane16);
  }

  if (a.n_ks == 1) {
    // out = O / l * sigmoid(G) for dims 128W .. 128W+127 of this lane's row.
    const float inv = 1.0f / lstar;
    const int64_t rows0 = (int64_t)b * a.R;
    const uint8_t* grow = sG + l16 * kGRow + 256 * W + 8 * g4;
    if (a.out_f32) {
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc(static_cast<float*>(a.out) + rows0 * kD, a.R * 2048);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint2 g2 = *reinterpret_cast<const uint2*>(grow + 32 * d);
        const float gv[4] = {bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                             bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16)};
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(acc[d][e] * inv * sigmoid(gv[e]));
        store16_buf(ro, row * 2048 + 512 * W + 64 * d + 16 * g4, v);
      }
    } else {
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc(static_cast<uint16_t*>(a.out) + rows0 * kD, a.R * 1024);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint2 g2 = *reinterpret_cast<const uint2*>(grow + 32 * d);
        const float gv[4] = {bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                             bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16)};
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[d][e] * inv * sigmoid(gv[e]);
        const u32x2 v = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, ro, row * 1024 + 256 * W + 32 * d + 8 * g4, 0, 0);
      }
    }
  } else if (row < a.R) {
    // This workgroup's partial: m*, l* and O (relative to 2^m*) of its rows.
    float* part = a.ws + ((int64_t)(b * a.n_hb + hb) * a.n_ks + ks) * kPart;
    if (W == 0 && g4 == 0) {
      part[l16] = mstar;
      part[16 + l16] = lstar;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<f32x4*>(part + 32 + l16 * kD + 128 * W + 16 * d + 4 * g4) = acc[d];
  }
}

// Merge of the n_ks partials of each (sequence, head block): workgroup
// (b, hb, 64-dim chunk dc), thread (row t / 16, dims 64 dc + 4 (t % 16) .. +3).
// The splits' loads are independent, so they are in flight together.
__global__ void __launch_bounds__(256) combine_kernel(SkArgs a) {
  const int dc = blockIdx.x & 7, bh = blockIdx.x >> 3;
  const int b = bh / a.n_hb, hb = bh % a.n_hb;
  const int rr = threadIdx.x >> 4, d = 64 * dc + 4 * (threadIdx.x & 15);
  const int row = 16 * hb + rr;
  if (row >= a.R) return;
  const float* part = a.ws + (int64_t)(b * a.n_hb + hb) * a.n_ks * kPart;
  constexpr int kMaxSplits = 16;
  float mk[kMaxSplits];
  float mstar = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) {
    mk[k] = k < a.n_ks ? part[k * kPart + rr] : -INFINITY;
    mstar = fmaxf(mstar, mk[k]);
  }
  float lstar = 0.0f;
  f32x4 acc = {};
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) {
    if (k < a.n_ks) {
      const float f = mk[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk[k] - mstar);
      lstar += f * part[k * kPart + 16 + rr];
      acc += f * *reinterpret_cast<const f32x4*>(part + k * kPart + 32 + rr * kD + d);
    }
  }
  const float inv = 1.0f / lstar;
  const int64_t orow = (int64_t)b * a.R + row;
  const uint2 g2 = *reinterpret_cast<const uint2*>(a.g + orow * kD + d);
  const float gv[4] = {bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                       bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16)};
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = acc[e] * inv * sigmoid(gv[e]);
  if (a.out_f32)
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * kD + d) =
        make_float4(r[0], r[1], r[2], r[3]);
  else
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * kD + d) =
        make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
}

}  // namespace

int decode_splits(int B, int H, int64_t nc_cap) {
  if (B <= 0) return 1;
  const int64_t wgs = (int64_t)B * ((H + 15) / 16);
  if (wgs >= 128) return 1;
  int n = (int)(256 / wgs);  // so that B * blocks * n <= 256
  // at least two 16-key tiles per stream (4 streams per split)
  const int64_t tiles = (nc_cap + kTile - 1) / kTile + kWindow / kTile;
  const int64_t cap = tiles / 8 > 1 ? tiles / 8 : 1;
  if (n > cap) n = (int)cap;
  if (n > 16) n = 16;  // combine_kernel merges at most 16 splits
  return n < 1 ? 1 : n;
}

size_t decode_workspace_bytes(int B, int H, int64_t nc_cap) {
  const int n = decode_splits(B, H, nc_cap);
  if (n <= 1) return 0;
  return (size_t)B * ((H + 15) / 16) * n * kPart * sizeof(float);
}

hipError_t launch_decode_sk(const DecodeProblem& p, const uint16_t* nk, const uint16_t* nv, int M,
                            void* ws, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  const bool multi = nk != nullptr;
  SkArgs a;
  a.q = p.q;
  a.g = p.g;
  a.ck = p.ck;
  a.cv = p.cv;
  a.wk = p.wk;
  a.wv = p.wv;
  a.nk = nk;
  a.nv = nv;
  a.pos = p.pos;
  a.out = p.out;
  a.ws = static_cast<float*>(ws);
  a.nc_cap = p.nc_cap;
  a.B = p.B;
  a.H = p.H;
  a.M = multi ? M : 1;
  a.R = a.M * p.H;
  a.n_hb = (a.R + 15) / 16;
  a.n_ks = multi ? 1 : decode_splits(p.B, p.H, p.nc_cap);
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  const int64_t pairs = (int64_t)p.B * a.n_ks;
  const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * a.n_hb)), block(256);
  if (multi)
    hipLaunchKernelGGL((decode_sk_kernel<true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_sk_kernel<false>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_ks == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.B * a.n_hb * 8)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
