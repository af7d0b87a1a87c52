// backward.hip - backward pass of HCA prefill attention on gfx950 (the training
// pass; the pages' attention kernel is measured on both passes:
// blog.derekhsu.net, section 訓練基礎設施).
//
// Whole sequence: queries and raw rows at positions 0 .. T-1, entries of the
// Nc = floor(T / 128) completed blocks (the forward's ck, cv).  For one query
// row (t, h), with x_j = scale <q, k_j> over its visible keys (entries b with
// 128 b + 127 <= t, raw rows t-127 .. t), p = softmax(x), a = sum_j p_j v_j,
// sig = sigmoid(g), o = a * sig and the upstream gradient dO:
//   dg = dO * a * sig (1 - sig),  da = dO * sig,  Dt = <da, a>,
//   ds_j = p_j (<da, v_j> - Dt),  dq = scale sum_j ds_j k_j,
//   dk_j += scale ds_j q,  dv_j += p_j da,
// and an entry's gradient reaches each row of its block divided by 128 (the
// derivative of the mean).
//
// Kernels (one wave = 16 query rows, or 16 keys; four waves per workgroup,
// each on its own work with its own LDS):
//   rows_kernel   per 16 flat rows (t, h): dA = dO * sig rounded to bf16 (kept
//                 in the workspace for the key kernel); pass A walks the keys
//                 with the decode kernel's fixed-reference softmax for the row
//                 sum, a (for dg) and Dt = sum_j p_j <dA, v_j> from the same dA
//                 and p the score gradients use, so that they sum to zero to fp32
//                 rounding; then dg, the row statistics lse and Dt; pass B walks
//                 the keys again for dq: S^T = K Q^T, P = 2^(x - lse),
//                 dP^T = V dA^T, dS^T = P (dP^T - Dt), dQ^T += K^T dS^T (K^T by
//                 transposing LDS reads);
//   keys_kernel   per 16 keys (raw rows, or entries with a chunk of queries):
//                 over the row blocks that see them, S = Q K^T, dP = dA V^T,
//                 dS, then dV^T += dA^T P and dK^T += Q^T dS with Q and dA rows
//                 copied into LDS and read transposed; raw keys are stored,
//                 entries are added atomically (several chunks per entry);
//   pool_kernel   dk, dv of raw rows += entry gradients / 128.
// fp32 accumulation throughout; MFMA operands are bf16 (P, dS and dA rounded
// to nearest even; P as in the forward).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kTile = 16;
constexpr int kRow = 1024 + 64;          // LDS rows read transposed (conflict free)
constexpr int kStage = kTile * kRow;     // 17408 bytes
constexpr float kHeadroom = 64.0f;
constexpr int kChunk = 4096;             // queries per entry task

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

struct BwArgs {
  const uint16_t *q, *g, *k, *v, *ck, *cv, *dout;
  float *dq, *dg, *dk, *dv;
  float *lse, *dt, *dck, *dcv;  // workspace: row statistics, entry gradients
  uint16_t* da;                 // workspace: dA rows, bf16 [T * H, 512]
  int64_t T;
  int H, Nc, n_rb;              // rows blocks of 16 flat rows
  int n_raw_tiles, n_ent_tasks, ent_chunks;
  float c, scale;               // c = scale * log2(e)
};

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
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// s_waitcnt vmcnt(0) / vmcnt(16) (vmcnt in bits 3:0 and 15:14), then a compiler
// barrier so that no memory access moves across the wait.
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vm16() {
  __builtin_amdgcn_s_waitcnt(0x4F70);
  asm volatile("" ::: "memory");
}

// The MFMAs are inline asm, so that accumulators and operands keep their
// register files (see decode_sk.hip): each carries the 2 wait states a VALU
// write of an operand needs, and the last of a chain the 16 a VALU read of its
// result needs.
//   score chain: d (VGPR) = A (VGPR) * B (AGPR)
__device__ __forceinline__ void mfma_va_first(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_va(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_va_last(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 15" : "+v"(d) : "v"(a), "a"(b));
}
//   same with both operands in VGPRs
__device__ __forceinline__ void mfma_vv_first(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vv(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vv_last(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 15" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15"); }

// O^T[512 dims x 16] += M^T P for a 16-row LDS tile M (rows kRow apart) read
// with transposing reads, P (B operand, keys x columns) in registers; the
// accumulators stay in AGPRs.  One asm block orders the 32 reads, their waits
// and the 32 MFMAs (8 reads in flight while the previous 8 MFMAs issue).
__device__ __forceinline__ void tr_tile(f32x4 (&o)[32], uint32_t ad, const i16x4& p) {
  i16x4 t[32];
#define HCA_RD(i) "ds_read_b64_tr_b16 %[t" #i "], %[ad] offset:" #i "*32\n\t"
#define HCA_MF(i) "v_mfma_f32_16x16x16_bf16 %[o" #i "], %[t" #i "], %[p], %[o" #i "]\n\t"
  asm volatile(
      HCA_RD(0) HCA_RD(1) HCA_RD(2) HCA_RD(3) HCA_RD(4) HCA_RD(5) HCA_RD(6) HCA_RD(7)
      HCA_RD(8) HCA_RD(9) HCA_RD(10) HCA_RD(11) HCA_RD(12) HCA_RD(13) HCA_RD(14) HCA_RD(15)
      "s_waitcnt lgkmcnt(8)\n\t"
      HCA_MF(0) HCA_MF(1) HCA_MF(2) HCA_MF(3) HCA_MF(4) HCA_MF(5) HCA_MF(6) HCA_MF(7)
      HCA_RD(16) HCA_RD(17) HCA_RD(18) HCA_RD(19) HCA_RD(20) HCA_RD(21) HCA_RD(22) HCA_RD(23)
      "s_waitcnt lgkmcnt(8)\n\t"
      HCA_MF(8) HCA_MF(9) HCA_MF(10) HCA_MF(11) HCA_MF(12) HCA_MF(13) HCA_MF(14) HCA_MF(15)
      HCA_RD(24) HCA_RD(25) HCA_RD(26) HCA_RD(27) HCA_RD(28) HCA_RD(29) HCA_RD(30) HCA_RD(31)
      "s_waitcnt lgkmcnt(8)\n\t"
      HCA_MF(16) HCA_MF(17) HCA_MF(18) HCA_MF(19) HCA_MF(20) HCA_MF(21) HCA_MF(22) HCA_MF(23)
      "s_waitcnt lgkmcnt(0)\n\t"
      HCA_MF(24) HCA_MF(25) HCA_MF(26) HCA_MF(27) HCA_MF(28) HCA_MF(29) HCA_MF(30) HCA_MF(31)
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
#undef HCA_RD
#undef HCA_MF
}

// ---------------------------------------------------------------- key lists
// The keys of a block of 16 flat rows whose queries run from t_lo to t_hi:
// entry tiles (entries 0 .. nc-1, nc = (t_hi + 1) / 128), then raw tiles
// (positions lo .. t_hi, lo = max(0, t_lo - 127)).
struct Keys {
  int nc, lo, nraw, n_et, n_tiles;
};
__device__ __forceinline__ Keys keys_of(int t_lo, int t_hi, int Nc) {
  Keys s;
  s.nc = (t_hi + 1) / kBlock;
  s.nc = s.nc < Nc ? s.nc : Nc;
  s.lo = t_lo - (kWindow - 1) > 0 ? t_lo - (kWindow - 1) : 0;
  s.nraw = t_hi - s.lo + 1;
  s.n_et = (s.nc + kTile - 1) / kTile;
  s.n_tiles = s.n_et + (s.nraw + kTile - 1) / kTile;
  return s;
}
// Tile j: buffer of its K (or V) rows (rows past the valid ones read as zeros)
// and its first key (entry index or position).
struct TileSrc {
  __amdgpu_buffer_rsrc_t r;
  bool ent;
  int first;
};
__device__ __forceinline__ TileSrc tile_src(const Keys& s, int j, const uint16_t* ent,
                                            const uint16_t* raw) {
  TileSrc t;
  t.ent = j < s.n_et;
  if (t.ent) {
    t.first = kTile * j;
    const int rows = s.nc - t.first < kTile ? s.nc - t.first : kTile;
    t.r = make_rsrc(ent + (int64_t)t.first * kD, rows * 1024);
  } else {
    t.first = s.lo + kTile * (j - s.n_et);
    const int rows = s.lo + s.nraw - t.first < kTile ? s.lo + s.nraw - t.first : kTile;
    t.r = make_rsrc(raw + (int64_t)t.first * kD, rows * 1024);
  }
  return t;
}
// 16 fragments of key row l16 (dims 32 ss + 8 g4 .. +7) into registers.
__device__ __forceinline__ void load_frags(__amdgpu_buffer_rsrc_t r, int l16, int g4,
                                           bf16x8 (&f)[16]) {
#pragma unroll
  for (int ss = 0; ss < 16; ++ss)
    f[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, l16 * 1024 + 64 * ss + 16 * g4, 0, 0));
}
// The 16 rows of a buffer into an LDS tile (rows kRow apart).
__device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t r, int lane16, uint8_t* st) {
#pragma unroll
  for (int rr = 0; rr < kTile; ++rr)
    dma16_buf(r, rr * 1024 + lane16, (lds_void*)(st + rr * kRow));
}

// ----------------------------------------------------------------- rows pass
__global__ void __launch_bounds__(256, 1) rows_kernel(BwArgs a) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[8 * kStage];
  const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = 4 * blockIdx.x + W;
  if (rb >= a.n_rb) return;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4, lane16 = lane * 16;
  uint8_t* const st[2] = {lds + (2 * W) * kStage, lds + (2 * W + 1) * kStage};
  const int64_t nrows = a.T * a.H;
  const int64_t r0 = (int64_t)rb * 16;
  const int nr = nrows - r0 < 16 ? (int)(nrows - r0) : 16;   // rows of the block
  const int64_t rmy = r0 + l16 < nrows ? r0 + l16 : nrows - 1;  // this lane's row (clamped)
  const bool valid = l16 < nr;
  const int t_my = (int)(rmy / a.H);
  const int t_lo = __builtin_amdgcn_readfirstlane((int)(r0 / a.H));
  const int t_hi = __builtin_amdgcn_readfirstlane((int)((r0 + nr - 1) / a.H));
  const Keys s = keys_of(t_lo, t_hi, a.Nc);
  const int nc_my = (t_my + 1) / kBlock < s.nc ? (t_my + 1) / kBlock : s.nc;
  const int lo_my = t_my - (kWindow - 1) > 0 ? t_my - (kWindow - 1) : 0;
  const int64_t ro = rmy * kD;

  // dA = dout * sigmoid(g) depends on the inputs alone: rounded to bf16 and
  // stored first (the key kernel reads it too), then read back as the B
  // operand of dP^T = V dA^T.  Lane (row l16, g4) handles dims 16 db + 4 g4.
  const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.da + r0 * kD, nr * 1024);
#pragma unroll 4
  for (int db = 0; db < 32; ++db) {
    const int d0 = 16 * db + 4 * g4;
    const uint2 g2 = *reinterpret_cast<const uint2*>(a.g + ro + d0);
    const uint2 o2 = *reinterpret_cast<const uint2*>(a.dout + ro + d0);
    const u32x2 w2 = {
        pack_bf16x2(bf16_bits_to_f32(o2.x & 0xFFFFu) * sigmoid(bf16_bits_to_f32(g2.x & 0xFFFFu)),
                    bf16_bits_to_f32(o2.x >> 16) * sigmoid(bf16_bits_to_f32(g2.x >> 16))),
        pack_bf16x2(bf16_bits_to_f32(o2.y & 0xFFFFu) * sigmoid(bf16_bits_to_f32(g2.y & 0xFFFFu)),
                    bf16_bits_to_f32(o2.y >> 16) * sigmoid(bf16_bits_to_f32(g2.y >> 16)))};
    __builtin_amdgcn_raw_buffer_store_b64(w2, rda, l16 * 1024 + 2 * d0, 0, 0);
  }
  wait_vm0();  // the stores have reached L2 (loads below bypass L1)
  bf16x8 daf[16], qf[16];
#pragma unroll
  for (int ss = 0; ss < 16; ++ss)
    daf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rda, l16 * 1024 + 64 * ss + 16 * g4, 0, 1));
  // Q^T fragments (B operand of the scores)
  load_frags(make_rsrc(a.q + r0 * kD, nr * 1024), l16, g4, qf);
  const int voff = (4 * g4 + (l16 >> 2)) * kRow + 8 * (l16 & 3);

  // visible range of key kk = 4 g4 + r of tile j: lo_v <= kk < hi_v
  auto vis = [&](int j, int& lo_v, int& hi_v) {
    if (j < s.n_et) {
      lo_v = 0;
      hi_v = nc_my - kTile * j;
    } else {
      const int p0 = s.lo + kTile * (j - s.n_et);
      lo_v = lo_my - p0;
      hi_v = t_my + 1 - p0;
    }
  };

  // ---- pass A: per row the maximum (fixed reference m), the weights
  // e_j = 2^(x_j - m) and, with them,
  //   l = sum e_j (fp32),  ldp = sum e_j dp_j,  dp_j = <dA, v_j>,
  //   the forward's ungated output a = (sum bf16(e_j) v_j) / (sum bf16(e_j)),
  // whence lse = m + log2 l and Dt = ldp / l = sum p_j dp_j: the same p and dp
  // the score gradients use, so that sum_j p_j (dp_j - Dt) = 0 holds to fp32
  // rounding (an exact-zero gradient stays zero).
  f32x4 o[32];
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f, lb = 0.0f, ldp = 0.0f;
  bool fixed_m = false, over = false;
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < 32; ++db) o[db] = f32x4{};
    l = lb = ldp = 0.0f;
    over = false;
    copy_rows(tile_src(s, 0, a.cv, a.v).r, lane16, st[0]);
    for (int j = 0; j < s.n_tiles; ++j) {
      bf16x8 kf[16], vf[16];
      sched_fence();
      load_frags(tile_src(s, j, a.ck, a.k).r, l16, g4, kf);
      load_frags(tile_src(s, j, a.cv, a.v).r, l16, g4, vf);
      if (j + 1 < s.n_tiles) copy_rows(tile_src(s, j + 1, a.cv, a.v).r, lane16, st[(j + 1) & 1]);
      sched_fence();
      f32x4 sc, dp;
      mfma_va_first(sc, kf[0], qf[0]);
#pragma unroll
      for (int ss = 1; ss < 15; ++ss) mfma_va(sc, kf[ss], qf[ss]);
      mfma_va_last(sc, kf[15], qf[15]);
      mfma_va_first(dp, vf[0], daf[0]);
#pragma unroll
      for (int ss = 1; ss < 15; ++ss) mfma_va(dp, vf[ss], daf[ss]);
      mfma_va_last(dp, vf[15], daf[15]);
      int lo_v, hi_v;
      vis(j, lo_v, hi_v);
      float x[4], mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 4 * g4 + r;
        x[r] = kk >= lo_v && kk < hi_v ? sc[r] * a.c : -INFINITY;
        mt = fmaxf(mt, x[r]);
      }
      mt = xmax32(xmax16(mt));
      if (!fixed_m && m == -INFINITY) m = mt;
      mseen = fmaxf(mseen, mt);
      over |= mt > m + kHeadroom;
      const float mx = m == -INFINITY ? 0.0f : m;
      f32x4 e;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = __builtin_amdgcn_exp2f(x[r] - mx);
        l += e[r];
        ldp += e[r] * dp[r];
      }
      const bf16x4 pb = __builtin_convertvector(e, bf16x4);
#pragma unroll
      for (int r = 0; r < 4; ++r) lb += (float)pb[r];
      // V(j) rows have landed once at most the 16 copies of V(j+1) (or the V(j)
      // fragment loads, on the last tile) are in flight.
      sched_fence();
      wait_vm16();
      sched_fence();
      tr_tile(o, (uint32_t)(uintptr_t)(st[j & 1] + voff), __builtin_bit_cast(i16x4, pb));
    }
    wait_vm0();
    if (pass == 1 || __builtin_amdgcn_ballot_w64(over) == 0) break;
    m = mseen;
    fixed_m = true;
  }
  mfma_drain();

  // ---- row statistics and dg
  const float lrow = xsum32(xsum16(l));
  const float inv_b = 1.0f / xsum32(xsum16(lb));
  const float lse = m + __builtin_amdgcn_logf(lrow);  // base 2: p_j = 2^(x_j - lse)
  const float dt = xsum32(xsum16(ldp)) / lrow;
  if (valid && g4 == 0) {
    a.lse[rmy] = lse;
    a.dt[rmy] = dt;
  }
#pragma unroll 4
  for (int db = 0; db < 32; ++db) {
    const int d0 = 16 * db + 4 * g4;
    const uint2 g2 = *reinterpret_cast<const uint2*>(a.g + ro + d0);
    const uint2 o2 = *reinterpret_cast<const uint2*>(a.dout + ro + d0);
    const float gv[4] = {bf16_bits_to_f32(g2.x & 0xFFFFu), bf16_bits_to_f32(g2.x >> 16),
                         bf16_bits_to_f32(g2.y & 0xFFFFu), bf16_bits_to_f32(g2.y >> 16)};
    const float dov[4] = {bf16_bits_to_f32(o2.x & 0xFFFFu), bf16_bits_to_f32(o2.x >> 16),
                          bf16_bits_to_f32(o2.y & 0xFFFFu), bf16_bits_to_f32(o2.y >> 16)};
    float dgv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = sigmoid(gv[e]);
      dgv[e] = dov[e] * (o[db][e] * inv_b) * sg * (1.0f - sg);
    }
    if (valid) *reinterpret_cast<float4*>(a.dg + ro + d0) = make_float4(dgv[0], dgv[1], dgv[2], dgv[3]);
  }

  // ---- pass B: dq
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4{};
  copy_rows(tile_src(s, 0, a.ck, a.k).r, lane16, st[0]);
  for (int j = 0; j < s.n_tiles; ++j) {
    bf16x8 kf[16], vf[16];
    sched_fence();
    load_frags(tile_src(s, j, a.ck, a.k).r, l16, g4, kf);
    load_frags(tile_src(s, j, a.cv, a.v).r, l16, g4, vf);
    if (j + 1 < s.n_tiles) copy_rows(tile_src(s, j + 1, a.ck, a.k).r, lane16, st[(j + 1) & 1]);
    sched_fence();
    f32x4 sc, dp;
    mfma_va_first(sc, kf[0], qf[0]);
#pragma unroll
    for (int ss = 1; ss < 15; ++ss) mfma_va(sc, kf[ss], qf[ss]);
    mfma_va_last(sc, kf[15], qf[15]);
    mfma_va_first(dp, vf[0], daf[0]);
#pragma unroll
    for (int ss = 1; ss < 15; ++ss) mfma_va(dp, vf[ss], daf[ss]);
    mfma_va_last(dp, vf[15], daf[15]);
    int lo_v, hi_v;
    vis(j, lo_v, hi_v);
    f32x4 ds;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 4 * g4 + r;
      const float p = kk >= lo_v && kk < hi_v ? __builtin_amdgcn_exp2f(sc[r] * a.c - lse) : 0.0f;
      ds[r] = p * (dp[r] - dt);
    }
    const bf16x4 db4 = __builtin_convertvector(ds, bf16x4);
    sched_fence();
    wait_vm16();  // K(j) rows in LDS: only K(j+1) (or this tile's V) may be in flight
    sched_fence();
    tr_tile(o, (uint32_t)(uintptr_t)(st[j & 1] + voff), __builtin_bit_cast(i16x4, db4));
  }
  wait_vm0();
  mfma_drain();
  if (valid) {
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const int d0 = 16 * db + 4 * g4;
      *reinterpret_cast<float4*>(a.dq + ro + d0) =
          make_float4(o[db][0] * a.scale, o[db][1] * a.scale, o[db][2] * a.scale, o[db][3] * a.scale);
    }
  }
}

// ----------------------------------------------------------------- keys pass
__global__ void __launch_bounds__(256, 1) keys_kernel(BwArgs a) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[8 * kStage];
  const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int task = 4 * blockIdx.x + W;
  if (task >= a.n_raw_tiles + a.n_ent_tasks) return;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4, lane16 = lane * 16;
  uint8_t* const sq = lds + (2 * W) * kStage;   // Q rows of the current row block
  uint8_t* const sa = lds + (2 * W + 1) * kStage;  // dA rows
  const int64_t nrows = a.T * a.H;

  // This task's 16 keys and the queries that can see them.
  const bool ent = task >= a.n_raw_tiles;
  int first, nkeys, t_from, t_to;
  if (!ent) {
    first = kTile * task;
    nkeys = a.T - first < kTile ? (int)(a.T - first) : kTile;
    t_from = first;
    t_to = first + nkeys - 1 + (kWindow - 1);
  } else {
    const int et = (task - a.n_raw_tiles) / a.ent_chunks, ch = (task - a.n_raw_tiles) % a.ent_chunks;
    first = kTile * et;
    nkeys = a.Nc - first < kTile ? a.Nc - first : kTile;
    t_from = kBlock * first + kBlock - 1;
    const int c0 = ch * kChunk;
    t_to = c0 + kChunk - 1;
    t_from = t_from > c0 ? t_from : c0;
  }
  t_to = t_to < a.T - 1 ? t_to : (int)(a.T - 1);
  if (t_from > t_to) return;  // an entry chunk before the entries' first query
  first = __builtin_amdgcn_readfirstlane(first);
  // K and V rows of the keys (B operands: lane (key l16, g4), dims 32 ss + 8 g4)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((ent ? a.ck : a.k) + (int64_t)first * kD, nkeys * 1024);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((ent ? a.cv : a.v) + (int64_t)first * kD, nkeys * 1024);
  bf16x8 kf[16], vf[16];
  load_frags(rk, l16, g4, kf);
  load_frags(rv, l16, g4, vf);
  // this lane's key (column l16 of S): first visible query
  const int key = first + l16;
  const int key_t0 = ent ? kBlock * key + kBlock - 1 : key;
  const bool key_ok = l16 < nkeys;

  f32x4 dk[32], dv[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    dk[db] = f32x4{};
    dv[db] = f32x4{};
  }
  const int voff = (4 * g4 + (l16 >> 2)) * kRow + 8 * (l16 & 3);
  {
    const int64_t rb0 = (int64_t)t_from * a.H / 16, rb1 = ((int64_t)t_to * a.H + a.H - 1) / 16;
    for (int64_t rb = rb0; rb <= rb1; ++rb) {
      const int64_t r0 = rb * 16;
      const int nr = nrows - r0 < 16 ? (int)(nrows - r0) : 16;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + r0 * kD, nr * 1024);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.da + r0 * kD, nr * 1024);
      sched_fence();
      copy_rows(rq, lane16, sq);
      copy_rows(rd, lane16, sa);
      // rows 4 g4 + r of the block: statistics (S layout: lane holds rows 4 g4 .. +3)
      float lse4[4], dt4[4];
      int t4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + 4 * g4 + r;
        const int64_t rr = row < nrows ? row : nrows - 1;
        lse4[r] = a.lse[rr];
        dt4[r] = a.dt[rr];
        t4[r] = row < nrows ? (int)(row / a.H) : -1;
      }
      wait_vm0();
      sched_fence();
      // S = Q K^T and dP = dA V^T, A operands (rows l16, dims 32 ss + 8 g4) from LDS
      f32x4 sc, dp;
      {
        bf16x8 qa[16];
#pragma unroll
        for (int ss = 0; ss < 16; ++ss)
          qa[ss] = *reinterpret_cast<const bf16x8*>(sq + l16 * kRow + 64 * ss + 16 * g4);
        mfma_vv_first(sc, qa[0], kf[0]);
#pragma unroll
        for (int ss = 1; ss < 15; ++ss) mfma_vv(sc, qa[ss], kf[ss]);
        mfma_vv_last(sc, qa[15], kf[15]);
      }
      {
        bf16x8 da[16];
#pragma unroll
        for (int ss = 0; ss < 16; ++ss)
          da[ss] = *reinterpret_cast<const bf16x8*>(sa + l16 * kRow + 64 * ss + 16 * g4);
        mfma_vv_first(dp, da[0], vf[0]);
#pragma unroll
        for (int ss = 1; ss < 15; ++ss) mfma_vv(dp, da[ss], vf[ss]);
        mfma_vv_last(dp, da[15], vf[15]);
      }
      // lane (key l16, g4) holds S[rows 4 g4 + r][key l16]
      f32x4 pp, ds;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t4[r];
        const bool v = key_ok && t >= 0 && t >= key_t0 && (ent || t - (kWindow - 1) <= key);
        const float p = v ? __builtin_amdgcn_exp2f(sc[r] * a.c - lse4[r]) : 0.0f;
        pp[r] = p;
        ds[r] = p * (dp[r] - dt4[r]);
      }
      const bf16x4 pb = __builtin_convertvector(pp, bf16x4);
      const bf16x4 dsb = __builtin_convertvector(ds, bf16x4);
      // dV^T += dA^T P, dK^T += Q^T dS (transposed LDS reads of the row tiles)
      tr_tile(dv, (uint32_t)(uintptr_t)(sa + voff), __builtin_bit_cast(i16x4, pb));
      tr_tile(dk, (uint32_t)(uintptr_t)(sq + voff), __builtin_bit_cast(i16x4, dsb));
      sched_fence();
    }
  }
  mfma_drain();
  // lane (key l16, g4) holds dims 16 db + 4 g4 .. +3 of key l16
  if (key_ok) {
    if (!ent) {
      float* dkr = a.dk + (int64_t)key * kD;
      float* dvr = a.dv + (int64_t)key * kD;
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const int d0 = 16 * db + 4 * g4;
        *reinterpret_cast<float4*>(dkr + d0) = make_float4(dk[db][0] * a.scale, dk[db][1] * a.scale,
                                                           dk[db][2] * a.scale, dk[db][3] * a.scale);
        *reinterpret_cast<float4*>(dvr + d0) = make_float4(dv[db][0], dv[db][1], dv[db][2], dv[db][3]);
      }
    } else {
      float* dkr = a.dck + (int64_t)key * kD;
      float* dvr = a.dcv + (int64_t)key * kD;
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const int d0 = 16 * db + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          atomicAdd(dkr + d0 + e, dk[db][e] * a.scale);
          atomicAdd(dvr + d0 + e, dv[db][e]);
        }
      }
    }
  }
}

// dk, dv of raw rows += the entry gradients of their block / 128; one thread
// per 4 dims of a row.
__global__ void pool_kernel(BwArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / (kD / 4);
  if (row >= (int64_t)a.Nc * kBlock) return;
  const int d0 = 4 * (int)(i % (kD / 4));
  const int64_t b = row / kBlock;
  const float4 ek = *reinterpret_cast<const float4*>(a.dck + b * kD + d0);
  const float4 ev = *reinterpret_cast<const float4*>(a.dcv + b * kD + d0);
  float4* pk = reinterpret_cast<float4*>(a.dk + row * kD + d0);
  float4* pv = reinterpret_cast<float4*>(a.dv + row * kD + d0);
  constexpr float s = 1.0f / kBlock;
  float4 x = *pk, y = *pv;
  x.x += ek.x * s; x.y += ek.y * s; x.z += ek.z * s; x.w += ek.w * s;
  y.x += ev.x * s; y.y += ev.y * s; y.z += ev.z * s; y.w += ev.w * s;
  *pk = x;
  *pv = y;
}

__global__ void zero_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

size_t backward_workspace_bytes(int64_t T, int H) {
  const int64_t rows = T * H, Nc = T / kBlock;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(rows * 4) * 2 + up(rows * kD * 2) + up(Nc * kD * 4) * 2 + 256;
}

hipError_t launch_backward(const BackwardProblem& p, void* ws, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  BwArgs a;
  a.q = p.q; a.g = p.g; a.k = p.k; a.v = p.v; a.ck = p.ck; a.cv = p.cv; a.dout = p.dout;
  a.dq = p.dq; a.dg = p.dg; a.dk = p.dk; a.dv = p.dv;
  a.T = p.T;
  a.H = p.H;
  a.Nc = (int)(p.T / kBlock);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t rows = p.T * p.H;
  uint8_t* w = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  a.lse = reinterpret_cast<float*>(w);
  w += up(rows * 4);
  a.dt = reinterpret_cast<float*>(w);
  w += up(rows * 4);
  a.da = reinterpret_cast<uint16_t*>(w);
  w += up(rows * kD * 2);
  a.dck = reinterpret_cast<float*>(w);
  w += up((size_t)a.Nc * kD * 4);
  a.dcv = reinterpret_cast<float*>(w);
  a.n_rb = (int)((rows + 15) / 16);
  a.n_raw_tiles = (int)((p.T + kTile - 1) / kTile);
  a.ent_chunks = (int)((p.T + kChunk - 1) / kChunk);
  a.n_ent_tasks = ((a.Nc + kTile - 1) / kTile) * a.ent_chunks;
  a.scale = p.scale;
  a.c = p.scale * 1.4426950408889634f;
  if (a.Nc > 0) {
    const unsigned blocks = (unsigned)(((int64_t)a.Nc * kD + 255) / 256);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, a.dck, (int64_t)a.Nc * kD);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, a.dcv, (int64_t)a.Nc * kD);
  }
  hipLaunchKernelGGL(rows_kernel, dim3((unsigned)((a.n_rb + 3) / 4)), dim3(256), 0, stream, a);
  const int tasks = a.n_raw_tiles + a.n_ent_tasks;
  hipLaunchKernelGGL(keys_kernel, dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, stream, a);
  if (a.Nc > 0) {
    const int64_t n = (int64_t)a.Nc * kBlock * (kD / 4);
    hipLaunchKernelGGL(pool_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace hca
