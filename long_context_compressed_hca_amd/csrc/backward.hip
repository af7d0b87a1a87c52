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
// Kernels (four waves per workgroup; one wave = 16 query rows, or 16 keys):
//   rows_kernel   per 64 flat rows (t, h) (wave w: rows 16w .. 16w+15): dA =
//                 dO * sig rounded to bf16 (kept in the workspace for the key
//                 kernel); pass A walks the 32-key tiles of the keys any of the
//                 64 rows sees, with the decode kernel's fixed-reference
//                 softmax, for the row sum, a (for dg) and Dt = sum_j p_j
//                 <dA, v_j> from the same dA and p the score gradients use, so
//                 that they sum to zero to fp32 rounding; then dg, the row
//                 statistics lse and Dt; pass B walks the tiles again for dq:
//                 S^T = K Q^T, P = 2^(x - lse), dP^T = V dA^T,
//                 dS^T = P (dP^T - Dt), dQ^T += K^T dS^T.
//   keys_kernel   per 64 keys (wave w: keys 16w .. 16w+15, K and V fragments
//                 in registers): over the 32-row blocks of queries that see
//                 them, S = Q K^T, dP = dA V^T, dS, then dV^T += dA^T P and
//                 dK^T += Q^T dS.  Raw keys are stored; entries are split into
//                 tasks of 512 row blocks whose sums are added atomically.
//   pool_kernel   dk, dv of raw rows += entry gradients / 128.
// Both main kernels stream their tiles (K and V; Q, dA and the row statistics)
// global -> LDS by DMA through two stages, each wave copying a quarter of
// every tile one tile ahead, and all four waves read every tile: as MFMA
// fragments (16x16x32 score-shaped chains) and, for the products that contract
// over keys or rows, with transposing reads (16x16x32 over the tile's 32 rows).
// One barrier per tile.  fp32 accumulation throughout; MFMA operands are bf16
// (P, dS and dA rounded to nearest even; P as in the forward).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kTile = 32;                // keys per tile (rows kernel), rows per block (keys kernel)
// LDS tile layout: row r at r * kRow, its 16-byte chunk c at chunk c ^ (r & 15)
// of the row.  Both read patterns then touch every bank once per phase: the
// b128 fragment reads (16 lanes: 16 rows, one chunk column each) and the
// transposing reads (32 lanes: 8 rows x 4 eight-byte pieces).  Every read
// address is one of a few per-lane bases plus an immediate offset.
constexpr int kRow = 1024 + 128;
constexpr int kStage = kTile * kRow;     // one 32-row tile: 36864 bytes
constexpr int kHalf = 16 * kRow;         // rows 16 .. 31 of a tile
// the asm helpers below carry these offsets as immediates
static_assert(kHalf == 18432 && kStage == 36864, "asm read offsets");
constexpr float kHeadroom = 64.0f;
constexpr int kRowsPerWg = 64;
constexpr int kKeysPerWg = 64;
constexpr int kChunkRb = 512;            // row blocks per entry task

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

struct BwArgs {
  const uint16_t *q, *g, *k, *v, *ck, *cv, *dout;
  float *dq, *dg, *dk, *dv;
  float *lse, *dt, *dck, *dcv;  // workspace: row statistics, entry gradients
  uint16_t* da;                 // workspace: dA rows, bf16 [T * H, 512]
  const void* out;              // saved state: the forward's gated output (bf16 or f32)
  const float* lse_in;          //   and its row log-sum-exp (natural log)
  int out_f32;
  int64_t T;
  int H, Nc, n_rb;              // n_rb: blocks of kTile flat rows
  int n_ent_tasks, n_chunks;    // entry tasks = entry groups x chunks of kChunkRb row blocks
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
// s_waitcnt vmcnt(N) (vmcnt in bits 3:0 and 15:14), then a compiler barrier so
// that no memory access moves across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// The MFMAs are inline asm, so that accumulators and operands keep their
// register files (the builtins let the register allocator move accumulators
// between AGPRs and VGPRs around loops).  mfma_drain gives the wait states a
// VALU read of accumulators written by the last MFMAs needs.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15"); }

// O^T[512 dims x 16] += M^T P over a 32-row LDS tile M, with 16x16x32 MFMAs
// (full rate; the 16x16x16 form costs about as many cycles for half the work).
// The contraction index of lane group g4 is the 8 rows {4 g4 .. 4 g4 + 3,
// 16 + 4 g4 .. 16 + 4 g4 + 3}: the A operand M^T comes from two transposing
// reads, of rows 4 g4 .. and of the same rows + 16, into the two halves of one
// 4-register group, and P (B operand, 8 bf16 per lane) holds
// the same rows in that order.  Dim block db = 8 a + b is read at ta[b] + 256 a
// (and + kHalf for rows 16 ..).  The groups are fixed registers (clobbered:
// inline asm cannot name the halves of an operand) used as a ring: the reads of
// one half of the ring are in flight while the other half's MFMAs issue, and a
// group is refilled only after the MFMA reading it has issued and the reads in
// between have been waited for.  Accumulators in AGPRs.  tr_rows: a ring of 16
// groups in v192 .. v255.  tr_keys2: both products of the key kernel in one
// block, o += (the stage's second tile)^T p then w += (its first tile)^T r,
// through 8 groups in v224 .. v255 (the key kernel keeps its K and V fragments
// in VGPRs), so the second product's reads overlap the first one's MFMAs.
__device__ __forceinline__ void tr_rows(f32x4 (&o)[32], const uint32_t (&ta)[8], const bf16x8& p) {
  asm volatile(
      "ds_read_b64_tr_b16 v[192:193], %[t0] offset:0\n\t"
      "ds_read_b64_tr_b16 v[194:195], %[t0] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[196:197], %[t1] offset:0\n\t"
      "ds_read_b64_tr_b16 v[198:199], %[t1] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[200:201], %[t2] offset:0\n\t"
      "ds_read_b64_tr_b16 v[202:203], %[t2] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[204:205], %[t3] offset:0\n\t"
      "ds_read_b64_tr_b16 v[206:207], %[t3] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[208:209], %[t4] offset:0\n\t"
      "ds_read_b64_tr_b16 v[210:211], %[t4] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[212:213], %[t5] offset:0\n\t"
      "ds_read_b64_tr_b16 v[214:215], %[t5] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[216:217], %[t6] offset:0\n\t"
      "ds_read_b64_tr_b16 v[218:219], %[t6] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[220:221], %[t7] offset:0\n\t"
      "ds_read_b64_tr_b16 v[222:223], %[t7] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:256\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:256\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:256\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:256\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:256\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:256\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:256\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:256\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:18688\n\t"
      "s_waitcnt lgkmcnt(15)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o0], v[192:195], %[p], %[o0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o1], v[196:199], %[p], %[o1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o2], v[200:203], %[p], %[o2]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o3], v[204:207], %[p], %[o3]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o4], v[208:211], %[p], %[o4]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o5], v[212:215], %[p], %[o5]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o6], v[216:219], %[p], %[o6]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o7], v[220:223], %[p], %[o7]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[192:193], %[t0] offset:512\n\t"
      "ds_read_b64_tr_b16 v[194:195], %[t0] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[196:197], %[t1] offset:512\n\t"
      "ds_read_b64_tr_b16 v[198:199], %[t1] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[200:201], %[t2] offset:512\n\t"
      "ds_read_b64_tr_b16 v[202:203], %[t2] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[204:205], %[t3] offset:512\n\t"
      "ds_read_b64_tr_b16 v[206:207], %[t3] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[208:209], %[t4] offset:512\n\t"
      "ds_read_b64_tr_b16 v[210:211], %[t4] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[212:213], %[t5] offset:512\n\t"
      "ds_read_b64_tr_b16 v[214:215], %[t5] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[216:217], %[t6] offset:512\n\t"
      "ds_read_b64_tr_b16 v[218:219], %[t6] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[220:221], %[t7] offset:512\n\t"
      "ds_read_b64_tr_b16 v[222:223], %[t7] offset:18944\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o8], v[224:227], %[p], %[o8]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o9], v[228:231], %[p], %[o9]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o10], v[232:235], %[p], %[o10]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o11], v[236:239], %[p], %[o11]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o12], v[240:243], %[p], %[o12]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o13], v[244:247], %[p], %[o13]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o14], v[248:251], %[p], %[o14]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o15], v[252:255], %[p], %[o15]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:768\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:768\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:768\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:768\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:768\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:768\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:768\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:768\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o16], v[192:195], %[p], %[o16]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o17], v[196:199], %[p], %[o17]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o18], v[200:203], %[p], %[o18]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o19], v[204:207], %[p], %[o19]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o20], v[208:211], %[p], %[o20]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o21], v[212:215], %[p], %[o21]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o22], v[216:219], %[p], %[o22]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o23], v[220:223], %[p], %[o23]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o24], v[224:227], %[p], %[o24]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o25], v[228:231], %[p], %[o25]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o26], v[232:235], %[p], %[o26]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o27], v[236:239], %[p], %[o27]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o28], v[240:243], %[p], %[o28]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o29], v[244:247], %[p], %[o29]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o30], v[248:251], %[p], %[o30]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o31], v[252:255], %[p], %[o31]"
      : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]),
        [o4] "+a"(o[4]), [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]),
        [o8] "+a"(o[8]), [o9] "+a"(o[9]), [o10] "+a"(o[10]), [o11] "+a"(o[11]),
        [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]), [o15] "+a"(o[15]),
        [o16] "+a"(o[16]), [o17] "+a"(o[17]), [o18] "+a"(o[18]), [o19] "+a"(o[19]),
        [o20] "+a"(o[20]), [o21] "+a"(o[21]), [o22] "+a"(o[22]), [o23] "+a"(o[23]),
        [o24] "+a"(o[24]), [o25] "+a"(o[25]), [o26] "+a"(o[26]), [o27] "+a"(o[27]),
        [o28] "+a"(o[28]), [o29] "+a"(o[29]), [o30] "+a"(o[30]), [o31] "+a"(o[31])
      : [t0] "v"(ta[0]), [t1] "v"(ta[1]), [t2] "v"(ta[2]), [t3] "v"(ta[3]),
        [t4] "v"(ta[4]), [t5] "v"(ta[5]), [t6] "v"(ta[6]), [t7] "v"(ta[7]),
        [p] "v"(p)
      : "memory", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}
__device__ __forceinline__ void tr_keys2(f32x4 (&o)[32], f32x4 (&w)[32], const uint32_t (&ta)[8], const bf16x8& p, const bf16x8& r) {
  asm volatile(
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:55296\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:36864\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:55296\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o0], v[224:227], %[p], %[o0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o1], v[228:231], %[p], %[o1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o2], v[232:235], %[p], %[o2]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o3], v[236:239], %[p], %[o3]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o4], v[240:243], %[p], %[o4]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o5], v[244:247], %[p], %[o5]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o6], v[248:251], %[p], %[o6]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o7], v[252:255], %[p], %[o7]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:55552\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:37120\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o8], v[224:227], %[p], %[o8]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o9], v[228:231], %[p], %[o9]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o10], v[232:235], %[p], %[o10]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o11], v[236:239], %[p], %[o11]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:55808\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o12], v[240:243], %[p], %[o12]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o13], v[244:247], %[p], %[o13]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o14], v[248:251], %[p], %[o14]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o15], v[252:255], %[p], %[o15]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:55808\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:37376\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:55808\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o16], v[224:227], %[p], %[o16]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o17], v[228:231], %[p], %[o17]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o18], v[232:235], %[p], %[o18]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o19], v[236:239], %[p], %[o19]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o20], v[240:243], %[p], %[o20]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o21], v[244:247], %[p], %[o21]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o22], v[248:251], %[p], %[o22]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o23], v[252:255], %[p], %[o23]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:56064\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:37632\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o24], v[224:227], %[p], %[o24]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o25], v[228:231], %[p], %[o25]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o26], v[232:235], %[p], %[o26]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o27], v[236:239], %[p], %[o27]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:0\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:0\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:0\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:0\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:18432\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o28], v[240:243], %[p], %[o28]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o29], v[244:247], %[p], %[o29]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o30], v[248:251], %[p], %[o30]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[o31], v[252:255], %[p], %[o31]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:0\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:0\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:0\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:18432\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:0\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:18432\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w0], v[224:227], %[r], %[w0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w1], v[228:231], %[r], %[w1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w2], v[232:235], %[r], %[w2]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w3], v[236:239], %[r], %[w3]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:256\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:256\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:256\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:256\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w4], v[240:243], %[r], %[w4]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w5], v[244:247], %[r], %[w5]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w6], v[248:251], %[r], %[w6]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w7], v[252:255], %[r], %[w7]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:256\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:256\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:256\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:18688\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:256\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w8], v[224:227], %[r], %[w8]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w9], v[228:231], %[r], %[w9]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w10], v[232:235], %[r], %[w10]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w11], v[236:239], %[r], %[w11]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:512\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:512\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:512\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:512\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:18944\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w12], v[240:243], %[r], %[w12]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w13], v[244:247], %[r], %[w13]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w14], v[248:251], %[r], %[w14]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w15], v[252:255], %[r], %[w15]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:512\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:512\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:512\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:18944\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:512\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:18944\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w16], v[224:227], %[r], %[w16]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w17], v[228:231], %[r], %[w17]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w18], v[232:235], %[r], %[w18]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w19], v[236:239], %[r], %[w19]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[224:225], %[t0] offset:768\n\t"
      "ds_read_b64_tr_b16 v[226:227], %[t0] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[228:229], %[t1] offset:768\n\t"
      "ds_read_b64_tr_b16 v[230:231], %[t1] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[232:233], %[t2] offset:768\n\t"
      "ds_read_b64_tr_b16 v[234:235], %[t2] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[236:237], %[t3] offset:768\n\t"
      "ds_read_b64_tr_b16 v[238:239], %[t3] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w20], v[240:243], %[r], %[w20]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w21], v[244:247], %[r], %[w21]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w22], v[248:251], %[r], %[w22]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w23], v[252:255], %[r], %[w23]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[t4] offset:768\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[t4] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[t5] offset:768\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[t5] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[t6] offset:768\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[t6] offset:19200\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[t7] offset:768\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[t7] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w24], v[224:227], %[r], %[w24]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w25], v[228:231], %[r], %[w25]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w26], v[232:235], %[r], %[w26]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w27], v[236:239], %[r], %[w27]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w28], v[240:243], %[r], %[w28]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w29], v[244:247], %[r], %[w29]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w30], v[248:251], %[r], %[w30]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[w31], v[252:255], %[r], %[w31]"
      : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]),
        [o4] "+a"(o[4]), [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]),
        [o8] "+a"(o[8]), [o9] "+a"(o[9]), [o10] "+a"(o[10]), [o11] "+a"(o[11]),
        [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]), [o15] "+a"(o[15]),
        [o16] "+a"(o[16]), [o17] "+a"(o[17]), [o18] "+a"(o[18]), [o19] "+a"(o[19]),
        [o20] "+a"(o[20]), [o21] "+a"(o[21]), [o22] "+a"(o[22]), [o23] "+a"(o[23]),
        [o24] "+a"(o[24]), [o25] "+a"(o[25]), [o26] "+a"(o[26]), [o27] "+a"(o[27]),
        [o28] "+a"(o[28]), [o29] "+a"(o[29]), [o30] "+a"(o[30]), [o31] "+a"(o[31]),
        [w0] "+a"(w[0]), [w1] "+a"(w[1]), [w2] "+a"(w[2]), [w3] "+a"(w[3]),
        [w4] "+a"(w[4]), [w5] "+a"(w[5]), [w6] "+a"(w[6]), [w7] "+a"(w[7]),
        [w8] "+a"(w[8]), [w9] "+a"(w[9]), [w10] "+a"(w[10]), [w11] "+a"(w[11]),
        [w12] "+a"(w[12]), [w13] "+a"(w[13]), [w14] "+a"(w[14]), [w15] "+a"(w[15]),
        [w16] "+a"(w[16]), [w17] "+a"(w[17]), [w18] "+a"(w[18]), [w19] "+a"(w[19]),
        [w20] "+a"(w[20]), [w21] "+a"(w[21]), [w22] "+a"(w[22]), [w23] "+a"(w[23]),
        [w24] "+a"(w[24]), [w25] "+a"(w[25]), [w26] "+a"(w[26]), [w27] "+a"(w[27]),
        [w28] "+a"(w[28]), [w29] "+a"(w[29]), [w30] "+a"(w[30]), [w31] "+a"(w[31])
      : [t0] "v"(ta[0]), [t1] "v"(ta[1]), [t2] "v"(ta[2]), [t3] "v"(ta[3]),
        [t4] "v"(ta[4]), [t5] "v"(ta[5]), [t6] "v"(ta[6]), [t7] "v"(ta[7]),
        [p] "v"(p), [r] "v"(r)
      : "memory", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}

// ---------------------------------------------------------------- key lists
// The keys of the rows whose queries run from t_lo to t_hi, in tiles of 32:
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
// A buffer descriptor as four words in scalar registers (what make_rsrc builds:
// base, stride 0, `bytes` bytes, 32-bit data format), for copies issued from
// inline asm.
__device__ __forceinline__ u32x4 desc_words(const void* base, int bytes) {
  const uint64_t ad = (uint64_t)(uintptr_t)base;
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)ad);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32) & 0xFFFFu);
  d[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  d[3] = 0x00020000u;
  return d;
}
// Tile j's K (or V) rows as descriptor words (the buffer tile_src makes).
__device__ __forceinline__ u32x4 tile_desc(const Keys& s, int j, const uint16_t* ent,
                                           const uint16_t* raw) {
  if (j < s.n_et) {
    const int first = kTile * j;
    const int rows = s.nc - first < kTile ? s.nc - first : kTile;
    return desc_words(ent + (int64_t)first * kD, rows * 1024);
  }
  const int first = s.lo + kTile * (j - s.n_et);
  const int rows = s.lo + s.nraw - first < kTile ? s.lo + s.nraw - first : kTile;
  return desc_words(raw + (int64_t)first * kD, rows * 1024);
}

// Rows 8w .. 8w+7 of a 32-row tile (buffer r of 1 KiB rows; rows past its end
// arrive as zeros) into the tile at st: 8 DMA instructions.  A copy writes 16
// bytes per lane to consecutive LDS chunks, so lane L of row rr fetches the
// row's chunk L ^ (rr & 15) (byte offset vo[u] = 16 (L ^ (rr & 15))).
__device__ __forceinline__ void copy8(__amdgpu_buffer_rsrc_t r, int w, const uint32_t (&vo)[8],
                                      uint8_t* st) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int rr = 8 * w + u;
    dma16_buf(r, rr * 1024 + (int)vo[u], (lds_void*)(st + rr * kRow));
  }
}

// Per-lane read bases within a tile (lane (l16, g4)):
//   fragment reads, 16 bytes of row x = l16 at byte 64 ss + 16 g4, ss = 4 a + b:
//     cb[b] + 256 a (+ kHalf for row 16 + x, + kStage for the stage's second tile);
//   transposing reads, 8 bytes of row y = 4 g4 + (l16 >> 2) at byte
//     32 db + 8 (l16 & 3), db = 8 a + b: tb[b] + 256 a (+ kHalf for row y + 16).
__device__ __forceinline__ void read_bases(int l16, int g4, uint32_t (&cb)[4], uint32_t (&tb)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b)
    cb[b] = (uint32_t)(l16 * kRow + 16 * (g4 ^ (l16 & 3)) + 64 * (b ^ (l16 >> 2)));
  const int y = 4 * g4 + (l16 >> 2), h = (l16 >> 1) & 1;
#pragma unroll
  for (int b = 0; b < 8; ++b) tb[b] = (uint32_t)(y * kRow + 16 * ((2 * b + h) ^ y) + 8 * (l16 & 1));
}

// Four score-shaped chains over the two 32-row tiles of a stage in LDS:
//   s0, s1 = sum_ss X_c[ss] b[ss] (c = 0, 1),  d0, d1 = sum_ss X_c[ss] c[ss] (c = 2, 3)
// (16 MFMA 16x16x32 each), X_0, X_1 rows 0 .. 15 and 16 .. 31 of the first
// tile, X_2, X_3 those of the second, with the A operands read from LDS (lane
// (l16, g4), fragment ss = 4 a + b: 16 bytes at ad[b] + 256 a + 0, kHalf,
// kStage, kStage + kHalf for c = 0 .. 3; ad = the stage + cb) and b, c in
// registers.  One asm block issues the 64
// reads through a ring of fixed registers, the reads of one group in flight
// while the previous group's MFMAs issue, and waits for everything it reads
// (the compiler does not see these LDS reads, so it inserts no wait for DMA
// copies in flight into the other stage).  It ends with the wait states a VALU
// read of the results needs.  chains_rows: b, c in AGPRs, a ring of 16 in
// v128 .. v191; chains_keys: b, c in VGPRs, a ring of 8 in v192 .. v223, after
// four 16-byte reads at sad + 64 i (row statistics).
__device__ __forceinline__ void chains_rows(f32x4& s0, f32x4& s1, f32x4& d0, f32x4& d1, const uint32_t (&ad)[4], const bf16x8 (&b)[16], const bf16x8 (&c)[16]) {
  asm volatile(
      "ds_read_b128 v[128:131], %[a0] offset:0\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:0\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:0\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:0\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:256\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:256\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:256\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:256\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:512\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:512\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:512\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:512\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:768\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:768\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:768\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:768\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[128:131], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[132:135], %[b1], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[136:139], %[b2], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[140:143], %[b3], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[144:147], %[b4], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[148:151], %[b5], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[152:155], %[b6], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[156:159], %[b7], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:18432\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:18432\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:18432\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:18432\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:18688\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:18688\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:18688\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[160:163], %[b8], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[164:167], %[b9], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[168:171], %[b10], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[172:175], %[b11], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[176:179], %[b12], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[180:183], %[b13], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[184:187], %[b14], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[188:191], %[b15], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:18944\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:18944\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:18944\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:18944\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:19200\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:19200\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:19200\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[128:131], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[132:135], %[b1], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[136:139], %[b2], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[140:143], %[b3], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[144:147], %[b4], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[148:151], %[b5], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[152:155], %[b6], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[156:159], %[b7], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:36864\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:36864\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:36864\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:36864\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:37120\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:37120\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:37120\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:37120\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[160:163], %[b8], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[164:167], %[b9], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[168:171], %[b10], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[172:175], %[b11], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[176:179], %[b12], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[180:183], %[b13], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[184:187], %[b14], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[188:191], %[b15], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:37376\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:37376\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:37376\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:37376\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:37632\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:37632\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:37632\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:37632\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[128:131], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[132:135], %[c1], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[136:139], %[c2], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[140:143], %[c3], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[144:147], %[c4], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[148:151], %[c5], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[152:155], %[c6], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[156:159], %[c7], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:55296\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:55296\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:55296\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:55296\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:55552\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:55552\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:55552\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[160:163], %[c8], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[164:167], %[c9], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[168:171], %[c10], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[172:175], %[c11], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[176:179], %[c12], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[180:183], %[c13], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[184:187], %[c14], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[188:191], %[c15], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:55808\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:55808\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:55808\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:55808\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:56064\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:56064\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:56064\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[128:131], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[132:135], %[c1], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[136:139], %[c2], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[140:143], %[c3], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[144:147], %[c4], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[148:151], %[c5], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[152:155], %[c6], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[156:159], %[c7], %[d1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[160:163], %[c8], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[164:167], %[c9], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[168:171], %[c10], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[172:175], %[c11], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[176:179], %[c12], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[180:183], %[c13], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[184:187], %[c14], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[188:191], %[c15], %[d1]\n\t"
      "s_nop 15\n\ts_nop 3"
      : [s0] "=&v"(s0), [s1] "=&v"(s1), [d0] "=&v"(d0), [d1] "=&v"(d1)
      : [a0] "v"(ad[0]), [a1] "v"(ad[1]), [a2] "v"(ad[2]), [a3] "v"(ad[3]),
        [b0] "a"(b[0]), [b1] "a"(b[1]), [b2] "a"(b[2]), [b3] "a"(b[3]),
        [b4] "a"(b[4]), [b5] "a"(b[5]), [b6] "a"(b[6]), [b7] "a"(b[7]),
        [b8] "a"(b[8]), [b9] "a"(b[9]), [b10] "a"(b[10]), [b11] "a"(b[11]),
        [b12] "a"(b[12]), [b13] "a"(b[13]), [b14] "a"(b[14]), [b15] "a"(b[15]),
        [c0] "a"(c[0]), [c1] "a"(c[1]), [c2] "a"(c[2]), [c3] "a"(c[3]),
        [c4] "a"(c[4]), [c5] "a"(c[5]), [c6] "a"(c[6]), [c7] "a"(c[7]),
        [c8] "a"(c[8]), [c9] "a"(c[9]), [c10] "a"(c[10]), [c11] "a"(c[11]),
        [c12] "a"(c[12]), [c13] "a"(c[13]), [c14] "a"(c[14]), [c15] "a"(c[15])
      : "memory", "v128", "v129", "v130", "v131", "v132", "v133", "v134", "v135", "v136", "v137", "v138", "v139", "v140", "v141", "v142", "v143", "v144", "v145", "v146", "v147", "v148", "v149", "v150", "v151", "v152", "v153", "v154", "v155", "v156", "v157", "v158", "v159", "v160", "v161", "v162", "v163", "v164", "v165", "v166", "v167", "v168", "v169", "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191");
}
__device__ __forceinline__ void chains_keys(f32x4& s0, f32x4& s1, f32x4& d0, f32x4& d1, const uint32_t (&ad)[4], const bf16x8 (&b)[16], const bf16x8 (&c)[16], uint32_t sad, f32x4 (&st)[4]) {
  asm volatile(
      "ds_read_b128 %[st0], %[sa] offset:0\n\t"
      "ds_read_b128 %[st1], %[sa] offset:64\n\t"
      "ds_read_b128 %[st2], %[sa] offset:128\n\t"
      "ds_read_b128 %[st3], %[sa] offset:192\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:0\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:0\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:0\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:0\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:256\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:256\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:256\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[192:195], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[196:199], %[b1], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[200:203], %[b2], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[204:207], %[b3], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:512\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:512\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:512\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:512\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[208:211], %[b4], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[212:215], %[b5], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[216:219], %[b6], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[220:223], %[b7], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:768\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:768\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:768\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:768\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[192:195], %[b8], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[196:199], %[b9], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[200:203], %[b10], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[204:207], %[b11], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:18432\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:18432\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:18432\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:18432\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[208:211], %[b12], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[212:215], %[b13], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[216:219], %[b14], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[220:223], %[b15], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:18688\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:18688\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:18688\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[192:195], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[196:199], %[b1], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[200:203], %[b2], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[204:207], %[b3], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:18944\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:18944\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:18944\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:18944\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[208:211], %[b4], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[212:215], %[b5], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[216:219], %[b6], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[220:223], %[b7], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:19200\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:19200\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:19200\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[192:195], %[b8], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[196:199], %[b9], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[200:203], %[b10], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[204:207], %[b11], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:36864\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:36864\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:36864\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:36864\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[208:211], %[b12], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[212:215], %[b13], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[216:219], %[b14], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[220:223], %[b15], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:37120\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:37120\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:37120\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:37120\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[192:195], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[196:199], %[c1], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[200:203], %[c2], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[204:207], %[c3], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:37376\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:37376\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:37376\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:37376\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[208:211], %[c4], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[212:215], %[c5], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[216:219], %[c6], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[220:223], %[c7], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:37632\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:37632\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:37632\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:37632\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[192:195], %[c8], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[196:199], %[c9], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[200:203], %[c10], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[204:207], %[c11], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:55296\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:55296\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:55296\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:55296\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[208:211], %[c12], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[212:215], %[c13], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[216:219], %[c14], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[220:223], %[c15], %[d0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:55552\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:55552\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:55552\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[192:195], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[196:199], %[c1], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[200:203], %[c2], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[204:207], %[c3], %[d1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:55808\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:55808\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:55808\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:55808\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[208:211], %[c4], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[212:215], %[c5], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[216:219], %[c6], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[220:223], %[c7], %[d1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:56064\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:56064\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:56064\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[192:195], %[c8], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[196:199], %[c9], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[200:203], %[c10], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[204:207], %[c11], %[d1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[208:211], %[c12], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[212:215], %[c13], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[216:219], %[c14], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[220:223], %[c15], %[d1]\n\t"
      "s_nop 15\n\ts_nop 3"
      : [s0] "=&v"(s0), [s1] "=&v"(s1), [d0] "=&v"(d0), [d1] "=&v"(d1),
        [st0] "=&v"(st[0]), [st1] "=&v"(st[1]), [st2] "=&v"(st[2]), [st3] "=&v"(st[3])
      : [a0] "v"(ad[0]), [a1] "v"(ad[1]), [a2] "v"(ad[2]), [a3] "v"(ad[3]),
        [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]),
        [b4] "v"(b[4]), [b5] "v"(b[5]), [b6] "v"(b[6]), [b7] "v"(b[7]),
        [b8] "v"(b[8]), [b9] "v"(b[9]), [b10] "v"(b[10]), [b11] "v"(b[11]),
        [b12] "v"(b[12]), [b13] "v"(b[13]), [b14] "v"(b[14]), [b15] "v"(b[15]),
        [c0] "v"(c[0]), [c1] "v"(c[1]), [c2] "v"(c[2]), [c3] "v"(c[3]),
        [c4] "v"(c[4]), [c5] "v"(c[5]), [c6] "v"(c[6]), [c7] "v"(c[7]),
        [c8] "v"(c[8]), [c9] "v"(c[9]), [c10] "v"(c[10]), [c11] "v"(c[11]),
        [c12] "v"(c[12]), [c13] "v"(c[13]), [c14] "v"(c[14]), [c15] "v"(c[15]),
        [sa] "v"(sad)
      : "memory", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223");
}

// The same chains with 16 LDS-DMA copies of the next tile issued from inside the
// asm, two after each group of MFMAs: an issuing copy stalls the wave while the
// CU's memory path is busy, and copies issued back to back by all four waves
// queue; spread out, the MFMAs already issued keep the pipe busy meanwhile.
// Copy u (0 .. 15) reads 16 bytes per lane at vo[u % 8] + so[u % 8] of buffer rk (u <
// 8) or rv (u >= 8) into LDS at m0 = mad[u] (plus 16 bytes per lane); m0 is
// saved first and restored last (the compiler keeps it for its own copies).
__device__ __forceinline__ void chains_rows_dma(f32x4& s0, f32x4& s1, f32x4& d0, f32x4& d1, const uint32_t (&ad)[4], const bf16x8 (&b)[16], const bf16x8 (&c)[16], const u32x4& rk, const u32x4& rv, const uint32_t (&vo)[8], const uint32_t (&so)[8], const uint32_t (&mad)[16]) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %[m0s], m0\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:0\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:0\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:0\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:0\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:256\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:256\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:256\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:256\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:512\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:512\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:512\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:512\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:768\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:768\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:768\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:768\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[128:131], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[132:135], %[b1], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[136:139], %[b2], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[140:143], %[b3], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[144:147], %[b4], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[148:151], %[b5], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[152:155], %[b6], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[156:159], %[b7], %[s0]\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo0], %[rk], %[so0] offen lds\n\t"
      "s_mov_b32 m0, %[m1]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo1], %[rk], %[so1] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:18432\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:18432\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:18432\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:18432\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:18688\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:18688\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:18688\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[160:163], %[b8], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[164:167], %[b9], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[168:171], %[b10], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[172:175], %[b11], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[176:179], %[b12], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[180:183], %[b13], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[184:187], %[b14], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[188:191], %[b15], %[s0]\n\t"
      "s_mov_b32 m0, %[m2]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo2], %[rk], %[so2] offen lds\n\t"
      "s_mov_b32 m0, %[m3]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo3], %[rk], %[so3] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:18944\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:18944\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:18944\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:18944\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:19200\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:19200\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:19200\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[128:131], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[132:135], %[b1], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[136:139], %[b2], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[140:143], %[b3], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[144:147], %[b4], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[148:151], %[b5], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[152:155], %[b6], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[156:159], %[b7], %[s1]\n\t"
      "s_mov_b32 m0, %[m4]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo4], %[rk], %[so4] offen lds\n\t"
      "s_mov_b32 m0, %[m5]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo5], %[rk], %[so5] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:36864\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:36864\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:36864\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:36864\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:37120\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:37120\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:37120\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:37120\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[160:163], %[b8], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[164:167], %[b9], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[168:171], %[b10], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[172:175], %[b11], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[176:179], %[b12], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[180:183], %[b13], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[184:187], %[b14], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[188:191], %[b15], %[s1]\n\t"
      "s_mov_b32 m0, %[m6]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo6], %[rk], %[so6] offen lds\n\t"
      "s_mov_b32 m0, %[m7]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo7], %[rk], %[so7] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:37376\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:37376\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:37376\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:37376\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:37632\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:37632\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:37632\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:37632\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[128:131], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[132:135], %[c1], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[136:139], %[c2], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[140:143], %[c3], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[144:147], %[c4], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[148:151], %[c5], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[152:155], %[c6], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[156:159], %[c7], %[d0]\n\t"
      "s_mov_b32 m0, %[m8]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo0], %[rv], %[so0] offen lds\n\t"
      "s_mov_b32 m0, %[m9]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo1], %[rv], %[so1] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[128:131], %[a0] offset:55296\n\t"
      "ds_read_b128 v[132:135], %[a1] offset:55296\n\t"
      "ds_read_b128 v[136:139], %[a2] offset:55296\n\t"
      "ds_read_b128 v[140:143], %[a3] offset:55296\n\t"
      "ds_read_b128 v[144:147], %[a0] offset:55552\n\t"
      "ds_read_b128 v[148:151], %[a1] offset:55552\n\t"
      "ds_read_b128 v[152:155], %[a2] offset:55552\n\t"
      "ds_read_b128 v[156:159], %[a3] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[160:163], %[c8], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[164:167], %[c9], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[168:171], %[c10], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[172:175], %[c11], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[176:179], %[c12], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[180:183], %[c13], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[184:187], %[c14], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[188:191], %[c15], %[d0]\n\t"
      "s_mov_b32 m0, %[m10]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo2], %[rv], %[so2] offen lds\n\t"
      "s_mov_b32 m0, %[m11]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo3], %[rv], %[so3] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[160:163], %[a0] offset:55808\n\t"
      "ds_read_b128 v[164:167], %[a1] offset:55808\n\t"
      "ds_read_b128 v[168:171], %[a2] offset:55808\n\t"
      "ds_read_b128 v[172:175], %[a3] offset:55808\n\t"
      "ds_read_b128 v[176:179], %[a0] offset:56064\n\t"
      "ds_read_b128 v[180:183], %[a1] offset:56064\n\t"
      "ds_read_b128 v[184:187], %[a2] offset:56064\n\t"
      "ds_read_b128 v[188:191], %[a3] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[128:131], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[132:135], %[c1], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[136:139], %[c2], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[140:143], %[c3], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[144:147], %[c4], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[148:151], %[c5], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[152:155], %[c6], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[156:159], %[c7], %[d1]\n\t"
      "s_mov_b32 m0, %[m12]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo4], %[rv], %[so4] offen lds\n\t"
      "s_mov_b32 m0, %[m13]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo5], %[rv], %[so5] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[160:163], %[c8], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[164:167], %[c9], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[168:171], %[c10], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[172:175], %[c11], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[176:179], %[c12], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[180:183], %[c13], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[184:187], %[c14], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[188:191], %[c15], %[d1]\n\t"
      "s_mov_b32 m0, %[m14]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo6], %[rv], %[so6] offen lds\n\t"
      "s_mov_b32 m0, %[m15]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo7], %[rv], %[so7] offen lds\n\t"
      "s_nop 15\n\ts_nop 3\n\t"
      "s_mov_b32 m0, %[m0s]"
      : [m0s] "=&s"(m0_saved), [s0] "=&v"(s0), [s1] "=&v"(s1), [d0] "=&v"(d0),
        [d1] "=&v"(d1)
      : [a0] "v"(ad[0]), [a1] "v"(ad[1]), [a2] "v"(ad[2]), [a3] "v"(ad[3]),
        [b0] "a"(b[0]), [b1] "a"(b[1]), [b2] "a"(b[2]), [b3] "a"(b[3]),
        [b4] "a"(b[4]), [b5] "a"(b[5]), [b6] "a"(b[6]), [b7] "a"(b[7]),
        [b8] "a"(b[8]), [b9] "a"(b[9]), [b10] "a"(b[10]), [b11] "a"(b[11]),
        [b12] "a"(b[12]), [b13] "a"(b[13]), [b14] "a"(b[14]), [b15] "a"(b[15]),
        [c0] "a"(c[0]), [c1] "a"(c[1]), [c2] "a"(c[2]), [c3] "a"(c[3]),
        [c4] "a"(c[4]), [c5] "a"(c[5]), [c6] "a"(c[6]), [c7] "a"(c[7]),
        [c8] "a"(c[8]), [c9] "a"(c[9]), [c10] "a"(c[10]), [c11] "a"(c[11]),
        [c12] "a"(c[12]), [c13] "a"(c[13]), [c14] "a"(c[14]), [c15] "a"(c[15]),
        [rk] "s"(rk), [rv] "s"(rv), [vo0] "v"(vo[0]), [vo1] "v"(vo[1]),
        [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]), [vo5] "v"(vo[5]),
        [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [so0] "s"(so[0]), [so1] "s"(so[1]),
        [so2] "s"(so[2]), [so3] "s"(so[3]), [so4] "s"(so[4]), [so5] "s"(so[5]),
        [so6] "s"(so[6]), [so7] "s"(so[7]), [m0] "s"(mad[0]), [m1] "s"(mad[1]),
        [m2] "s"(mad[2]), [m3] "s"(mad[3]), [m4] "s"(mad[4]), [m5] "s"(mad[5]),
        [m6] "s"(mad[6]), [m7] "s"(mad[7]), [m8] "s"(mad[8]), [m9] "s"(mad[9]),
        [m10] "s"(mad[10]), [m11] "s"(mad[11]), [m12] "s"(mad[12]), [m13] "s"(mad[13]),
        [m14] "s"(mad[14]), [m15] "s"(mad[15])
      : "memory", "v128", "v129", "v130", "v131", "v132", "v133", "v134", "v135", "v136", "v137", "v138", "v139", "v140", "v141", "v142", "v143", "v144", "v145", "v146", "v147", "v148", "v149", "v150", "v151", "v152", "v153", "v154", "v155", "v156", "v157", "v158", "v159", "v160", "v161", "v162", "v163", "v164", "v165", "v166", "v167", "v168", "v169", "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191");
}
__device__ __forceinline__ void chains_keys_dma(f32x4& s0, f32x4& s1, f32x4& d0, f32x4& d1, const uint32_t (&ad)[4], const bf16x8 (&b)[16], const bf16x8 (&c)[16], uint32_t sad, f32x4 (&st)[4], const u32x4& rk, const u32x4& rv, const uint32_t (&vo)[8], const uint32_t (&so)[8], const uint32_t (&mad)[16]) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %[m0s], m0\n\t"
      "ds_read_b128 %[st0], %[sa] offset:0\n\t"
      "ds_read_b128 %[st1], %[sa] offset:64\n\t"
      "ds_read_b128 %[st2], %[sa] offset:128\n\t"
      "ds_read_b128 %[st3], %[sa] offset:192\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:0\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:0\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:0\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:0\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:256\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:256\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:256\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[192:195], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[196:199], %[b1], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[200:203], %[b2], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[204:207], %[b3], %[s0]\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo0], %[rk], %[so0] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:512\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:512\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:512\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:512\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[208:211], %[b4], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[212:215], %[b5], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[216:219], %[b6], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[220:223], %[b7], %[s0]\n\t"
      "s_mov_b32 m0, %[m1]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo1], %[rk], %[so1] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:768\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:768\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:768\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:768\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[192:195], %[b8], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[196:199], %[b9], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[200:203], %[b10], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[204:207], %[b11], %[s0]\n\t"
      "s_mov_b32 m0, %[m2]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo2], %[rk], %[so2] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:18432\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:18432\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:18432\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:18432\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[208:211], %[b12], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[212:215], %[b13], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[216:219], %[b14], %[s0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s0], v[220:223], %[b15], %[s0]\n\t"
      "s_mov_b32 m0, %[m3]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo3], %[rk], %[so3] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:18688\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:18688\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:18688\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:18688\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[192:195], %[b0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[196:199], %[b1], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[200:203], %[b2], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[204:207], %[b3], %[s1]\n\t"
      "s_mov_b32 m0, %[m4]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo4], %[rk], %[so4] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:18944\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:18944\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:18944\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:18944\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[208:211], %[b4], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[212:215], %[b5], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[216:219], %[b6], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[220:223], %[b7], %[s1]\n\t"
      "s_mov_b32 m0, %[m5]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo5], %[rk], %[so5] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:19200\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:19200\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:19200\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:19200\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[192:195], %[b8], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[196:199], %[b9], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[200:203], %[b10], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[204:207], %[b11], %[s1]\n\t"
      "s_mov_b32 m0, %[m6]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo6], %[rk], %[so6] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:36864\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:36864\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:36864\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:36864\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[208:211], %[b12], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[212:215], %[b13], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[216:219], %[b14], %[s1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[s1], v[220:223], %[b15], %[s1]\n\t"
      "s_mov_b32 m0, %[m7]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo7], %[rk], %[so7] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:37120\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:37120\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:37120\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:37120\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[192:195], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[196:199], %[c1], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[200:203], %[c2], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[204:207], %[c3], %[d0]\n\t"
      "s_mov_b32 m0, %[m8]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo0], %[rv], %[so0] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:37376\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:37376\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:37376\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:37376\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[208:211], %[c4], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[212:215], %[c5], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[216:219], %[c6], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[220:223], %[c7], %[d0]\n\t"
      "s_mov_b32 m0, %[m9]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo1], %[rv], %[so1] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:37632\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:37632\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:37632\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:37632\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[192:195], %[c8], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[196:199], %[c9], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[200:203], %[c10], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[204:207], %[c11], %[d0]\n\t"
      "s_mov_b32 m0, %[m10]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo2], %[rv], %[so2] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:55296\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:55296\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:55296\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:55296\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[208:211], %[c12], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[212:215], %[c13], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[216:219], %[c14], %[d0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d0], v[220:223], %[c15], %[d0]\n\t"
      "s_mov_b32 m0, %[m11]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo3], %[rv], %[so3] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:55552\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:55552\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:55552\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:55552\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[192:195], %[c0], 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[196:199], %[c1], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[200:203], %[c2], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[204:207], %[c3], %[d1]\n\t"
      "s_mov_b32 m0, %[m12]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo4], %[rv], %[so4] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[192:195], %[a0] offset:55808\n\t"
      "ds_read_b128 v[196:199], %[a1] offset:55808\n\t"
      "ds_read_b128 v[200:203], %[a2] offset:55808\n\t"
      "ds_read_b128 v[204:207], %[a3] offset:55808\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[208:211], %[c4], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[212:215], %[c5], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[216:219], %[c6], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[220:223], %[c7], %[d1]\n\t"
      "s_mov_b32 m0, %[m13]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo5], %[rv], %[so5] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "ds_read_b128 v[208:211], %[a0] offset:56064\n\t"
      "ds_read_b128 v[212:215], %[a1] offset:56064\n\t"
      "ds_read_b128 v[216:219], %[a2] offset:56064\n\t"
      "ds_read_b128 v[220:223], %[a3] offset:56064\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[192:195], %[c8], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[196:199], %[c9], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[200:203], %[c10], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[204:207], %[c11], %[d1]\n\t"
      "s_mov_b32 m0, %[m14]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo6], %[rv], %[so6] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[208:211], %[c12], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[212:215], %[c13], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[216:219], %[c14], %[d1]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[d1], v[220:223], %[c15], %[d1]\n\t"
      "s_mov_b32 m0, %[m15]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo7], %[rv], %[so7] offen lds\n\t"
      "s_nop 15\n\ts_nop 3\n\t"
      "s_mov_b32 m0, %[m0s]"
      : [m0s] "=&s"(m0_saved), [s0] "=&v"(s0), [s1] "=&v"(s1), [d0] "=&v"(d0),
        [d1] "=&v"(d1), [st0] "=&v"(st[0]), [st1] "=&v"(st[1]), [st2] "=&v"(st[2]),
        [st3] "=&v"(st[3])
      : [a0] "v"(ad[0]), [a1] "v"(ad[1]), [a2] "v"(ad[2]), [a3] "v"(ad[3]),
        [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]),
        [b4] "v"(b[4]), [b5] "v"(b[5]), [b6] "v"(b[6]), [b7] "v"(b[7]),
        [b8] "v"(b[8]), [b9] "v"(b[9]), [b10] "v"(b[10]), [b11] "v"(b[11]),
        [b12] "v"(b[12]), [b13] "v"(b[13]), [b14] "v"(b[14]), [b15] "v"(b[15]),
        [c0] "v"(c[0]), [c1] "v"(c[1]), [c2] "v"(c[2]), [c3] "v"(c[3]),
        [c4] "v"(c[4]), [c5] "v"(c[5]), [c6] "v"(c[6]), [c7] "v"(c[7]),
        [c8] "v"(c[8]), [c9] "v"(c[9]), [c10] "v"(c[10]), [c11] "v"(c[11]),
        [c12] "v"(c[12]), [c13] "v"(c[13]), [c14] "v"(c[14]), [c15] "v"(c[15]),
        [sa] "v"(sad), [rk] "s"(rk), [rv] "s"(rv), [vo0] "v"(vo[0]),
        [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]),
        [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [so0] "s"(so[0]),
        [so1] "s"(so[1]), [so2] "s"(so[2]), [so3] "s"(so[3]), [so4] "s"(so[4]),
        [so5] "s"(so[5]), [so6] "s"(so[6]), [so7] "s"(so[7]), [m0] "s"(mad[0]),
        [m1] "s"(mad[1]), [m2] "s"(mad[2]), [m3] "s"(mad[3]), [m4] "s"(mad[4]),
        [m5] "s"(mad[5]), [m6] "s"(mad[6]), [m7] "s"(mad[7]), [m8] "s"(mad[8]),
        [m9] "s"(mad[9]), [m10] "s"(mad[10]), [m11] "s"(mad[11]), [m12] "s"(mad[12]),
        [m13] "s"(mad[13]), [m14] "s"(mad[14]), [m15] "s"(mad[15])
      : "memory", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)p;
}

// ----------------------------------------------------------------- rows pass
// kSaved: the forward's output o and row log-sum-exp are given, so there is no
// pass A: Dt = <dO, o> (= <dA, a>), dg = dO o (1 - sigmoid(g)) and lse come
// from the saved state in the loop that forms dA.
template <bool kSaved>
__global__ void __launch_bounds__(256, 1) rows_kernel(BwArgs a) {
  // stage s (0, 1): the K rows of a 32-key tile at lds + 2 s kStage, its V rows after them
  __shared__ __attribute__((aligned(256))) uint8_t lds[4 * kStage];
  const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int64_t nrows = a.T * a.H;
  const int64_t g0 = (int64_t)blockIdx.x * kRowsPerWg;  // the workgroup's rows g0 .. glast
  const int64_t glast = g0 + kRowsPerWg - 1 < nrows ? g0 + kRowsPerWg - 1 : nrows - 1;
  const int64_t r0 = g0 + 16 * W;                       // this wave's rows (none past nrows)
  const int nr = r0 >= nrows ? 0 : (nrows - r0 < 16 ? (int)(nrows - r0) : 16);
  const int64_t rmy = r0 + l16 < nrows ? r0 + l16 : nrows - 1;  // this lane's row (clamped)
  const bool valid = l16 < nr;
  const int t_my = (int)(rmy / a.H);
  const Keys s = keys_of(__builtin_amdgcn_readfirstlane((int)(g0 / a.H)),
                         __builtin_amdgcn_readfirstlane((int)(glast / a.H)), a.Nc);
  const int nt = s.n_tiles;
  const int nc_my = (t_my + 1) / kBlock < s.nc ? (t_my + 1) / kBlock : s.nc;
  const int lo_my = t_my - (kWindow - 1) > 0 ? t_my - (kWindow - 1) : 0;
  const int64_t ro = rmy * kD;

  // dA = dout * sigmoid(g) depends on the inputs alone (rounded to bf16; the
  // key kernel reads it from the workspace too).  With the saved state lane
  // (row l16, g4) forms dims 32 ss + 8 g4 .. +7, exactly its B operand fragment
  // ss of dP^T = V dA^T, so dA stays in registers and nothing waits for its
  // stores; the same loop forms dg and the lane's part of <dO, o>.
  const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.da + r0 * kD, nr * 1024);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + r0 * kD, nr * 1024);
  bf16x8 daf[16], qf[16];
  float dsum = 0.0f;
  if constexpr (kSaved) {
#pragma unroll
  for (int ss = 0; ss < 16; ++ss)
    qf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, l16 * 1024 + 64 * ss + 16 * g4, 0, 0));
  // Four batches of four fragments; the loads of batch b+1 are issued before
  // batch b is formed and stored (the stores could alias later loads, so the
  // compiler would not move those loads above them).
  uint4 gb[2][4], ob[2][4], xb[2][4][2];
  auto load_batch = [&](int b, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * (4 * b + i) + 8 * g4;
      gb[slot][i] = *reinterpret_cast<const uint4*>(a.g + ro + d0);
      ob[slot][i] = *reinterpret_cast<const uint4*>(a.dout + ro + d0);
      if constexpr (kSaved) {
        if (a.out_f32) {
          xb[slot][i][0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.out) + ro + d0);
          xb[slot][i][1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.out) + ro + d0 + 4);
        } else {
          xb[slot][i][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.out) + ro + d0);
        }
      }
    }
  };
  auto form_batch = [&](int b, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ss = 4 * b + i, d0 = 32 * ss + 8 * g4;
      const uint32_t gw[4] = {gb[slot][i].x, gb[slot][i].y, gb[slot][i].z, gb[slot][i].w};
      const uint32_t ow[4] = {ob[slot][i].x, ob[slot][i].y, ob[slot][i].z, ob[slot][i].w};
      float dov[8], sg[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dov[2 * e] = bf16_bits_to_f32(ow[e] & 0xFFFFu);
        dov[2 * e + 1] = bf16_bits_to_f32(ow[e] >> 16);
        sg[2 * e] = sigmoid(bf16_bits_to_f32(gw[e] & 0xFFFFu));
        sg[2 * e + 1] = sigmoid(bf16_bits_to_f32(gw[e] >> 16));
      }
      const u32x4 w4 = {pack_bf16x2(dov[0] * sg[0], dov[1] * sg[1]), pack_bf16x2(dov[2] * sg[2], dov[3] * sg[3]),
                        pack_bf16x2(dov[4] * sg[4], dov[5] * sg[5]), pack_bf16x2(dov[6] * sg[6], dov[7] * sg[7])};
      daf[ss] = __builtin_bit_cast(bf16x8, w4);
      __builtin_amdgcn_raw_buffer_store_b128(w4, rda, l16 * 1024 + 2 * d0, 0, 0);
      if constexpr (kSaved) {
        float ov[8];
        if (a.out_f32) {
          const uint32_t xw[8] = {xb[slot][i][0].x, xb[slot][i][0].y, xb[slot][i][0].z, xb[slot][i][0].w,
                                  xb[slot][i][1].x, xb[slot][i][1].y, xb[slot][i][1].z, xb[slot][i][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[e] = __uint_as_float(xw[e]);
        } else {
          const uint32_t uw[4] = {xb[slot][i][0].x, xb[slot][i][0].y, xb[slot][i][0].z, xb[slot][i][0].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ov[2 * e] = bf16_bits_to_f32(uw[e] & 0xFFFFu);
            ov[2 * e + 1] = bf16_bits_to_f32(uw[e] >> 16);
          }
        }
        float dgv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dsum += dov[e] * ov[e];
          dgv[e] = dov[e] * ov[e] * (1.0f - sg[e]);
        }
        if (valid) {
          *reinterpret_cast<float4*>(a.dg + ro + d0) = make_float4(dgv[0], dgv[1], dgv[2], dgv[3]);
          *reinterpret_cast<float4*>(a.dg + ro + d0 + 4) = make_float4(dgv[4], dgv[5], dgv[6], dgv[7]);
        }
      }
    }
  };
  load_batch(0, 0);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b + 1 < 4) load_batch(b + 1, (b + 1) & 1);
    form_batch(b, b & 1);
  }
  } else {
  // Without the saved state dA is stored, then read back into the operand
  // registers with the Q fragments (forming it in registers here leaves pass A
  // short of registers).
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
  wait_vm<0>();  // the stores have reached L2 (the loads below bypass L1)
#pragma unroll
  for (int ss = 0; ss < 16; ++ss) {
    daf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rda, l16 * 1024 + 64 * ss + 16 * g4, 0, 1));
    qf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, l16 * 1024 + 64 * ss + 16 * g4, 0, 0));
  }
  }

  // visible range of key kk (0 .. 31) of tile j for this lane's row: lo_v <= kk < hi_v
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
  // Tile j's stage; this wave's quarter of its K and V rows into it.
  // Copies of this wave's rows 8W .. 8W+7 of a tile: per-lane (swizzled) and
  // per-row buffer offsets.
  uint32_t vo[8], soff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    vo[u] = (uint32_t)(16 * (lane ^ ((8 * W + u) & 15)));
    soff[u] = (uint32_t)((8 * W + u) * 1024);
  }
  auto kst = [&](int j) { return lds + (j & 1) * (2 * kStage); };
  auto issue_k = [&](int j) { copy8(tile_src(s, j, a.ck, a.k).r, W, vo, kst(j)); };
  auto issue_v = [&](int j) { copy8(tile_src(s, j, a.cv, a.v).r, W, vo, kst(j) + kStage); };
  // Top of tile j: this wave's copies of it (issued during tile j-1) have
  // landed, then every wave's; every wave is also done with tile j-1, whose
  // stage tile j+1 takes.
  auto arrive = [&]() {
    wait_vm<0>();
    barrier_no_fence();
  };
  uint32_t cb[4], tb[8];
  read_bases(l16, g4, cb, tb);
  // LDS rows of this wave's copies of tile j (K rows, then V rows)
  auto next_rows = [&](int j, uint32_t (&mad)[16]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mad[u] = __builtin_amdgcn_readfirstlane(lds_addr(kst(j) + (8 * W + u) * kRow));
      mad[8 + u] = __builtin_amdgcn_readfirstlane(lds_addr(kst(j) + kStage + (8 * W + u) * kRow));
    }
  };
  auto chain_bases = [&](const uint8_t* st, uint32_t (&ad)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) ad[b] = lds_addr(st) + cb[b];
  };
  auto tr_bases = [&](const uint8_t* tile, uint32_t (&ta)[8]) {
#pragma unroll
    for (int b = 0; b < 8; ++b) ta[b] = lds_addr(tile) + tb[b];
  };

  // ---- pass A: per row the maximum (fixed reference m), the weights
  // e_j = 2^(x_j - m) and, with them,
  //   l = sum e_j (fp32),  ldp = sum e_j dp_j,  dp_j = <dA, v_j>,
  //   the forward's ungated output a = (sum bf16(e_j) v_j) / (sum bf16(e_j)),
  // whence lse = m + log2 l and Dt = ldp / l = sum p_j dp_j: the same p and dp
  // the score gradients use, so that sum_j p_j (dp_j - Dt) = 0 holds to fp32
  // rounding (an exact-zero gradient stays zero).  K is read as fragments,
  // V as fragments and transposed.  Keys 16h + 4 g4 + r of a tile are in
  // sc[h][r] (h = 0, 1).
  f32x4 o[32];
  float lse, dt;  // row statistics: log-sum-exp in base-2 score units, Dt = <dA, a>
  if constexpr (kSaved) {
    dt = xsum32(xsum16(dsum));
    lse = a.lse_in[rmy] * 1.4426950408889634f;
    if (valid && g4 == 0) {  // the key kernel reads them from the workspace
      a.lse[rmy] = lse;
      a.dt[rmy] = dt;
    }
  } else {
  float m = -INFINITY, mseen = -INFINITY, l = 0.0f, lb = 0.0f, ldp = 0.0f;
  bool fixed_m = false;
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < 32; ++db) o[db] = f32x4{};
    l = lb = ldp = 0.0f;
    bool over = false;
    barrier_no_fence();  // every wave is done with the stages
    issue_k(0);
    issue_v(0);
    for (int j = 0; j < nt; ++j) {
      arrive();
      uint8_t* const sk = kst(j);
      f32x4 sc[2], dp[2];  // S^T = K Q^T, dP^T = V dA^T
      uint32_t ad[4];
      chain_bases(sk, ad);
      if (j + 1 < nt) {
        uint32_t mad[16];
        next_rows(j + 1, mad);
        chains_rows_dma(sc[0], sc[1], dp[0], dp[1], ad, qf, daf, tile_desc(s, j + 1, a.ck, a.k),
                        tile_desc(s, j + 1, a.cv, a.v), vo, soff, mad);
      } else {
        chains_rows(sc[0], sc[1], dp[0], dp[1], ad, qf, daf);
      }
      int lo_v, hi_v;
      vis(j, lo_v, hi_v);
      float x[8], mt = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = 16 * h + 4 * g4 + r;
          x[4 * h + r] = kk >= lo_v && kk < hi_v ? sc[h][r] * a.c : -INFINITY;
          mt = fmaxf(mt, x[4 * h + r]);
        }
      mt = xmax32(xmax16(mt));
      if (!fixed_m && m == -INFINITY) m = mt;
      mseen = fmaxf(mseen, mt);
      over |= mt > m + kHeadroom;
      const float mx = m == -INFINITY ? 0.0f : m;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(x[i] - mx);
        l += e;
        ldp += e * dp[i >> 2][i & 3];
        pb[i] = (__bf16)e;
        lb += (float)pb[i];
      }
      uint32_t ta[8];
      tr_bases(sk + kStage, ta);
      tr_rows(o, ta, pb);
    }
    // the workgroup walks the tiles again (all waves, barriers in step) if a
    // score of any row rose more than 2^64 above its reference
    if (pass == 1 || !__syncthreads_or(over)) break;
    m = mseen;
    fixed_m = true;
  }
  mfma_drain();

  // ---- row statistics and dg
  const float lrow = xsum32(xsum16(l));
  const float inv_b = 1.0f / xsum32(xsum16(lb));
  lse = m + __builtin_amdgcn_logf(lrow);  // base 2: p_j = 2^(x_j - lse)
  dt = xsum32(xsum16(ldp)) / lrow;
  if (valid && g4 == 0) {
    a.lse[rmy] = lse;
    a.dt[rmy] = dt;
  }
#pragma unroll
  for (int db = 0; db < 32; ++db) {  // fully unrolled: o[db] stays in registers
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
  }  // recompute (no saved state)

  // ---- pass B: dq.  K is read as fragments and transposed, V as fragments.
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4{};
  barrier_no_fence();  // every wave is done with the stages
  issue_k(0);
  issue_v(0);
  for (int j = 0; j < nt; ++j) {
    arrive();
    uint8_t* const sk = kst(j);
    f32x4 sc[2], dp[2];
    uint32_t ad[4];
    chain_bases(sk, ad);
    if (j + 1 < nt) {
      uint32_t mad[16];
      next_rows(j + 1, mad);
      chains_rows_dma(sc[0], sc[1], dp[0], dp[1], ad, qf, daf, tile_desc(s, j + 1, a.ck, a.k),
                      tile_desc(s, j + 1, a.cv, a.v), vo, soff, mad);
    } else {
      chains_rows(sc[0], sc[1], dp[0], dp[1], ad, qf, daf);
    }
    int lo_v, hi_v;
    vis(j, lo_v, hi_v);
    bf16x8 dsb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 16 * (i >> 2) + 4 * g4 + (i & 3);
      const float p = kk >= lo_v && kk < hi_v ? __builtin_amdgcn_exp2f(sc[i >> 2][i & 3] * a.c - lse) : 0.0f;
      dsb[i] = (__bf16)(p * (dp[i >> 2][i & 3] - dt));
    }
    uint32_t ta[8];
    tr_bases(sk, ta);
    tr_rows(o, ta, dsb);
  }
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
  // stage s (0, 1): Q rows of a 32-row block, its dA rows, then lse[32], Dt[32]
  constexpr int kKStage = 2 * kStage + 256;
  __shared__ __attribute__((aligned(256))) uint8_t lds[2 * kKStage];
  const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4, lane16 = lane * 16;
  const int64_t nrows = a.T * a.H;

  // Task -> 64 keys and the row blocks rb0 .. rb1 of queries that can see
  // them (the entry tasks first: they are the long ones).  The entry tasks of
  // one row chunk (every entry group's) are consecutive among the workgroups
  // of one XCD (blockIdx % 8), so they run together and read the chunk's Q and
  // dA rows, in the same order, through that XCD's L2: the rows come from HBM
  // about once rather than once per entry group.
  const int task = blockIdx.x;
  const bool ent = task < a.n_ent_tasks;
  int first, nkeys;
  int64_t rb0, rb1;
  if (ent) {
    const int n_grp = a.n_ent_tasks / a.n_chunks;  // n_chunks is a multiple of 8
    const int k = task >> 3;
    const int grp = k % n_grp, ch = 8 * (k / n_grp) + (task & 7);
    first = kKeysPerWg * grp;
    nkeys = a.Nc - first < kKeysPerWg ? a.Nc - first : kKeysPerWg;
    const int64_t t0 = (int64_t)kBlock * first + kBlock - 1;  // first query seeing entry `first`
    const int64_t c0 = (int64_t)ch * kChunkRb, c1 = c0 + kChunkRb - 1;
    rb0 = t0 * a.H / kTile;
    rb0 = rb0 > c0 ? rb0 : c0;
    rb1 = c1 < a.n_rb - 1 ? c1 : a.n_rb - 1;
  } else {
    first = kKeysPerWg * (task - a.n_ent_tasks);
    nkeys = a.T - first < kKeysPerWg ? (int)(a.T - first) : kKeysPerWg;
    int64_t t1 = (int64_t)first + kKeysPerWg - 1 + (kWindow - 1);
    t1 = t1 < a.T - 1 ? t1 : a.T - 1;
    rb0 = (int64_t)first * a.H / kTile;
    rb1 = (t1 * a.H + a.H - 1) / kTile;
  }
  if (rb0 > rb1) return;  // the whole workgroup: an entry chunk before the entries' first query

  // This wave's 16 keys (none past the last): K and V rows as the B operands
  // of S = Q K^T and dP = dA V^T, lane (key l16, g4) dims 32 ss + 8 g4 .. +7.
  const int wfirst = first + 16 * W;
  const int wkeys = nkeys - 16 * W < 0 ? 0 : (nkeys - 16 * W < 16 ? nkeys - 16 * W : 16);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((ent ? a.ck : a.k) + (int64_t)wfirst * kD, wkeys * 1024);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((ent ? a.cv : a.v) + (int64_t)wfirst * kD, wkeys * 1024);
  bf16x8 kf[16], vf[16];
#pragma unroll
  for (int ss = 0; ss < 16; ++ss) {
    kf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, l16 * 1024 + 64 * ss + 16 * g4, 0, 0));
    vf[ss] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, l16 * 1024 + 64 * ss + 16 * g4, 0, 0));
  }
  const int key = wfirst + l16;  // this lane's key (column l16 of S)
  const int key_t0 = ent ? kBlock * key + kBlock - 1 : key;  // its first query
  const bool key_ok = l16 < wkeys;
  // The flat rows (t, h) that see the key, row = t H + h: row_lo <= row < row_hi
  // (a raw key is seen by queries key .. key + 127, an entry by all from key_t0),
  // so the per-row test needs no division by H.
  const int64_t row_lo = key_ok ? (int64_t)key_t0 * a.H : nrows;
  int64_t row_hi = ent ? nrows : ((int64_t)key + kWindow) * a.H;
  row_hi = row_hi < nrows ? row_hi : nrows;

  f32x4 dk[32], dv[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    dk[db] = f32x4{};
    dv[db] = f32x4{};
  }
  // Row block i's stage; this wave's quarter of its Q and dA rows, and of its
  // statistics (lanes 0, 1: 8 rows' lse, then their Dt): 18 DMA instructions.
  const int nb = (int)(rb1 - rb0 + 1);
  uint32_t vo[8], soff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    vo[u] = (uint32_t)(16 * (lane ^ ((8 * W + u) & 15)));
    soff[u] = (uint32_t)((8 * W + u) * 1024);
  }
  auto st = [&](int i) { return lds + (i & 1) * kKStage; };
  auto issue_q = [&](int i) {
    const int64_t r0 = (rb0 + i) * kTile;
    const int nr = nrows - r0 < kTile ? (int)(nrows - r0) : kTile;
    uint8_t* sp = st(i);
    copy8(make_rsrc(a.q + r0 * kD, nr * 1024), W, vo, sp);
    if (lane < 2) {
      dma16_buf(make_rsrc(a.lse + r0, nr * 4), 32 * W + lane16, (lds_void*)(sp + 2 * kStage + 32 * W));
      dma16_buf(make_rsrc(a.dt + r0, nr * 4), 32 * W + lane16,
                (lds_void*)(sp + 2 * kStage + 128 + 32 * W));
    }
  };
  auto issue_a = [&](int i) {
    const int64_t r0 = (rb0 + i) * kTile;
    const int nr = nrows - r0 < kTile ? (int)(nrows - r0) : kTile;
    copy8(make_rsrc(a.da + r0 * kD, nr * 1024), W, vo, st(i) + kStage);
  };
  uint32_t cb[4], tb[8];
  read_bases(l16, g4, cb, tb);
  issue_q(0);
  issue_a(0);
  for (int i = 0; i < nb; ++i) {
    wait_vm<0>();        // this wave's copies of block i (issued during block i-1)
    barrier_no_fence();  // every wave's; every wave is done with block i-1
    uint8_t* const sp = st(i);
    const int64_t r0 = (rb0 + i) * kTile;
    // S = Q K^T and dP = dA V^T: lane (key l16, g4) gets rows 16h + 4 g4 + r in
    // sc[h][r]; the statistics of rows 4 g4 .. and 16 + 4 g4 .. (lse, then Dt)
    f32x4 sc[2], dp[2], stt[4];
    uint32_t ad[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) ad[b] = lds_addr(sp) + cb[b];
    if (i + 1 < nb) {
      // block i+1's statistics (2 copies, lanes 0 and 1), then its Q and dA rows
      // from inside the chains
      const int64_t n0 = (rb0 + i + 1) * kTile;
      const int nr = nrows - n0 < kTile ? (int)(nrows - n0) : kTile;
      uint8_t* const sq = st(i + 1);
      if (lane < 2) {
        dma16_buf(make_rsrc(a.lse + n0, nr * 4), 32 * W + lane16, (lds_void*)(sq + 2 * kStage + 32 * W));
        dma16_buf(make_rsrc(a.dt + n0, nr * 4), 32 * W + lane16,
                  (lds_void*)(sq + 2 * kStage + 128 + 32 * W));
      }
      uint32_t mad[16];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        mad[u] = __builtin_amdgcn_readfirstlane(lds_addr(sq + (8 * W + u) * kRow));
        mad[8 + u] = __builtin_amdgcn_readfirstlane(lds_addr(sq + kStage + (8 * W + u) * kRow));
      }
      chains_keys_dma(sc[0], sc[1], dp[0], dp[1], ad, kf, vf, lds_addr(sp + 2 * kStage + 16 * g4),
                      stt, desc_words(a.q + n0 * kD, nr * 1024), desc_words(a.da + n0 * kD, nr * 1024),
                      vo, soff, mad);
    } else {
      chains_keys(sc[0], sc[1], dp[0], dp[1], ad, kf, vf, lds_addr(sp + 2 * kStage + 16 * g4), stt);
    }
    bf16x8 pb, dsb;
    // the block's rows r0 + off (off 0 .. 31) that see this lane's key: lo <= off < hi
    const int64_t lo64 = row_lo - r0, hi64 = row_hi - r0;
    const int lo = lo64 < 0 ? 0 : (lo64 > kTile ? kTile : (int)lo64);
    const int hi = hi64 < 0 ? 0 : (hi64 > kTile ? kTile : (int)hi64);
#pragma unroll
    for (int i8 = 0; i8 < 8; ++i8) {
      const int h = i8 >> 2, r = i8 & 3;
      const int off = 16 * h + 4 * g4 + r;
      const bool v = off >= lo && off < hi;
      const float p = v ? __builtin_amdgcn_exp2f(sc[h][r] * a.c - stt[h][r]) : 0.0f;
      pb[i8] = (__bf16)p;
      dsb[i8] = (__bf16)(p * (dp[h][r] - stt[2 + h][r]));
    }
    // dV^T += dA^T P, dK^T += Q^T dS (transposing reads of the row tiles)
    uint32_t ta[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) ta[b] = lds_addr(sp) + tb[b];
    tr_keys2(dv, dk, ta, pb, dsb);
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
  a.out = p.out; a.lse_in = p.lse; a.out_f32 = p.out_f32 ? 1 : 0;
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
  a.n_rb = (int)((rows + kTile - 1) / kTile);
  a.n_chunks = ((a.n_rb + kChunkRb - 1) / kChunkRb + 7) / 8 * 8;  // chunks past the rows are empty
  a.n_ent_tasks = ((a.Nc + kKeysPerWg - 1) / kKeysPerWg) * a.n_chunks;
  a.scale = p.scale;
  a.c = p.scale * 1.4426950408889634f;
  if (a.Nc > 0) {
    const unsigned blocks = (unsigned)(((int64_t)a.Nc * kD + 255) / 256);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, a.dck, (int64_t)a.Nc * kD);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, a.dcv, (int64_t)a.Nc * kD);
  }
  const dim3 rows_grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg));
  if (p.out != nullptr)
    hipLaunchKernelGGL(rows_kernel<true>, rows_grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(rows_kernel<false>, rows_grid, dim3(256), 0, stream, a);
  const int64_t raw_tasks = (p.T + kKeysPerWg - 1) / kKeysPerWg;
  hipLaunchKernelGGL(keys_kernel, dim3((unsigned)(a.n_ent_tasks + raw_tasks)), dim3(256), 0, stream,
                     a);
  if (a.Nc > 0) {
    const int64_t n = (int64_t)a.Nc * kBlock * (kD / 4);
    hipLaunchKernelGGL(pool_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace hca
