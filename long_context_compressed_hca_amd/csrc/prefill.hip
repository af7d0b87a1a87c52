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
// Work decomposition.  The query tensor is viewed as a flat list of Tq*H rows
// (row = query*H + head); a workgroup owns 128 consecutive rows, 4 waves of 32.
// All rows of a workgroup share one K/V head, so every 32-key tile of K and V
// is staged once in LDS and read by the four waves (for H = 64 that is 2
// queries x 64 heads).  The workgroup walks the compressed entries it can see
// (one set for all its rows except at block ends) and then the raw window,
// in one online softmax.
//
// Per wave and 32-key tile:
//   S^T[key][row] = K . Q^T      32 MFMA 32x32x16 (A = K from LDS, B = Q in VGPRs)
//   mask, online softmax         each lane owns one row and 16 of the 32 keys
//   O^T[dv][row] += V^T . P^T    32 MFMA 32x32x16 (A = V^T via LDS transpose reads)
// Computing the transposes keeps a row in one lane (a 2-lane max/sum per tile)
// and makes P^T the B operand straight from the S^T accumulator layout.
//
// LDS: two stages x (K tile + V tile) x 32 rows x 1 KiB = 128 KiB.  Tiles are
// copied global -> LDS by DMA (global_load_lds_dwordx4, no VGPRs), one 1 KiB
// row per wave instruction, with an XOR swizzle of the 16-byte chunks chosen
// so the two read patterns are bank-conflict free:
//   K: chunk c of key r stored at c ^ (r & 15)   (b128 reads, 16 keys x 1 chunk)
//   V: chunk c of key r stored at c ^ 4(r & 3)   (b64 transpose reads, 4 keys x 4 chunks)
// The tile i+1 copy is in flight while tile i is computed.
//
// Softmax: scores are kept in the exp2 domain (x = s * scale * log2 e).  Each
// row fixes its reference m at its first tile with a visible key and weighs
// every key by p = 2^(x - m); O is never rescaled in the loop (a rescale of
// 256 accumulator registers per lane would cost more than the tile's MFMAs).
// If any score rises more than 2^64 above its reference, the workgroup runs
// its tiles again with the exact row maximum as reference.  P is rounded to
// bf16 for the MFMA and the row sum l adds the rounded values, so O/l is an
// exact weighted mean of V rows up to fp32 accumulation.
//
// Epilogue: out = O / l * sigmoid(G), sigmoid(x) = 1/(1 + 2^(-x log2 e)),
// which gives exactly 0 at G = -inf and 1 at G = +inf.  bf16 (nearest even)
// or f32 output.
//
// Roofline: 4*512 flop per (row, visible key); at 128K context the kernel is
// MFMA bound (about 420 flop per HBM byte).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kRowsPerWG = 128;
constexpr int kTile = 32;
constexpr int kRun = 16;  // consecutive workgroups kept on one XCD
constexpr float kHeadroom = 64.0f;  // p = 2^(x - m) stays below 2^64 in a pass

struct Args {
  const uint16_t* q;
  const uint16_t* g;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  void* out;
  int rows;  // Tq * H
  int q_start, kv_start, Nc;  // positions and counts fit in 31 bits (checked on the host)
  int n_wg;
  int H;
  float c;  // scale * log2(e)
  int out_f32;
};

__device__ __forceinline__ int n_entries(int t, int Nc) {
  const int n = (t + 1) / kBlock;
  return n < Nc ? n : Nc;
}

// Describes the tile sequence of one workgroup.
struct Tiles {
  int nc_wg;  // entries visible to the last row of the workgroup
  int w_lo;   // first raw position of the window union
  int t_max;  // last position of the workgroup
  int n_ct;       // compressed tiles
  int n_tiles;
};

// Copy tile `it` into (sK, sV).  Each wave copies 8 of the 32 key rows of K and
// of V; the row pointers are wave-uniform (SGPRs), the lane offset is 32-bit.
__device__ __forceinline__ void issue_tile(const Args& a, const Tiles& ts, int it, uint8_t* sK,
                                           uint8_t* sV, int wave, int lane) {
  const uint8_t* kb;
  const uint8_t* vb;
  int first, last;
  if (it < ts.n_ct) {
    kb = reinterpret_cast<const uint8_t*>(a.ck);
    vb = reinterpret_cast<const uint8_t*>(a.cv);
    first = it * kTile;
    last = ts.nc_wg - 1;
  } else {
    kb = reinterpret_cast<const uint8_t*>(a.k);
    vb = reinterpret_cast<const uint8_t*>(a.v);
    first = ts.w_lo + (it - ts.n_ct) * kTile - a.kv_start;
    last = ts.t_max - a.kv_start;
  }
#pragma unroll
  for (int u = 0; u < kTile / 4; ++u) {
    const int r = wave * (kTile / 4) + u;  // key row within the tile
    int src = first + r;
    src = src < last ? src : last;  // rows past the end repeat a valid row; they are masked
    const uint8_t* krow = kb + (size_t)src * (kD * 2);
    const uint8_t* vrow = vb + (size_t)src * (kD * 2);
    dma16(krow + ((lane ^ (r & 15)) << 4), (lds_void*)(sK + r * 1024));
    dma16(vrow + ((lane ^ ((r & 3) << 2)) << 4), (lds_void*)(sV + r * 1024));
  }
}

__device__ __forceinline__ float max16(const f32x16& s) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
  return m;
}

struct WaveState {
  f32x16 o[16];  // O^T accumulators: dv block b, lane row l%32
  float m;       // row reference max (exp2 domain), -inf before the first visible key
  float mseen;   // largest score of the row seen so far
  float l;       // this lane's partial row sum (its 16 keys of every tile)
  bool over;     // a score exceeded m + kHeadroom in this pass
};

// Process one 32-key tile for this wave.
//   kind 0: compressed entries e0 .. e0+31;  kind 1: raw positions p0 .. p0+31.
__device__ __forceinline__ void compute_tile(const Args& a, WaveState& st, const bf16x8 (&qf)[32],
                                             const uint8_t* sK, const uint8_t* sV, int kind,
                                             int first, int t, int tw_min, int tw_max,
                                             int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  bool need, full;
  if (kind == 0) {
    need = first < n_entries(tw_max, a.Nc);
    full = first + kTile <= n_entries(tw_min, a.Nc);
  } else {
    need = first <= tw_max && first + kTile - 1 >= tw_min - (kWindow - 1);
    full = first >= tw_max - (kWindow - 1) && first + kTile - 1 <= tw_min;
  }
  if (!need) return;

  // ---- S^T = K . Q^T
  // Step ss reads logical chunk 2ss+g of key row l32, stored at (2ss+g) ^ (l32&15).
  // With ss = 8j + i that is 16j + ((2i + g) ^ (l32&15)): 8 lane offsets, and j
  // becomes an immediate offset of 256 bytes.
  f32x16 s = {};
  const uint8_t* krow = sK + l32 * 1024;
  int koff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) koff[i] = ((2 * i + g) ^ (l32 & 15)) << 4;
#pragma unroll
  for (int ss = 0; ss < 32; ++ss) {
    const bf16x8 kf =
        *reinterpret_cast<const bf16x8*>(krow + koff[ss & 7] + 256 * (ss >> 3));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ss], s, 0, 0, 0);
  }

  // ---- mask (only on tiles where some row of this wave sees part of the tile)
  if (!full) {
    const int nc = n_entries(t, a.Nc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = first + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool vis = kind == 0 ? key < nc : (key <= t && key >= t - (kWindow - 1));
      s[r] = vis ? s[r] : -INFINITY;
    }
  }

  // ---- softmax weights against the row's reference max (exp2 domain)
  float mt = max16(s) * a.c;
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  st.mseen = fmaxf(st.mseen, mt);
  st.m = st.m == -INFINITY ? mt : st.m;  // fixed at the row's first visible key
  st.over |= mt > st.m + kHeadroom;
  const float msub = st.m == -INFINITY ? 0.0f : st.m;
  uint32_t pk[8];
  float lsum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -msub));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], a.c, -msub));
    const uint32_t w = pack_bf16x2(p0, p1);
    pk[r >> 1] = w;
    lsum += bf16_bits_to_f32(w & 0xFFFFu) + bf16_bits_to_f32(w >> 16);
  }
  st.l += lsum;

  // ---- O^T += V^T . P^T
  const int s16 = lane & 15, q4 = lane >> 4;
  const int gq = q4 >> 1, h = q4 & 1;
  const int krow_lo = 4 * gq + (s16 >> 2);                 // + 16*c2 + 8*r
  const int sw = (s16 >> 2) & 3;                            // V swizzle (in 4-chunk units)
  const int cbase = 2 * h + ((s16 & 3) >> 1);               // + 4*b
  const int half = (s16 & 1) << 3;
  // dv block b = 4j + i reads chunk (4b + cbase) ^ 4sw = 16j + 4(i ^ sw) + cbase:
  // 4 lane offsets, j is an immediate offset of 256 bytes.
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = ((4 * (i ^ sw) + cbase) << 4) + half;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    bf16x8 pf;
    {
      const uint32_t w[4] = {pk[4 * c2], pk[4 * c2 + 1], pk[4 * c2 + 2], pk[4 * c2 + 3]};
      pf = *reinterpret_cast<const bf16x8*>(w);
    }
    const uint8_t* v0 = sV + (16 * c2 + krow_lo) * 1024;
    const uint8_t* v1 = v0 + 8 * 1024;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int off = voff[b & 3] + 256 * (b >> 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + off));
      const short w8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(w8);
      st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, st.o[b], 0, 0, 0);
    }
  }
}

__global__ void __launch_bounds__(256, 1) prefill_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTile * 1024];

  // Block -> workgroup: runs of kRun consecutive workgroups stay on one XCD
  // (blocks are dealt to the 8 XCDs round robin), and the heaviest
  // workgroups (latest positions, most entries) are dispatched first.
  const int bid = blockIdx.x;
  const int jx = bid >> 3, xcd = bid & 7;
  const int logical = (jx / kRun) * (8 * kRun) + xcd * kRun + (jx % kRun);
  if (logical >= a.n_wg) return;
  const int wg = a.n_wg - 1 - logical;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  const int row0 = wg * kRowsPerWG;
  const int last = (row0 + kRowsPerWG < a.rows ? row0 + kRowsPerWG : a.rows) - 1;
  const int wr0 = row0 + wave * 32 < last ? row0 + wave * 32 : last;
  const int wr1 = row0 + wave * 32 + 31 < last ? row0 + wave * 32 + 31 : last;
  const int my_row_raw = row0 + wave * 32 + l32;
  const int my_row = my_row_raw < last ? my_row_raw : last;
  const int t = a.q_start + my_row / a.H;
  const int tw_min = a.q_start + wr0 / a.H, tw_max = a.q_start + wr1 / a.H;

  Tiles ts;
  const int t_min = a.q_start + row0 / a.H;
  ts.t_max = a.q_start + last / a.H;
  ts.nc_wg = n_entries(ts.t_max, a.Nc);
  ts.w_lo = t_min - (kWindow - 1) > 0 ? t_min - (kWindow - 1) : 0;
  ts.n_ct = (ts.nc_wg + kTile - 1) / kTile;
  ts.n_tiles = ts.n_ct + (ts.t_max - ts.w_lo + 1 + kTile - 1) / kTile;

  // Q fragments (B operand of S^T): lane holds row l%32, dims 16ss + 8g .. +8.
  bf16x8 qf[32];
  {
    const uint16_t* qrow = a.q + (size_t)my_row * kD + 8 * (lane >> 5);
#pragma unroll
    for (int ss = 0; ss < 32; ++ss) qf[ss] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ss);
  }

  auto tile_first = [&](int it, int& kind) -> int {
    if (it < ts.n_ct) {
      kind = 0;
      return it * kTile;
    }
    kind = 1;
    return ts.w_lo + (it - ts.n_ct) * kTile;
  };

  WaveState st;
  st.m = -INFINITY;
  st.mseen = -INFINITY;
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int b = 0; b < 16; ++b) st.o[b] = f32x16{};
    st.l = 0.0f;
    st.over = false;

    issue_tile(a, ts, 0, sK0, sV0, wave, lane);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < ts.n_tiles; it += 2) {
      int kind;
      int first;
      if (it + 1 < ts.n_tiles) issue_tile(a, ts, it + 1, sK1, sV1, wave, lane);
      first = tile_first(it, kind);
      compute_tile(a, st, qf, sK0, sV0, kind, first, t, tw_min, tw_max, lane);
      wait_vmem();
      __syncthreads();
      if (it + 1 >= ts.n_tiles) break;
      if (it + 2 < ts.n_tiles) issue_tile(a, ts, it + 2, sK0, sV0, wave, lane);
      first = tile_first(it + 1, kind);
      compute_tile(a, st, qf, sK1, sV1, kind, first, t, tw_min, tw_max, lane);
      wait_vmem();
      __syncthreads();
    }
    // Scores are weighted against a reference fixed at each row's first
    // visible tile, so O is never rescaled inside the loop.  Only if some
    // score rose more than 2^kHeadroom above its reference (possible only
    // for extreme score ranges) is the workgroup's pass repeated, with the
    // exact row maximum of the first pass as reference; that cannot overflow.
    if (pass == 1 || !__syncthreads_or(st.over)) break;
    st.m = st.mseen;
  }

  // ---- epilogue: out = O / l * sigmoid(G)
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = 1.0f / l_tot;
  if (my_row_raw > last) return;
  const int g = lane >> 5;
  const uint16_t* grow = a.g + (size_t)my_row * kD;
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int b = 0; b < 16; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dv = 32 * b + 8 * i + 4 * g;
      const uint2 gw = *reinterpret_cast<const uint2*>(grow + dv);
      const float gv[4] = {bf16_bits_to_f32(gw.x & 0xFFFFu), bf16_bits_to_f32(gw.x >> 16),
                           bf16_bits_to_f32(gw.y & 0xFFFFu), bf16_bits_to_f32(gw.y >> 16)};
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
        r[e] = st.o[b][4 * i + e] * inv * sig;
      }
      if (a.out_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)my_row * kD + dv) =
            make_float4(r[0], r[1], r[2], r[3]);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (size_t)my_row * kD + dv) =
            make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
      }
    }
  }
}

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
  a.n_wg = (a.rows + kRowsPerWG - 1) / kRowsPerWG;
  if (a.n_wg == 0) return hipSuccess;
  const int per = 8 * kRun;
  const int grid = (a.n_wg + per - 1) / per * per;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
