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
// and from that XCD's L2 for the other groups.  The key list (entries, then
// window positions) is walked in 16-key tiles that the four waves copy into
// LDS together by DMA, three tiles ahead of the one being computed (four LDS
// stages of K + V), so about 96 KiB per CU are in flight.  Per tile, every
// wave computes the full scores S^T[key][head] (16 MFMA 16x16x32, K from LDS,
// Q of the 16 heads in VGPRs) and the same online softmax; wave w then adds
// the tile to O^T[dv][head] for dims 128w .. 128w+127 (8 MFMA 16x16x16, V^T
// by one LDS transpose read each, P^T straight from the score registers) and
// at the end gates and stores those dims.  Memory bound: per sequence
// (nc + window) * 2 KiB of K/V plus 3 * H KiB of q, g and out.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kHeads = 16;  // heads per workgroup
constexpr int kTile = 16;
constexpr int kAhead = 3;  // tiles copied ahead of the one computed

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

// Sources of one sequence's keys: its entries (rows 0 .. nc-1 of its cache
// block) and its 128-row window ring, as buffer descriptors.
struct KeySrc {
  __amdgpu_buffer_rsrc_t ek, ev, wk, wv;
  int nc, lo, n_keys;  // key j < nc is entry j, else ring slot (lo + j - nc) % 128
};

// Copy rows 4w .. 4w+3 of tile i into (sK, sV): chunk c of a K row stored at
// c ^ (r & 15), of a V row at c ^ 4(r & 3).  Rows past the last key repeat it
// (finite data; those keys are masked).  Row choice and offsets are
// wave-uniform scalar arithmetic.
__device__ __forceinline__ void copy_tile(const KeySrc& ks, int i, uint8_t* sK, uint8_t* sV,
                                          int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * wave + u;
    int j = i * kTile + r;
    j = j < ks.n_keys ? j : ks.n_keys - 1;
    const bool entry = j < ks.nc;
    const int row = entry ? j : ((ks.lo + j - ks.nc) & (kWindow - 1));
    dma16_buf(entry ? ks.ek : ks.wk, row * 1024 + ((lane ^ (r & 15)) << 4),
              (lds_void*)(sK + r * 1024));
    dma16_buf(entry ? ks.ev : ks.wv, row * 1024 + ((lane ^ ((r & 3) << 2)) << 4),
              (lds_void*)(sV + r * 1024));
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

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__global__ void __launch_bounds__(256, 1) decode_kernel(Args a) {
  // Four stages of (K, V) tiles, separate arrays so the compiler can tell a
  // copy into one stage from reads of another.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK2[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sK3[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV2[kTile * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t sV3[kTile * 1024];

  // blockIdx -> (sequence, head group): XCD x = blockIdx % 8 takes sequences
  // x, x + 8, ... with all their head groups.
  const int L = blockIdx.x;
  const int k8 = L >> 3;
  const int hg = k8 % a.n_hg;
  const int b = (k8 / a.n_hg) * 8 + (L & 7);
  if (b >= a.B) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;

  // Positions below 2^31 (negative ones read as 0); wave-uniform.
  int64_t t64 = a.pos[b];
  t64 = t64 < 0 ? 0 : (t64 > 0x7FFFFFFF ? 0x7FFFFFFF : t64);
  const int t = __builtin_amdgcn_readfirstlane((int)t64);
  KeySrc ks;
  ks.nc = (int)(((int64_t)t + 1) / kBlock);
  if ((int64_t)ks.nc > a.nc_cap) ks.nc = (int)a.nc_cap;  // out-of-contract: never read past the cache
  ks.lo = t - (kWindow - 1) > 0 ? t - (kWindow - 1) : 0;
  ks.n_keys = ks.nc + (t - ks.lo + 1);
  const int n_tiles = (ks.n_keys + kTile - 1) / kTile;
  ks.ek = make_rsrc(a.ck + (int64_t)b * a.nc_cap * kD, ks.nc * 1024);
  ks.ev = make_rsrc(a.cv + (int64_t)b * a.nc_cap * kD, ks.nc * 1024);
  ks.wk = make_rsrc(a.wk + (int64_t)b * kWindow * kD, kWindow * 1024);
  ks.wv = make_rsrc(a.wv + (int64_t)b * kWindow * kD, kWindow * 1024);
  const int64_t head0 = (int64_t)b * a.H + hg * kHeads;

  // Q fragments (B operand of S^T): lane holds head l16, dims 32ss + 8g4 .. +8.
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q + (head0 + l16) * kD + 8 * g4;
#pragma unroll
    for (int ss = 0; ss < 16; ++ss) qf[ss] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ss);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // Q in (copies below are counted from here)
  copy_tile(ks, 0, sK0, sV0, wave, lane);
  if (n_tiles > 1) copy_tile(ks, 1, sK1, sV1, wave, lane);
  if (n_tiles > 2) copy_tile(ks, 2, sK2, sV2, wave, lane);

  // O^T blocks: o[db] lane (head l16, g4), reg r -> dim 128w + 16db + 4g4 + r
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{};
  float m = -INFINITY, l = 0.0f;

  // Tile i in (sK, sV); the copy of tile i+3 goes to (dK, dV), the stage of
  // tile i-1.
  auto tile = [&](int i, const uint8_t* sK, const uint8_t* sV, uint8_t* dK, uint8_t* dV) {
    int pending = n_tiles - 1 - i;  // copies issued after tile i's
    wait_tiles_pending(pending < 2 ? pending : 2);
    // Every wave's rows of tile i have landed and tile i-1 is done: the
    // copies of tiles i+1, i+2 stay in flight across this barrier.
    barrier_no_fence();
    // All LDS reads of the tile first (a read after a copy would wait for it).
    bf16x8 kf[16];
    {
      const uint8_t* krow = sK + l16 * 1024;
#pragma unroll
      for (int ss = 0; ss < 16; ++ss)
        kf[ss] = *reinterpret_cast<const bf16x8*>(krow + (((4 * ss + g4) ^ l16) << 4));
    }
    // V^T fragment of dim block 8w + db: source lane l16 addresses key row
    // 4g4 + l16/4, dims 16(8w+db) + 4(l16&3); the result lane (dim l16 of the
    // block) holds keys 4g4 .. 4g4+3.
    i16x4 vf[8];
    {
      const int krow = 4 * g4 + (l16 >> 2);
      const int sw = ((l16 >> 2) & 3) << 2;
      const uint8_t* v0 = sV + krow * 1024;
      const int half = (l16 & 1) << 3;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int chunk = 2 * (8 * wave + db) + ((l16 & 3) >> 1);
        vf[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + ((chunk ^ sw) << 4) + half));
      }
    }
    if (i + kAhead < n_tiles) copy_tile(ks, i + kAhead, dK, dV, wave, lane);
    // scores: lane holds head l16, keys 4g4 + r of the tile (four independent
    // accumulator chains over the 16 dim steps)
    f32x4 sc[4] = {};
#pragma unroll
    for (int ss = 0; ss < 16; ++ss)
      sc[ss & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ss], qf[ss], sc[ss & 3], 0, 0, 0);
    f32x4 s = (sc[0] + sc[1]) + (sc[2] + sc[3]);
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = i * kTile + 4 * g4 + r;
      s[r] = j < ks.n_keys ? s[r] * a.c : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    mt = xmax32(xmax16(mt));
    if (mt > m) {  // same decision for every lane of a head
      const float alpha = __builtin_amdgcn_exp2f(m - mt);
      m = mt;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    const uint32_t w0 = pack_bf16x2(__builtin_amdgcn_exp2f(s[0] - m), __builtin_amdgcn_exp2f(s[1] - m));
    const uint32_t w1 = pack_bf16x2(__builtin_amdgcn_exp2f(s[2] - m), __builtin_amdgcn_exp2f(s[3] - m));
    l += bf16_bits_to_f32(w0 & 0xFFFFu) + bf16_bits_to_f32(w0 >> 16) +
         bf16_bits_to_f32(w1 & 0xFFFFu) + bf16_bits_to_f32(w1 >> 16);
    // P^T (B operand): lane (head l16, g4) holds keys 4g4 .. 4g4+3, the same
    // keys as the V^T fragments' k-slots.
    const uint32_t pw[2] = {w0, w1};
    const i16x4 pf = *reinterpret_cast<const i16x4*>(pw);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[db], pf, o[db], 0, 0, 0);
  };
  for (int i = 0; i < n_tiles; i += 4) {
    tile(i, sK0, sV0, sK3, sV3);
    if (i + 1 >= n_tiles) break;
    tile(i + 1, sK1, sV1, sK0, sV0);
    if (i + 2 >= n_tiles) break;
    tile(i + 2, sK2, sV2, sK1, sV1);
    if (i + 3 >= n_tiles) break;
    tile(i + 3, sK3, sV3, sK2, sV2);
  }

  // out = O / l * sigmoid(G) for this wave's 128 dims.
  l = xsum32(xsum16(l));
  const float inv = 1.0f / l;
  constexpr float kLog2e = 1.4426950408889634f;
  const int64_t rowo = (head0 + l16) * kD + 128 * wave + 4 * g4;
  uint2 gw[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) gw[db] = *reinterpret_cast<const uint2*>(a.g + rowo + 16 * db);
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
