// decode.hip - HCA decode attention on gfx950: one new query per sequence.
//
// For sequence b with its new token at position t (already written into its
// ring slot t % 128), the keys are the floor((t+1)/128) cached entries and the
// raw rows of positions max(0, t-127) .. t, read from the ring (aitest123.com,
// "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B", section 模型结构; lininn.cn,
// section 43 层里，37 层只读摘要).  The output is gated by sigmoid(G)
// (blog.derekhsu.net, section 低秩閘控注意力).
//
// Decomposition.  One workgroup per (sequence, group of 16 heads).  Its four
// waves split the key list (split-K): wave w takes 32-key tiles w, w+4, ...
// Each wave keeps its own online softmax (m, l, O) and the four partial
// results are merged through LDS at the end (max of m, rescale, sum):
//   m* = max_w m_w,  O = sum_w 2^(m_w - m*) O_w / sum_w 2^(m_w - m*) l_w.
// The four head groups of a sequence read the same keys; consecutive blocks
// (heads of one sequence) are dealt to different XCDs, so the K/V bytes come
// from HBM once and from the MALL after that.
//
// Per wave and 32-key tile (16 heads):
//   S^T[key][head] = K . Q^T   2 x 16 MFMA 16x16x32 (K fragments straight from
//                              global memory, Q fragments in VGPRs)
//   P^T                        each lane holds one head and 8 of the 32 keys
//   O^T[dv][head] += V^T P^T   32 MFMA 16x16x32, V^T through LDS transpose reads
//                              of a 32-row V tile the wave copied by DMA
// Memory bound: per sequence (nc + window) * 2 KiB of K/V plus 3 * H KiB of
// q, g and out.
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kHeads = 16;  // heads per workgroup
constexpr int kTile = 32;

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
  int H;
  float c;  // scale * log2(e)
  int out_f32;
};

// Row pointer of key j of a sequence: entries first, then window positions.
__device__ __forceinline__ const uint16_t* key_row(const uint16_t* entries, const uint16_t* ring,
                                                   int64_t j, int64_t nc, int64_t lo) {
  if (j < nc) return entries + j * kD;
  const int64_t p = lo + (j - nc);
  return ring + (p % kWindow) * kD;
}

__global__ void __launch_bounds__(256, 1) decode_kernel(Args a) {
  // V tiles, 32 KiB per wave; reused for the partial results of the merge.
  __shared__ __attribute__((aligned(1024))) uint8_t sV[4][kTile * 1024];
  __shared__ float sM[4][kHeads];
  __shared__ float sL[4][kHeads];

  const int b = blockIdx.x;
  const int hg = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g4 = lane >> 4;

  int64_t t = a.pos[b];
  if (t < 0) t = 0;
  int64_t nc = (t + 1) / kBlock;
  if (nc > a.nc_cap) nc = a.nc_cap;  // out-of-contract input: never read past the cache
  const int64_t lo = t - (kWindow - 1) > 0 ? t - (kWindow - 1) : 0;
  const int64_t n_keys = nc + (t - lo + 1);
  const int n_tiles = (int)((n_keys + kTile - 1) / kTile);

  const uint16_t* ckb = a.ck + (int64_t)b * a.nc_cap * kD;
  const uint16_t* cvb = a.cv + (int64_t)b * a.nc_cap * kD;
  const uint16_t* wkb = a.wk + (int64_t)b * kWindow * kD;
  const uint16_t* wvb = a.wv + (int64_t)b * kWindow * kD;
  const int64_t head0 = (int64_t)b * a.H + hg * kHeads;

  // Q fragments: lane holds head l16, dims 32ss + 8g4 .. +8.
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q + (head0 + l16) * kD + 8 * g4;
#pragma unroll
    for (int ss = 0; ss < 16; ++ss) qf[ss] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ss);
  }

  f32x4 o[32];
#pragma unroll
  for (int bd = 0; bd < 32; ++bd) o[bd] = f32x4{};
  float m = -INFINITY, l = 0.0f;
  uint8_t* myV = sV[wave];

  for (int it = wave; it < n_tiles; it += 4) {
    const int64_t j0 = (int64_t)it * kTile;
    // V tile -> LDS (rows past the end repeat the last key; they are masked)
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      int64_t j = j0 + r;
      j = j < n_keys ? j : n_keys - 1;
      const uint16_t* vrow = key_row(cvb, wvb, j, nc, lo);
      dma16(vrow + 8 * (lane ^ ((r & 3) << 2)), (lds_void*)(myV + r * 1024));
    }
    // S^T for the two 16-key blocks
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int64_t j = j0 + 16 * blk + l16;
      j = j < n_keys ? j : n_keys - 1;
      const uint16_t* krow = key_row(ckb, wkb, j, nc, lo) + 8 * g4;
      bf16x8 kf[16];
#pragma unroll
      for (int ss = 0; ss < 16; ++ss) kf[ss] = *reinterpret_cast<const bf16x8*>(krow + 32 * ss);
      f32x4 acc = {};
#pragma unroll
      for (int ss = 0; ss < 16; ++ss)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ss], qf[ss], acc, 0, 0, 0);
      s[blk] = acc;
    }
    // mask keys past the end; lane holds keys 16*blk + 4*g4 + r
    float mt = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t j = j0 + 16 * blk + 4 * g4 + r;
        s[blk][r] = j < n_keys ? s[blk][r] * a.c : -INFINITY;
        mt = fmaxf(mt, s[blk][r]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (mt > m) {  // same decision for the four lanes of a head
      const float alpha = exp2f(m - mt);
      m = mt;
      l *= alpha;
#pragma unroll
      for (int bd = 0; bd < 32; ++bd) o[bd] *= alpha;
    }
    uint32_t pk[4];
    float lsum = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[blk][r] - m);
        const float p1 = __builtin_amdgcn_exp2f(s[blk][r + 1] - m);
        const uint32_t w = pack_bf16x2(p0, p1);
        pk[2 * blk + (r >> 1)] = w;
        lsum += bf16_bits_to_f32(w & 0xFFFFu) + bf16_bits_to_f32(w >> 16);
      }
    l += lsum;
    bf16x8 pf;
    {
      const uint32_t w[4] = {pk[0], pk[1], pk[2], pk[3]};
      pf = *reinterpret_cast<const bf16x8*>(w);
    }
    wait_vmem();  // this wave's V tile has landed (LDS private to the wave)
    // V^T fragments: source lane (l16) addresses key row 16*blk + 4*g4 + l16/4,
    // dims 16*bd + 4*(l16 & 3) .. +4.
    const int krow = 4 * g4 + (l16 >> 2);
    const int sw = ((l16 >> 2) & 3) << 2;
    const uint8_t* v0 = myV + krow * 1024;
    const uint8_t* v1 = v0 + 16 * 1024;
    const int half = (l16 & 1) << 3;
#pragma unroll
    for (int bd = 0; bd < 32; ++bd) {
      const int chunk = 2 * bd + ((l16 & 3) >> 1);
      const int off = ((chunk ^ sw) << 4) + half;
      const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + off));
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + off));
      const short w8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(w8);
      o[bd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[bd], 0, 0, 0);
    }
    // all lanes done reading this tile before the next DMA overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four waves (split-K combine through LDS)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // every wave is done with its V tiles
  float* part = reinterpret_cast<float*>(sV[wave]);  // [512 dv][16 heads]
  if (g4 == 0) {
    sM[wave][l16] = m;
    sL[wave][l16] = l;
  }
#pragma unroll
  for (int bd = 0; bd < 32; ++bd)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[(16 * bd + 4 * g4 + r) * kHeads + l16] = o[bd][r];
  __syncthreads();

  // thread -> (head, 32 consecutive dims)
  const int hh = threadIdx.x & 15;
  const int d0 = (threadIdx.x >> 4) * 32;
  float mw[4], ms = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = sM[w][hh];
    ms = fmaxf(ms, mw[w]);
  }
  float wgt[4], lt = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = mw[w] == -INFINITY ? 0.0f : exp2f(mw[w] - ms);
    lt += wgt[w] * sL[w][hh];
  }
  const float inv = 1.0f / lt;
  const uint16_t* grow = a.g + (head0 + hh) * kD;
  constexpr float kLog2e = 1.4426950408889634f;
  for (int d = d0; d < d0 + 32; d += 4) {
    const uint2 gw = *reinterpret_cast<const uint2*>(grow + d);
    const float gv[4] = {bf16_bits_to_f32(gw.x & 0xFFFFu), bf16_bits_to_f32(gw.x >> 16),
                         bf16_bits_to_f32(gw.y & 0xFFFFu), bf16_bits_to_f32(gw.y >> 16)};
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc += wgt[w] * reinterpret_cast<const float*>(sV[w])[(d + e) * kHeads + hh];
      const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
      r[e] = acc * inv * sig;
    }
    if (a.out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (head0 + hh) * kD + d) =
          make_float4(r[0], r[1], r[2], r[3]);
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (head0 + hh) * kD + d) =
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
  a.H = p.H;
  a.c = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_f32 ? 1 : 0;
  hipLaunchKernelGGL(decode_kernel, dim3((unsigned)p.B, (unsigned)(p.H / kHeads)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace hca
