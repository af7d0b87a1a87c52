// gate.hip - gate logits of the low-rank gate on gfx950: G = latent * W_g^T.
//
// The gate that multiplies the attention output is computed from the query's
// low-rank latent, several times narrower than the hidden state
// (blog.derekhsu.net, section 潛在閘控稀疏注意力, the 低秩閘控注意力 item;
// yilup.net, section 架構設計): G[t, n] = sum_r latent[t, r] * W_g[n, r], with
// n = h * 512 + d indexing the (head, dim) of the gate.  The prefill kernel
// applies sigmoid(G) in its epilogue.
//
// A plain bf16 GEMM with fp32 accumulation, both operands K-contiguous
// (latent [T, R] row major, W_g [N, R] like a linear layer's weight):
//   * a workgroup computes a 256 (n) x 256 (t) tile of G^T, four waves of
//     128 x 128, each 4 x 4 MFMA 32x32x16 blocks with the accumulators in
//     AGPRs; computing G^T puts four consecutive n of one t in each lane, and
//     the epilogue turns the wave's block into rows of G through LDS (the
//     buffers of the tile's last step, 32 rows at a time) so that it stores
//     whole 128-byte lines;
//   * K advances 64 at a time.  Each operand's 256 x 64 slice of a step (32
//     KiB: 128-byte row pieces, whole cache lines) is copied into LDS by DMA,
//     W_g two steps ahead through three buffers, the latent one step ahead
//     through two (five buffers, 160 KiB).  A copy instruction fetches 8 rows
//     x 128 bytes: whole lines, which the copy path moves faster than the
//     half-line pieces of a 32-wide step (the steps are bound by the copies
//     more than by the MFMAs).  The 16-byte chunks of
//     a row are permuted (chunk c of row i at c ^ ((i >> 1) & 7)), applied on
//     the global side of the copy, so the fragment reads of 16 lanes hit 16
//     different bank groups;
//   * one persistent workgroup per CU; in each round the 32 workgroups of an
//     XCD take a group of 4 (t) x 8 (n) tiles, so they read their latent and
//     W_g slices from that XCD's L2 (12 slices instead of 64 per step), and
//     the K steps of a workgroup's tiles form one stream through the buffers.
// Bound: MFMA (arithmetic intensity about 128 flop per byte per tile, more
// with the L2 sharing).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kBT = 256, kBN = 256, kBK = 64;
constexpr int kRowB = kBK * 2;              // 128 bytes per row per step
constexpr int kOpBytes = 256 * kRowB;       // one operand's slice of a step: 32 KiB
constexpr int kWBufs = 3, kLBufs = 2;       // W_g buffers, then latent buffers
constexpr int kLdsBytes = (kWBufs + kLBufs) * kOpBytes;
constexpr int kEpiRow = 256 + 16;           // LDS row of the epilogue's transpose
static_assert(2 * 32 * kEpiRow <= kOpBytes, "two waves' epilogue rows fit a buffer");

struct GateArgs {
  const uint16_t* lat;  // [T, R]
  const uint16_t* w;    // [N, R]
  uint16_t* g;          // [T, N]
  int64_t T;
  int R, N;
  int n_tiles_t, n_tiles_n;
};

// Position of 16-byte chunk c of row i inside its 128-byte LDS row.
__device__ __forceinline__ int chunk_pos(int i, int c) { return c ^ ((i >> 1) & 7); }

// DMA of one operand's 256 x 64 slice (columns k0 .. k0+63) into an LDS
// buffer: wave `wave` copies rows 64 wave .. 64 wave + 63, 8 rows (1 KiB) per
// instruction u (0..7); lane L writes LDS row r0 + L / 8, position L % 8, and
// fetches the chunk stored there.
__device__ __forceinline__ void dma_rows8(__amdgpu_buffer_rsrc_t src, int ld_bytes, int k0,
                                          uint8_t* dst, int wave, int lane, int u) {
  const int row = 64 * wave + 8 * u + (lane >> 3), pos = lane & 7;
  const int c = pos ^ ((row >> 1) & 7);
  dma16_buf(src, row * ld_bytes + 2 * k0 + 16 * c, (lds_void*)(dst + (64 * wave + 8 * u) * kRowB));
}

// MFMA with the accumulator pinned to AGPRs (inline asm: the builtin lets the
// register allocator move accumulators between register files around the
// loop).  The operands come from LDS reads, whose waits the compiler inserts;
// no VALU instruction writes them.  The accumulators are zeroed long before
// the first MFMA and read after mfma_drain().
__device__ __forceinline__ void mfma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Tile q (0, 1, ...) of workgroup L: in round q, XCD x = L % 8 takes group
// 8 q + x of 4 (t) x 8 (n) tiles, and its workgroup L / 8 takes tile L / 8 of
// the group.  False past the workgroup's last tile (t tiles are rounded up to
// a multiple of 4 per group; the tiles past the last are skipped).
__device__ __forceinline__ bool tile_of(const GateArgs& a, int L, int q, int& tt, int& nt) {
  const int groups_n = a.n_tiles_n / 8;
  const int grp = q * 8 + (L & 7), w32 = L >> 3;
  tt = (grp / groups_n) * 4 + (w32 >> 3);
  nt = (grp % groups_n) * 8 + (w32 & 7);
  return tt < a.n_tiles_t;
}

// Persistent: one workgroup per CU walks its tiles, and the K steps of all of
// them form one stream through the five buffers (a tile's first copies are
// issued during the previous tile's last steps and land during its
// epilogue), so the copy path, which bounds the steps, stays busy across
// tiles.
__global__ void __launch_bounds__(256, 1) gate_kernel(GateArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

  const int L = blockIdx.x;
  int tt, nt;
  if (!tile_of(a, L, 0, tt, nt)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wa = wave >> 1, wb = wave & 1;  // n half, t half
  const int ld = a.R * 2;
  const int nk = a.R / kBK;
  const int fi = lane & 31, fh = lane >> 5;
  uint8_t* const wbuf = lds;                       // W_g of stream step j: buffer j % 3
  uint8_t* const lbuf = lds + kWBufs * kOpBytes;   // latent of stream step j: buffer j % 2

  auto w_rsrc = [&](int n_t) { return make_rsrc(a.w + (int64_t)n_t * kBN * a.R, kBN * ld); };
  auto t_rows_of = [&](int t_t) {
    const int64_t t0 = (int64_t)t_t * kBT;
    return (int)(a.T - t0 < kBT ? a.T - t0 : kBT);
  };
  auto l_rsrc = [&](int t_t) {
    return make_rsrc(a.lat + (int64_t)t_t * kBT * a.R, t_rows_of(t_t) * ld);
  };

  // Copy cursors: the next stream step j whose W_g (latent) slice is to be
  // copied, as tile number q and K step k; live while that tile exists.
  int wq = 0, wk = 0, wj = 0, lq = 0, lk = 0, lj = 0;
  bool w_live = true, l_live = true;
  __amdgpu_buffer_rsrc_t wrs = w_rsrc(nt), lrs = l_rsrc(tt);
  auto copy_w = [&](int u) { dma_rows8(wrs, ld, wk * kBK, wbuf + (wj % kWBufs) * kOpBytes, wave, lane, u); };
  auto copy_l = [&](int u) { dma_rows8(lrs, ld, lk * kBK, lbuf + (lj % kLBufs) * kOpBytes, wave, lane, u); };
  auto adv_w = [&]() {
    ++wj;
    if (++wk == nk) {
      wk = 0;
      int t2, n2;
      w_live = tile_of(a, L, ++wq, t2, n2);
      if (w_live) wrs = w_rsrc(n2);
    }
  };
  auto adv_l = [&]() {
    ++lj;
    if (++lk == nk) {
      lk = 0;
      int t2, n2;
      l_live = tile_of(a, L, ++lq, t2, n2);
      if (l_live) lrs = l_rsrc(t2);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Prologue: W_g of stream steps 0 and 1, the latent of step 0.
#pragma unroll
  for (int u = 0; u < 8; ++u) copy_w(u);
  adv_w();
#pragma unroll
  for (int u = 0; u < 8; ++u) copy_l(u);
  adv_l();
  const bool w1 = w_live;
  if (w1) {
#pragma unroll
    for (int u = 0; u < 8; ++u) copy_w(u);
    adv_w();
  }
  // Fragment offsets: lane (i = lane % 32, k half = lane / 32) of 32-row block
  // bi reads row 32 bi + i, logical chunk 2 kk + lane / 32 (kk = 0..3: the
  // four 16-wide k slices of a step).
  auto read_frags = [&](int j, int kk, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const uint8_t* sw = wbuf + (j % kWBufs) * kOpBytes;
    const uint8_t* sl = lbuf + (j % kLBufs) * kOpBytes;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int r = 128 * wa + 32 * bi + fi;
      af[bi] = *reinterpret_cast<const bf16x8*>(sw + r * kRowB + 16 * chunk_pos(r, 2 * kk + fh));
    }
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int r = 128 * wb + 32 * bj + fi;
      bfr[bj] = *reinterpret_cast<const bf16x8*>(sl + r * kRowB + 16 * chunk_pos(r, 2 * kk + fh));
    }
  };
  // s_waitcnt vmcnt(8) / vmcnt(0), expcnt and lgkmcnt left at "no wait".
  auto wait_vm8 = [&]() { __builtin_amdgcn_s_waitcnt(0x0F78); };
  auto wait_vm0 = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

  // Stream step g runs four k slices of 16 MFMAs each, the fragments of slice
  // kk+1 read during slice kk:
  //   slice 0   issues the latent copies of step g+1, one after every other
  //             MFMA (an issuing copy stalls the wave; spread out, the MFMAs
  //             already issued keep the pipe busy);
  //   slice 1   issues the W_g copies of step g+2 the same way;
  //   sync      after slice 2: this wave's copies of step g+1 have landed
  //             (only the W_g copies of step g+2 may still be in flight;
  //             vector-memory operations complete in issue order, so older
  //             stores are done too) and its reads of step g are done (slice
  //             3's fragments were read during slice 2); barrier: every
  //             wave's, so step g+1 may be read and the buffers of step g
  //             refilled (latent by step g+2, W_g by step g+3);
  //   slice 3   while step g+1's slice-0 fragments are read.
  bf16x8 af[2][4], bf[2][4];
  if (w1) wait_vm8(); else wait_vm0();
  barrier_no_fence();
  read_frags(0, 0, af[0], bf[0]);
  int g = 0;  // stream step
  int q = 0;  // tile number
  for (;;) {
    for (int s = 0; s < nk; ++s, ++g) {
      const bool do_l = l_live, do_w = w_live;  // the latent of step g+1, W_g of step g+2
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cur = kk & 1;
        if (kk == 3) {
          if (do_w) wait_vm8(); else wait_vm0();
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's reads are done
          barrier_no_fence();
          if (do_l) read_frags(g + 1, 0, af[0], bf[0]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          mfma32(acc[m >> 2][m & 3], af[cur][m >> 2], bf[cur][m & 3]);
          if (m == 1 && kk < 3) {
            // after the first MFMAs (which wait for this slice's reads): a
            // wait placed by the compiler for those would otherwise cover
            // these too
            __builtin_amdgcn_sched_barrier(0);
            read_frags(g, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (kk == 0 && (m & 1) && do_l) copy_l(m >> 1);
          if (kk == 1 && (m & 1) && do_w) copy_w(m >> 1);
        }
        if (kk == 0 && do_l) adv_l();
        if (kk == 1 && do_w) adv_w();
      }
    }

    // Epilogue of tile (tt, nt), whose last step was g - 1.  D[n][t] block
    // (bi, bj): lane (t = lane % 32, half h), register r -> n = 8 (r / 4) +
    // 4 h + r % 4, so each lane holds 8-byte pieces of 32 rows of G; stored
    // as they are, every instruction would write 16 bytes of each of 32 rows,
    // which stores at about half the rate of whole lines.  So the wave's
    // block goes through LDS, 32 rows (one bj) at a time, and is stored as
    // whole rows, 4 rows of 256 bytes per instruction.  The buffers of step
    // g - 1 are free (the barrier of its slice 3 followed every wave's last
    // reads of them; their next copies come in step g): waves 0, 1 use its
    // W_g buffer, waves 2, 3 its latent buffer, 32 rows of 256 bytes plus 16
    // bytes of padding each (a piece write of 16 rows hits distinct banks).
    asm volatile("s_nop 15\n\ts_nop 15");  // wait states before VALU reads of the accumulators
    {
      uint8_t* region = (wave < 2 ? wbuf + ((g - 1) % kWBufs) * kOpBytes
                                  : lbuf + ((g - 1) % kLBufs) * kOpBytes) +
                        (wave & 1) * 32 * kEpiRow;
      const int64_t t0 = (int64_t)tt * kBT;
      // Rows past the last one are range checked.
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + t0 * a.N, t_rows_of(tt) * a.N * 2);
      const int n0 = nt * kBN, c16 = lane & 15;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          const f32x16& c = acc[bi][bj];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const u32x2 v = {pack_bf16x2(c[4 * qq], c[4 * qq + 1]), pack_bf16x2(c[4 * qq + 2], c[4 * qq + 3])};
            *reinterpret_cast<u32x2*>(region + fi * kEpiRow + (32 * bi + 8 * qq + 4 * fh) * 2) = v;
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int row = 4 * k + (lane >> 4);
          const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * kEpiRow + 16 * c16);
          store16_buf(rg, ((128 * wb + 32 * bj + row) * a.N + n0 + 128 * wa + 8 * c16) * 2, v);
        }
      }
    }
    if (!tile_of(a, L, ++q, tt, nt)) break;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // every wave is done with the free buffers before step g's copies refill them
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_no_fence();
  }
}

}  // namespace

hipError_t launch_gate(const uint16_t* latent, const uint16_t* w, uint16_t* g, int64_t T, int R,
                       int N, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  GateArgs a;
  a.lat = latent;
  a.w = w;
  a.g = g;
  a.T = T;
  a.R = R;
  a.N = N;
  a.n_tiles_t = (int)((T + kBT - 1) / kBT);
  a.n_tiles_n = N / kBN;
  // one persistent workgroup per CU, 32 per XCD (workgroup L on XCD L % 8);
  // a workgroup with no tile exits at once
  hipLaunchKernelGGL(gate_kernel, dim3(256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
