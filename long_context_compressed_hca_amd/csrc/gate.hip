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
//     the epilogue turns the wave's block into rows of G through LDS so that
//     it stores whole 128-byte lines;
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
//   * tiles are dealt in groups of 4 (t) x 8 (n) per XCD, so the 32
//     workgroups of a group read their latent and W_g slices from that XCD's
//     L2 (12 slices instead of 64 per step).
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
static_assert(4 * 128 * kEpiRow <= kLdsBytes, "the epilogue fits the buffers");

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

__global__ void __launch_bounds__(256, 1) gate_kernel(GateArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

  // blockIdx -> (t tile, n tile): consecutive workgroups of one XCD (blockIdx
  // % 8) fill a group of 4 t tiles x 8 n tiles.
  const int L = blockIdx.x;
  const int x = L & 7, li = L >> 3;
  const int grp = (li >> 5) * 8 + x, w32 = li & 31;
  const int groups_n = a.n_tiles_n / 8;
  const int tt = (grp / groups_n) * 4 + (w32 >> 3);
  const int nt = (grp % groups_n) * 8 + (w32 & 7);
  if (tt >= a.n_tiles_t) return;
  const int64_t t0 = (int64_t)tt * kBT;
  const int n0 = nt * kBN;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wa = wave >> 1, wb = wave & 1;  // n half, t half
  const int ld = a.R * 2;
  const int64_t t_rows = a.T - t0 < kBT ? a.T - t0 : kBT;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (int64_t)n0 * a.R, kBN * ld);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lat + t0 * a.R, (int)t_rows * ld);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = a.R / kBK;
  uint8_t* const wbuf = lds;                       // W_g of step s: buffer s % 3
  uint8_t* const lbuf = lds + kWBufs * kOpBytes;   // latent of step s: buffer s % 2
  auto w_dst = [&](int s) { return wbuf + (s % kWBufs) * kOpBytes; };
  auto l_dst = [&](int s) { return lbuf + (s % kLBufs) * kOpBytes; };
  // Prologue: W_g of steps 0 and 1, the latent of step 0.
#pragma unroll
  for (int u = 0; u < 8; ++u) dma_rows8(rw, ld, 0, w_dst(0), wave, lane, u);
#pragma unroll
  for (int u = 0; u < 8; ++u) dma_rows8(rl, ld, 0, l_dst(0), wave, lane, u);
  if (nk > 1) {
#pragma unroll
    for (int u = 0; u < 8; ++u) dma_rows8(rw, ld, kBK, w_dst(1), wave, lane, u);
  }
  // Fragment offsets: lane (i = lane % 32, k half = lane / 32) of 32-row block
  // bi reads row 32 bi + i, logical chunk 2 kk + lane / 32 (kk = 0..3: the
  // four 16-wide k slices of a step).
  const int fi = lane & 31, fh = lane >> 5;
  auto read_frags = [&](int s, int kk, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const uint8_t* sw = w_dst(s);
    const uint8_t* sl = l_dst(s);
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

  // Step s runs four k slices of 16 MFMAs each, the fragments of slice kk+1
  // read during slice kk:
  //   slice 0   issues the latent copies of step s+1, one after every other
  //             MFMA (an issuing copy stalls the wave; spread out, the MFMAs
  //             already issued keep the pipe busy);
  //   slice 1   issues the W_g copies of step s+2 the same way;
  //   sync      after slice 2: this wave's copies of step s+1 have landed
  //             (only the W_g copies of step s+2 may still be in flight) and
  //             its reads of step s are done (slice 3's fragments were read
  //             during slice 2); barrier: every wave's, so step s+1 may be
  //             read and the buffers of step s refilled (latent by step s+2,
  //             W_g by step s+3);
  //   slice 3   while step s+1's slice-0 fragments are read.
  bf16x8 af[2][4], bf[2][4];
  if (nk > 1) wait_vm8(); else wait_vm0();
  barrier_no_fence();
  read_frags(0, 0, af[0], bf[0]);
  for (int s = 0; s < nk; ++s) {
    const bool copy_l = s + 1 < nk, copy_w = s + 2 < nk;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk == 3) {
        if (copy_w) wait_vm8(); else wait_vm0();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's reads are done
        barrier_no_fence();
        if (s + 1 < nk) read_frags(s + 1, 0, af[0], bf[0]);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma32(acc[m >> 2][m & 3], af[cur][m >> 2], bf[cur][m & 3]);
        if (m == 1 && kk < 3) {
          // after the first MFMAs (which wait for this slice's reads): a wait
          // placed by the compiler for those would otherwise cover these too
          __builtin_amdgcn_sched_barrier(0);
          read_frags(s, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kk == 0 && (m & 1) && copy_l) dma_rows8(rl, ld, (s + 1) * kBK, l_dst(s + 1), wave, lane, m >> 1);
        if (kk == 1 && (m & 1) && copy_w) dma_rows8(rw, ld, (s + 2) * kBK, w_dst(s + 2), wave, lane, m >> 1);
      }
    }
  }

  asm volatile("s_nop 15\n\ts_nop 15");  // wait states before VALU reads of the accumulators
  // Epilogue through LDS.  D[n][t] block (bi, bj): lane (t = lane % 32, half
  // h), register r -> n = 8 (r / 4) + 4 h + r % 4, so each lane holds 8-byte
  // pieces of 32 rows of G; stored as they are, every instruction writes 16
  // bytes of each of 32 rows, which stores at about half the rate of whole
  // lines.  So each wave writes its 128 x 128 block into its own LDS region
  // (rows t of 256 bytes, 16 bytes of padding so a piece write of 16 rows
  // hits distinct banks) and stores it as whole rows, 4 rows of 256 bytes
  // per instruction.  The stages are free: every wave's last LDS reads were
  // waited for before the loop's last barrier.
  uint8_t* region = lds + wave * 128 * kEpiRow;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const f32x16& c = acc[bi][bj];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
        const u32x2 v = {pack_bf16x2(c[4 * qq], c[4 * qq + 1]), pack_bf16x2(c[4 * qq + 2], c[4 * qq + 3])};
        *reinterpret_cast<u32x2*>(region + (32 * bj + fi) * kEpiRow + (32 * bi + 8 * qq + 4 * fh) * 2) = v;
      }
    }
  // Rows past the last one are range checked.
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + t0 * a.N, (int)t_rows * a.N * 2);
  const int c16 = lane & 15;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int row = 4 * k + (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * kEpiRow + 16 * c16);
    store16_buf(rg, ((128 * wb + row) * a.N + n0 + 128 * wa + 8 * c16) * 2, v);
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
  // groups of 4 x 8 tiles; t tiles rounded up to a multiple of 4 (the extra
  // workgroups exit at once), n tiles are a multiple of 8 (N % 2048 == 0)
  const int64_t groups = (int64_t)((a.n_tiles_t + 3) / 4) * (a.n_tiles_n / 8);
  const int64_t wgs = ((groups + 7) / 8) * 8 * 32;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hca
