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
//   * K advances 32 at a time through four LDS stages (32 KiB each), filled by
//     DMA three steps ahead; 64-byte rows are stored with their 16-byte chunks
//     permuted (chunk c of row i at c ^ ((i >> 2) & 3)), so the fragment reads
//     of 8 lanes hit 8 different bank groups; the permutation is applied on
//     the global side of the copy (each lane fetches the chunk that belongs at
//     its LDS position);
//   * tiles are dealt in groups of 4 (t) x 8 (n) per XCD, so the 32
//     workgroups of a group read their latent and W_g slices from that XCD's
//     L2 (12 slices instead of 64 per step).
// Bound: MFMA (arithmetic intensity about 128 flop per byte per tile, more
// with the L2 sharing).
#include "hca_common.h"
#include "hca_kernels.h"

namespace hca {
namespace {

constexpr int kBT = 256, kBN = 256, kBK = 32;
constexpr int kRowB = kBK * 2;              // 64 bytes per row per stage
constexpr int kOpBytes = 256 * kRowB;       // one operand of one stage: 16 KiB
constexpr int kStageB = 2 * kOpBytes;       // W_g then latent
constexpr int kStages = 4;
constexpr int kEpiRow = 256 + 16;           // LDS row of the epilogue's transpose
constexpr int kLdsBytes = kStages * kStageB > 4 * 128 * kEpiRow ? kStages * kStageB : 4 * 128 * kEpiRow;

struct GateArgs {
  const uint16_t* lat;  // [T, R]
  const uint16_t* w;    // [N, R]
  uint16_t* g;          // [T, N]
  int64_t T;
  int R, N;
  int n_tiles_t, n_tiles_n;
};

// Position of 16-byte chunk c of row i inside its 64-byte LDS row.
__device__ __forceinline__ int chunk_pos(int i, int c) { return c ^ ((i >> 2) & 3); }

// DMA of one operand's 256 x 32 slice (columns k0 .. k0+31) into an LDS
// stage: wave `wave` copies rows 64 wave .. 64 wave + 63, 16 rows (1 KiB) per
// instruction; lane L writes LDS row r0 + L / 4, position L % 4, and fetches
// the chunk stored there.
__device__ __forceinline__ void dma_slice(__amdgpu_buffer_rsrc_t src, int ld_bytes, int k0,
                                          uint8_t* dst, int wave, int lane) {
  const int rr = lane >> 2, pos = lane & 3;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 64 * wave + 16 * u + rr;
    const int c = pos ^ ((row >> 2) & 3);
    dma16_buf(src, row * ld_bytes + 2 * k0 + 16 * c, (lds_void*)(dst + (64 * wave + 16 * u) * kRowB));
  }
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
  // Prologue: steps 0, 1, 2.
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    if (s < nk) {
      dma_slice(rw, ld, s * kBK, lds + s * kStageB, wave, lane);
      dma_slice(rl, ld, s * kBK, lds + s * kStageB + kOpBytes, wave, lane);
    }
  }
  // Fragment offsets: lane (i = lane % 32, k half = lane / 32) of 32-row block
  // bi reads row 32 bi + i, logical chunk 2 kk + lane / 32.
  const int fi = lane & 31, fh = lane >> 5;
  auto read_frags = [&](int s, int kk, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const uint8_t* sw = lds + (s % kStages) * kStageB;
    const uint8_t* sl = sw + kOpBytes;
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
  // This wave's copies of step s have landed: the copies of the steps after
  // it that are already issued (up to s + 2, 8 each) may still be in flight.
  // (s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at "no wait")
  auto wait_step = [&](int s) {
    if (s + 2 < nk)
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    else if (s + 1 < nk)
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };
  // One DMA instruction of step t's copies (u = 0..7: W_g rows, then latent rows).
  auto dma_one = [&](int t, int u) {
    uint8_t* st = lds + (t % kStages) * kStageB + (u < 4 ? 0 : kOpBytes);
    const int uu = u & 3, rr = lane >> 2, pos = lane & 3;
    const int row = 64 * wave + 16 * uu + rr;
    const int c = pos ^ ((row >> 2) & 3);
    dma16_buf(u < 4 ? rw : rl, row * ld + 2 * t * kBK + 16 * c, (lds_void*)(st + (64 * wave + 16 * uu) * kRowB));
  };

  // Step s runs in two halves of 16 MFMAs (k = 0..15, then 16..31):
  //   first half   MFMAs on the k 0..15 fragments (read during the previous
  //                step), while this step's k 16..31 fragments are read and
  //                step s+3's 8 copies issue, one after every other MFMA (an
  //                issuing copy stalls the wave; spread out, the MFMAs already
  //                issued keep the pipe busy);
  //   sync         this wave's copies of step s+1 have landed and its reads of
  //                step s are done; barrier: every wave's, so step s+1 may be
  //                read and step s's stage may be refilled by step s+4;
  //   second half  MFMAs on the k 16..31 fragments, while step s+1's k 0..15
  //                fragments are read.
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  wait_step(0);
  barrier_no_fence();
  read_frags(0, 0, a0, b0);
  for (int s = 0; s < nk; ++s) {
    const bool copy = s + 3 < nk;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      mfma32(acc[m >> 2][m & 3], a0[m >> 2], b0[m & 3]);
      if (m == 1) {
        // after the first MFMAs (which wait for the k 0..15 reads): a wait
        // placed by the compiler for those would otherwise cover these too
        __builtin_amdgcn_sched_barrier(0);
        read_frags(s, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((m & 1) && copy) dma_one(s + 3, m >> 1);
    }
    if (s + 1 < nk) wait_step(s + 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's reads are done
    barrier_no_fence();
    if (s + 1 < nk) read_frags(s + 1, 0, a0, b0);
#pragma unroll
    for (int m = 0; m < 16; ++m) mfma32(acc[m >> 2][m & 3], a1[m >> 2], b1[m & 3]);
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
