// gemm_pp_kernel.hpp -- the 256 x 256 tile on eight waves in two alternating
// groups ("ping-pong"), TN layout: a measured alternative to the production
// schedule, never chosen automatically.
//
// The production loop (gemm_kernel.hpp) issues every fragment read and every
// direct-to-LDS load between the MFMAs of the same wave.  Here no memory
// instruction sits in an MFMA stream: waves 0-3 (group 0) and 4-7 (group 1),
// one of each group per SIMD, each own a 128 x 64 block of C (2 x 4 wave
// grid) and walk K in half steps of 32, alternating
//   a memory phase: the 12 fragment reads of the half step and 4 direct-to-LDS
//     loads of a later step, then
//   a compute phase: the half step's 32 MFMAs and nothing else,
// each closed by a workgroup barrier.  Group 1 starts one phase late, so that
// on every SIMD one wave issues matrix-core instructions while the other
// issues memory instructions (the role split of the tcgen05 translation's
// warp-specialisation section, done by time instead of by wave).
//
// LDS holds whole 64-k steps in the production layout (rows of 128 bytes,
// chunk c of row r at c ^ ((r >> 1) & 7), chunk_pos<kLdsXor>) and the
// production ring: three A stages and two B stages of 32 KiB.  Every load
// instruction therefore moves eight whole 128-byte rows, so no cache line is
// requested twice, and the fragment reads are the production kernel's
// (kmajor_frag_offset, half step h of step s reading slice h & 1).
//
// Half steps 2s and 2s+1 read step s.  With "interval" the span between two
// consecutive barriers, group 0's memory phase of half h falls in interval
// 2h and its compute phase in 2h+1; group 1's one interval later.  The memory
// phase of half 2s issues B of step s+1, that of half 2s+1 issues A of step
// s+2; each memory phase ends by waiting for its own fragment reads, and the
// odd ones also for every load but the four just issued, i.e. for A and B of
// step s+1.  So:
//   - step s+1 is complete in LDS at the barrier that opens interval 4s+4,
//     where group 0 first reads it;
//   - B of step s+1 goes into the stage of step s-1, whose last reads (group
//     1, half 2s-1, interval 4s-1) were waited for before the barrier that
//     closes interval 4s-1, the earliest of those loads being issued in
//     interval 4s; A of step s+2 goes into the stage of step s-1 as well
//     (three A stages), two intervals later.
//
// The half steps are summed in the same order as the production kernel's K
// slices (k ascending, 32 at a time, one accumulator per 16 x 16 tile), so the
// two give the same bits.
#pragma once

#include "gemm_kernel.hpp"

namespace hgemm {

struct PpCfg {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int NT = 512;
  static constexpr int LDS = kLdsXor;
  static constexpr int NSA = 3, NSB = 2;              // ring stages of A and of B
  static constexpr int STAGE = 256 * 128;             // one 64-k step of one operand
  static constexpr int B_BASE = NSA * STAGE;
  static constexpr int PIPE_BYTES = (NSA + NSB) * STAGE;
  using Epi = TileCfg<256, 256, kLdsXor, 1, 2, 4>;    // wave grid and epilogue layout
  static constexpr int FM = Epi::FM, FN = Epi::FN;    // 8 x 4 MFMA tiles per wave
  static constexpr int LDS_BYTES = PIPE_BYTES > Epi::EPI_BYTES ? PIPE_BYTES : Epi::EPI_BYTES;
  static_assert(Epi::NW == 8 && Epi::WTM == 128 && Epi::WTN == 64, "wave grid");
  static_assert(LDS_BYTES <= 163840, "160 KiB of LDS");
};

// TIMED: a measurement copy that, like the production kernel's kTimed mode,
// writes workgroup b's shader clock and 100 MHz real-time clock, before its
// tile and after its stores of C are issued, to ((uint64_t *)ws)[4b ..].
template <int DT, bool TIMED = false>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs args) {
  using T = PpCfg;
  constexpr int FM = T::FM, FN = T::FN;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  uint64_t c0 = 0, r0 = 0;
  if constexpr (TIMED) {
    c0 = clock64();
    r0 = wall_clock64();
  }

  const int M = args.M, N = args.N, K = args.K;
  const int lda = args.lda, ldb = args.ldb;
  const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  const int p = __builtin_amdgcn_readfirstlane(xcd_position(blockIdx.x, args.grid, args.xcd_remap));
  int tm, tn;
  tile_of(args.tile_begin + p, tiles_m, tiles_n, args.group_m, tm, tn);
  const int m0 = __builtin_amdgcn_readfirstlane(tm * 256);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * 256);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int wm = wave / T::Epi::WVN, wn = wave % T::Epi::WVN;
  const int rows_a = min(256, M - m0), rows_b = min(256, N - n0);
  const int NS = (K + 63) / 64;  // K steps

  // ---- loads: wave w fills segments 4w .. 4w+3 (rows 32w .. 32w+31) of each
  // stage, four loads sharing one M0 (immediate offsets 0 .. 3072), placed by
  // kmajor_load_offset.  As in the production kernel, the descriptors' base
  // sits kShift bytes low and every offset kShift bytes high, so that no offset
  // goes below zero; chunks past K get an offset past any range.
  constexpr uint32_t kShift = 4096;
  uint32_t off_a[4], off_b[4];
  int chunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int ca, cb;
    off_a[i] = kmajor_load_offset<kLdsXor>(4 * wave + i, lane, lda, ca) + kShift - 1024u * i;
    off_b[i] = kmajor_load_offset<kLdsXor>(4 * wave + i, lane, ldb, cb) + kShift - 1024u * i;
    chunk[i] = ca;  // the same row and lane give the same chunk for A and B
  }
  const uint16_t *a_panel = args.A + (size_t)m0 * lda;
  const uint16_t *b_panel = args.B + (size_t)n0 * ldb;
  // rows past the tile edge and every step past K read as zero
  auto rsrc = [&](const uint16_t *panel, int ld, int rows, int k0) {
    const int krem = K - k0;
    const char *base = (const char *)(panel + k0) - kShift;
    const uint32_t bytes = krem <= 0 ? 0u : (uint32_t)((rows - 1) * ld + krem) * 2u + kShift;
    return make_rsrc(base, bytes);
  };
  auto load_op = [&](const uint16_t *panel, int ld, int rows, const uint32_t *off,
                     uint32_t stage, int s) {
    const int k0 = 64 * s, krem = K - k0;
    const __amdgpu_buffer_rsrc_t r = rsrc(panel, ld, rows, k0);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)  // K % 8 == 0: a chunk is all in or all out
      o[i] = 8 * chunk[i] < krem ? off[i] : kOutOfRange + kShift - 1024u * i;
    char *dst = smem + stage + wave * 4096;
    load16_lds_imm<0>(r, o[0], dst);
    load16_lds_imm<1>(r, o[1], dst);
    load16_lds_imm<2>(r, o[2], dst);
    load16_lds_imm<3>(r, o[3], dst);
  };
  auto load_a = [&](int s) { load_op(a_panel, lda, rows_a, off_a, (uint32_t)(s % T::NSA) * T::STAGE, s); };
  auto load_b = [&](int s) {
    load_op(b_panel, ldb, rows_b, off_b, (uint32_t)(T::B_BASE + (s % T::NSB) * T::STAGE), s);
  };

  // ---- fragment reads: 16 rows x 32 k per fragment (kmajor_frag_offset)
  uint32_t rd[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) rd[sl] = kmajor_frag_offset<kLdsXor>(lane, sl);
  const uint32_t rd_a = wm * 128 * 128, rd_b = T::B_BASE + wn * 64 * 128;
  u32x4 fa[FM], fb[FN];
  auto read_half = [&](int s, int sl) {
    const uint32_t sa = (uint32_t)(s % T::NSA) * T::STAGE + rd_a + rd[sl];
    const uint32_t sb = (uint32_t)(s % T::NSB) * T::STAGE + rd_b + rd[sl];
#pragma unroll
    for (int q = 0; q < FN; ++q) fb[q] = *(const u32x4 *)(smem + sb + q * 16 * 128);
#pragma unroll
    for (int q = 0; q < FM; ++q) fa[q] = *(const u32x4 *)(smem + sa + q * 16 * 128);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

  // compute phase (operands swapped, as in the production kernel, so that
  // each lane ends with four consecutive columns of one row of C), closed by
  // the barrier that hands the matrix cores to the other group
  auto compute = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = mfma16x16x32<DT>(fb[b], fa[a], acc[a][b]);
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: A and B of step 0 landed, A of step 1 in flight; group 1
  // then passes one barrier more, which puts it one phase behind
  load_a(0);
  load_b(0);
  load_a(1);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 15));
  wg_barrier();
  if (grp) wg_barrier();
  __builtin_amdgcn_sched_barrier(0);

  for (int s = 0; s < NS; ++s) {
    // half 2s: memory phase (loads past the last step read nothing)
    read_half(s, 0);
    load_b(s + 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // own fragment reads done
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    compute();
    // half 2s+1
    read_half(s, 1);
    load_a(s + 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0));  // and A, B of step s+1 landed
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    compute();
  }
  // group 0 passes the barrier it skipped at the start: equal counts, and the
  // epilogue's own wait and barrier find every wave done with the ring
  if (!grp) wg_barrier();

  store_tile<T::Epi, DT>(args, acc, smem, m0, n0, wave, lane);
  if constexpr (TIMED) {
    const uint64_t c1 = clock64(), r1 = wall_clock64();
    if (threadIdx.x == 0) {
      uint64_t *t = reinterpret_cast<uint64_t *>(args.ws) + 4 * (size_t)blockIdx.x;
      t[0] = c0;
      t[1] = r0;
      t[2] = c1;
      t[3] = r1;
    }
  }
}

}  // namespace hgemm
