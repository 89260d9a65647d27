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
  int chunk[4];  // logical k-chunk of each load: the same for A and B (same row and lane)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    off_a[i] = kmajor_load_offset<kLdsXor>(4 * wave + i, lane, lda, chunk[i]) + kShift - 1024u * i;
    off_b[i] = kmajor_load_offset<kLdsXor>(4 * wave + i, lane, ldb, chunk[i]) + kShift - 1024u * i;
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


// ---------------------------------------------------------------------------
// The 128 x 128 tile on eight waves in two groups that split K: a measured
// alternative to the 128 x 128 deeper-ring kernel for a single round of
// tiles, TN layout.
//
// That kernel's loop is bound by issue, not by the matrix cores: a 64 x 64
// wave block issues 16 fragment reads and 8 loads per 32 MFMAs, and the MFMAs
// wait behind them.  Here both groups hold the whole tile, one 64 x 64 block
// per wave (waves w and w + 4 the same block), so the reads per MFMA do not
// grow; group 0 takes the even K steps and group 1 the odd ones, and each
// wave alternates
//   a memory phase: the 16 fragment reads of its step and 8 direct-to-LDS
//     loads (4 A and 4 B segments) of the step three later, then
//   a compute phase: the step's 32 MFMAs and nothing else,
// each closed by a workgroup barrier, group 1 one phase late.  So in interval
// s (between two barriers) the group of step s reads it while the other
// group computes step s - 1.
//
// LDS: four stages per operand of one 64-k step (128 rows of 128 bytes,
// chunk c of row r at chunk_pos<kLdsXor>), A then B: 128 KiB.  Step t is
// loaded by group (t + 1) % 2 (steps 0..2 in the prologue, step s + 3 in the
// memory phase of step s) into the stage of step t - 4, which the other
// group read in interval t - 4 and waited for before that interval's
// barrier.  Each memory phase ends by waiting for its own reads and for its
// group's loads of step s + 1 (issued in interval s - 2, or the prologue),
// so step s + 1 is complete at the barrier that opens interval s + 1.
// (A five-stage ring in which each group loads the steps it reads, with a
// lead of four intervals, measured 3-8 % slower still.)
//
// At the end group 1 adds its sums into group 0's through LDS and group 0
// writes C.  The sum of an element is therefore (even steps) + (odd steps),
// each in k order: not the production kernel's order, so the two differ in
// the last bits (both within the tolerance against the oracle); run to run
// it is the same.
//
// Measured against the deeper-ring kernel on single-round TN shapes
// (1536^3 to 2048^2 x 8192, 256 x 16384 x 4096): 0.85-0.95 of its rate.
// Halving the MFMAs between two barriers leaves each phase short against
// the barrier and the fixed costs (prologue, the reduction through LDS, the
// epilogue by half the waves) grow relative to the loop, so the kernel stays
// an ablation and is never chosen automatically.
struct PpkCfg {
  static constexpr int BM = 128, BN = 128, BK = 64;
  static constexpr int NT = 512;
  static constexpr int LDS = kLdsXor;
  static constexpr int NST = 4;                        // ring stages per operand
  static constexpr int STAGE = 128 * 128;              // one 64-k step of one operand
  static constexpr int B_BASE = NST * STAGE;
  static constexpr int PIPE_BYTES = 2 * NST * STAGE;
  using Epi = TileCfg<128, 128>;                       // group 0's wave grid and epilogue
  static constexpr int FM = Epi::FM, FN = Epi::FN;     // 4 x 4 MFMA tiles per wave
  static constexpr int RED_BYTES = 4 * FM * FN * 64 * 16;  // group 1's sums
  static constexpr int LDS_BYTES = PIPE_BYTES;
  static_assert(Epi::NW == 4 && Epi::WTM == 64 && Epi::WTN == 64, "wave grid");
  static_assert(RED_BYTES <= LDS_BYTES && Epi::EPI_BYTES <= LDS_BYTES, "LDS reuse");
  static_assert(LDS_BYTES <= 163840, "160 KiB of LDS");
};

template <int DT>
__global__ __launch_bounds__(512) void gemm_ppk_kernel(GemmArgs args) {
  using T = PpkCfg;
  constexpr int FM = T::FM, FN = T::FN, NST = T::NST;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int M = args.M, N = args.N, K = args.K;
  const int lda = args.lda, ldb = args.ldb;
  const int tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  const int p = __builtin_amdgcn_readfirstlane(xcd_position(blockIdx.x, args.grid, args.xcd_remap));
  int tm, tn;
  tile_of(args.tile_begin + p, tiles_m, tiles_n, args.group_m, tm, tn);
  const int m0 = __builtin_amdgcn_readfirstlane(tm * 128);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * 128);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, wl = wave & 3;  // group, wave within the group
  const int wm = wl >> 1, wn = wl & 1;
  const int rows_a = min(128, M - m0), rows_b = min(128, N - n0);
  const int KT = (K + 63) / 64;

  // ---- loads: wave wl of the loading group fills segments 4wl .. 4wl+3
  // (rows 32wl .. 32wl+31) of a stage of A and of B, four loads sharing one M0
  // (immediate offsets 0 .. 3072), placed by kmajor_load_offset; descriptors
  // kShift bytes low and offsets kShift high, as in the production kernel
  constexpr uint32_t kShift = 4096;
  uint32_t off_a[4], off_b[4];
  int chunk[4];  // the same for A and B (same row and lane)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    off_a[i] = kmajor_load_offset<kLdsXor>(4 * wl + i, lane, lda, chunk[i]) + kShift - 1024u * i;
    off_b[i] = kmajor_load_offset<kLdsXor>(4 * wl + i, lane, ldb, chunk[i]) + kShift - 1024u * i;
  }
  const uint16_t *a_panel = args.A + (size_t)m0 * lda;
  const uint16_t *b_panel = args.B + (size_t)n0 * ldb;
  auto rsrc = [&](const uint16_t *panel, int ld, int rows, int k0) {
    const int krem = K - k0;
    const char *base = (const char *)(panel + k0) - kShift;
    const uint32_t bytes = krem <= 0 ? 0u : (uint32_t)((rows - 1) * ld + krem) * 2u + kShift;
    return make_rsrc(base, bytes);
  };
  auto load_op = [&](const uint16_t *panel, int ld, int rows, const uint32_t *off,
                     uint32_t stage, int s) {
    const int krem = K - 64 * s;
    const __amdgpu_buffer_rsrc_t r = rsrc(panel, ld, rows, 64 * s);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)  // K % 8 == 0: a chunk is all in or all out
      o[i] = 8 * chunk[i] < krem ? off[i] : kOutOfRange + kShift - 1024u * i;
    char *dst = smem + stage + wl * 4096;
    load16_lds_imm<0>(r, o[0], dst);
    load16_lds_imm<1>(r, o[1], dst);
    load16_lds_imm<2>(r, o[2], dst);
    load16_lds_imm<3>(r, o[3], dst);
  };
  auto load_step = [&](int s) {  // 8 loads; steps past K read nothing
    const uint32_t st = (uint32_t)(s % NST) * T::STAGE;
    load_op(a_panel, lda, rows_a, off_a, st, s);
    load_op(b_panel, ldb, rows_b, off_b, T::B_BASE + st, s);
  };

  // ---- fragment reads of one step (both 32-k slices), production offsets
  uint32_t rd[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) rd[sl] = kmajor_frag_offset<kLdsXor>(lane, sl);
  const uint32_t rd_a = wm * 64 * 128, rd_b = T::B_BASE + wn * 64 * 128;
  u32x4 fa[2][FM], fb[2][FN];
  auto read_step = [&](int s) {
    const uint32_t st = (uint32_t)(s % NST) * T::STAGE;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int q = 0; q < FN; ++q) fb[sl][q] = *(const u32x4 *)(smem + st + rd_b + q * 2048 + rd[sl]);
#pragma unroll
      for (int q = 0; q < FM; ++q) fa[sl][q] = *(const u32x4 *)(smem + st + rd_a + q * 2048 + rd[sl]);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

  // memory phase of step s: its reads, the loads of step s + 3, then wait for
  // the own reads and for the group's loads of step s + 1 (all but the 8 just
  // issued), and the barrier
  auto memory = [&](int s) {
    read_step(s);
    load_step(s + 3);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 0));
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // compute phase: slice 0 then slice 1 (k ascending), operands swapped as in
  // the production kernel, then the barrier
  auto compute = [&]() {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = mfma16x16x32<DT>(fb[sl][b], fa[sl][a], acc[a][b]);
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: step t loaded by group (t + 1) % 2: group 1 steps 0 and 2,
  // group 0 step 1; group 1 waits for step 0 (step 2 may stay in flight)
  if (grp) {
    load_step(0);
    load_step(2);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 15));
  } else {
    load_step(1);
  }
  __builtin_amdgcn_sched_barrier(0);
  wg_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // ---- main loop: intervals 0 .. KT, each closed by one barrier of every
  // wave; group g reads step s in interval s (s = g mod 2) and computes it in
  // interval s + 1
  if (grp) wg_barrier();  // interval 0: group 1 has nothing to compute
  for (int s = grp; s < KT; s += 2) {
    memory(s);
    compute();
  }
  // both groups have passed KT + 1 interval barriers
  if (((KT & 1) == 0) != (grp == 1)) wg_barrier();

  // ---- group 1's sums into group 0's, through LDS (every load has landed:
  // the last ones, past K, still write their zeros)
  __builtin_amdgcn_s_waitcnt(0);
  wg_barrier();
  f32x4 *red = reinterpret_cast<f32x4 *>(smem) + (size_t)wl * FM * FN * 64 + lane;
  if (grp) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) red[(i * FN + j) * 64] = acc[i][j];
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();
  if (!grp) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const f32x4 v = red[(i * FN + j) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] += v[e];
      }
    store_tile<T::Epi, DT>(args, acc, smem, m0, n0, wl, lane);
  } else {
    wg_barrier();  // the epilogue's barrier (group 0's reads of the sums are done)
  }
}

}  // namespace hgemm
