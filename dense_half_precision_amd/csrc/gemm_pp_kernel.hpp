// gemm_pp_kernel.hpp -- the 256 x 256 tile on eight waves in two alternating
// groups ("ping-pong"), TN layout: a measured alternative to the production
// schedule, never chosen automatically.
//
// The production loop (gemm_kernel.hpp) issues every fragment read and every
// direct-to-LDS load between the MFMAs of the same wave.  Here no memory
// instruction sits in an MFMA stream: waves 0-3 (group 0) and 4-7 (group 1),
// one of each group per SIMD, each own a 128 x 64 block of C (2 x 4 wave
// grid) and walk K in slices of 32, alternating
//   a memory phase: the 12 fragment reads of the slice and the 4
//     direct-to-LDS loads of the slice three ahead, then
//   a compute phase: the slice's 32 MFMAs and nothing else,
// each closed by a workgroup barrier.  Group 1 starts one phase late, so that
// on every SIMD one wave issues matrix-core instructions while the other
// issues memory instructions (the role split of the tcgen05 translation's
// warp-specialisation section, done by time instead of by wave).
//
// LDS: a ring of five slices per operand (256 rows x 32 k = 16 KiB each; A,
// then B; 160 KiB).  A row of a slice is 64 bytes, four 16-byte chunks; chunk c
// of row r is stored at c ^ ((r >> 2) & 3), so that the 16 lanes of a fragment
// read (rows r0 .. r0+15, one chunk) cover the 64 banks once, and each load
// instruction writes 1 KiB of consecutive LDS.  Slice j lives in slot j % 5.
// The loads of slice i + 3 are issued in the memory phase of slice i, into the
// slot of slice i - 2, which both groups finished reading (their compute
// phases waited for those reads) before the barrier that ends the compute
// phase of group 1 on slice i - 2.  At the end of the memory phase of slice i
// each wave waits for its own loads of slice i + 1, so that slice i + 1 is
// complete in LDS at the barrier before group 0 reads it.
//
// The slices are summed in the same order as the production kernel's K steps
// (k ascending, 32 at a time, one accumulator per 16 x 16 tile), so the two
// give the same bits.
#pragma once

#include "gemm_kernel.hpp"

namespace hgemm {

struct PpCfg {
  static constexpr int BM = 256, BN = 256, BK = 64;  // BK: the table's K step
  static constexpr int NT = 512;
  static constexpr int LDS = kLdsXor;
  static constexpr int NSLOT = 5;                     // ring slots per operand
  static constexpr int SLOT = 256 * 64;               // one 32-k slice of one operand
  static constexpr int B_BASE = NSLOT * SLOT;
  static constexpr int PIPE_BYTES = 2 * NSLOT * SLOT;
  using Epi = TileCfg<256, 256, kLdsXor, 1, 2, 4>;    // wave grid and epilogue layout
  static constexpr int FM = Epi::FM, FN = Epi::FN;    // 8 x 4 MFMA tiles per wave
  static constexpr int LDS_BYTES = PIPE_BYTES > Epi::EPI_BYTES ? PIPE_BYTES : Epi::EPI_BYTES;
  static_assert(Epi::NW == 8 && Epi::WTM == 128 && Epi::WTN == 64, "wave grid");
  static_assert(LDS_BYTES <= 163840, "160 KiB of LDS");
};

// Direct-to-LDS placement of one slice: lane l of 1 KiB segment s (of 16)
// writes LDS bytes s*1024 + 16*l of the slot, which hold row 16s + l/4,
// stored chunk l%4, that is logical chunk (l%4) ^ ((row >> 2) & 3).
__host__ __device__ __forceinline__ void pp_load_place(int s, int lane, int &row, int &chunk) {
  row = 16 * s + (lane >> 2);
  chunk = (lane & 3) ^ ((row >> 2) & 3);
}

// LDS byte offset within a slot that lane l reads for the fragment of rows
// 16f .. 16f+15: row 16f + l%16, logical chunk l/16 (k = 8*(l/16) .. +7 of
// the slice), i.e. f*1024 + pp_frag_offset(l).
__host__ __device__ __forceinline__ uint32_t pp_frag_offset(int lane) {
  const int row = lane & 15, chunk = lane >> 4;
  return (uint32_t)(row * 64 + ((chunk ^ ((row >> 2) & 3)) * 16));
}

template <int DT>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs args) {
  using T = PpCfg;
  constexpr int FM = T::FM, FN = T::FN;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

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
  const int NS = (K + 31) / 32;  // slices

  // ---- loads: wave w fills segments 2w and 2w+1 (rows 32w .. 32w+31) of
  // each slice of A and of B, sharing one M0 (immediate offsets 0 and 1024),
  // placed by pp_load_place.  As in the production kernel, the descriptors'
  // base sits kShift bytes low and every offset kShift bytes high, so that no
  // offset goes below zero; chunks past K get an offset past any range.
  constexpr uint32_t kShift = 4096;
  uint32_t off_a[2], off_b[2], off_out[2];
  int chunk[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    int row;
    pp_load_place(2 * wave + s, lane, row, chunk[s]);
    off_a[s] = (uint32_t)(row * lda + 8 * chunk[s]) * 2u + kShift - 1024u * s;
    off_b[s] = (uint32_t)(row * ldb + 8 * chunk[s]) * 2u + kShift - 1024u * s;
    off_out[s] = kOutOfRange + kShift - 1024u * s;
  }
  const uint16_t *a_panel = args.A + (size_t)m0 * lda;
  const uint16_t *b_panel = args.B + (size_t)n0 * ldb;
  // rows past the tile edge and every slice past K read as zero
  auto rsrc = [&](const uint16_t *panel, int ld, int rows, int k0) {
    const int krem = K - k0;
    const char *base = (const char *)(panel + k0) - kShift;
    const uint32_t bytes = krem <= 0 ? 0u : (uint32_t)((rows - 1) * ld + krem) * 2u + kShift;
    return make_rsrc(base, bytes);
  };
  auto load_slice = [&](int j) {
    const int k0 = 32 * j, krem = K - k0;
    const __amdgpu_buffer_rsrc_t ra = rsrc(a_panel, lda, rows_a, k0);
    const __amdgpu_buffer_rsrc_t rb = rsrc(b_panel, ldb, rows_b, k0);
    const uint32_t slot = (uint32_t)(j % T::NSLOT) * T::SLOT + wave * 2048;
    uint32_t oa[2], ob[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool in = 8 * chunk[s] < krem;  // K % 8 == 0: a chunk is all in or all out
      oa[s] = in ? off_a[s] : off_out[s];
      ob[s] = in ? off_b[s] : off_out[s];
    }
    load16_lds_imm<0>(ra, oa[0], smem + slot);
    load16_lds_imm<1>(ra, oa[1], smem + slot);
    load16_lds_imm<0>(rb, ob[0], smem + T::B_BASE + slot);
    load16_lds_imm<1>(rb, ob[1], smem + T::B_BASE + slot);
  };

  // ---- fragment reads (pp_frag_offset): the MFMA operand layout
  const uint32_t rd = pp_frag_offset(lane);
  const uint32_t rd_a = wm * 128 * 64 + rd;
  const uint32_t rd_b = T::B_BASE + wn * 64 * 64 + rd;
  u32x4 fa[FM], fb[FN];
  auto read_slice = [&](int j) {
    const uint32_t slot = (uint32_t)(j % T::NSLOT) * T::SLOT;
#pragma unroll
    for (int q = 0; q < FN; ++q) fb[q] = *(const u32x4 *)(smem + slot + rd_b + q * 16 * 64);
#pragma unroll
    for (int q = 0; q < FM; ++q) fa[q] = *(const u32x4 *)(smem + slot + rd_a + q * 16 * 64);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

  // ---- prologue: slices 0, 1 and 2 in flight, slice 0 complete everywhere;
  // group 1 then passes one barrier more, which puts it one phase behind
  load_slice(0);
  load_slice(1);
  load_slice(2);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 15));
  wg_barrier();
  if (grp) wg_barrier();
  __builtin_amdgcn_sched_barrier(0);

  for (int i = 0; i < NS; ++i) {
    // memory phase (loads past the last slice read nothing)
    read_slice(i);
    load_slice(i + 3);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 15));  // own loads of slice i+1 landed
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase (operands swapped, as in the production kernel, so that
    // each lane ends with four consecutive columns of one row of C)
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = mfma16x16x32<DT>(fb[b], fa[a], acc[a][b]);
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  // group 0 passes the barrier it skipped at the start: equal counts, and the
  // epilogue's own barrier finds every wave done with the ring
  if (!grp) wg_barrier();

  store_tile<T::Epi, DT>(args, acc, smem, m0, n0, wave, lane);
}

}  // namespace hgemm
