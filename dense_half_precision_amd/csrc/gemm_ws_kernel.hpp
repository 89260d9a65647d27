// HGEMM with producer/consumer wave specialisation (TN: A[M][K], Bt[N][K]).
//
// The tcgen05 translation's warp-specialisation section splits a workgroup
// into a load warp, an MMA warp and epilogue warps that hand shared-memory
// buffers to each other; the S4000 post names the same idea as its next step.
// On gfx950 the loads need no producer registers at all (direct-to-LDS
// buffer loads), but in the single-role kernel each wave still spends issue
// slots on them: address and descriptor arithmetic, the M0 register, the load
// instructions themselves, which the matrix core waits behind.  Here four
// loader waves issue every load of the workgroup and four MFMA waves only
// read LDS and issue MFMAs.
//
// Register budget decides the shape: eight waves on four SIMDs is two waves
// per SIMD, 256 registers each, so an MFMA wave holds 64 x 128 of C (128
// accumulators + 96 fragment registers) and the tile is 128 x 256.
//
// LDS: a ring of three stages of one K step (A 16 KiB, then B 32 KiB; rows of
// 128 bytes with the XOR swizzle of the single-role kernel), 144 KiB.
// Loads run two steps ahead.  One workgroup barrier per step, in the middle
// of the second k-slice as in the single-role kernel:
//   loader waves, iteration kt (after barrier kt-1, which freed the stage of
//     step kt-1): loads of step kt+2 into that stage; wait for step kt+1;
//     barrier kt.
//   MFMA waves, step kt: slice 0 (reading slice 1 of step kt), the first half
//     of slice 1, own reads drained, barrier kt, the second half of slice 1
//     (reading slice 0 of step kt+1, complete since barrier kt).
// Both roles pass the same barriers: one before the loop, one per step and
// the epilogue's.
#pragma once

#include "gemm_kernel.hpp"

namespace hgemm {

template <int BM_, int BN_>
struct WsCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int NT = 512;                      // 4 MFMA waves (2 x 2) + 4 loader waves
  static constexpr int WVM = 2, WVN = 2, NW = 4;      // the MFMA waves
  static constexpr int WTM = BM / 2, WTN = BN / 2;    // MFMA wave block
  static constexpr int FM = WTM / 16, FN = WTN / 16;  // 16x16 MFMA tiles per wave
  static constexpr int NMF = FM * FN;                 // MFMAs per 32-k slice
  static constexpr int LDS = kLdsXor;
  static constexpr int EPI = 1;
  static constexpr int A_STAGE = BM * 128, B_STAGE = BN * 128;
  static constexpr int STAGE = A_STAGE + B_STAGE;     // A rows, then B rows
  static constexpr int NSTAGE = 3;
  static constexpr int PIPE_BYTES = NSTAGE * STAGE;
  static constexpr int CROW = WTN * 2 + 16;
  static constexpr int EPI_BYTES = 4 * WTM * CROW;
  static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  static constexpr int SEG_A = BM / 8;                // 1 KiB segments of A per step
  static constexpr int SEGS = (BM + BN) / 8;          // ... of A and B
  static constexpr int SEG_W = SEGS / 4;              // per loader wave
  static_assert(SEGS % 4 == 0 && FM % 2 == 0, "tile");
  static_assert(LDS_BYTES <= 163840, "160 KiB of LDS");
};

template <class T, int DT>
__global__ __launch_bounds__(512) void gemm_ws_kernel(GemmArgs args) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  constexpr int FM = T::FM, FN = T::FN, NMF = T::NMF, NR = FM + FN;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int M = args.M, N = args.N, K = args.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int p = __builtin_amdgcn_readfirstlane(xcd_position(blockIdx.x, args.grid, args.xcd_remap));
  int tm, tn;
  tile_of(args.tile_begin + p, tiles_m, tiles_n, args.group_m, tm, tn);
  const int m0 = __builtin_amdgcn_readfirstlane(tm * BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);
  const int KT = (K + BK - 1) / BK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto stage = [](int s) { return (uint32_t)((s % 3) * T::STAGE); };

  if (wave >= 4) {
    // ---- loader waves: segments pw*SEG_W .. of each step (A first, then B)
    const int pw = wave - 4;
    const int lda = args.lda, ldb = args.ldb;
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const uint16_t *a_panel = args.A + (size_t)m0 * lda;
    const uint16_t *b_panel = args.B + (size_t)n0 * ldb;
    uint32_t off[T::SEG_W];
    int chunk[T::SEG_W];
#pragma unroll
    for (int i = 0; i < T::SEG_W; ++i) {
      const int s = pw * T::SEG_W + i;
      off[i] = s < T::SEG_A ? kmajor_load_offset<T::LDS>(s, lane, lda, chunk[i])
                            : kmajor_load_offset<T::LDS>(s - T::SEG_A, lane, ldb, chunk[i]);
    }
    // rows past the tile edge and, from the partial step on, k past K read
    // zero; steps past K have an empty range
    const int tail = (K % BK) ? (K - 1) / BK : -1;
    auto issue = [&](int step) {
      const int k0 = step * BK, krem = K - k0;
      if (step == tail) {
#pragma unroll
        for (int i = 0; i < T::SEG_W; ++i) off[i] = chunk[i] * 8 < krem ? off[i] : kOutOfRange;
      }
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(a_panel + k0, krem > 0 ? (uint32_t)((rows_a - 1) * lda + krem) * 2u : 0u);
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(b_panel + k0, krem > 0 ? (uint32_t)((rows_b - 1) * ldb + krem) * 2u : 0u);
      char *dst = smem + stage(step) + pw * T::SEG_W * 1024;
#pragma unroll
      for (int i = 0; i < T::SEG_W; ++i)
        load16_lds(pw * T::SEG_W + i < T::SEG_A ? ra : rb, off[i], dst + i * 1024);
    };
    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(T::SEG_W, 0));  // step 0 in LDS
    wg_barrier();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 2 < KT) {
        issue(kt + 2);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(T::SEG_W, 0));  // step kt+1 in LDS
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      }
      wg_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();  // the MFMA waves' epilogue barrier
    return;
  }

  // ---- MFMA waves ------------------------------------------------------------
  const int wm = wave >> 1, wn = wave & 1;
  uint32_t rd_off[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) rd_off[sl] = kmajor_frag_offset<T::LDS>(lane, sl);
  const uint32_t rd_a = (wm * T::WTM) * 128;
  const uint32_t rd_b = T::A_STAGE + (wn * T::WTN) * 128;
  u32x4 f[2][FN + FM];  // [set][B fragments 0..FN-1, A fragments FN..FN+FM-1]
  // read op q of slice sl of the step at `st` into set S: B fragments first
  auto read_op = [&](auto S_, uint32_t st, int sl, int q) {
    constexpr int S = decltype(S_)::value;
    if (q < FN) f[S][q] = *(const u32x4 *)(smem + st + rd_b + q * 16 * 128 + rd_off[sl]);
    else f[S][q] = *(const u32x4 *)(smem + st + rd_a + (q - FN) * 16 * 128 + rd_off[sl]);
  };
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};
  auto mfma = [&](auto S_, int t) {
    constexpr int S = decltype(S_)::value;
    const int i = t / FN, j = t % FN;
    acc[i][j] = mfma16x16x32<DT>(f[S][j], f[S][FN + i], acc[i][j]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  wg_barrier();  // step 0 in LDS
#pragma unroll
  for (int q = 0; q < NR; ++q) read_op(I0{}, stage(0), 0, q);
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < KT; ++kt) {
    const uint32_t cs = stage(kt), ns = stage(kt + 1);
    // slice 0; read slice 1
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      mfma(I0{}, t);
#pragma unroll
      for (int q = t * NR / NMF; q < (t + 1) * NR / NMF; ++q) read_op(I1{}, cs, 1, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first half of slice 1
#pragma unroll
    for (int t = 0; t < NMF / 2; ++t) {
      mfma(I1{}, t);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // own reads of step kt done
    wg_barrier();
    // second half of slice 1; read slice 0 of step kt+1
#pragma unroll
    for (int t = NMF / 2; t < NMF; ++t) {
      mfma(I1{}, t);
      constexpr int H = NMF / 2;
      const int u = t - H;
#pragma unroll
      for (int q = u * NR / H; q < (u + 1) * NR / H; ++q) read_op(I0{}, ns, 0, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  store_tile<T, DT>(args, acc, smem, m0, n0, wave, lane);
}

}  // namespace hgemm
