// gemm_regstage.hpp -- register-staged HGEMM kernel (32x32x16 MFMA, 2-stage
// LDS ring filled through registers).  Kept as the baseline design the
// direct-to-LDS kernel in gemm_kernel.hpp is measured against.
//
// One workgroup computes a BM x BN tile of C with four 64-wide waves, each
// owning a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks whose FP32
// accumulators stay in registers for the whole K loop (the output-stationary
// tiling of the tcgen05 translation's "tiled_matmul" recap; the block -> warp
// -> MMA hierarchy of the HGEMM MMA note, section on the fractal structure;
// the S4000 post's section 3.1 on block and warp tiling).
//
// Per K step of BK = 64:
//   global -> registers : 16-byte buffer loads, 8 lanes per 128-byte row, so
//                         each wave reads whole cache lines (S4000 post 3.2,
//                         vectorised loads); rows past M/N and k past K read
//                         as zero through the buffer range check.
//   registers -> LDS    : 16-byte stores into a 2-stage ring (the multi-stage
//                         pipeline of the HGEMM MMA note and the tcgen05
//                         translation's pipelining section).  Each 128-byte
//                         row of 8 chunks is stored with chunk c at position
//                         c ^ ((row >> 1) & 7), an XOR swizzle in the spirit
//                         of the CuTe note's Swizzle<3,3,3> and the ablation
//                         draft's section 3 bank analysis, re-derived for the
//                         64 banks and 16-byte reads of gfx950 (see LdsLayout).
//   LDS -> registers    : one 16-byte read per operand fragment and lane
//                         (8 consecutive k of one row).
//   MFMA                : v_mfma_f32_32x32x16_{f16,bf16}.
// The operands are fed swapped (B tile as the MFMA's first operand), so each
// lane ends up holding four consecutive columns of one row of C, which the
// epilogue converts to FP16/BF16 (round to nearest even) and stores with 8-byte
// writes: the fused FP32 -> half epilogue.
//
// NN: B[K][N] arrives n-contiguous; each thread loads an 8 (k) x 8 (n) block
// with eight 16-byte loads and transposes it in registers, so the LDS image of
// the B tile is k-contiguous exactly as in TN and the inner loop is shared.
//
// Workgroup order: an XCD-aware remap gives each of the 8 XCDs (which receive
// workgroups round-robin) a contiguous range of tile ids, and the tile ids are
// walked in groups of GROUP_M tile rows, so the tiles resident on one XCD at
// the same time share A row panels and B column panels in its L2 (the block
// swizzle of the HGEMM notes and the grouped order of the tcgen05
// translation's 2-SM section).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace hgemm {

template <int BM_, int BN_, int WM_, int WN_, int LDS_, int PGR_ = 2>
struct RsCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int LDS = LDS_;
  static constexpr int ROWB = (LDS == kLdsPad) ? 144 : 128;  // LDS bytes per tile row
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int ROWS_PER_PASS = NT / 8;           // rows covered by one load pass
  static constexpr int LA = BM / ROWS_PER_PASS;           // A chunks per thread
  static constexpr int LB = BN / ROWS_PER_PASS;           // Bt chunks per thread (TN)
  static constexpr int NN_BLOCKS = BN;                    // 8x8 blocks in a 64 x BN tile (NN)
  static constexpr int PGR = PGR_;                        // register sets of global prefetch
  static_assert(WM * WN == 4, "four waves per workgroup");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is made of 32x32 blocks");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load passes");
  static_assert(NN_BLOCKS <= NT, "one 8x8 block per thread at most");
  static_assert(PGR == 1 || PGR == 2, "one or two register sets");
};

template <class T, int LAYOUT, int DT>
__global__ __launch_bounds__(T::NT, 1) void regstage_kernel(GemmArgs args) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  constexpr int FM = T::FM, FN = T::FN, ROWB = T::ROWB;
  constexpr int LA = T::LA, LB = T::LB;
  __shared__ __attribute__((aligned(16))) char smem[T::LDS_BYTES];

  const int M = args.M, N = args.N, K = args.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, args.group_m, args.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  // ---- global load addressing -------------------------------------------
  // A panel: rows m0 .. m0+BM of A[M][K]; thread loads chunk kc = tid % 8 of
  // rows tid/8 + i*ROWS_PER_PASS.
  const int ld_row = tid >> 3, ld_kc = tid & 7;
  const int rows_a = min(BM, M - m0);
  const uint16_t *a_panel = args.A + (size_t)m0 * K;
  uint32_t a_off[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) a_off[i] = (uint32_t)((ld_row + i * T::ROWS_PER_PASS) * K + ld_kc * 8) * 2u;

  // TN: Bt panel rows n0 .. n0+BN of Bt[N][K], same pattern as A.
  // NN: thread owns the 8x8 block (k = nn_kg*8.., n = nn_nc*8..) of the 64 x BN tile.
  const int rows_b = min(BN, N - n0);
  uint32_t b_off[LAYOUT == kTN ? LB : 8];
  const int nn_kg = tid & 7, nn_nc = tid >> 3;
  const bool nn_active = (LAYOUT == kNN) && (T::NN_BLOCKS == T::NT || tid < T::NN_BLOCKS);
  if constexpr (LAYOUT == kTN) {
#pragma unroll
    for (int i = 0; i < LB; ++i) b_off[i] = (uint32_t)((ld_row + i * T::ROWS_PER_PASS) * K + ld_kc * 8) * 2u;
  } else {
    const bool col_ok = nn_active && (n0 + nn_nc * 8 < N);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      b_off[j] = col_ok ? (uint32_t)((nn_kg * 8 + j) * N + nn_nc * 8) * 2u : kOutOfRange;
  }

  // ---- LDS addressing ----------------------------------------------------
  // Stage s: A rows at s*STAGE, B rows at s*STAGE + BM*ROWB.
  // Store position of this thread's chunk (A, and Bt for TN): row ld_row + i*RPP.
  const uint32_t st_a = ld_row * ROWB + chunk_pos<T::LDS>(ld_row, ld_kc) * 16;
  const uint32_t st_b = BM * ROWB + st_a;
  // Fragment reads: lane reads row (sub-tile base + lane%32), logical chunk 2*ks + lane/32.
  uint32_t rd_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    rd_off[ks] = (lane & 31) * ROWB + chunk_pos<T::LDS>(lane & 31, 2 * ks + (lane >> 5)) * 16;
  const uint32_t rd_a = (wm * T::WTM) * ROWB;            // + i*32*ROWB
  const uint32_t rd_b = BM * ROWB + (wn * T::WTN) * ROWB;  // + j*32*ROWB

  // Global tiles are staged through registers, PGR sets deep: the loads for
  // K step d are issued PGR steps ahead and stored to LDS one step ahead.
  constexpr int PGR = T::PGR;
  constexpr int NRB = (LAYOUT == kTN) ? LB : 8;
  u32x4 ra[PGR][LA];
  u32x4 rb[PGR][NRB];

  // Loads of K step d (k0 = d*BK) into register set P.  Steps at or past K
  // get an empty resource (every load reads zero, no memory is touched), so
  // the steady-state loop needs no branches.
  auto gload = [&](auto P_, int k0) {
    constexpr int P = decltype(P_)::value;
    const int krem = K - k0;  // may be <= 0
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(a_panel + k0, krem > 0 ? (uint32_t)(rows_a * K - k0) * 2u : 0u);
    // chunks past K inside a valid row would read the next row: force them out of range
    const uint32_t kmask = (ld_kc * 8 < krem) ? 0u : kOutOfRange;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[P][i] = load16(rsa, a_off[i] | kmask);
    if constexpr (LAYOUT == kTN) {
      const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
          args.B + (size_t)n0 * K + k0, krem > 0 ? (uint32_t)(rows_b * K - k0) * 2u : 0u);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[P][i] = load16(rsb, b_off[i] | kmask);
    } else {
      // rows k0 .. min(K, k0+64) of B[K][N], columns from n0; rows past K
      // fall outside the resource and read as zero.
      const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
          args.B + (size_t)k0 * N + n0, krem > 0 ? (uint32_t)(min(krem, BK) * N) * 2u : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) rb[P][j] = load16(rsb, b_off[j]);
    }
  };

  // Register set P -> LDS stage.
  auto swrite = [&](auto P_, int stage) {
    constexpr int P = decltype(P_)::value;
    char *base = smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *(u32x4 *)(base + st_a + i * T::ROWS_PER_PASS * ROWB) = ra[P][i];
    if constexpr (LAYOUT == kTN) {
#pragma unroll
      for (int i = 0; i < LB; ++i)
        *(u32x4 *)(base + st_b + i * T::ROWS_PER_PASS * ROWB) = rb[P][i];
    } else {
      if (nn_active) {
        // transpose the 8x8 block: rb[j] holds n = nn_nc*8 + 0..7 at k = nn_kg*8 + j;
        // tile row n gets the 8 k values as one 16-byte chunk (logical chunk nn_kg).
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = i >> 1;
          u32x4 w;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = rb[P][2 * p][d], hi = rb[P][2 * p + 1][d];
            w[p] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          const int row = nn_nc * 8 + i;
          *(u32x4 *)(base + BM * ROWB + row * ROWB + chunk_pos<T::LDS>(row, nn_kg) * 16) = w;
        }
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // Operand fragments of two k slices (16 k each) in flight.
  u32x4 fa[2][FM], fb[2][FN];
  auto read_frags = [&](auto F_, int stage, int ks) {
    constexpr int F = decltype(F_)::value;
    const char *base = smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[F][i] = *(const u32x4 *)(base + rd_a + i * 32 * ROWB + rd_off[ks]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[F][j] = *(const u32x4 *)(base + rd_b + j * 32 * ROWB + rd_off[ks]);
  };
  auto mfmas = [&](auto F_) {
    constexpr int F = decltype(F_)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16<DT>(fb[F][j], fa[F][i], acc[i][j]);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr int NMF = FM * FN, NDSR = FM + FN, NVM = LA + NRB;
  constexpr int NDSW = (LAYOUT == kTN) ? LA + LB : LA + 8;

  const int KT = (K + BK - 1) / BK;

  // Prologue: step 0 in LDS stage 0, steps 1 .. PGR in flight, slice 0 read.
  gload(I0{}, 0);
  swrite(I0{}, 0);
  if constexpr (PGR == 2) gload(I1{}, BK);
  __syncthreads();
  read_frags(I0{}, 0, 0);
  gload(I0{}, PGR * BK);  // register set PGR % PGR = 0
  __builtin_amdgcn_sched_barrier(0);

  // One K step, four phases of FM*FN MFMAs each.  Step kt computes from LDS
  // stage kt&1 while step kt+1 is stored into the other stage and the global
  // loads of step kt+1+PGR are in flight; the barrier sits before the last
  // slice so that slice's MFMAs cover the first LDS reads of the next stage.
  auto kstep = [&](auto S_, int kt) {
    constexpr int S = decltype(S_)::value;  // = kt % 2, the LDS stage computed from
    constexpr int Q = S % PGR;              // = kt % PGR, the register set of step kt
    using Next = std::integral_constant<int, (Q + 1) % PGR>;
    // slice 0 (fragments read before the barrier), read slice 1
    read_frags(I1{}, S, 1);
    mfmas(I0{});
    sched_interleave<NMF, NDSR, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // slice 1, read slice 2
    read_frags(I0{}, S, 2);
    mfmas(I1{});
    sched_interleave<NMF, NDSR, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // slice 2, read slice 3, store step kt+1 into the other stage
    read_frags(I1{}, S, 3);
    swrite(Next{}, S ^ 1);
    mfmas(I0{});
    sched_interleave<NMF, NDSR, NDSW, 0>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // slice 3, read slice 0 of step kt+1, issue the loads of step kt+1+PGR
    read_frags(I0{}, S ^ 1, 0);
    gload(Next{}, (kt + 1 + PGR) * BK);
    mfmas(I1{});
    sched_interleave<NMF, NDSR, 0, NVM>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Steps go in pairs so that the stage and register-set indices are constants.
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    kstep(I0{}, kt);
    kstep(I1{}, kt + 1);
  }
  if (kt < KT) kstep(I0{}, kt);

  // ---- epilogue: FP32 -> FP16/BF16, 8-byte stores -------------------------
  // lane holds, for block (i, j) and group g, C[m][n .. n+3] with
  // m = m0 + wm*WTM + i*32 + lane%32, n = n0 + wn*WTN + j*32 + 8g + 4*(lane/32).
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * T::WTM + i * 32 + (lane & 31);
    if (m >= M) continue;
    uint16_t *crow = args.C + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * T::WTN + j * 32 + 8 * g + 4 * (lane >> 5);
        if (n < N) {
          u32x2 v;
          v[0] = pack2<DT>(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v[1] = pack2<DT>(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *(u32x2 *)(crow + n) = v;
        }
      }
    }
  }
}

}  // namespace hgemm
