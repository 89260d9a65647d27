// gemm_kernel.hpp -- the HGEMM kernel template for gfx950.
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
//                         c ^ (row & 7), an XOR swizzle in the spirit of the
//                         CuTe note's Swizzle<3,3,3> and the ablation draft's
//                         section 3 bank analysis, re-derived for the 16-byte
//                         LDS reads below.
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

#include "device.hpp"

namespace hgemm {

enum LdsLayout { kLdsXor = 0, kLdsPlain = 1, kLdsPad = 2 };
enum Layout { kTN = 0, kNN = 1 };

struct GemmArgs {
  const uint16_t *A;
  const uint16_t *B;
  uint16_t *C;
  int M, N, K;
  int group_m;   // >= 1
  int xcd_remap; // 0 or 1
};

template <int BM_, int BN_, int WM_, int WN_, int LDS_>
struct TileCfg {
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
  static_assert(WM * WN == 4, "four waves per workgroup");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is made of 32x32 blocks");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load passes");
  static_assert(NN_BLOCKS <= NT, "one 8x8 block per thread at most");
};

// Physical 16-byte chunk position of logical chunk c in tile row r.
template <int LDS>
__device__ __forceinline__ int chunk_pos(int r, int c) {
  if constexpr (LDS == kLdsXor) return c ^ (r & 7);
  else return c;
}

// Map the dispatch index to (tile_m, tile_n).
__host__ __device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n,
                                                     int group_m, int xcd_remap, int &tm,
                                                     int &tn) {
  const int total = tiles_m * tiles_n;
  if (xcd_remap) {
    // workgroup i runs on XCD i % 8; give XCD x the ids [x*per, (x+1)*per)
    const int per = total >> 3;
    if (pid < (per << 3)) pid = (pid & 7) * per + (pid >> 3);
  }
  const int width = group_m * tiles_n;
  const int g = pid / width;
  const int first_m = g * group_m;
  const int gsz = (tiles_m - first_m < group_m) ? tiles_m - first_m : group_m;
  const int in = pid - g * width;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

template <class T, int LAYOUT, int DT>
__global__ __launch_bounds__(T::NT, 1) void gemm_kernel(GemmArgs args) {
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
  const bool nn_active = (LAYOUT == kNN) && (tid < T::NN_BLOCKS);
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

  u32x4 ra[LA];
  u32x4 rb[LAYOUT == kTN ? LB : 8];

  auto gload = [&](int k0, bool tail) {
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(a_panel + k0, (uint32_t)(rows_a * K - k0) * 2u);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      uint32_t off = a_off[i];
      if (tail && (k0 + ld_kc * 8 >= K)) off = kOutOfRange;
      ra[i] = load16(rsa, off);
    }
    if constexpr (LAYOUT == kTN) {
      const __amdgpu_buffer_rsrc_t rsb =
          make_rsrc(args.B + (size_t)n0 * K + k0, (uint32_t)(rows_b * K - k0) * 2u);
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        uint32_t off = b_off[i];
        if (tail && (k0 + ld_kc * 8 >= K)) off = kOutOfRange;
        rb[i] = load16(rsb, off);
      }
    } else {
      // rows k0 .. min(K, k0+64) of B[K][N], columns from n0; rows past K
      // fall outside the resource and read as zero.
      const __amdgpu_buffer_rsrc_t rsb =
          make_rsrc(args.B + (size_t)k0 * N + n0, (uint32_t)(min(K - k0, BK) * N) * 2u);
      if (nn_active) {
#pragma unroll
        for (int j = 0; j < 8; ++j) rb[j] = load16(rsb, b_off[j]);
      }
    }
  };

  auto swrite = [&](int stage) {
    char *base = smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *(u32x4 *)(base + st_a + i * T::ROWS_PER_PASS * ROWB) = ra[i];
    if constexpr (LAYOUT == kTN) {
#pragma unroll
      for (int i = 0; i < LB; ++i)
        *(u32x4 *)(base + st_b + i * T::ROWS_PER_PASS * ROWB) = rb[i];
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
            const uint32_t lo = rb[2 * p][d], hi = rb[2 * p + 1][d];
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

  const int KT = (K + BK - 1) / BK;
  const bool has_tail = (K % BK) != 0;
  if (KT > 0) {
    gload(0, has_tail && KT == 1);
    swrite(0);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK, has_tail && (kt + 2 == KT));
    const char *base = smem + cur * T::STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = *(const u32x4 *)(base + rd_a + i * 32 * ROWB + rd_off[ks]);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = *(const u32x4 *)(base + rd_b + j * 32 * ROWB + rd_off[ks]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16<DT>(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < KT) swrite(cur ^ 1);
    __syncthreads();
  }

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
