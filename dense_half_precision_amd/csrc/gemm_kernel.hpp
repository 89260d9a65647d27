// gemm_kernel.hpp -- the HGEMM kernel for gfx950.
//
// One workgroup of four 64-wide waves (2 x 2; the wave grid is a parameter,
// and a 2 x 4 grid of eight waves, two per SIMD, is kept as a measured
// variant) computes a BM x BN tile of C; each wave owns a block made of 16x16
// MFMA tiles whose FP32 accumulators stay in registers for the whole K loop
// (a (BM/2) x (BN/2) block with four waves): the output-stationary
// tiling of the tcgen05 translation's tiled_matmul recap and the block ->
// warp -> MMA hierarchy of the HGEMM MMA note (fractal-structure section) and
// of section 3.1 of the S4000 post.
//
// Matrix cores: v_mfma_f32_16x16x32_{f16,bf16}.  Under the MI355X power limit
// it sustains a higher clock than the 32x32x16 form on random data (it moves
// half the accumulator bytes per FLOP), which is what the throughput of a
// dense half-precision GEMM on this part is bound by.
//
// Global -> LDS: direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds), one
// 1 KiB segment per wave instruction, no registers involved (the pages'
// asynchronous gmem -> smem copies: cp.async in the HGEMM MMA note's main
// loop section, TMA in the tcgen05 translation).  Rows past M/N and k past K
// read as zero through the buffer range check.  The LDS holds a ring of NSB
// + 1 A stages and NSB B stages, three and two for a 256 x 256 tile (A and B
// of one K step of 64 are 32 KiB each there, 160 KiB in all): the loads of
// step s are issued during step s - NSB, those of A before that step's
// barrier and those of B after it (the SPREAD configurations: NSB A and NSB B
// stages, both loaded during step s - NSB + 1, evenly among the MFMAs before
// its barrier) -- the multi-stage pipeline of the HGEMM MMA note and
// of the tcgen05 translation's pipelining section, sized to the 160 KiB LDS of
// gfx950.  Each 128-byte row of a K step is stored with its
// 16-byte chunks XOR-swizzled (chunk ^ ((row >> 1) & 7)), an LDS layout that
// keeps both the 16-byte fragment reads and the direct-to-LDS writes free of
// bank conflicts (the swizzle of the CuTe note's first step and the ablation
// draft's section 3 bank analysis, redone for 64 banks).
//
// NN: B arrives k-major (n contiguous).  It is loaded into LDS as is and the
// MFMA operand (8 consecutive k of one n per lane) is assembled with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16, two per fragment), so no
// pass over the data transposes it.
//
// Schedule: one K step is 2 k-slices of 32, 2 * FM * FN MFMAs per wave.  The
// instruction stream is ordered by hand (each MFMA followed by at most one
// LDS read and/or one load, fenced with sched_barrier) so that every memory
// instruction issues while the matrix core is busy.  The fragments of the
// next slice are read during the current one (double buffer in registers);
// the single workgroup barrier per step sits before the last half slice so
// those MFMAs cover the first LDS reads of the next step.  The barrier is a
// bare s_barrier with explicit waits: __syncthreads() would wait for every
// load still in flight.
//
// Epilogue: C = alpha * sums + beta * C, converted to FP16/BF16 (round to
// nearest even) into a wave-private, padded LDS region, then 16-byte stores
// of whole 256-byte row segments (the LDS-staged epilogue of the CuTe note and
// of the S4000 post).
//
// Workgroup order: XCD-aware remap plus grouping by group_m tile rows
// (xcd_position, tile_of), so the tiles resident on one XCD share A and B
// panels in its L2 (the block swizzle of the HGEMM notes, the grouped order of
// the tcgen05 translation's 2-SM section).
//
// Launch modes (gemm_kernel's last parameter): whole-K tiles; K segments of
// the tail tiles, whose FP32 partial sums gemm_sk_fixup adds up; the whole
// rounds followed by the segments in one launch; or one workgroup per CU
// looping over whole-K tiles.  A segment runs the same tile code on a K
// sub-range.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace hgemm {

template <int BM_, int BN_, int LDS_ = kLdsXor, int EPI_ = 1, int WVM_ = 2, int WVN_ = 2,
          int NSB_ = 2, int SPREAD_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WVM = WVM_, WVN = WVN_;        // waves along M and N
  // LDS ring: NSA stages of A and NSB of B.  SPREAD 0: A is loaded NSA - 1
  // steps ahead (in slice 0), B NSB steps ahead (after the barrier), NSA =
  // NSB + 1.  SPREAD 1: both are loaded NSB - 1 steps ahead, spread evenly
  // over the step's MFMAs before the barrier, NSA = NSB.
  static constexpr int SPREAD = SPREAD_;
  static constexpr int NSB = NSB_, NSA = SPREAD_ ? NSB_ : NSB_ + 1;
  static constexpr int NW = WVM * WVN;                // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WVM, WTN = BN / WVN;  // wave block
  static constexpr int FM = WTM / 16, FN = WTN / 16;  // 16x16 MFMA tiles per wave
  static constexpr int NMF = FM * FN;                 // MFMAs per 32-k slice
  static constexpr int LDS = LDS_;
  static constexpr int EPI = EPI_;                    // 1: C through LDS, 0: direct stores
  static constexpr int A_STAGE = BM * 128;            // BM rows x 64 k x 2 bytes
  static constexpr int B_STAGE = BN * 128;            // TN: BN rows x 64 k; NN: 64 rows x BN
  static constexpr int B_BASE = NSA * A_STAGE;        // the A stages, then the B stages
  static constexpr int PIPE_BYTES = NSA * A_STAGE + NSB * B_STAGE;
  static constexpr int CROW = WTN * 2 + 16;           // epilogue row pitch (bytes)
  static constexpr int EPI_BYTES = EPI ? NW * WTM * CROW : 0;
  static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  static constexpr int SEG_A = BM / (8 * NW);         // 1 KiB A segments per wave and step
  static constexpr int SEG_B = BN / (8 * NW);         // 1 KiB B segments per wave and step
  static_assert(BM % 64 == 0 && BN % 64 == 0 && BM <= 256 && BN <= 256, "tile");
  static_assert(SEG_A * 8 * NW == BM && SEG_B * 8 * NW == BN, "whole segments per wave");
  static_assert(WTM % 32 == 0 && WTN % 16 == 0 && (NW == 4 || NW == 8), "wave grid");
  static_assert((WVN & (WVN - 1)) == 0, "wave index split by shift and mask");
  static_assert(FM % 2 == 0, "the slice is split in halves by A block");
  static_assert(LDS_BYTES <= 163840, "160 KiB of LDS");
  static_assert(LDS == kLdsXor || LDS == kLdsPlain, "layouts of this kernel");
  static_assert(!SPREAD || NSB >= 3, "the spread loads need two steps of lead");
};

// Epilogue of a BM x BN tile whose FP32 sums a workgroup holds in acc (wave
// w: block (w/WVN, w%WVN) of WTM x WTN; lane l, tile (i, j): C[m][n .. n+3],
// m = block row + 16i + l%16, n = block column + 16j + 4*(l/16)).
// C = alpha * acc + beta * C, rounded once to the output type; with alpha ==
// 1 and beta == 0 the sums are converted as they are and C is not read.
template <class T, int DT>
__device__ __forceinline__ void store_tile(const GemmArgs &args, f32x4 (&acc)[T::FM][T::FN],
                                           char *smem, int m0, int n0, int wave, int lane) {
  constexpr int FM = T::FM, FN = T::FN;
  const int M = args.M, N = args.N, ldc = args.ldc;
  const int wm = (unsigned)wave / T::WVN, wn = (unsigned)wave % T::WVN;
  const int wm0 = m0 + wm * T::WTM, wn0 = n0 + wn * T::WTN;
  const float alpha = args.alpha, beta = args.beta;
  // packed output of tile (i, j) for this lane; c: the old C there (GEN with
  // beta != 0)
  auto out2 = [&](auto GEN_, int i, int j, u32x2 c) {
    constexpr bool GEN = decltype(GEN_)::value;
    float x[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
    if constexpr (GEN) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= alpha;
      if (beta != 0.0f) {
        float c0, c1, c2, c3;
        unpack2<DT>(c[0], c0, c1);
        unpack2<DT>(c[1], c2, c3);
        x[0] = __builtin_fmaf(beta, c0, x[0]);
        x[1] = __builtin_fmaf(beta, c1, x[1]);
        x[2] = __builtin_fmaf(beta, c2, x[2]);
        x[3] = __builtin_fmaf(beta, c3, x[3]);
      }
    }
    u32x2 v;
    v[0] = pack2<DT>(x[0], x[1]);
    v[1] = pack2<DT>(x[2], x[3]);
    return v;
  };
  // In the general form the old C of CB row blocks of fragments is read at
  // once (at most 128 registers a lane, free after the main loop: the operand
  // fragments are dead by then), so that the latencies of those reads overlap;
  // one row block at a time, they cost 8-22 % (TN f16 8192^3 to 2048^3 with
  // beta = 1).  Elements outside M x N read as 0 and are not stored.
  constexpr int CB = FM < 64 / FN ? FM : 64 / FN;
  static_assert(FM % CB == 0, "row blocks of old C per batch");
  auto epilogue = [&](auto GEN_) {
    constexpr bool GEN = decltype(GEN_)::value;
    if constexpr (T::EPI) {
      __builtin_amdgcn_s_waitcnt(0);  // no load still writing LDS, no read pending
      wg_barrier();                   // every wave is done with the pipeline stages
      char *cw = smem + wave * (T::WTM * T::CROW);
#pragma unroll
      for (int i0 = 0; i0 < FM; i0 += CB) {
        u32x2 cold[CB][FN];
#pragma unroll
        for (int i = 0; i < CB; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) cold[i][j] = u32x2{0u, 0u};
        if (GEN && beta != 0.0f) {
#pragma unroll
          for (int i = 0; i < CB; ++i) {
            const int m = wm0 + (i0 + i) * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int n = wn0 + j * 16 + 4 * (lane >> 4);
              if (m < M && n < N) cold[i][j] = *(const u32x2 *)(args.C + (size_t)m * ldc + n);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < CB; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            *(u32x2 *)(cw + ((i0 + i) * 16 + (lane & 15)) * T::CROW + (j * 16 + 4 * (lane >> 4)) * 2) =
                out2(GEN_, i0 + i, j, cold[i][j]);
        if constexpr (GEN) asm volatile("" ::: "memory");
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      // each row of the wave block is WTN*2 bytes = WTN/8 lanes of 16 bytes.
      // C is written once and not read again by this launch: nontemporal
      // stores stream it past the L2, where it would otherwise evict the A and
      // B panel lines that neighbouring tiles still read, and leave dirty
      // lines for the end of the launch to write back (measured: TN f16 8192^3
      // 740 -> 725 us, NN bf16 4096^3 98.4 -> 97.4, TN f16 2048^3 18.3 -> 18.0;
      // the same bits)
      // The LDS reads go out in batches of up to 8 before their stores, so
      // that their latencies overlap (one read, wait, store at a time took
      // 9k cycles a 256 x 256 tile), and the row pointer steps by RPI rows.
      // A wave block inside M x N stores without per-lane predicates.  A row
      // of WTN = 96 (12 chunks) takes 16 lanes, the last 4 idle.
      constexpr int CPR = T::WTN / 8;                // 16-byte chunks per row
      constexpr int LPR = CPR > 8 ? 16 : CPR;        // lanes per row (a power of two)
      constexpr bool FULL = LPR == CPR;              // every lane stores
      constexpr int RPI = 64 / LPR;
      constexpr int NROW = T::WTM / RPI, BATCH = NROW < 8 ? NROW : 8;
      static_assert((LPR & (LPR - 1)) == 0 && CPR <= LPR && 2 * CPR > LPR, "lanes per row");
      static_assert(NROW % BATCH == 0, "store batches");
      const bool lane_on = FULL || (lane % LPR) < CPR;
      const int row0 = lane / LPR, col = lane_on ? 8 * (lane % LPR) : 0;
      const char *src = cw + row0 * T::CROW + col * 2;
      uint16_t *dst = args.C + (size_t)(wm0 + row0) * ldc + (wn0 + col);
      const size_t step = (size_t)RPI * ldc;
      const bool inside = wm0 + T::WTM <= M && wn0 + T::WTN <= N;  // uniform
      const int rows_left = M - wm0 - row0;  // this lane's rows: r * RPI < rows_left
      const bool col_in = lane_on && wn0 + col < N;
#pragma unroll
      for (int r0 = 0; r0 < NROW; r0 += BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
          v[b] = *(const u32x4 *)(src + (r0 + b) * RPI * T::CROW);
        if (inside) {
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            if (lane_on) __builtin_nontemporal_store(v[b], (u32x4 *)dst);
            dst += step;
          }
        } else {
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            if (col_in && (r0 + b) * RPI < rows_left) __builtin_nontemporal_store(v[b], (u32x4 *)dst);
            dst += step;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = wm0 + i * 16 + (lane & 15);
        if (m < M) {
          uint16_t *crow = args.C + (size_t)m * ldc;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = wn0 + j * 16 + 4 * (lane >> 4);
            if (n < N) {
              u32x2 c = {0u, 0u};
              if (GEN && beta != 0.0f) c = *(const u32x2 *)(crow + n);
              *(u32x2 *)(crow + n) = out2(GEN_, i, j, c);
            }
          }
        }
        if constexpr (GEN) asm volatile("" ::: "memory");
      }
    }
  };
  if (alpha == 1.0f && beta == 0.0f)
    epilogue(std::false_type{});
  else
    epilogue(std::true_type{});
}

// One tile (position `tile` of the grouped tile order) by one workgroup.
// SPLIT: only K segment `seg` of sk_split, whose FP32 partial sums go to
// workspace slot `slot` (a separate instantiation, so that whole-K tiles
// carry none of the segment bookkeeping in registers).
// PH: a measurement copy that reads the shader clock (s_memtime) at three
// points of every K step, and at the tile's start and end, and writes each
// wave's per-phase cycle sums to ((uint32_t *)args.ws)[16 * (NW * blockIdx.x
// + wave) ..] (see the main loop and the kPhases launch mode).
template <class T, int LAYOUT, int DT, bool SPLIT, bool OPAQUE = false, bool PH = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs &args, char *smem, int tile, int seg,
                                          int slot) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  constexpr int FM = T::FM, FN = T::FN, NMF = T::NMF;
  constexpr int SEG_A = T::SEG_A, SEG_B = T::SEG_B;
  constexpr bool A_MN = a_mn_major(LAYOUT);  // A stored K x M: transposing reads
  constexpr bool B_MN = b_mn_major(LAYOUT);  // B stored K x N: transposing reads
  // an m/n-contiguous operand is loaded as k-rows of 2*BM or 2*BN bytes laid
  // end to end over the 1 KiB segments; the XOR layout covers rows of 128,
  // 256, 384 or 512 bytes
  static_assert(!A_MN || BM == 64 || BM == 128 || BM == 192 || BM == 256, "m-contiguous A width");
  static_assert(!B_MN || BN == 64 || BN == 128 || BN == 192 || BN == 256, "n-contiguous B width");
  constexpr int NRA = A_MN ? 2 * FM : FM;    // LDS reads for the A fragments of a slice
  constexpr int NRB = B_MN ? 2 * FN : FN;    // ... and for the B fragments
  constexpr int NR = NRA + NRB;              // LDS reads per slice
  // Read order within a slice: the transposing reads (inline assembly, not
  // tracked by the compiler's wait-count pass) go first, so that the wait the
  // compiler places for a later, tracked read of the same slice also covers
  // them (LDS reads complete in order).  With both operands transposed there
  // is no tracked read, and an explicit wait opens each slice instead.
  constexpr bool A_FIRST = A_MN && !B_MN;
  constexpr bool ALL_TR = A_MN && B_MN;

  // (PH) the tile's start, retired by the prologue's wait
  uint32_t ph_start = 0;
  if constexpr (PH) ph_start = (uint32_t)__builtin_amdgcn_s_memtime();
  const int M = args.M, N = args.N;
  const int lda = args.lda, ldb = args.ldb;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // K range of this workgroup: all of it, or steps [seg*KT/S, (seg+1)*KT/S)
  // of a split.  A segment is computed as a GEMM of its own: the operand
  // panels start at its first k and K is its length, so that the main loop
  // below is the same code either way.
  const int KT_all = (args.K + BK - 1) / BK;
  const int S = SPLIT ? args.sk_split : 1;
  const int k_begin = SPLIT ? __builtin_amdgcn_readfirstlane(seg * KT_all / S) * BK : 0;
  const int K = SPLIT ? __builtin_amdgcn_readfirstlane(
                            min(args.K, (seg + 1) * KT_all / S * BK) - k_begin)
                      : args.K;
  int tm, tn;
  tile_of(tile, tiles_m, tiles_n, args.group_m, tm, tn);
  // the tile order divides on the vector unit; the results are uniform and are
  // moved to scalar registers explicitly, so that the buffer descriptors built
  // from them stay scalar (a descriptor held in vector registers turns every
  // load into a per-lane loop)
  const int m0 = __builtin_amdgcn_readfirstlane(tm * BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);
  int tid = threadIdx.x;
  // called in a loop over tiles: hide the thread index, so that per-lane
  // offsets are recomputed per tile instead of being kept live across the
  // epilogue
  if constexpr (OPAQUE) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (unsigned)wave / T::WVN, wn = (unsigned)wave % T::WVN;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);

  // ---- direct-to-LDS loads ------------------------------------------------
  // k-contiguous operand (A[M][K], Bt[N][K]): segment s = 8 tile rows of 128
  // bytes; lane -> (row s*8 + lane/8, stored chunk lane%8), which holds logical
  // k-chunk (lane%8) ^ swizzle(row).
  // m/n-contiguous operand (At[K][M], B[K][N]): k-rows of 2*BX bytes end to
  // end; LDS byte b = s*1024 + 16*lane -> (k-row b / (2*BX), stored chunk
  // (b % (2*BX)) / 16) holding m/n-chunk stored-chunk ^ nn_chunk_xor(k);
  // chunks past the M/N edge (a multiple of 8) read out of range.
  // Wave w loads segments w*SEG .. w*SEG+SEG-1 of each operand.
  auto kmaj_off = [&](int part, int ld, int &chunk) {
    return kmajor_load_offset<T::LDS>(part, lane, ld, chunk);
  };
  auto mnmaj_off = [&](int part, int ld, int rowb, int x0, int xdim, int &chunk) {
    return mnmajor_load_offset<T::LDS>(part, lane, ld, rowb, x0, xdim, chunk);
  };
  uint32_t a_off[SEG_A];
  int a_chunk[SEG_A];
#pragma unroll
  for (int i = 0; i < SEG_A; ++i)
    a_off[i] = A_MN ? mnmaj_off(wave * SEG_A + i, lda, 2 * BM, m0, M, a_chunk[i])
                    : kmaj_off(wave * SEG_A + i, lda, a_chunk[i]);
  uint32_t b_off[SEG_B];
  int b_chunk[SEG_B];
#pragma unroll
  for (int i = 0; i < SEG_B; ++i)
    b_off[i] = B_MN ? mnmaj_off(wave * SEG_B + i, ldb, 2 * BN, n0, N, b_chunk[i])
                    : kmaj_off(wave * SEG_B + i, ldb, b_chunk[i]);
  // Loads 4j .. 4j+3 of an operand (four consecutive 1 KiB LDS segments)
  // share one LDS base address (M0): the immediate offset 1024*(i%4) moves
  // both the LDS destination and the global address, so each lane's offset
  // is lowered by it.  The descriptors' base is lowered by kShift
  // bytes and every offset raised by as much, so that no offset goes below
  // zero however small the leading dimension; out-of-range offsets stay out
  // of range.
  constexpr uint32_t kShift = 4096;
  auto imm_of = [](int i) { return 1024u * (uint32_t)(i & 3); };
#pragma unroll
  for (int i = 0; i < SEG_A; ++i) a_off[i] += kShift - imm_of(i);
#pragma unroll
  for (int i = 0; i < SEG_B; ++i) b_off[i] += kShift - imm_of(i);
  const uint16_t *a_panel =
      A_MN ? args.A + m0 + (size_t)k_begin * lda : args.A + (size_t)m0 * lda + k_begin;
  const uint16_t *b_panel =
      B_MN ? args.B + n0 + (size_t)k_begin * ldb : args.B + (size_t)n0 * ldb + k_begin;

  // A stage of step s at (s % NSA) * A_STAGE, B stage at B_BASE + (s % NSB) * B_STAGE
  constexpr int NSA = T::NSA, NSB = T::NSB;
  auto a_base = [&](int s) { return (uint32_t)((s % NSA) * T::A_STAGE); };
  auto b_base = [&](int s) { return (uint32_t)(T::B_BASE + (s % NSB) * T::B_STAGE); };
  // Loads still in flight at each step's barrier: those issued after the
  // loads of step kt+1 (A of NSB-1 later steps, B of NSB-2; spread: A and B
  // of NSB-2 later steps), which the wait there lets run on.
  constexpr bool SPREAD = T::SPREAD != 0;
  constexpr int AHEAD = SPREAD ? (NSB - 2) * (SEG_A + SEG_B) : (NSB - 1) * SEG_A + (NSB - 2) * SEG_B;
  static_assert(AHEAD < 64, "vmcnt range");

  // Buffer resource of one operand for the K step starting at k0: rows past
  // the tile edge (k-contiguous) or k-rows past this workgroup's K range
  // (m/n-contiguous) fall outside it and read as zero, and so does every step
  // past the range (no traffic for the loads the pipeline runs ahead).
  // (One descriptor built from selected base and size: descriptors merged from
  // branches lose their uniformity and end up in a per-lane loop.)
  auto rsrc_of = [&](bool mn, const uint16_t *panel, int ld, int rows, int k0) {
    const int krem = K - k0;
    const char *base = (const char *)(mn ? panel + (size_t)k0 * ld : panel + k0) - kShift;
    const uint32_t bytes = krem <= 0 ? 0u
                           : mn      ? (uint32_t)(min(krem, BK) * ld) * 2u + kShift
                                     : (uint32_t)((rows - 1) * ld + K - k0) * 2u + kShift;
    return make_rsrc(base, bytes);
  };
  __amdgpu_buffer_rsrc_t rs_a, rs_b;
  auto prep_a = [&](int step) { rs_a = rsrc_of(A_MN, a_panel, lda, rows_a, step * BK); };
  auto prep_b = [&](int step) { rs_b = rsrc_of(B_MN, b_panel, ldb, rows_b, step * BK); };
  auto load_seg = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, char *group_base, int i) {
    switch (i & 3) {
      case 0: load16_lds_imm<0>(r, voff, group_base); break;
      case 1: load16_lds_imm<1>(r, voff, group_base); break;
      case 2: load16_lds_imm<2>(r, voff, group_base); break;
      default: load16_lds_imm<3>(r, voff, group_base); break;
    }
  };
  auto load_a = [&](uint32_t stage, int i) {
    load_seg(rs_a, a_off[i], smem + stage + (wave * SEG_A + (i & ~3)) * 1024, i);
  };
  auto load_b = [&](uint32_t stage, int i) {
    load_seg(rs_b, b_off[i], smem + stage + (wave * SEG_B + (i & ~3)) * 1024, i);
  };
  // K tail: on the one partial step (K % 64 != 0) a k-chunk past K inside a
  // valid row of a k-contiguous operand would read past the row's end, so from
  // that step on those chunks point out of range (every later step is out of
  // range as a whole).  The offsets are masked once, not per load: a select
  // feeding each load would sit in the MFMA stream and stall it.
  const int tail = (K % BK) ? (K - 1) / BK : -1;
  auto mask_tail = [&]() {
    // (a side effect keeps this a branch: executed as selects on every step it
    // would sit in the MFMA stream and hold both offset sets in registers)
    asm volatile("" ::: "memory");
    const int kr = K - tail * BK;
    if constexpr (!A_MN) {
#pragma unroll
      for (int i = 0; i < SEG_A; ++i)
        a_off[i] = (a_chunk[i] * 8 < kr) ? a_off[i] : kOutOfRange + kShift - imm_of(i);
    }
    if constexpr (!B_MN) {
#pragma unroll
      for (int i = 0; i < SEG_B; ++i)
        b_off[i] = (b_chunk[i] * 8 < kr) ? b_off[i] : kOutOfRange + kShift - imm_of(i);
    }
  };

  // ---- fragment reads -------------------------------------------------------
  // k-contiguous: 16 rows x 32 k; lane reads row (lane & 15), logical k-chunk
  // 4*slice + lane/16 of that row.
  uint32_t rd_off[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) rd_off[sl] = kmajor_frag_offset<T::LDS>(lane, sl);
  const uint32_t rd_a = (wm * T::WTM) * 128;
  const uint32_t rd_b = (wn * T::WTN) * 128;
  // m/n-contiguous: two transposing reads per fragment (see mnmajor_frag_offset)
  auto tr_offsets = [&](uint32_t *off, int nfrag, int x_wave, int rowb) {
#pragma unroll
    for (int j = 0; j < nfrag; ++j) off[j] = mnmajor_frag_offset<T::LDS>(lane, x_wave + 16 * j, rowb);
  };
  uint32_t tra_off[A_MN ? FM : 1], trb_off[B_MN ? FN : 1];
  if constexpr (A_MN) tr_offsets(tra_off, FM, wm * T::WTM, 2 * BM);
  if constexpr (B_MN) tr_offsets(trb_off, FN, wn * T::WTN, 2 * BN);

  u32x4 f[2][FN + FM];  // [set][B fragments 0..FN-1, A fragments FN..FN+FM-1]
  auto read_a = [&](auto S_, uint32_t ab, int sl, int qa) {
    constexpr int S = decltype(S_)::value;
    if constexpr (A_MN) {
      const int i = qa >> 1, h = qa & 1;
      const u32x2 v = lds_read_tr16(lds_addr(smem + ab + tra_off[i]), (32 * sl + 4 * h) * 2 * BM);
      f[S][FN + i][2 * h] = v[0];
      f[S][FN + i][2 * h + 1] = v[1];
    } else {
      f[S][FN + qa] = *(const u32x4 *)(smem + ab + rd_a + qa * 16 * 128 + rd_off[sl]);
    }
  };
  auto read_b = [&](auto S_, uint32_t bb, int sl, int qb) {
    constexpr int S = decltype(S_)::value;
    if constexpr (B_MN) {
      const int j = qb >> 1, h = qb & 1;
      const u32x2 v = lds_read_tr16(lds_addr(smem + bb + trb_off[j]), (32 * sl + 4 * h) * 2 * BN);
      f[S][j][2 * h] = v[0];
      f[S][j][2 * h + 1] = v[1];
    } else {
      f[S][qb] = *(const u32x4 *)(smem + bb + rd_b + qb * 16 * 128 + rd_off[sl]);
    }
  };
  // read op q (0..NR-1) of slice sl into set S, in the order stated above
  auto read_op = [&](auto S_, uint32_t ab, uint32_t bb, int sl, int q) {
    if constexpr (A_FIRST) {
      if (q < NRA) read_a(S_, ab, sl, q);
      else read_b(S_, bb, sl, q - NRA);
    } else {
      if (q < NRB) read_b(S_, bb, sl, q);
      else read_a(S_, ab, sl, q - NRB);
    }
  };
  // With no tracked read in a slice: wait for all of its reads before its
  // first MFMA, the fragment registers tied to the wait so that neither an
  // MFMA nor another value can use them earlier.
  auto wait_set = [&](auto S_) {
    constexpr int S = decltype(S_)::value;
    if constexpr (ALL_TR) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[S][0]));
#pragma unroll
      for (int q = 1; q < FN + FM; ++q) asm volatile("" : "+v"(f[S][q]));
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};
  // MFMA t of a slice: A tile i = t / FN, B tile j = t % FN, j running backwards
  // on odd i, so that every MFMA shares an operand with the one before it (at a
  // change of i the B fragment, else the A fragment); operands swapped so each
  // lane ends with 4 consecutive columns of one row of C.  Each accumulator
  // still sums its slices in k order, so the results are the same bits; the
  // order runs 0.2-1.4 % faster than plain row order (interleaved timing,
  // 8192^3, NN 4096^3, 2048^3).  The persistent loop keeps the row order, with
  // which its registers fit without scratch.
  auto mfma = [&](auto S_, int t) {
    constexpr int S = decltype(S_)::value;
    const int i = t / FN, jj = t % FN, j = (!OPAQUE && (i & 1)) ? FN - 1 - jj : jj;
    acc[i][j] = mfma16x16x32<DT>(f[S][j], f[S][FN + i], acc[i][j]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  const int KT = (K + BK - 1) / BK;

  // ---- prologue: the loads the loop's earlier steps would have issued, in
  // the same order (A of step s, then B of step s, for s = 0 .. NSB-1), the
  // last B after the first barrier, where it overlaps the reads of slice 0
  // (spread: steps 0 .. NSB-2, all before the barrier) ----
  constexpr int LEAD = SPREAD ? NSB - 1 : NSB;  // steps loaded ahead of the loop
#pragma unroll
  for (int st = 0; st < LEAD; ++st) {
    if (tail == st) mask_tail();
    prep_a(st);
#pragma unroll
    for (int i = 0; i < SEG_A; ++i) load_a(a_base(st), i);
    if (SPREAD || st < NSB - 1) {
      prep_b(st);
#pragma unroll
      for (int i = 0; i < SEG_B; ++i) load_b(b_base(st), i);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(AHEAD, 0));  // step 0 in LDS
  wg_barrier();
  if constexpr (!SPREAD) prep_b(NSB - 1);
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    read_op(I0{}, a_base(0), b_base(0), 0, q);
    if constexpr (!SPREAD) {
      if (q * SEG_B / NR != (q + 1) * SEG_B / NR) load_b(b_base(NSB - 1), q * SEG_B / NR);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- phase clocks (PH only) ------------------------------------------------
  // Stamps per step: c before the wait that ends Y, d after it, e after the
  // barrier.  s_memtime counts on the LDS/scalar counter, and while one is
  // outstanding every wait the compiler places for an LDS read becomes a
  // wait for all of them; so c sits just before the loop's own lgkmcnt(0)
  // wait, and d and e are retired by one more lgkmcnt(0) after Z's first
  // MFMA, before Z's first LDS read (the only cost the stamps add: their
  // round trip, less one MFMA).  Phase sums over the steps:
  //   W = d - c: the wait for the next step's loads and the own reads,
  //   B = e - d: the barrier,
  //   R = next c - e: everything else, i.e. 128 MFMAs with the fragment
  //       reads, loads and address arithmetic among them (KT - 1 of these).
  uint32_t ph_w = 0, ph_b = 0, ph_r = 0;
  uint32_t pc = 0, pd = 0, pe = 0, ph_first = 0;
  uint32_t ph_out[9];
  auto stamp = [&]() { return (uint32_t)__builtin_amdgcn_s_memtime(); };

  // ---- main loop -------------------------------------------------------------
  // stage offsets of steps kt, kt+1, ..., rotated at the end of each step
  // (no division in the loop); ra[NSA-1] is also the stage of step kt-1
  uint32_t ra[NSA], rb[NSB];
#pragma unroll
  for (int i = 0; i < NSA; ++i) ra[i] = a_base(i);
#pragma unroll
  for (int i = 0; i < NSB; ++i) rb[i] = b_base(i);
  // Spread loads: the SEG_A + SEG_B loads of a step (A, then B) go after
  // MFMAs spread_pos(0), spread_pos(1), ... of the step's first NMF + NMF/2
  // (X and Y below), evenly spaced.
  constexpr int SP_MF = NMF + NMF / 2, SP_LD = SEG_A + SEG_B;
  auto spread_load = [&](int pos, uint32_t la, uint32_t lb) {
#pragma unroll
    for (int g = 0; g < SP_LD; ++g) {
      if (g * SP_MF / SP_LD + SP_MF / SP_LD / 2 == pos) {
        if (g < SEG_A) load_a(la, g);
        else load_b(lb, g - SEG_A);
      }
    }
  };
  for (int kt = 0; kt < KT; ++kt) {
    // loads of steps kt+LEAD on are issued below
    if (__builtin_expect(kt + LEAD == tail, 0)) mask_tail();
    const uint32_t ca = ra[0], cb = rb[0];
    const uint32_t na = ra[1], nb = rb[1];
    // X: slice 0; read slice 1; A of step kt+NSA-1 into the stage step kt-1
    // used (spread: A and B of step kt+NSB-1, in X and Y)
    prep_a(kt + NSA - 1);
    const uint32_t la = ra[NSA - 1];
    if constexpr (SPREAD) prep_b(kt + NSB - 1);
    const uint32_t lb_x = rb[NSB - 1];
    wait_set(I0{});
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      mfma(I0{}, t);
#pragma unroll
      for (int q = t * NR / NMF; q < (t + 1) * NR / NMF; ++q) read_op(I1{}, ca, cb, 1, q);
      if constexpr (SPREAD) {
        spread_load(t, la, lb_x);
      } else if constexpr (SEG_A > 0) {
        constexpr int SP = NMF / SEG_A;  // one A load every SP MFMAs, after MFMA 2 mod SP
        if (t % SP == (SP > 2 ? 2 : 0)) load_a(la, t / SP);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Y: first half of slice 1
    wait_set(I1{});
#pragma unroll
    for (int t = 0; t < NMF / 2; ++t) {
      mfma(I1{}, t);
      if constexpr (SPREAD) spread_load(NMF + t, la, lb_x);
      __builtin_amdgcn_sched_barrier(0);
    }
    // step kt+1 complete in LDS (later steps' loads may stay in flight), own
    // reads done
    if constexpr (PH) pc = stamp();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(AHEAD, 0));
    if constexpr (PH) {
      if (kt > 0) ph_r += pc - pe;  // e of the step before is in
      else ph_first = pc;
      pd = stamp();
      wg_barrier();
      pe = stamp();
    } else {
      wg_barrier();
    }
    // Z: second half of slice 1; read slice 0 of step kt+1; B of step kt+NSB
    // (spread: no loads)
    if constexpr (!SPREAD) prep_b(kt + NSB);
    const uint32_t lb = rb[0];  // step kt+NSB reuses the B stage of step kt
#pragma unroll
    for (int t = NMF / 2; t < NMF; ++t) {
      mfma(I1{}, t);
      if constexpr (PH) {
        if (t == NMF / 2) {  // d and e in, before the first read of Z
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
          ph_w += pd - pc;
          ph_b += pe - pd;
        }
      }
      constexpr int H = NMF / 2;
      const int u = t - H;
#pragma unroll
      for (int q = u * NR / H; q < (u + 1) * NR / H; ++q) read_op(I0{}, na, nb, 0, q);
      if constexpr (SEG_B > 0 && !SPREAD) {
        constexpr int SP = H / SEG_B > 0 ? H / SEG_B : 1;
        if (u % SP == (SP > 1 ? 1 : 0) && u / SP < SEG_B) load_b(lb, u / SP);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NSA - 1; ++i) ra[i] = ra[i + 1];
    ra[NSA - 1] = ca;
#pragma unroll
    for (int i = 0; i < NSB - 1; ++i) rb[i] = rb[i + 1];
    rb[NSB - 1] = cb;
  }

  if constexpr (PH) {
    // the last step's second half of slice 1, up to the end of the loop; then
    // one stamp's round trip (issue to result), which the wait after c and
    // the wait after e also contain
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    const uint32_t end = stamp();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    const uint32_t rt0 = stamp();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    const uint32_t rt1 = stamp();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    ph_out[0] = ph_w;
    ph_out[1] = ph_b;
    ph_out[2] = ph_r;
    ph_out[3] = (uint32_t)KT;
    ph_out[4] = KT > 0 ? end - ph_first : 0u;  // first step's c to the loop's end
    ph_out[5] = KT > 0 ? end - pe : 0u;        // the last step's Z
    ph_out[6] = rt1 - rt0;
    ph_out[7] = KT > 0 ? ph_first - ph_start : 0u;  // tile start to the first step's c
    ph_out[8] = rt1;  // where the epilogue starts
  }

  // The last step (or, for K = 0, the prologue) read fragments for a step that
  // does not exist; the compiler sees those values dead and may hand their
  // registers to the epilogue while the transposing reads, which it does not
  // track, still write them.  Wait for them here, and keep the fragment
  // registers alive up to the wait.
  if constexpr (A_MN || B_MN) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0][0]));
#pragma unroll
    for (int q = 1; q < FN + FM; ++q) asm volatile("" : "+v"(f[0][q]));
  }

  // ---- epilogue --------------------------------------------------------------
  if constexpr (SPLIT) {
    // a K segment: its FP32 sums go to workspace slot `slot`, each wave's block
    // in lane order (16-byte stores, 1 KiB per instruction); the fixup kernel
    // adds the segments of the tile in order and writes C
    // (stored straight from the accumulator registers: a plain store made the
    // compiler shuttle accumulators between register files inside the loop.
    // The compiler does not pad inline assembly for the matrix-core result
    // latency, so 24 wait states first: more than the 19 the slowest MFMA
    // needs before a memory instruction may read its result.)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float *dst = args.ws + ((size_t)slot * T::NW + wave) * (FM * FN * 256) + lane * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        asm volatile("global_store_dwordx4 %0, %1, off"
                     :
                     : "v"(dst + (i * FN + j) * 256), "a"(acc[i][j])
                     : "memory");
  } else {
    store_tile<T, DT>(args, acc, smem, m0, n0, wave, lane);
  }
  if constexpr (PH) {
    const uint32_t done = (uint32_t)__builtin_amdgcn_s_memtime();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    if (lane == 0) {
      uint32_t *o = reinterpret_cast<uint32_t *>(args.ws) + 16 * ((size_t)T::NW * blockIdx.x + wave);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = ph_out[i];
      o[8] = done - ph_out[8];  // the epilogue, up to its stores of C issued
#pragma unroll
      for (int i = 9; i < 16; ++i) o[i] = 0;
    }
  }
}

// Launch modes (the position of a workgroup is its index after the XCD remap
// of its part of the grid):
//   kWhole: `grid` whole-K tiles, positions tile_begin + p;
//   kSegments: sk_tiles * sk_split K segments, position p = segment
//     p / sk_tiles of tile tile_begin + p % sk_tiles, written to slot p;
//   kMixed: `grid` whole-K tiles 0 .. grid-1 (whole rounds: a multiple of
//     the 8 XCDs, so the segments after them keep the XCD placement the
//     remap assumes), then the segments of kSegments, in one launch: the
//     short segments fill the CUs as the last whole tiles finish, with no
//     launch boundary between them, and their partial sums are written last,
//     while the caches still hold them for the fixup.
//   kPersistent: whole-K tiles, gridDim.x workgroups (one per CU) each taking
//     positions b, b + gridDim.x, ... of `grid`: the same tile on the same XCD
//     in the same round as kWhole, but the next tile's loads start while the
//     last one's stores of C drain, and no workgroup is launched per tile.
//   kTimed: kWhole, and workgroup b writes four 64-bit counters to
//     ((uint64_t *)ws)[4b ..]: the shader clock (s_memtime) and the 100 MHz
//     real-time clock (s_memrealtime) before its tile and after its stores
//     of C are issued.  Their ratio is the engine clock the tiles ran at (a
//     measurement copy: the power limit of the part sets that clock).
//   kPhases: kWhole, and wave w of workgroup b writes sixteen 32-bit values
//     to ((uint32_t *)ws)[16 * (NW*b + w) ..]: the shader cycles it spent in
//     the main loop's wait for the next step's loads (W) and its barrier
//     (B), summed over its KT K steps, and between one step's barrier and
//     the next step's wait (R: a step's MFMAs with the fragment reads, loads
//     and address arithmetic among them), summed over KT - 1 steps; KT; the
//     cycles from the first step's wait to the loop's end; the last step's
//     cycles after its barrier; one clock read's round trip; the cycles from
//     the tile's start to the first step's wait (the prologue and the first
//     step's MFMAs before its wait); the epilogue's cycles up to its stores
//     of C issued; and seven 0s (a measurement copy: the clock reads and one
//     extra wait per step).
enum LaunchMode { kWhole = 0, kSegments = 1, kMixed = 2, kPersistent = 3, kTimed = 4,
                  kPhases = 5 };

template <class T, int LAYOUT, int DT, int MODE>
__global__ __launch_bounds__(T::NT) void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const int b = blockIdx.x;
  if constexpr (MODE == kWhole) {
    const int p = __builtin_amdgcn_readfirstlane(xcd_position(b, args.grid, args.xcd_remap));
    gemm_tile<T, LAYOUT, DT, false>(args, smem, args.tile_begin + p, 0, 0);
  } else if constexpr (MODE == kTimed) {
    const uint64_t c0 = clock64(), r0 = wall_clock64();
    const int p = __builtin_amdgcn_readfirstlane(xcd_position(b, args.grid, args.xcd_remap));
    gemm_tile<T, LAYOUT, DT, false>(args, smem, args.tile_begin + p, 0, 0);
    const uint64_t c1 = clock64(), r1 = wall_clock64();
    if (threadIdx.x == 0) {
      uint64_t *t = reinterpret_cast<uint64_t *>(args.ws) + 4 * (size_t)b;
      t[0] = c0;
      t[1] = r0;
      t[2] = c1;
      t[3] = r1;
    }
  } else if constexpr (MODE == kPhases) {
    const int p = __builtin_amdgcn_readfirstlane(xcd_position(b, args.grid, args.xcd_remap));
    gemm_tile<T, LAYOUT, DT, false, false, true>(args, smem, args.tile_begin + p, 0, 0);
  } else if constexpr (MODE == kPersistent) {
    for (int v = b; v < args.grid; v += gridDim.x) {
      const int p = __builtin_amdgcn_readfirstlane(xcd_position(v, args.grid, args.xcd_remap));
      gemm_tile<T, LAYOUT, DT, false, true>(args, smem, args.tile_begin + p, 0, 0);
      // every wave has read its epilogue rows back from LDS before the next
      // tile's loads overwrite them (the stores of C may still be in flight)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      wg_barrier();
    }
  } else {
    const int dp = MODE == kMixed ? args.grid : 0;  // whole tiles ahead of the segments
    if (MODE == kMixed && b < dp) {
      const int p = __builtin_amdgcn_readfirstlane(xcd_position(b, dp, args.xcd_remap));
      gemm_tile<T, LAYOUT, DT, false>(args, smem, p, 0, 0);
    } else {
      const int nseg = args.sk_tiles * args.sk_split;
      const int p = __builtin_amdgcn_readfirstlane(xcd_position(b - dp, nseg, args.xcd_remap));
      gemm_tile<T, LAYOUT, DT, true>(args, smem, args.tile_begin + p % args.sk_tiles,
                                     p / args.sk_tiles, p);
    }
  }
}

// Second half of a K-split launch: the S FP32 partial sums of each split tile
// are added in segment order (so the result does not depend on which segment
// finished first) and written to C with alpha and beta, rounded once.  A
// tile's partial sums are NW*FM*FN chunks of 1 KiB (wave block, then MFMA tile
// (i, j); one accumulator quad per lane); workgroup b handles the 16 chunks
// 16*(b % P) .. of split tile b / P, each thread 4 chunks of one lane, with the
// loads of four segments in flight before they are added (the sums are
// bandwidth work: few registers a lane, many loads outstanding).
template <class T, int DT>
__global__ __launch_bounds__(256) void gemm_sk_fixup(GemmArgs args) {
  constexpr int FM = T::FM, FN = T::FN;
  constexpr int CHUNKS = T::NW * FM * FN;
  constexpr int P = fixup_parts(T::BM, T::BN);
  static_assert(CHUNKS == 16 * P, "16 chunks a workgroup");
  constexpr int SLOT = CHUNKS * 256;  // floats of one segment's partial sums
  const int M = args.M, N = args.N, ldc = args.ldc;
  const int tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
  const int tile = blockIdx.x / P, part = blockIdx.x % P;
  int tm, tn;
  tile_of(args.tile_begin + tile, tiles_m, tiles_n, args.group_m, tm, tn);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = part * 16 + wave * 4;  // this thread's chunks c0 .. c0+3
  const float *src = args.ws + (size_t)tile * SLOT + (size_t)c0 * 256 + lane * 4;
  const size_t seg_stride = (size_t)args.sk_tiles * SLOT;
  const int S = args.sk_split;
  f32x4 acc[4] = {};
  int sg = 0;
  for (; sg + 4 <= S; sg += 4) {
    f32x4 p[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) p[b][c] = *(const f32x4 *)(src + (sg + b) * seg_stride + c * 256);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += p[b][c];
  }
  for (; sg < S; ++sg) {
    f32x4 p[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) p[c] = *(const f32x4 *)(src + sg * seg_stride + c * 256);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += p[c];
  }
  const float alpha = args.alpha, beta = args.beta;
  const bool plain = alpha == 1.0f && beta == 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = c0 + c, w = ch / (FM * FN), ij = ch % (FM * FN);
    const int m = tm * T::BM + ((unsigned)w / T::WVN) * T::WTM + (ij / FN) * 16 + (lane & 15);
    const int n = tn * T::BN + ((unsigned)w % T::WVN) * T::WTN + (ij % FN) * 16 + 4 * (lane >> 4);
    if (m >= M || n >= N) continue;  // N % 8 == 0: n < N covers n .. n+3
    uint16_t *cp = args.C + (size_t)m * ldc + n;
    float x[4] = {acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
    if (!plain) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= alpha;
      if (beta != 0.0f) {
        const u32x2 old = *(const u32x2 *)cp;
        float c0f, c1f, c2f, c3f;
        unpack2<DT>(old[0], c0f, c1f);
        unpack2<DT>(old[1], c2f, c3f);
        x[0] = __builtin_fmaf(beta, c0f, x[0]);
        x[1] = __builtin_fmaf(beta, c1f, x[1]);
        x[2] = __builtin_fmaf(beta, c2f, x[2]);
        x[3] = __builtin_fmaf(beta, c3f, x[3]);
      }
    }
    u32x2 v;
    v[0] = pack2<DT>(x[0], x[1]);
    v[1] = pack2<DT>(x[2], x[3]);
    __builtin_nontemporal_store(v, (u32x2 *)cp);  // written once, as in store_tile
  }
}

}  // namespace hgemm
