// common.hpp -- pieces shared by the HGEMM kernels: arguments, LDS layouts,
// workgroup-to-tile order.
#pragma once

#include "device.hpp"

namespace hgemm {

// LDS image of a tile: rows of 64 16-bit values (128 bytes = 8 chunks of 16).
//   kLdsXor    chunk c of row r at chunk c ^ ((r >> 1) & 7)   (default)
//   kLdsPlain  chunk c at c (no swizzle)
//   kLdsPad    chunk c at c, rows padded to 144 bytes
//   kLdsXorRow chunk c at c ^ (r & 7)
// gfx950 LDS serves 16-byte lane reads 16 lanes (256 bytes, 64 banks) at a
// time.  The operand-fragment read has lanes 0..15 on rows r0..r0+15 of one
// logical chunk: two consecutive 128-byte rows fill the 64 banks once, so the
// 16 lanes are conflict-free exactly when (r & 1, position) is distinct, which
// c ^ ((r >> 1) & 7) guarantees; c ^ (r & 7) repeats every 8 rows (two-way
// conflict) and the plain layout puts all 16 lanes on one bank group
// (eight-way).  The writes (8 lanes per row, all 8 chunks) stay conflict-free
// under every layout.
enum LdsLayout { kLdsXor = 0, kLdsPlain = 1, kLdsPad = 2, kLdsXorRow = 3 };
// Operand orientations (row-major storage).  Bit 0: B is stored K x N (n
// contiguous) instead of N x K (k contiguous); bit 1: A is stored K x M (m
// contiguous) instead of M x K.  TN and NN are the pages' two layouts.
enum Layout {
  kTN = 0,    // A[M][K], B stored as Bt[N][K]
  kNN = 1,    // A[M][K], B[K][N]
  kAtTN = 2,  // A stored as At[K][M], Bt[N][K]
  kAtNN = 3,  // A stored as At[K][M], B[K][N]
};
constexpr bool a_mn_major(int layout) { return (layout & 2) != 0; }
constexpr bool b_mn_major(int layout) { return (layout & 1) != 0; }

struct GemmArgs {
  const uint16_t *A;
  const uint16_t *B;
  uint16_t *C;
  int M, N, K;
  int lda, ldb, ldc;  // row strides (elements) of the stored A, B, C
  float alpha, beta;  // C = alpha * A B + beta * C; beta == 0: C is not read
  int group_m;        // >= 1
  int xcd_remap;      // 0 or 1
};

// Scheduling hints for one phase: after each of the NMF matrix-core
// instructions place one LDS read (first NDSR), one LDS write (first NDSW) and
// one global load (first NVM); the rest are placed freely.
template <int NMF, int NDSR, int NDSW, int NVM>
__device__ __forceinline__ void sched_interleave() {
#pragma unroll
  for (int i = 0; i < NMF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (i < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if (i < NDSW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    if (i < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
  }
}

// Physical 16-byte chunk position of logical chunk c in tile row r.
template <int LDS>
__host__ __device__ __forceinline__ int chunk_pos(int r, int c) {
  if constexpr (LDS == kLdsXor) return c ^ ((r >> 1) & 7);
  else if constexpr (LDS == kLdsXorRow) return c ^ (r & 7);
  else return c;
}

// An m- or n-contiguous operand in LDS (NN's B, a stored-transposed A): k-rows
// of `row_bytes` (2*BN or 2*BM) bytes, 16-byte chunks.  The transposing fragment read (lds_read_tr16) has the 16
// lanes of a group on k-rows 8g + 0..3 (and 8g + 4..7 for the second read),
// four lanes per row on two adjacent chunks; with 256 bytes of banks a 512-
// or 256-byte row maps every row onto the same banks, so the chunk is XORed
// with 2*(k & 3) + 8*((k >> 3) & 1): the eight rows a 32-lane half reads land
// on distinct bank pairs.  128-byte rows already alternate between the two
// bank halves and only need 2*((k >> 1) & 1) + 4*((k >> 3) & 1).
template <int LDS>
__host__ __device__ __forceinline__ int nn_chunk_xor(int k, int row_bytes) {
  if constexpr (LDS == kLdsPlain) {
    return 0;
  } else {
    return row_bytes >= 256 ? 2 * (k & 3) + 8 * ((k >> 3) & 1)
                            : 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1);
  }
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

}  // namespace hgemm
