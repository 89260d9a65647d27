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
// gfx950 LDS serves a 16-byte-per-lane read in four passes of 16 lanes (256
// bytes over 64 banks of 4 bytes), measured with the LDS read probes: lanes
// {0-3, 12-15, 20-23, 24-27}, then {4-7, 8-11, 16-19, 28-31}, then the same
// plus 32.  The operand-fragment read puts lane l on row r0 + l%16, logical
// chunk c + l/16, so one pass reads rows r0 + {0-3, 12-15} at chunk c and rows
// r0 + {4-11} at chunk c+1.  Two consecutive 128-byte rows fill the 64 banks
// once, and c ^ ((r >> 1) & 7) gives the 16 lanes of a pass 16 distinct
// 16-byte bank groups; the plain layout leaves a four-way conflict.  (64-byte
// rows with c ^ ((r >> 2) & 3), conflict-free if lanes 0-15 formed a pass,
// conflict two-way.)  The writes (8 lanes per row, all 8 chunks) measure
// conflict-free under every layout.
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
  // The launch covers positions tile_begin .. of the grouped tile order with
  // `grid` workgroups.  sk_split == 0: one tile per workgroup, whole K.
  // sk_split = S >= 2: sk_tiles tiles, each split into S K-segments, one
  // workgroup per segment, whose FP32 partial sums go to `ws` (the fixup
  // kernel adds them up and writes C).
  int tile_begin, grid;
  int sk_split, sk_tiles;
  float *ws;
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
// on distinct bank pairs.  128- and 384-byte rows already alternate between
// the two bank halves and only need 2*((k >> 1) & 1) + 4*((k >> 3) & 1), a
// value below 8 that keeps the chunk inside its 128-byte group of the row.
template <int LDS>
__host__ __device__ __forceinline__ int nn_chunk_xor(int k, int row_bytes) {
  if constexpr (LDS == kLdsPlain) {
    return 0;
  } else {
    return row_bytes % 256 == 0 ? 2 * (k & 3) + 8 * ((k >> 3) & 1)
                            : 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1);
  }
}

// ---- operand tiles: direct-to-LDS placement and fragment reads ------------
// One K step of an operand tile in LDS, as the kernels load and read it.
//
// K-contiguous operand (A[M][K], Bt[N][K]): rows of 64 k = 128 bytes, chunk c
// of row r at chunk_pos(r, c).  Load segment `seg` (1 KiB, one wave
// instruction) covers rows 8*seg .. 8*seg+7; lane l writes LDS bytes
// seg*1024 + 16*l, i.e. row 8*seg + l/8, physical chunk l%8, and so loads the
// logical chunk (l%8) ^ chunk_pos(row, 0) (the XOR layouts are involutions).
// Returns the global byte offset of that chunk (row stride `ld` elements);
// the logical chunk goes to `chunk`.
template <int LDS>
__host__ __device__ __forceinline__ uint32_t kmajor_load_offset(int seg, int lane, int ld,
                                                                int &chunk) {
  const int row = seg * 8 + (lane >> 3);
  chunk = (lane & 7) ^ chunk_pos<LDS>(row, 0);
  return (uint32_t)(row * ld + chunk * 8) * 2u;
}

// M/N-contiguous operand (At[K][M], B[K][N]): k-rows of `rowb` (2 * tile
// width) bytes laid end to end; lane l of segment `seg` writes LDS byte
// b = seg*1024 + 16*l, i.e. k-row b / rowb, physical chunk (b % rowb) / 16,
// which holds logical chunk ((b % rowb) / 16) ^ nn_chunk_xor(k).  A 64-,
// 128- or 256-wide tile fits whole k-rows in a segment; a 384-byte k-row
// (192 wide) straddles segments, which changes nothing for a lane.  Chunks
// at or past `xdim` (the M or N edge, a multiple of 8) relative to the tile
// origin x0 get an out-of-range offset.
template <int LDS>
__host__ __device__ __forceinline__ uint32_t mnmajor_load_offset(int seg, int lane, int ld,
                                                                 int rowb, int x0, int xdim,
                                                                 int &chunk) {
  const unsigned b = (unsigned)(seg * 1024 + 16 * lane), rb = (unsigned)rowb;
  const int k = (int)(b / rb);
  const int c = (int)((b % rb) / 16u) ^ nn_chunk_xor<LDS>(k, rowb);
  chunk = c;
  return (x0 + c * 8 < xdim) ? (uint32_t)(k * ld + c * 8) * 2u : kOutOfRange;
}

// Matrix-core operand fragment: lane l holds 8 consecutive k (k = 32*sl +
// 8*(l/16) + e, e = 0..7) of row/column 16*f + l%16 of the tile.
// K-contiguous: one 16-byte read at f*16*128 + kmajor_frag_offset(l, sl).
template <int LDS>
__host__ __device__ __forceinline__ uint32_t kmajor_frag_offset(int lane, int sl) {
  return (lane & 15) * 128 + chunk_pos<LDS>(lane & 15, 4 * sl + (lane >> 4)) * 16;
}

// M/N-contiguous: two transposing reads (ds_read_b64_tr_b16) at
// mnmajor_frag_offset(l, x, rowb) + (32*sl + 4*h) * rowb, h = 0, 1, for the
// fragment at columns x .. x+15 (x a multiple of 16): within each 16-lane
// group, lane i points at k-row 8g + i/4 (+4h), columns x + 4*(i%4) .. +3.
template <int LDS>
__host__ __device__ __forceinline__ uint32_t mnmajor_frag_offset(int lane, int x, int rowb) {
  const int g = lane >> 4, i = lane & 15;
  const int k = 8 * g + (i >> 2);
  const int c = ((x / 8) ^ nn_chunk_xor<LDS>(k, rowb)) + ((i & 3) >> 1);
  return k * rowb + c * 16 + (i & 1) * 8;
}

// Position of workgroup `pid` in the tile sequence of a launch of `grid`
// workgroups.  Workgroup i runs on XCD i % 8; with the remap, XCD x receives
// the contiguous positions [x*per, (x+1)*per) (per = grid / 8), so that the
// tiles resident on one XCD are neighbours in the grouped order below and
// share A and B panels in its L2.  Positions past 8*per keep their index.
__host__ __device__ __forceinline__ int xcd_position(int pid, int grid, int xcd_remap) {
  if (xcd_remap) {
    const int per = grid >> 3;
    if (pid < (per << 3)) return (pid & 7) * per + (pid >> 3);
  }
  return pid;
}

// Tile at position v of the grouped order: groups of group_m tile rows, each
// walked column by column (down the group's rows first).
__host__ __device__ __forceinline__ void tile_of(int v, int tiles_m, int tiles_n, int group_m,
                                                 int &tm, int &tn) {
  const int width = group_m * tiles_n;
  const int g = v / width;
  const int first_m = g * group_m;
  const int gsz = (tiles_m - first_m < group_m) ? tiles_m - first_m : group_m;
  const int in = v - g * width;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Workgroups of the K-split fixup per tile: a BM x BN tile's FP32 partial
// sums are BM*BN/256 chunks of 1 KiB, 16 chunks a workgroup.
__host__ __device__ constexpr int fixup_parts(int bm, int bn) { return bm * bn / 4096; }

// Dispatch index -> (tile_m, tile_n) for a launch over the whole tile grid.
__host__ __device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n,
                                                     int group_m, int xcd_remap, int &tm,
                                                     int &tn) {
  tile_of(xcd_position(pid, tiles_m * tiles_n, xcd_remap), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace hgemm
