/*
 * hgemm_probe.h -- test-support entry points of libhgemm.so.  They run the
 * library's own device building blocks in isolation so that tests can check
 * the assumptions the GEMM kernels rest on.  Not needed to compute a GEMM.
 *
 * All pointers are device pointers on the current HIP device; calls enqueue
 * on `stream` (a hipStream_t, NULL = default) without synchronising and
 * return an hgemm_status_t (see hgemm.h).
 */
#ifndef HGEMM_PROBE_H
#define HGEMM_PROBE_H

#include <stdint.h>

#include "hgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One 32x32x16 matrix-core instruction on one wave (the instruction behind
 * the per-lane fragment maps that the HGEMM MMA note and the ablation draft
 * spell out for their MMA shapes, section 3.1 of the draft).
 * x, y: 64 lanes x 8 elements of `dtype` (lane-major, 1024 bytes each), the
 *       first and second operand as each lane holds it.
 * d:    64 lanes x 16 floats (lane-major, 4096 bytes): the accumulator
 *       registers after D = X * Y with a zero input accumulator.
 */
hgemm_status_t hgemm_probe_mfma(int dtype, const void *x, const void *y, float *d,
                                void *stream);

/*
 * One 16x16x32 matrix-core instruction on one wave (the shape of the
 * production kernels).
 * x, y: 64 lanes x 8 elements of `dtype` (lane-major, 1024 bytes each), the
 *       first and second operand as each lane holds it.
 * d:    64 lanes x 4 floats (lane-major, 1024 bytes): the accumulator
 *       registers after D = X * Y with a zero input accumulator.
 */
hgemm_status_t hgemm_probe_mfma16(int dtype, const void *x, const void *y, float *d,
                                  void *stream);

/*
 * One K step of an operand tile through the production kernels' path: one
 * wave loads it into LDS with their direct-to-LDS placement and XOR layout,
 * then reads every matrix-core operand fragment back with their fragment
 * reads (16-byte reads for a K-contiguous operand, transposing reads for an
 * M/N-contiguous one).
 *   mn_major 0: src holds a bx x 64 tile, element (row, k) at src[row*ld + k]
 *               (ld >= 64);
 *   mn_major 1: src holds the same tile stored 64 x bx, element (row, k) at
 *               src[k*ld + row] (ld >= bx);
 *   bx in {64, 128, 192, 256}; ld a multiple of 8, at most 2^20.
 * dst: (bx/16) x 2 x 64 entries of 16 bytes: entry [f][sl][lane] holds the 8
 *      values lane `lane` feeds the matrix core for fragment f and k-slice sl,
 *      which must be tile (16f + lane%16, 32sl + 8(lane/16) + e), e = 0..7.
 * The check of the fragment-to-operand map of the ablation draft's section
 * 3.1-3.2 for this hardware.
 */
hgemm_status_t hgemm_probe_fragments(int mn_major, int bx, const void *src, int64_t ld,
                                     void *dst, void *stream);

/*
 * Host-side: the production kernels' placement of one K step of an operand
 * tile (bx in {64, 128, 192, 256}; XOR layout), computed by the same functions
 * the kernels use.
 *   load_row[s*64 + l], load_chunk[s*64 + l] (bx/8 segments x 64 lanes): the
 *     tile row (mn_major 0) or k-row (mn_major 1) and the logical 16-byte
 *     chunk that lane l of direct-to-LDS segment s loads; it lands at LDS byte
 *     s*1024 + 16*l.
 *   read_off[((f*2 + sl)*R + r)*64 + l] ((bx/16) x 2 x R x 64; R = 1 for
 *     mn_major 0, 2 for mn_major 1): the LDS byte offset lane l reads with
 *     read r of fragment f, k-slice sl (16-byte reads, or 8-byte transposing
 *     reads).
 */
hgemm_status_t hgemm_probe_operand_offsets(int mn_major, int bx, int *load_row, int *load_chunk,
                                           int *read_off);

/*
 * LDS layout round trip for a 256-row x 64-column tile of 16-bit values:
 * the tile is written to LDS with the register-staged baseline's store pattern and LDS layout
 * `lds_layout` (0 = XOR swizzle on row/2, 1 = plain rows, 2 = padded rows,
 * 3 = XOR swizzle on the row), read back
 * with the kernels' operand-fragment pattern, and each fragment is stored
 * to `dst` at the logical position it is meant to hold.  dst must equal src
 * (the round-trip check of the tcgen05 translation's swizzle section).
 * src, dst: 256 x 64 16-bit values, row-major (32 KiB each).
 */
hgemm_status_t hgemm_probe_lds_roundtrip(int lds_layout, const void *src, void *dst,
                                         void *stream);

/*
 * Matrix-core throughput ceiling: `waves` 64-lane waves (in workgroups of 4)
 * each issue `iters` x 16 independent 32x32x16 FP16 MFMAs with no memory
 * traffic in the loop.  FLOPs = waves * iters * 16 * 32768.  out receives
 * one float per lane (a sum that keeps the work alive), waves*64 floats.
 * clocks (may be NULL): per wave, the shader-clock cycles and the ticks of
 * the constant-rate real-time counter its loop took (2*waves uint64), from
 * which the sustained engine clock follows.
 */
hgemm_status_t hgemm_probe_mfma_peak(int waves, int iters, float *out, uint64_t *clocks,
                                     void *stream);

/*
 * Matrix-core issue rate per shape and operand data: `waves` waves (in
 * workgroups of 4) each issue `iters` x 16 (iters a multiple of 8) FP16
 * MFMAs on 16 independent
 * accumulators, shape 0 = 32x32x16 (32768 FLOP each), 1 = 16x16x32 (16384
 * FLOP each); random 1: operands rotate over 8 + 8 registers of
 * pseudo-random values in (-1, 1), as a GEMM's do, 0: one constant pair.
 * The sustained clock under the board's power limit depends on both.
 * out: waves*64 floats; clocks (may be NULL): per wave, shader-clock cycles
 * and constant-rate real-time ticks (2*waves uint64).
 */
hgemm_status_t hgemm_probe_mfma_rate(int shape, int random, int waves, int iters, float *out,
                                     uint64_t *clocks, void *stream);

/*
 * LDS read throughput of one 16-byte-per-lane access pattern, over a
 * 64 KiB buffer per workgroup of 256 threads, `iters` x 16 reads per lane:
 *   pattern 0: lane-contiguous (lane l reads bytes 16*l .. of a 1 KiB row),
 *   pattern 1: the GEMM operand-fragment read with the XOR swizzle,
 *   pattern 2: the same read on plain (unswizzled) 128-byte rows,
 *   pattern 3: the same read with the chunk ^ (row & 7) swizzle
 *   (patterns 1-3: the 32-row fragments of the register-staged baseline);
 *   pattern 4: the production 16-row fragment read (k-contiguous operand)
 *              with the XOR layout,  pattern 5: the same on plain rows,
 *   pattern 6: the production transposing fragment read (two 8-byte
 *              ds_read_b64_tr_b16 per 16 bytes) on 256-byte k-rows with the
 *              XOR layout,  pattern 7: the same without it;
 *   pattern 8: the 16-row fragment read on 64-byte rows (32 k per row, chunk
 *              c of row r at c ^ ((r >> 2) & 3)).
 * Bytes read = workgroups * 256 * iters * 16 * 16 for every pattern.
 * out: workgroups*256 floats.
 */
hgemm_status_t hgemm_probe_lds_read(int workgroups, int iters, int pattern, float *out,
                                    void *stream);

/*
 * LDS read throughput of an arbitrary lane-to-address map: 256 threads per
 * workgroup, each wave in its own 16 KiB quarter of a 64 KiB buffer; lane l
 * reads 16 bytes at (lane_offsets[l] & 1008) + 1024 * j, j = 0..15, `iters`
 * times.  lane_offsets: 64 uint32_t in device memory (offsets into the first
 * KiB; the mask keeps every read inside the quarter).  Bytes read = workgroups * 256 * iters *
 * 16 * 16.  out: workgroups*256 floats.
 */
hgemm_status_t hgemm_probe_lds_lanes(int workgroups, int iters, const uint32_t *lane_offsets,
                                     float *out, void *stream);

/*
 * Global-to-CU streaming throughput: every workgroup of 256 threads moves
 * 64 KiB per iteration (16 x 16 bytes per lane) out of the window
 * [buf, buf + window_bytes) (a power of two between 64 KiB and 1 GiB; small
 * windows stay resident in L2), for `iters` iterations.  Each wave-wide load
 * reads 8 rows of 128 bytes whose starts are row_stride bytes apart (a
 * multiple of 16, >= 128; 128 = contiguous, 2*K = one K-step of a GEMM
 * operand); successive iterations move to the next 128-byte column.
 *   mode 0: into registers, 16 loads per lane in flight,
 *   mode 1: straight into LDS (direct-to-LDS loads), 16 in flight,
 *   mode 2: into registers, 8 in flight,  mode 3: into LDS, 8 in flight;
 *   mode 4 / 5: as mode 0 / 1, but each load reads 16 half rows of 64 bytes
 *   and two consecutive iterations read the two halves of the same rows, so
 *   that every 128-byte line is requested twice.
 * Bytes moved = workgroups * iters * 65536.  out: workgroups*256 floats.
 */
hgemm_status_t hgemm_probe_l2_read(int workgroups, int iters, int mode, const void *buf,
                                   uint32_t window_bytes, uint32_t row_stride, float *out,
                                   void *stream);

/*
 * Matrix-core issue rate with memory instructions mixed in (one wave per
 * SIMD, four waves per workgroup): every iteration issues 64 16x16x32 FP16
 * MFMAs with random operands and, spread evenly among them, `nload` loads
 * (0, 2, 4, 8 or 16) out of the L2-resident window [buf, buf + window_bytes)
 * (a power of two, 64 KiB .. 1 GiB) and `nread` (0 or 16) 16-byte LDS reads:
 *   kind 0: 16-byte-per-lane loads straight into LDS (1 KiB each),
 *   kind 1: 16-byte-per-lane loads into registers, then written to LDS,
 *   kind 2: 4-byte-per-lane loads straight into LDS (256 bytes each).
 * nread + 256 (kind 0 only) adds a workgroup barrier every 128 MFMAs, in the
 * middle of every other iteration, after waiting for the previous iteration's
 * loads and this wave's LDS reads (the waits of a pipelined GEMM step).
 * clocks[2w], clocks[2w+1] (device, 2 * 4 * workgroups uint64_t): shader clock
 * cycles and 100 MHz real-time ticks of wave w over its loop; cycles divided
 * by 64 * iters is the time per MFMA, 16 at full rate.  out: workgroups*256
 * floats (results kept live).
 */
hgemm_status_t hgemm_probe_mix(int kind, int nload, int nread, int workgroups, int iters,
                               const void *buf, uint32_t window_bytes, float *out,
                               uint64_t *clocks, void *stream);

/*
 * Host-only: byte offset, inside one LDS stage, of 16-byte chunk c of tile
 * row r under LDS layout `lds_layout` (as in hgemm_probe_lds_roundtrip), for
 * r < rows and c < 8: offsets[r * 8 + c].  No GPU work.
 */
hgemm_status_t hgemm_probe_lds_offsets(int lds_layout, int rows, int *offsets);

/*
 * Host-only: the workgroup -> output-tile order the GEMM kernels use for a
 * grid of tiles_m x tiles_n tiles (XCD remap on/off, grouped by group_m tile
 * rows).  Writes, for every workgroup id i < tiles_m * tiles_n, its tile row
 * tm[i] and tile column tn[i] (host arrays).  No GPU work.
 */
hgemm_status_t hgemm_probe_tile_order(int tiles_m, int tiles_n, int group_m, int xcd_remap,
                                      int *tm, int *tn);

#ifdef __cplusplus
}
#endif

#endif /* HGEMM_PROBE_H */
