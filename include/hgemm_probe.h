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
 * LDS layout round trip for a 256-row x 64-column tile of 16-bit values:
 * the tile is written to LDS with the kernels' store pattern and LDS layout
 * `lds_layout` (0 = XOR swizzle, 1 = plain rows, 2 = padded rows), read back
 * with the kernels' operand-fragment pattern, and each fragment is stored
 * to `dst` at the logical position it is meant to hold.  dst must equal src
 * (the round-trip check of the tcgen05 translation's swizzle section).
 * src, dst: 256 x 64 16-bit values, row-major (32 KiB each).
 */
hgemm_status_t hgemm_probe_lds_roundtrip(int lds_layout, const void *src, void *dst,
                                         void *stream);

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
