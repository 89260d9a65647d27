/*
 * hgemm.h -- C ABI of libhgemm.so: dense half-precision GEMM on AMD Instinct
 * MI355X (gfx950).
 *
 * Operation (the naive matmul of the "tcgen05 for dummies" translation,
 * "[译] tcgen05 入门：从零实现 B200 GEMM", section "Recap: how to write a
 * high-performance matmul kernel"; the TN/NN layouts of the kernel header in
 * "HGEMM: WMMA 与 MMA PTX 代码学习", full-listing section):
 *
 *     C[m][n] = round_to_dtype( sum_{k<K} A[m][k] * Bop[k][n] )
 *
 * with FP16 or BF16 inputs, products and sums carried in FP32 by the matrix
 * cores (the FP32-accumulate-then-convert outline of section 3 of
 * "MTT S4000 张量核心 GEMM 优化…"), and one round-to-nearest-even conversion
 * of each FP32 sum to the output type.  C is overwritten (never read): there
 * is no alpha/beta.
 *
 * Layouts (all dense, packed, row-major, element size 2 bytes):
 *   TN: A is M x K (lda = K); B is stored as Bt, N x K (ldb = K), so
 *       Bop[k][n] = Bt[n][k]; C is M x N (ldc = N).
 *   NN: A is M x K (lda = K); B is K x N (ldb = N); C is M x N (ldc = N).
 *
 * Accepted shapes: M, N, K >= 0; N % 8 == 0 and K % 8 == 0 so that every row
 * of every operand starts on a 16-byte boundary; M <= 2^30, N <= 2^23,
 * K <= 2^21, and the grid of output tiles below 2^31 workgroups (these keep
 * every per-tile byte offset in 32 bits).  M and N need not be multiples of any tile:
 * edge tiles are predicated.  M == 0 or N == 0 is a no-op; K == 0 writes
 * +0 to all of C (the empty sum).
 *
 * Pointers: A, B and C are device pointers on the current HIP device, each
 * 16-byte aligned, owned and allocated by the caller.  A and B are read-only
 * here; C must not overlap A or B.  The library allocates nothing and keeps
 * no pointer after a call returns.
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call
 * only enqueues work on that stream and returns without synchronising; the
 * caller orders and waits with events or stream syncs.  Calls are re-entrant
 * and thread-safe.
 *
 * Errors: every entry point returns an hgemm_status_t and never prints or
 * throws.  Arguments are validated before anything is launched, so a non-OK
 * status other than HGEMM_ERR_HIP means nothing was enqueued.  The torch
 * binding of "HGEMM: WMMA 与 MMA PTX 代码学习" (full-listing section) checks
 * the operands' dtype and shapes before launching and throws a C++ exception
 * on a mismatch; across a C ABI an exception cannot be caught, so the same
 * checks return these codes instead (HGEMM_ERR_INVALID_ARG for what that
 * binding rejects; HGEMM_ERR_UNSUPPORTED for what this library adds:
 * alignment, N % 8, K % 8 and the size limits).
 */
#ifndef HGEMM_H
#define HGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hgemm_dtype {
  HGEMM_F16 = 0,  /* IEEE binary16 inputs and output */
  HGEMM_BF16 = 1  /* bfloat16 inputs and output */
} hgemm_dtype_t;

typedef enum hgemm_status {
  HGEMM_OK = 0,
  HGEMM_ERR_INVALID_ARG = 1, /* negative dimension, unknown dtype, NULL
                                pointer while M*N > 0 (or M*N*K > 0 for
                                A and B), bad config */
  HGEMM_ERR_UNSUPPORTED = 2, /* N or K not a multiple of 8, a pointer not
                                16-byte aligned, a dimension over the limits
                                above, or a config that does not fit */
  HGEMM_ERR_HIP = 3,         /* the HIP runtime refused a launch; the
                                hipError_t is kept per thread, see
                                hgemm_last_hip_error() */
  HGEMM_ERR_SCRATCH = 4      /* hgemm_gemm_noalloc: the call needs more than
                                the library's static scratch */
} hgemm_status_t;

typedef enum hgemm_op {
  HGEMM_OP_N = 0, /* operand used as stored */
  HGEMM_OP_T = 1  /* operand stored transposed */
} hgemm_op_t;

/* C[M,N] = A[M,K] * Bt[N,K]^T.  A, Bt, C as described above.  (The pages'
 * "TN": the B operand is read as stored N x K, as the kernel of the HGEMM MMA
 * note, full-listing section, reads it.) */
hgemm_status_t hgemm_tn(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                        const void *A, const void *Bt, void *C, void *stream);

/* C[M,N] = A[M,K] * B[K,N].  A, B, C as described above.  (The pages' "NN":
 * A, B and C all row-major, the HGEMM MMA note's kernel header.) */
hgemm_status_t hgemm_nn(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                        const void *A, const void *B, void *C, void *stream);

/*
 * General form (the BLAS gemm update on row-major storage):
 *
 *     C[m][n] = round( alpha * sum_k opA(A)[m][k] * opB(B)[k][n] + beta * C[m][n] )
 *
 *   opA = HGEMM_OP_N: A is M x K, element (m, k) at A[m*lda + k], lda >= K;
 *   opA = HGEMM_OP_T: A is stored K x M, element (m, k) at A[k*lda + m], lda >= M;
 *   opB = HGEMM_OP_N: B is K x N, element (k, n) at B[k*ldb + n], ldb >= N;
 *   opB = HGEMM_OP_T: B is stored N x K, element (k, n) at B[n*ldb + k], ldb >= K;
 *   C is M x N, element (m, n) at C[m*ldc + n], ldc >= N.
 *
 * hgemm_tn is (OP_N, OP_T) and hgemm_nn is (OP_N, OP_N), with packed leading
 * dimensions, alpha = 1 and beta = 0.  The pages stop at C = A*B; alpha and
 * beta follow the usual BLAS gemm meaning: the FP32 sum is scaled by alpha,
 * beta times the old C (converted exactly to FP32) is added with one fused
 * multiply-add, and the result is rounded once to the output type.  With
 * beta == 0 the old C is not read (it may hold anything, NaN included); with
 * K == 0 the call computes beta * C.  Leading dimensions are in elements.
 *
 * Accepted arguments, beyond those of hgemm_tn: leading dimensions at least
 * the minimums above (else HGEMM_ERR_INVALID_ARG) and multiples of 8; M a
 * multiple of 8 when opA is HGEMM_OP_T; lda/ldb at most 2^22 for a K-contiguous
 * operand (OP_N A, OP_T B) and 2^23 for an M/N-contiguous one, ldc below 2^31
 * (else HGEMM_ERR_UNSUPPORTED).  With beta != 0, C must not overlap A or B.
 */
hgemm_status_t hgemm_gemm(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K,
                          hgemm_dtype_t dtype, float alpha, const void *A, int64_t lda,
                          const void *B, int64_t ldb, float beta, void *C, int64_t ldc,
                          void *stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *hgemm_status_string(hgemm_status_t status);

/* hipError_t of this thread's last HGEMM_ERR_HIP (0 if none yet). */
int hgemm_last_hip_error(void);

/* Library version string, e.g. "hgemm-gfx950 1.5". */
const char *hgemm_version(void);

/*
 * Explicit kernel selection, for tuning and for the ablations that back each
 * design choice with counters (tile shape, LDS layout, block-index swizzle).
 * The pages' launchers expose the same kind of knobs at run time (stages,
 * block swizzle on/off and its stride) in the torch bindings of the HGEMM
 * MMA note and the CuTe note.  Here the tile, the LDS stage ring and the LDS
 * layout (XOR swizzle, unswizzled, padded rows) are compile-time properties of
 * a kernel, so they are chosen together by a kernel-table index, whose name
 * (hgemm_kernel_info) states them; the block-index swizzle is chosen at run
 * time by group_m and xcd_remap.
 */
typedef struct hgemm_config {
  int32_t kernel;    /* index into the kernel table, or -1 for the automatic
                        choice; the entry's layout and dtype must match the
                        call */
  int32_t group_m;   /* tile rows per group of the grouped block order
                        (>= 1), or 0 for the kernel's default */
  int32_t xcd_remap; /* 1: give each XCD a contiguous range of tiles;
                        0: plain dispatch order; -1: default (on) */
  int32_t split;     /* K split of the tail (see hgemm_gemm_ws): 0 = automatic
                        (no split without a workspace), -1 = none, S >= 2 =
                        S segments per tail tile (needs a workspace and a
                        256 x 256 kernel) */
} hgemm_config_t;

/* As hgemm_tn / hgemm_nn, with an explicit configuration (NULL = automatic). */
hgemm_status_t hgemm_tn_ex(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                           const void *A, const void *Bt, void *C, void *stream,
                           const hgemm_config_t *cfg);
hgemm_status_t hgemm_nn_ex(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                           const void *A, const void *B, void *C, void *stream,
                           const hgemm_config_t *cfg);
/*
 * General form with a workspace, for shapes whose tiles leave the last round
 * of workgroups under-filled (the idle units of the MTT S4000 post, section
 * 3.9.2, and the persistent-kernel section of the tcgen05 translation; here a
 * K split rather than a persistent kernel): when the tiles of the 256 x 256
 * kernel do not fill whole rounds of the 256 CUs, the tiles of the last,
 * partial round (the tail) are each cut into S K segments that run side by
 * side; each segment writes its FP32 partial sums (256 KiB) to the
 * workspace, and a second kernel adds the S segments of a tile in segment
 * order and writes C with alpha, beta and one rounding.
 * The result is deterministic; it differs from the unsplit one only in the
 * FP32 summation order.  Up to three launches are enqueued on `stream` (the
 * whole rounds, the segments, the sums); the workspace must stay untouched
 * until they complete, and calls that overlap in time must not share one.
 * Status codes as for hgemm_gemm, plus HGEMM_ERR_UNSUPPORTED for a workspace
 * that is not 16-byte aligned.
 *
 * With cfg->split == 0 (automatic; hgemm_gemm_ws) the library splits only
 * when its cost estimate for the split is below 0.86 of the best unsplit
 * tile's, choosing S by the same estimate.
 * hgemm_gemm_ws_size returns the workspace bytes the automatic choice would
 * use for this call (0 when it would not split; 0 for an invalid operation
 * flag, dtype or dimension <= 0).  With a workspace smaller than that (or
 * NULL) the call runs unsplit.
 * workspace: device memory, 16-byte aligned, owned by the caller.
 */
size_t hgemm_gemm_ws_size(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K,
                          hgemm_dtype_t dtype);

hgemm_status_t hgemm_gemm_ws(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K,
                             hgemm_dtype_t dtype, float alpha, const void *A, int64_t lda, const void *B,
                             int64_t ldb, float beta, void *C, int64_t ldc, void *workspace,
                             size_t ws_bytes, void *stream);

/* As hgemm_gemm_ws, with an explicit configuration (NULL = automatic);
 * cfg->split > 0 forces that split (HGEMM_ERR_UNSUPPORTED when there is no
 * tail, S exceeds the K steps, or the workspace is too small).  A "_clk"
 * kernel (a measurement copy of a production kernel or of the two-group
 * "_pp" kernel) writes four uint64_t
 * per workgroup b to the workspace at index 4b: shader clock and 100 MHz
 * real-time clock before the tile, then both after its stores of C are
 * issued; it needs 32 bytes per workgroup (HGEMM_ERR_UNSUPPORTED otherwise).
 * A "_ph" kernel (a measurement copy of a production kernel whose main loop
 * reads the shader clock around each step's wait and barrier) writes sixteen
 * uint32_t per wave w of workgroup b at index 16*(4b + w): the cycles the
 * wave spent in the wait for the next step's loads and in the barrier, each
 * summed over the K steps, the cycles between a step's barrier and the next
 * step's wait summed over all but the last step, the number of K steps, the
 * cycles from the first step's wait to the loop's end, the last step's cycles
 * after its barrier, the round trip of one clock read, the cycles from the
 * tile's start to the first step's wait, the epilogue's cycles up to its
 * stores of C issued, and seven zeros; it needs 256 bytes per workgroup. */
hgemm_status_t hgemm_gemm_ws_ex(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N,
                                int64_t K, hgemm_dtype_t dtype, float alpha, const void *A, int64_t lda, const void *B,
                                int64_t ldb, float beta, void *C, int64_t ldc, void *workspace,
                                size_t ws_bytes, void *stream, const hgemm_config_t *cfg);

/*
 * No-allocation variant of hgemm_gemm_ws, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, result
 * and kernels as hgemm_gemm_ws with a large enough workspace (bit-identical
 * output), but the K split's partial sums go to a static device array of the
 * library, HGEMM_NOALLOC_SCRATCH_BYTES (64 MiB) on each device it runs on,
 * held from the library's first use there until the process ends.  The call
 * allocates nothing.
 *   - Calls whose automatic split needs more (hgemm_gemm_ws_size above the
 *     limit) return HGEMM_ERR_SCRATCH and enqueue nothing.
 *   - The array is shared by every call on a device and keeps the last
 *     call's contents: calls that overlap in time on one device (concurrent
 *     streams, threads) race and give wrong results; order them.
 *   - The first call on a device looks up the array's device address
 *     (HGEMM_ERR_HIP if the runtime refuses), with that device current: the
 *     stream must belong to the current device.
 */
#define HGEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hgemm_status_t hgemm_gemm_noalloc(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N,
                                  int64_t K, hgemm_dtype_t dtype, float alpha, const void *A,
                                  int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                                  int64_t ldc, void *stream);

/* As hgemm_gemm, with an explicit configuration (NULL = automatic). */
hgemm_status_t hgemm_gemm_ex(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K,
                             hgemm_dtype_t dtype, float alpha, const void *A, int64_t lda,
                             const void *B, int64_t ldb, float beta, void *C,
                             int64_t ldc, void *stream, const hgemm_config_t *cfg);

/* Number of entries in the kernel table. */
int hgemm_kernel_count(void);

/* Description of kernel table entry `index` (NULL if out of range):
 * "<layout>_<dtype>_<BM>x<BN>x<BK>" for the production kernels (the ones the
 * automatic choice uses: entries 0..11, 20..31, the deeper-ring "_r3"
 * entries 38..45, the 256 x 128 entries 65..72, the 192 x 256 entries
 * 73..76 (TN and NN), the deeper-ring 64 x 64 "_r4" entries 77..84, the
 * 256 x 192 and 192 x 192 entries 85..90 and the entries 91..104 that
 * complete the 192-wide tiles for the other layouts, see hgemm_auto_kernel;
 * "at_" layouts take A stored
 * transposed), with a suffix naming what an
 * ablation changes ("_plainlds": LDS without the XOR swizzle, "_directepi":
 * epilogue without LDS staging, "_pp": eight waves in two groups alternating
 * memory and MFMA phases), and an "rs_" prefix for the register-staged
 * 32x32x16 baseline design (suffix: its LDS layout), and "_clk" and "_ph"
 * suffixes for measurement copies that record per-workgroup clocks and
 * per-wave main-loop phase cycles (see hgemm_gemm_ws_ex).
 * The integers describing
 * it are written through the non-NULL pointers: layout 0 = TN (A[M][K],
 * Bt[N][K]), 1 = NN (A[M][K], B[K][N]), 2 = at_tn (At[K][M], Bt[N][K]), 3 =
 * at_nn (At[K][M], B[K][N]); dtype
 * as hgemm_dtype_t; the workgroup tile BM x BN x BK. */
const char *hgemm_kernel_info(int index, int *layout, int *dtype, int *bm,
                              int *bn, int *bk);

/* Kernel table index the automatic choice would use for this call (layout
 * as in hgemm_kernel_info), or -1 for invalid arguments.  The choice takes the
 * tile (256 x 256, 192 x 256, 256 x 192, 192 x 192, 256 x 128, 128 x 128 or
 * 64 x 64, among those the layout has) with the least estimated time: rounds
 * of workgroups over the 256 CUs, times the K steps of 64 plus 3 for a tile's
 * prologue and epilogue (fewer where 128 x 128 or 64 x 64 workgroups share a
 * CU and overlap theirs), times the tile's area over its measured relative
 * throughput; ties go to the earlier tile in that list.  A single round of
 * 128 x 128 tiles (at most 256) over 24 or more K steps takes that tile's
 * entry with one more LDS stage per operand (the "_r3" names), and a single
 * round of 64 x 64 tiles whose A and B pass 6 MiB the entry with two more
 * (the "_r4" names).  This is the choice of hgemm_tn, hgemm_nn and
 * hgemm_gemm; hgemm_gemm_ws may split K instead. */
int hgemm_auto_kernel(int layout, hgemm_dtype_t dtype, int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* HGEMM_H */
