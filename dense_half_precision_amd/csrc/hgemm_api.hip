// hgemm_api.hip -- C ABI of libhgemm.so (declared in include/hgemm.h):
// argument validation, the kernel table, the per-shape choice and the launch
// on the caller's stream.  Nothing here allocates device memory or
// synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "hgemm.h"
#include "gemm_kernel.hpp"
#include "gemm_regstage.hpp"

namespace {

using namespace hgemm;

thread_local int g_last_hip_error = 0;

typedef void (*kernel_fn)(GemmArgs);

struct KernelEntry {
  const char *name;
  int layout, dtype, bm, bn, bk, lds, default_group_m;
  bool production;  // candidate of the automatic choice
  bool general;     // honours leading dimensions, alpha and beta
  kernel_fn fn;
};

template <class T, int LAYOUT, int DT>
constexpr KernelEntry entry(const char *name, int group_m, bool production) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, production, true,
                     &gemm_kernel<T, LAYOUT, DT>};
}
// the register-staged baseline assumes packed TN/NN operands, alpha 1, beta 0
template <class T, int LAYOUT, int DT>
constexpr KernelEntry rs_entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, false, false,
                     &regstage_kernel<T, LAYOUT, DT>};
}

using T256 = TileCfg<256, 256>;
using T128 = TileCfg<128, 128>;
using T64 = TileCfg<64, 64>;
using T256Plain = TileCfg<256, 256, kLdsPlain>;
using T256Direct = TileCfg<256, 256, kLdsXor, 0>;
using R256 = RsCfg<256, 256, 2, 2, kLdsXor>;
using R256Plain = RsCfg<256, 256, 2, 2, kLdsPlain>;
using R256Pad = RsCfg<256, 256, 2, 2, kLdsPad>;
using R256XorRow = RsCfg<256, 256, 2, 2, kLdsXorRow>;

// Index order is part of the ablation interface (hgemm_kernel_info lists it);
// new entries are appended.
const KernelEntry kTable[] = {
    entry<T256, kTN, kF16>("tn_f16_256x256x64", 4, true),
    entry<T256, kTN, kBF16>("tn_bf16_256x256x64", 4, true),
    entry<T256, kNN, kF16>("nn_f16_256x256x64", 4, true),
    entry<T256, kNN, kBF16>("nn_bf16_256x256x64", 4, true),
    entry<T128, kTN, kF16>("tn_f16_128x128x64", 4, true),
    entry<T128, kTN, kBF16>("tn_bf16_128x128x64", 4, true),
    entry<T128, kNN, kF16>("nn_f16_128x128x64", 4, true),
    entry<T128, kNN, kBF16>("nn_bf16_128x128x64", 4, true),
    entry<T64, kTN, kF16>("tn_f16_64x64x64", 4, true),
    entry<T64, kTN, kBF16>("tn_bf16_64x64x64", 4, true),
    entry<T64, kNN, kF16>("nn_f16_64x64x64", 4, true),
    entry<T64, kNN, kBF16>("nn_bf16_64x64x64", 4, true),
    // ablations of the production kernel: unswizzled LDS, direct epilogue stores
    entry<T256Plain, kTN, kF16>("tn_f16_256x256x64_plainlds", 4, false),
    entry<T256Plain, kNN, kBF16>("nn_bf16_256x256x64_plainlds", 4, false),
    entry<T256Direct, kTN, kF16>("tn_f16_256x256x64_directepi", 4, false),
    // baseline design: register-staged loads, 32x32x16 MFMA, LDS layout variants
    rs_entry<R256, kTN, kF16>("rs_tn_f16_256x256x64_xor", 8),
    rs_entry<R256Plain, kTN, kF16>("rs_tn_f16_256x256x64_plain", 8),
    rs_entry<R256Pad, kTN, kF16>("rs_tn_f16_256x256x64_pad", 8),
    rs_entry<R256XorRow, kTN, kF16>("rs_tn_f16_256x256x64_xorrow", 8),
    rs_entry<R256, kNN, kBF16>("rs_nn_bf16_256x256x64_xor", 8),
    // A stored transposed (At[K][M]) with Bt[N][K] or B[K][N]
    entry<T256, kAtTN, kF16>("at_tn_f16_256x256x64", 4, true),
    entry<T256, kAtTN, kBF16>("at_tn_bf16_256x256x64", 4, true),
    entry<T256, kAtNN, kF16>("at_nn_f16_256x256x64", 4, true),
    entry<T256, kAtNN, kBF16>("at_nn_bf16_256x256x64", 4, true),
    entry<T128, kAtTN, kF16>("at_tn_f16_128x128x64", 4, true),
    entry<T128, kAtTN, kBF16>("at_tn_bf16_128x128x64", 4, true),
    entry<T128, kAtNN, kF16>("at_nn_f16_128x128x64", 4, true),
    entry<T128, kAtNN, kBF16>("at_nn_bf16_128x128x64", 4, true),
    entry<T64, kAtTN, kF16>("at_tn_f16_64x64x64", 4, true),
    entry<T64, kAtTN, kBF16>("at_tn_bf16_64x64x64", 4, true),
    entry<T64, kAtNN, kF16>("at_nn_f16_64x64x64", 4, true),
    entry<T64, kAtNN, kBF16>("at_nn_bf16_64x64x64", 4, true),
};
constexpr int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

constexpr int64_t kMaxM = int64_t(1) << 30;
constexpr int64_t kMaxN = int64_t(1) << 23;
constexpr int64_t kMaxK = int64_t(1) << 21;
// leading dimensions: a k-contiguous operand (A[M][K], Bt[N][K]) is addressed
// 256 rows at a time with 32-bit byte offsets; an m/n-contiguous one (At[K][M],
// B[K][N]) 64 k-rows at a time; C with 64-bit offsets
constexpr int64_t kMaxLdK = int64_t(1) << 22;
constexpr int64_t kMaxLdMN = int64_t(1) << 23;
constexpr int64_t kMaxLdC = (int64_t(1) << 31) - 8;

int find_kernel(int layout, int dtype, int bm) {
  for (int i = 0; i < kTableSize; ++i)
    if (kTable[i].production && kTable[i].layout == layout && kTable[i].dtype == dtype &&
        kTable[i].bm == bm)
      return i;
  return -1;
}

// Automatic choice: the tile size with the least estimated time, taken as
// (waves of workgroups over the 256 CUs, one workgroup per CU) x (time of
// one tile), a tile's time being its area over the per-CU throughput of that
// tile size at full occupancy, measured relative to the 256 x 256 kernel
// (128: 0.8, 64: 0.5).  Ties go to the larger tile.
int auto_kernel(int layout, int dtype, int64_t M, int64_t N) {
  constexpr int64_t kCUs = 256;
  const int sizes[3] = {256, 128, 64};
  const int64_t rate10[3] = {10, 8, 5};  // relative throughput x 10
  int best = 256;
  int64_t best_cost = -1;
  for (int i = 0; i < 3; ++i) {
    const int64_t t = sizes[i];
    const int64_t tiles = ((M + t - 1) / t) * ((N + t - 1) / t);
    const int64_t cost = ((tiles + kCUs - 1) / kCUs) * t * t * 40 / rate10[i];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = sizes[i];
    }
  }
  return find_kernel(layout, dtype, best);
}

struct Call {
  int layout;  // kTN, kNN, kAtTN, kAtNN
  int64_t M, N, K;
  int dtype;
  float alpha, beta;
  const void *A, *B;
  void *C;
  int64_t lda, ldb, ldc;
};

hgemm_status_t validate(const Call &c) {
  if (c.M < 0 || c.N < 0 || c.K < 0) return HGEMM_ERR_INVALID_ARG;
  if (c.dtype != HGEMM_F16 && c.dtype != HGEMM_BF16) return HGEMM_ERR_INVALID_ARG;
  const bool a_mn = a_mn_major(c.layout), b_mn = b_mn_major(c.layout);
  if (c.lda < (a_mn ? c.M : c.K) || c.ldb < (b_mn ? c.N : c.K) || c.ldc < c.N)
    return HGEMM_ERR_INVALID_ARG;
  if (c.M == 0 || c.N == 0) return HGEMM_OK;
  if (c.C == nullptr) return HGEMM_ERR_INVALID_ARG;
  if (c.K > 0 && (c.A == nullptr || c.B == nullptr)) return HGEMM_ERR_INVALID_ARG;
  if (c.N % 8 != 0 || c.K % 8 != 0 || (a_mn && c.M % 8 != 0)) return HGEMM_ERR_UNSUPPORTED;
  if (c.lda % 8 != 0 || c.ldb % 8 != 0 || c.ldc % 8 != 0) return HGEMM_ERR_UNSUPPORTED;
  if (c.M > kMaxM || c.N > kMaxN || c.K > kMaxK) return HGEMM_ERR_UNSUPPORTED;
  if (c.lda > (a_mn ? kMaxLdMN : kMaxLdK) || c.ldb > (b_mn ? kMaxLdMN : kMaxLdK) ||
      c.ldc > kMaxLdC)
    return HGEMM_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(c.C) & 15) != 0) return HGEMM_ERR_UNSUPPORTED;
  if (c.K > 0 &&
      (((reinterpret_cast<uintptr_t>(c.A) | reinterpret_cast<uintptr_t>(c.B)) & 15) != 0))
    return HGEMM_ERR_UNSUPPORTED;
  return HGEMM_OK;
}

hgemm_status_t run(const Call &c, void *stream, const hgemm_config_t *cfg) {
  hgemm_status_t st = validate(c);
  if (st != HGEMM_OK) return st;
  int kidx = -1, group_m = 0, xcd = 1;
  if (cfg != nullptr) {
    if (cfg->reserved != 0 || cfg->group_m < 0 || cfg->xcd_remap < -1 || cfg->xcd_remap > 1 ||
        cfg->kernel < -1 || cfg->kernel >= kTableSize)
      return HGEMM_ERR_INVALID_ARG;
    kidx = cfg->kernel;
    group_m = cfg->group_m;
    if (cfg->xcd_remap >= 0) xcd = cfg->xcd_remap;
  }
  if (kidx >= 0 && (kTable[kidx].layout != c.layout || kTable[kidx].dtype != c.dtype))
    return HGEMM_ERR_INVALID_ARG;
  if (c.M == 0 || c.N == 0) return HGEMM_OK;
  if (kidx < 0) kidx = auto_kernel(c.layout, c.dtype, c.M, c.N);
  if (kidx < 0) return HGEMM_ERR_UNSUPPORTED;
  const KernelEntry &e = kTable[kidx];
  if (!e.general) {
    const bool packed = c.lda == c.K && c.ldb == (b_mn_major(c.layout) ? c.N : c.K) &&
                        c.ldc == c.N;
    if (!packed || c.alpha != 1.0f || c.beta != 0.0f) return HGEMM_ERR_UNSUPPORTED;
  }
  if (group_m == 0) group_m = e.default_group_m;

  const int64_t tiles = ((c.M + e.bm - 1) / e.bm) * ((c.N + e.bn - 1) / e.bn);
  if (tiles > INT32_MAX) return HGEMM_ERR_UNSUPPORTED;
  GemmArgs a;
  a.A = static_cast<const uint16_t *>(c.A);
  a.B = static_cast<const uint16_t *>(c.B);
  a.C = static_cast<uint16_t *>(c.C);
  a.M = (int)c.M;
  a.N = (int)c.N;
  a.K = (int)c.K;
  a.lda = (int)c.lda;
  a.ldb = (int)c.ldb;
  a.ldc = (int)c.ldc;
  a.alpha = c.alpha;
  a.beta = c.beta;
  a.group_m = group_m;
  a.xcd_remap = xcd;
  // hipGetLastError() reports the last error of any earlier runtime call on
  // this thread too: clear it so that only the launch's own result is seen
  (void)hipGetLastError();
  hipLaunchKernelGGL(e.fn, dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return HGEMM_ERR_HIP;
  }
  return HGEMM_OK;
}

// The pages' two layouts: packed storage, alpha 1, beta 0.
Call packed(int layout, int64_t M, int64_t N, int64_t K, int dtype, const void *A, const void *B,
            void *C) {
  return Call{layout, M, N, K, dtype, 1.0f, 0.0f, A, B, C,
              K, layout == kNN ? N : K, N};
}

// op flags -> layout; -1 if invalid
int layout_of(int opA, int opB) {
  if ((opA != HGEMM_OP_N && opA != HGEMM_OP_T) || (opB != HGEMM_OP_N && opB != HGEMM_OP_T))
    return -1;
  return (opA == HGEMM_OP_T ? 2 : 0) | (opB == HGEMM_OP_N ? 1 : 0);
}

}  // namespace

extern "C" {

hgemm_status_t hgemm_tn(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                        const void *Bt, void *C, void *stream) {
  return run(packed(kTN, M, N, K, dtype, A, Bt, C), stream, nullptr);
}

hgemm_status_t hgemm_nn(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                        const void *B, void *C, void *stream) {
  return run(packed(kNN, M, N, K, dtype, A, B, C), stream, nullptr);
}

hgemm_status_t hgemm_tn_ex(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                           const void *Bt, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(packed(kTN, M, N, K, dtype, A, Bt, C), stream, cfg);
}

hgemm_status_t hgemm_nn_ex(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                           const void *B, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(packed(kNN, M, N, K, dtype, A, B, C), stream, cfg);
}

hgemm_status_t hgemm_gemm_ex(int opA, int opB, int64_t M, int64_t N, int64_t K, int dtype,
                             float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                             float beta, void *C, int64_t ldc, void *stream,
                             const hgemm_config_t *cfg) {
  const int layout = layout_of(opA, opB);
  if (layout < 0) return HGEMM_ERR_INVALID_ARG;
  return run(Call{layout, M, N, K, dtype, alpha, beta, A, B, C, lda, ldb, ldc}, stream, cfg);
}

hgemm_status_t hgemm_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K, int dtype,
                          float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                          float beta, void *C, int64_t ldc, void *stream) {
  return hgemm_gemm_ex(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                       nullptr);
}

const char *hgemm_status_string(int status) {
  switch (status) {
    case HGEMM_OK: return "ok";
    case HGEMM_ERR_INVALID_ARG: return "invalid argument";
    case HGEMM_ERR_UNSUPPORTED: return "unsupported shape, alignment or config";
    case HGEMM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int hgemm_last_hip_error(void) { return g_last_hip_error; }

const char *hgemm_version(void) { return "hgemm-gfx950 1.1"; }

int hgemm_kernel_count(void) { return kTableSize; }

const char *hgemm_kernel_info(int index, int *layout, int *dtype, int *bm, int *bn, int *bk) {
  if (index < 0 || index >= kTableSize) return nullptr;
  const KernelEntry &e = kTable[index];
  if (layout) *layout = e.layout;
  if (dtype) *dtype = e.dtype;
  if (bm) *bm = e.bm;
  if (bn) *bn = e.bn;
  if (bk) *bk = e.bk;
  return e.name;
}

int hgemm_auto_kernel(int layout, int dtype, int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (layout < kTN || layout > kAtNN || (dtype != HGEMM_F16 && dtype != HGEMM_BF16) || M <= 0 ||
      N <= 0)
    return -1;
  return auto_kernel(layout, dtype, M, N);
}

}  // extern "C"
