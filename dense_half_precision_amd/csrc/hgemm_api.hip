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
  kernel_fn fn;
};

template <class T, int LAYOUT, int DT>
constexpr KernelEntry entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m,
                     &gemm_kernel<T, LAYOUT, DT>};
}
template <class T, int LAYOUT, int DT>
constexpr KernelEntry rs_entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m,
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

// Index order is part of the ablation interface (hgemm_kernel_info lists it).
// Entries 0..11 are the production kernels the automatic choice picks from.
const KernelEntry kTable[] = {
    entry<T256, kTN, kF16>("tn_f16_256x256x64", 4),
    entry<T256, kTN, kBF16>("tn_bf16_256x256x64", 4),
    entry<T256, kNN, kF16>("nn_f16_256x256x64", 4),
    entry<T256, kNN, kBF16>("nn_bf16_256x256x64", 4),
    entry<T128, kTN, kF16>("tn_f16_128x128x64", 4),
    entry<T128, kTN, kBF16>("tn_bf16_128x128x64", 4),
    entry<T128, kNN, kF16>("nn_f16_128x128x64", 4),
    entry<T128, kNN, kBF16>("nn_bf16_128x128x64", 4),
    entry<T64, kTN, kF16>("tn_f16_64x64x64", 4),
    entry<T64, kTN, kBF16>("tn_bf16_64x64x64", 4),
    entry<T64, kNN, kF16>("nn_f16_64x64x64", 4),
    entry<T64, kNN, kBF16>("nn_bf16_64x64x64", 4),
    // ablations of the production kernel: unswizzled LDS, direct epilogue stores
    entry<T256Plain, kTN, kF16>("tn_f16_256x256x64_plainlds", 4),
    entry<T256Plain, kNN, kBF16>("nn_bf16_256x256x64_plainlds", 4),
    entry<T256Direct, kTN, kF16>("tn_f16_256x256x64_directepi", 4),
    // baseline design: register-staged loads, 32x32x16 MFMA, LDS layout variants
    rs_entry<R256, kTN, kF16>("rs_tn_f16_256x256x64_xor", 8),
    rs_entry<R256Plain, kTN, kF16>("rs_tn_f16_256x256x64_plain", 8),
    rs_entry<R256Pad, kTN, kF16>("rs_tn_f16_256x256x64_pad", 8),
    rs_entry<R256XorRow, kTN, kF16>("rs_tn_f16_256x256x64_xorrow", 8),
    rs_entry<R256, kNN, kBF16>("rs_nn_bf16_256x256x64_xor", 8),
};
constexpr int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

constexpr int64_t kMaxM = int64_t(1) << 30;
constexpr int64_t kMaxN = int64_t(1) << 23;
constexpr int64_t kMaxK = int64_t(1) << 21;

constexpr int kProductionKernels = 12;

int find_kernel(int layout, int dtype, int bm) {
  for (int i = 0; i < kProductionKernels; ++i)
    if (kTable[i].layout == layout && kTable[i].dtype == dtype && kTable[i].bm == bm) return i;
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

hgemm_status_t validate(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                        const void *B, const void *C) {
  if (M < 0 || N < 0 || K < 0) return HGEMM_ERR_INVALID_ARG;
  if (dtype != HGEMM_F16 && dtype != HGEMM_BF16) return HGEMM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return HGEMM_OK;
  if (C == nullptr) return HGEMM_ERR_INVALID_ARG;
  if (K > 0 && (A == nullptr || B == nullptr)) return HGEMM_ERR_INVALID_ARG;
  if (N % 8 != 0 || K % 8 != 0) return HGEMM_ERR_UNSUPPORTED;
  if (M > kMaxM || N > kMaxN || K > kMaxK) return HGEMM_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(C) & 15) != 0) return HGEMM_ERR_UNSUPPORTED;
  if (K > 0 && (((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) != 0))
    return HGEMM_ERR_UNSUPPORTED;
  return HGEMM_OK;
}

hgemm_status_t run(int layout, int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                   const void *B, void *C, void *stream, const hgemm_config_t *cfg) {
  hgemm_status_t st = validate(M, N, K, dtype, A, B, C);
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
  if (kidx >= 0 && (kTable[kidx].layout != layout || kTable[kidx].dtype != dtype))
    return HGEMM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return HGEMM_OK;
  if (kidx < 0) kidx = auto_kernel(layout, dtype, M, N);
  if (kidx < 0) return HGEMM_ERR_UNSUPPORTED;
  const KernelEntry &e = kTable[kidx];
  if (group_m == 0) group_m = e.default_group_m;

  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
  if (tiles > INT32_MAX) return HGEMM_ERR_UNSUPPORTED;
  GemmArgs a;
  a.A = static_cast<const uint16_t *>(A);
  a.B = static_cast<const uint16_t *>(B);
  a.C = static_cast<uint16_t *>(C);
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.group_m = group_m;
  a.xcd_remap = xcd;
  hipLaunchKernelGGL(e.fn, dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return HGEMM_ERR_HIP;
  }
  return HGEMM_OK;
}

}  // namespace

extern "C" {

hgemm_status_t hgemm_tn(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                        const void *Bt, void *C, void *stream) {
  return run(kTN, M, N, K, dtype, A, Bt, C, stream, nullptr);
}

hgemm_status_t hgemm_nn(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                        const void *B, void *C, void *stream) {
  return run(kNN, M, N, K, dtype, A, B, C, stream, nullptr);
}

hgemm_status_t hgemm_tn_ex(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                           const void *Bt, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(kTN, M, N, K, dtype, A, Bt, C, stream, cfg);
}

hgemm_status_t hgemm_nn_ex(int64_t M, int64_t N, int64_t K, int dtype, const void *A,
                           const void *B, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(kNN, M, N, K, dtype, A, B, C, stream, cfg);
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

const char *hgemm_version(void) { return "hgemm-gfx950 1.0"; }

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
  if ((layout != kTN && layout != kNN) || (dtype != HGEMM_F16 && dtype != HGEMM_BF16) || M <= 0 ||
      N <= 0)
    return -1;
  return auto_kernel(layout, dtype, M, N);
}

}  // extern "C"
