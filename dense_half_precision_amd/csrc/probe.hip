// probe.hip -- test-support kernels (declared in include/hgemm_probe.h): run
// the MFMA wrapper and the LDS store/read addressing of the GEMM kernels in
// isolation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hgemm_probe.h"
#include "gemm_kernel.hpp"

namespace {

using namespace hgemm;

template <int DT>
__global__ __launch_bounds__(64) void probe_mfma_kernel(const u32x4 *x, const u32x4 *y, float *d) {
  const int l = threadIdx.x;
  f32x16 acc = f32x16{};
  acc = mfma32x32x16<DT>(x[l], y[l], acc);
#pragma unroll
  for (int r = 0; r < 16; ++r) d[l * 16 + r] = acc[r];
}

// Same store/read pattern as gemm_kernel's A region with BM = 256, 256 threads.
template <int LDS>
__global__ __launch_bounds__(256) void probe_lds_kernel(const u32x4 *src, u32x4 *dst) {
  using T = TileCfg<256, 256, 2, 2, LDS>;
  constexpr int ROWB = T::ROWB;
  __shared__ __attribute__((aligned(16))) char smem[256 * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ld_row = tid >> 3, ld_kc = tid & 7;
  const uint32_t st = ld_row * ROWB + chunk_pos<LDS>(ld_row, ld_kc) * 16;
#pragma unroll
  for (int i = 0; i < T::LA; ++i)
    *(u32x4 *)(smem + st + i * T::ROWS_PER_PASS * ROWB) =
        src[(ld_row + i * T::ROWS_PER_PASS) * 8 + ld_kc];
  __syncthreads();
  // wave w reads rows [64w, 64w+64) as two 32-row fragments, all four k steps
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t off = (lane & 31) * ROWB + chunk_pos<LDS>(lane & 31, 2 * ks + (lane >> 5)) * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row0 = wave * 64 + i * 32;
      const u32x4 v = *(const u32x4 *)(smem + row0 * ROWB + off);
      dst[(row0 + (lane & 31)) * 8 + 2 * ks + (lane >> 5)] = v;
    }
  }
}

hgemm_status_t launched() {
  return hipGetLastError() == hipSuccess ? HGEMM_OK : HGEMM_ERR_HIP;
}

}  // namespace

extern "C" {

hgemm_status_t hgemm_probe_mfma(int dtype, const void *x, const void *y, float *d, void *stream) {
  if (dtype != HGEMM_F16 && dtype != HGEMM_BF16) return HGEMM_ERR_INVALID_ARG;
  if (!x || !y || !d) return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)d) & 15) return HGEMM_ERR_UNSUPPORTED;
  if (dtype == HGEMM_F16)
    hipLaunchKernelGGL(probe_mfma_kernel<kF16>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (const u32x4 *)y, d);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<kBF16>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (const u32x4 *)y, d);
  return launched();
}

hgemm_status_t hgemm_probe_lds_roundtrip(int lds_layout, const void *src, void *dst,
                                         void *stream) {
  if (!src || !dst) return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return HGEMM_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  switch (lds_layout) {
    case kLdsXor:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsXor>, dim3(1), dim3(256), 0, s, (const u32x4 *)src,
                         (u32x4 *)dst);
      break;
    case kLdsPlain:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsPlain>, dim3(1), dim3(256), 0, s,
                         (const u32x4 *)src, (u32x4 *)dst);
      break;
    case kLdsPad:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsPad>, dim3(1), dim3(256), 0, s, (const u32x4 *)src,
                         (u32x4 *)dst);
      break;
    default:
      return HGEMM_ERR_INVALID_ARG;
  }
  return launched();
}

hgemm_status_t hgemm_probe_tile_order(int tiles_m, int tiles_n, int group_m, int xcd_remap,
                                      int *tm, int *tn) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || (xcd_remap != 0 && xcd_remap != 1) ||
      !tm || !tn)
    return HGEMM_ERR_INVALID_ARG;
  if ((int64_t)tiles_m * tiles_n > INT32_MAX) return HGEMM_ERR_UNSUPPORTED;
  const int total = tiles_m * tiles_n;
  for (int i = 0; i < total; ++i) tile_coords(i, tiles_m, tiles_n, group_m, xcd_remap, tm[i], tn[i]);
  return HGEMM_OK;
}

}  // extern "C"
