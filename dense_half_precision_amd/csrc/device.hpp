// device.hpp -- gfx950 device primitives for the HGEMM kernels: vector
// types, the FP16/BF16 matrix-core (MFMA) instructions, range-checked buffer
// loads and the FP32 -> FP16/BF16 round-to-nearest-even packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hgemm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dtype { kF16 = 0, kBF16 = 1 };

// 32x32x16 MFMA, FP32 accumulate: D[i][j] = sum_k X[i][k] * Y[k][j] + Cin.
// Each lane holds 8 consecutive-k elements of X (row i = lane % 32) and of Y
// (column j = lane % 32), lanes 32..63 holding the second half of the 16 k;
// lane l, accumulator r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].  Only the
// k index matters symmetrically for X and Y, so any fixed k order of the 16
// elements gives the same sum; the output map is checked by a probe test.
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 x, u32x4 y, f32x16 c) {
  if constexpr (DT == kF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
  }
}

// Two FP32 values -> packed pair of 16-bit values, round to nearest even
// (the default round mode of the FP32 -> FP16 and FP32 -> BF16 converts).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == kF16) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (_Float16)lo);
    const uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
  } else {
    const uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
  }
}

// Buffer resource over [base, base + nbytes): 128-bit loads whose byte offset
// is at or beyond nbytes return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// Offset that is always out of range for make_rsrc() (nbytes < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
}

}  // namespace hgemm
