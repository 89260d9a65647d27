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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16x16x32 MFMA, FP32 accumulate: D[i][j] = sum_k X[i][k] * Y[k][j] + Cin.
// Lane l holds 8 consecutive-k elements of X (row i = l % 16) and of Y
// (column j = l % 16), lane group l / 16 holding k = 8*(l/16) .. +7; lane l,
// accumulator r holds D[4*(l/16) + r][l % 16].
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 x, u32x4 y, f32x4 c) {
  if constexpr (DT == kF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
  }
}

// Byte address of a location in the workgroup's LDS (the 32-bit address that
// ds_* instructions take).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)(p);
}

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16) at LDS byte address
// addr + off (off a constant below 65536 after inlining; the build fails
// otherwise).  Within each group of 16 lanes, lane i points at 4 consecutive
// elements; lane l receives element (l % 4) of the row that lane 4*j + l/4
// points at, for j = 0..3.  Addresses are 8-byte aligned.
//
// Issued as inline assembly: the compiler's wait-count pass cannot tell this
// instruction's builtin form apart from a read of memory that a pending
// direct-to-LDS load may still be writing, and drains every load in flight
// (vmcnt(0)) before it, which serialises the load pipeline.  The pass does not
// see the assembly either, so it inserts no wait for the destination: the
// caller must issue a compiler-visible LDS read after this one and consume the
// destination only in instructions that also need that later read.  LDS reads
// complete in order, so the wait the compiler places for the later read also
// covers this one.  The memory clobber keeps the two in program order.
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr, int off) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(off) : "memory");
  return v;
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

// Packed pair of 16-bit values -> two FP32 values (exact).
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t v, float &lo, float &hi) {
  if constexpr (DT == kF16) {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
  } else {
    lo = __builtin_bit_cast(float, v << 16);
    hi = __builtin_bit_cast(float, v & 0xFFFF0000u);
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

// 16-byte buffer load of every lane straight into LDS: lane l's data lands at
// lds_base + 16*l (lds_base must be the same for the whole wave);
// out-of-range offsets read zero.
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                           void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset, 0, 0, 0);
}

// load16_lds with the instruction's immediate offset 1024 * J, which moves
// the LDS destination and the global address alike: four loads into
// consecutive 1 KiB segments share one lds_base (one M0), each lane's voffset
// lowered by the immediate.
template <int J>
__device__ __forceinline__ void load16_lds_imm(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                               void *lds_base) {
  static_assert(J >= 0 && J < 4, "immediate offsets 0, 1024, 2048, 3072");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset, 0, 1024 * J, 0);
}

// Workgroup barrier without the memory fence of __syncthreads(): the caller
// waits (s_waitcnt) for exactly the LDS reads/writes other waves depend on.
// __syncthreads() would also drain every outstanding direct-to-LDS load
// (it counts as a pending LDS write), which would serialise the pipeline.
// The empty asm statements keep the compiler from moving memory operations
// across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate (gfx9 encoding): wait until at most vm outstanding
// vector-memory operations and at most lgkm LDS/scalar operations remain.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | (((vm >> 4) & 0x3) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}

}  // namespace hgemm
