// probe.hip -- test-support kernels (declared in include/hgemm_probe.h): run
// the GEMM kernels' building blocks in isolation (MFMA lane maps, LDS
// placement and fragment reads, tile order) and measure the hardware rates
// the design rests on (matrix-core issue rate and clock per shape and data,
// LDS read throughput per access pattern, L2-to-CU streaming).
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "hgemm_probe.h"
#include "gemm_regstage.hpp"

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

// One 16x16x32 matrix-core instruction on one wave.
template <int DT>
__global__ __launch_bounds__(64) void probe_mfma16_kernel(const u32x4 *x, const u32x4 *y,
                                                          float *d) {
  const int l = threadIdx.x;
  const f32x4 acc = mfma16x16x32<DT>(x[l], y[l], f32x4{});
#pragma unroll
  for (int r = 0; r < 4; ++r) d[l * 4 + r] = acc[r];
}

// One wave loads one K step of an operand tile (BX rows x 64 k, or 64 k-rows
// x BX for the m/n-contiguous form) into LDS with the kernels' direct-to-LDS
// placement and XOR layout, then reads every operand fragment back with the
// kernels' fragment reads: dst[f][sl][lane] = the 16 bytes lane `lane` holds
// for fragment f (rows/columns 16f..16f+15) of k-slice sl.
template <int MN, int BX>
__global__ __launch_bounds__(64) void probe_fragments_kernel(const uint16_t *src, int ld,
                                                             u32x4 *dst) {
  __shared__ __attribute__((aligned(1024))) char smem[BX * 128];
  const int lane = threadIdx.x;
  constexpr int ROWB = 2 * BX;
  const uint32_t bytes = (uint32_t)((MN ? 63 * ld + BX : (BX - 1) * ld + 64) * 2);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, bytes);
#pragma unroll
  for (int seg = 0; seg < BX / 8; ++seg) {  // BX * 128 bytes = BX / 8 segments of 1 KiB
    int chunk;
    const uint32_t off = MN ? mnmajor_load_offset<kLdsXor>(seg, lane, ld, ROWB, 0, BX, chunk)
                            : kmajor_load_offset<kLdsXor>(seg, lane, ld, chunk);
    load16_lds(r, off, smem + seg * 1024);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // the segments have landed in LDS
#pragma unroll
  for (int f = 0; f < BX / 16; ++f) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      u32x4 v;
      if constexpr (MN) {
        const uint32_t a = lds_addr(smem + mnmajor_frag_offset<kLdsXor>(lane, 16 * f, ROWB));
        const u32x2 lo = lds_read_tr16(a, (32 * sl) * ROWB);
        const u32x2 hi = lds_read_tr16(a, (32 * sl + 4) * ROWB);
        v[0] = lo[0];
        v[1] = lo[1];
        v[2] = hi[0];
        v[3] = hi[1];
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v));  // the reads are not compiler-tracked
      } else {
        v = *(const u32x4 *)(smem + f * 16 * 128 + kmajor_frag_offset<kLdsXor>(lane, sl));
      }
      dst[(f * 2 + sl) * 64 + lane] = v;
    }
  }
}

// Same store/read pattern as the register-staged baseline's A region with
// BM = 256, 256 threads.
template <int LDS>
__global__ __launch_bounds__(256) void probe_lds_kernel(const u32x4 *src, u32x4 *dst) {
  using T = RsCfg<256, 256, 2, 2, LDS>;
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

__global__ __launch_bounds__(256) void probe_mfma_peak_kernel(int iters, float *out,
                                                              uint64_t *clocks) {
  const int t = threadIdx.x;
  const uint64_t c0 = clock64(), r0 = wall_clock64();
  u32x4 a = {0x3c003c00u ^ (uint32_t)t, 0x3c00u, 0x3c003c00u, 0x0u};
  u32x4 b = {0x3c00u, 0x3c003c00u ^ (uint32_t)t, 0x0u, 0x3c003c00u};
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j & 3] = mfma32x32x16<kF16>(a, b, acc[j & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * 256 + t] = s;
  const uint64_t c1 = clock64(), r1 = wall_clock64();
  if (clocks != nullptr && (t & 63) == 0) {
    const int w = blockIdx.x * 4 + (t >> 6);
    clocks[2 * w] = c1 - c0;      // shader clock cycles
    clocks[2 * w + 1] = r1 - r0;  // constant-rate real-time ticks
  }
}

// Production fragment reads over one wave's 16 KiB quarter: 4 k-contiguous
// 16-row fragments (rows of 128 bytes, one 16-byte read each) or, with the
// transposing read, a 64 x 128 m/n-contiguous tile (rows of 256 bytes, two
// 8-byte reads per fragment), with the XOR layout (XOR) or without.
template <bool TR, bool XOR>
__global__ __launch_bounds__(256) void probe_lds_frag_kernel(int iters, float *out) {
  __shared__ __attribute__((aligned(1024))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 65536 / 16; i += 256) ((u32x4 *)smem)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  constexpr int L = XOR ? kLdsXor : kLdsPlain;
  char *q = smem + wave * 16384;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if constexpr (!TR) {
    uint32_t off[2];
    for (int sl = 0; sl < 2; ++sl) off[sl] = kmajor_frag_offset<L>(lane, sl);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {  // fragment j % 8 of a 128-row block, slice j / 8
        const u32x4 v = *(const u32x4 *)(q + (j & 7) * 16 * 128 + off[j >> 3]);
        acc ^= v;
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    }
  } else {
    uint32_t off[8];
    for (int f = 0; f < 8; ++f) off[f] = mnmajor_frag_offset<L>(lane, 16 * f, 256);
    for (int i = 0; i < iters; ++i) {
      // 16 fragments of 16 bytes per lane = 32 transposing reads, in groups of
      // 8; the reads are not compiler-tracked, so each group ends in an
      // explicit wait tied to all eight destinations
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2 v[8];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * jg + jj;
          v[2 * jj] = lds_read_tr16(lds_addr(q + off[j & 7]), (j >> 3) * 32 * 256);
          v[2 * jj + 1] = lds_read_tr16(lds_addr(q + off[j & 7]), ((j >> 3) * 32 + 4) * 256);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]));
#pragma unroll
        for (int r = 1; r < 8; ++r) asm volatile("" : "+v"(v[r]));
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          acc[0] ^= v[r][0];
          acc[1] ^= v[r][1];
        }
      }
    }
  }
  out[blockIdx.x * 256 + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// Matrix-core issue rate of one shape: each wave runs iters x 16 MFMAs over
// 16 independent accumulators.  With RANDOM the operands are 8 + 8 registers
// of pseudo-random FP16 values in (-1, 1): x changes from one MFMA to the
// next and y every 16, so that consecutive MFMAs see different bits (as in a
// GEMM); otherwise one constant pair.  The MFMAs are inline assembly with the
// accumulators pinned to AGPRs and the operands to VGPRs: compiled from the
// builtins, this loop picks up register moves between the MFMAs that would be
// measured instead of the matrix core.  Each accumulator is reused 16 MFMAs
// later, far past the instruction's latency.
template <int SHAPE>
__device__ __forceinline__ void mfma_pinned(f32x16 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int SHAPE>
__device__ __forceinline__ void mfma_pinned(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <int SHAPE, bool RANDOM>
__global__ __launch_bounds__(256) void probe_mfma_rate_kernel(int iters, float *out,
                                                              uint64_t *clocks) {
  const int t = threadIdx.x;
  u32x4 x[8], y[8];
  uint32_t h = 0x9E3779B9u * (uint32_t)(t + 1);
  for (int i = 0; i < 8; ++i)
    for (int e = 0; e < 4; ++e) {
      uint32_t w = 0x3C003C00u;  // 1.0, 1.0
      if (RANDOM) {
        h = h * 1664525u + 1013904223u;  // LCG: random sign and mantissa, exponent -1
        w = (h & 0x83FF83FFu) | 0x38003800u;
      }
      x[i][e] = w;
      y[i][e] = RANDOM ? (w ^ 0x80008000u) + (uint32_t)i : w;
    }
  using Acc = std::conditional_t<SHAPE == 0, f32x16, f32x4>;
  constexpr int R = SHAPE == 0 ? 16 : 4;
  Acc acc[16];
  for (int j = 0; j < 16; ++j) acc[j] = Acc{};
  // the compiler inserts no hazard wait states around inline assembly: let the
  // zeroing writes of the accumulators settle before the first MFMA reads them
  // (the empty statements pin the writes before the wait)
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" : "+a"(acc[j]));
  // operands opaque to the compiler: held in VGPRs, never rebuilt in the loop
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(x[i]), "+v"(y[i]));
  asm volatile("s_nop 7" ::: "memory");
  const uint64_t c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j) mfma_pinned<SHAPE>(acc[j], x[j & 7], y[u]);
  }
  // nor after it: wait out the last MFMAs' latency (256 wait states) before
  // the accumulators are read
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("s_nop 15" ::: "memory");
  const uint64_t c1 = clock64(), r1 = wall_clock64();
  float s = 0.0f;
  for (int j = 0; j < 16; ++j)
    for (int r = 0; r < R; ++r) s += acc[j][r];
  out[blockIdx.x * 256 + t] = s;
  if (clocks != nullptr && (t & 63) == 0) {
    const int w = blockIdx.x * 4 + (t >> 6);
    clocks[2 * w] = c1 - c0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// Matrix-core issue rate with memory instructions mixed in, one wave per SIMD
// (four per workgroup, one workgroup per CU): each iteration issues 64
// 16x16x32 MFMAs (random FP16 operands, 16 independent accumulators) and,
// spread evenly among them,
//   NLOAD loads of kind KIND out of an L2-resident window:
//     0: buffer_load_dwordx4 ... lds (1 KiB into LDS per instruction; four
//        loads share one LDS base through the immediate offset),
//     1: buffer_load_dwordx4 into registers (1 KiB per instruction), written
//        to LDS with ds_write_b128 in the second half of the iteration,
//     2: buffer_load_dword ... lds (256 bytes into LDS per instruction);
//   NREAD 16-byte LDS reads (ds_read_b128) of a region no load writes.
// Kinds 0 and 2 wait at the end of an iteration only for the previous
// iteration's loads; reads are consumed at the end of their iteration.
// clocks[2w], clocks[2w+1]: shader clock cycles and real-time ticks of wave w
// over the loop; cycles / (64 * iters) is the time per MFMA (16 at full rate).
template <int KIND, int NLOAD, int NREAD, bool BAR = false>
__global__ __launch_bounds__(256) void probe_mix_kernel(const uint16_t *buf, uint32_t window,
                                                        int iters, float *out, uint64_t *clocks) {
  __shared__ __attribute__((aligned(1024))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  u32x4 x[8], y[8];
  uint32_t h = 0x9E3779B9u * (uint32_t)(t + 1);
  for (int i = 0; i < 8; ++i)
    for (int e = 0; e < 4; ++e) {
      h = h * 1664525u + 1013904223u;
      const uint32_t w = (h & 0x83FF83FFu) | 0x38003800u;
      x[i][e] = w;
      y[i][e] = (w ^ 0x80008000u) + (uint32_t)i;
    }
  f32x4 acc[16];
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{};
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" : "+a"(acc[j]));
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(x[i]), "+v"(y[i]));
  // LDS: wave w owns [16w KiB, 16w+16 KiB): loads land in its first 8 KiB,
  // reads come from its last 8 KiB
  for (int i = t; i < 65536 / 16; i += 256) ((u32x4 *)smem)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  char *dst = smem + wave * 16384;
  const uint32_t rd = (uint32_t)(wave * 16384 + 8192 + lane * 16);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, window);
  const uint32_t mask = window - 1;  // a power of two
  uint32_t base = ((blockIdx.x * 4u + (uint32_t)wave) * 16384u) & mask;
  constexpr int LSP = (KIND == 1 ? 32 : 64) / (NLOAD > 0 ? NLOAD : 64);  // MFMAs per load
  constexpr int RSP = 64 / (NREAD > 0 ? NREAD : 64);                     // MFMAs per read
  u32x4 gv[KIND == 1 && NLOAD > 0 ? NLOAD : 1];
  u32x4 rv[NREAD > 0 ? NREAD : 1];
  asm volatile("s_nop 7" ::: "memory");
  const uint64_t c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      if constexpr (BAR) {
        // a workgroup barrier every 128 MFMAs, in the middle of every other
        // iteration, after the waits a pipelined GEMM step has there
        if (j == 32 && (it & 1)) {
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(KIND == 1 ? 0 : NLOAD, 0));
          wg_barrier();
        }
      }
      mfma_pinned<1>(acc[j & 15], x[j & 7], y[(j >> 3) & 7]);
      if constexpr (NLOAD > 0) {
        if (j % LSP == 0 && j / LSP < NLOAD) {
          const int i = j / LSP;
          const uint32_t so = (base + (uint32_t)i * 1024u) & mask;
          if constexpr (KIND == 0) {
            auto *l = (__attribute__((address_space(3))) void *)(dst + ((i >> 2) & 1) * 4096);
            const uint32_t vo = (uint32_t)lane * 16u;
            switch (i & 3) {
              case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vo, so, 0, 0); break;
              case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vo, so, 1024, 0); break;
              case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vo, so, 2048, 0); break;
              default: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vo, so, 3072, 0); break;
            }
          } else if constexpr (KIND == 2) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void *)(dst + (i & 31) * 256), 4,
                (uint32_t)lane * 4u, so, 0, 0);
          } else {
            gv[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)lane * 16u, so, 0);
          }
        }
        if constexpr (KIND == 1) {
          if (j >= 32 && (j - 32) % LSP == 0 && (j - 32) / LSP < NLOAD) {
            const int i = (j - 32) / LSP;
            *(u32x4 *)(dst + (i & 7) * 1024 + lane * 16) = gv[i];
          }
        }
      }
      if constexpr (NREAD > 0) {
        if (j % RSP == RSP / 2 && j / RSP < NREAD) {
          const int k = j / RSP;
          rv[k] = *(const u32x4 *)(smem + rd + (k & 7) * 1024);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    base = (base + (uint32_t)NLOAD * 1024u) & mask;
    if constexpr (NREAD > 0) {
#pragma unroll
      for (int k = 0; k < NREAD; ++k) asm volatile("" ::"v"(rv[k]));
    }
    if constexpr (KIND != 1 && NLOAD > 0) {
      // the previous iteration's loads have landed (this one's may run on)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(NLOAD, 63));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("s_nop 15" ::: "memory");
  const uint64_t c1 = clock64(), r1 = wall_clock64();
  float sum = 0.0f;
  for (int j = 0; j < 16; ++j)
    for (int e = 0; e < 4; ++e) sum += acc[j][e];
  out[blockIdx.x * 256 + t] = sum + (float)((const uint32_t *)smem)[t];
  if (clocks != nullptr && lane == 0) {
    const int w = blockIdx.x * 4 + wave;
    clocks[2 * w] = c1 - c0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

using MixFn = void (*)(const uint16_t *, uint32_t, int, float *, uint64_t *);
template <int KIND, int NREAD, bool BAR = false>
MixFn mix_fn(int nload) {
  switch (nload) {
    case 0: return &probe_mix_kernel<KIND, 0, NREAD, BAR>;
    case 2: return &probe_mix_kernel<KIND, 2, NREAD, BAR>;
    case 4: return &probe_mix_kernel<KIND, 4, NREAD, BAR>;
    case 8: return &probe_mix_kernel<KIND, 8, NREAD, BAR>;
    case 16: return &probe_mix_kernel<KIND, 16, NREAD, BAR>;
    default: return nullptr;
  }
}

template <int PATTERN>
__global__ __launch_bounds__(256) void probe_lds_read_kernel(int iters, float *out) {
  __shared__ __attribute__((aligned(16))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 65536 / 16; i += 256) ((u32x4 *)smem)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  uint32_t off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if constexpr (PATTERN == 0)
      off[ks] = wave * 16384 + ks * 4096 + lane * 16;
    else
      off[ks] = wave * 16384 + (lane & 31) * 128 +
                chunk_pos<PATTERN == 1 ? kLdsXor : (PATTERN == 2 ? kLdsPlain : kLdsXorRow)>(
                    lane & 31, 2 * ks + (lane >> 5)) * 16;
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      // each wave stays inside its own 16 KiB quarter: pattern 0 spans
      // 4 x 4096 + 3 x 1024 + 1024 bytes, patterns 1/2 span 4 x 4096 (32 rows each)
      constexpr int kStep = (PATTERN == 0) ? 1024 : 4096;
      const u32x4 v = *(const u32x4 *)(smem + off[j & 3] + (j >> 2) * kStep);
      acc ^= v;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): keep reads of one iteration together
  }
  out[blockIdx.x * 256 + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// The 16-row fragment read on 64-byte rows (32 k per row, chunk c of row r
// at c ^ ((r >> 2) & 3)): lane l reads row l % 16, logical chunk l / 16.
// That layout is conflict-free if 16-byte reads were served lanes 0-15,
// 16-31, ... at a time, and measures at half the rate of the production
// layout: the hardware groups the lanes otherwise.  16 fragments of 16 rows
// per iteration, each wave in its own 16 KiB quarter.
__global__ __launch_bounds__(256) void probe_lds_half_row_kernel(int iters, float *out) {
  __shared__ __attribute__((aligned(1024))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 65536 / 16; i += 256) ((u32x4 *)smem)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int row = lane & 15, chunk = (lane >> 4) ^ ((row >> 2) & 3);
  const char *q = smem + wave * 16384 + row * 64 + chunk * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= *(const u32x4 *)(q + j * 1024);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  }
  out[blockIdx.x * 256 + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// 16-byte LDS reads at per-lane byte offsets given by the caller (lane l reads
// offs[l] + 1024 * j, j = 0..15, within its wave's 16 KiB quarter; every
// read of an iteration at its own address, so that none can be folded into
// another): the read rate of any lane-to-address map, for the bank model.
__global__ __launch_bounds__(256) void probe_lds_lanes_kernel(int iters, const uint32_t *offs,
                                                              float *out) {
  __shared__ __attribute__((aligned(1024))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 65536 / 16; i += 256) ((u32x4 *)smem)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const char *q = smem + wave * 16384 + (offs[lane] & 1008u);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= *(const u32x4 *)(q + j * 1024);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  }
  out[blockIdx.x * 256 + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// Streams 64 KiB per workgroup per iteration out of an L2-resident window:
// MODE 0 into registers, MODE 1 straight into LDS; NF loads per lane in flight.
// HALF: every load covers 16 half rows of 64 bytes instead of 8 rows of 128,
// and two consecutive iterations take the two halves of the same rows, so
// that each 128-byte line is requested twice.
template <int MODE, int NF, bool HALF = false>
__global__ __launch_bounds__(256) void probe_l2_kernel(const uint16_t *buf, uint32_t window,
                                                       uint32_t row_stride, int iters, float *out) {
  __shared__ __attribute__((aligned(1024))) char smem[65536];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, window);
  const uint32_t mask = window - 1;  // window is a power of two
  uint32_t base = (blockIdx.x * 65536u) & mask;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; j += NF) {
      u32x4 v[NF];
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        // 1 KiB per wave and load: 8 rows of 128 bytes (or 16 of 64), rows
        // row_stride bytes apart
        const uint32_t off =
            HALF ? (base + (uint32_t)(it & 1) * 64u +
                    ((uint32_t)(wave * 16 + j + i) * 16u + (uint32_t)(lane >> 2)) * row_stride +
                    (uint32_t)(lane & 3) * 16u) & mask
                 : (base + (uint32_t)(wave * 16 + j + i) * 8u * row_stride +
                    (uint32_t)(lane >> 3) * row_stride + (uint32_t)(lane & 7) * 16u) & mask;
        if constexpr (MODE == 0) v[i] = load16(r, off);
        else load16_lds(r, off, smem + (wave * 16 + j + i) * 1024);
      }
      if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < NF; ++i) acc ^= v[i];
      }
    }
    if constexpr (MODE == 1) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (!HALF || (it & 1)) base = (base + 128u * 8u) & mask;  // 1 KiB further along the rows
  }
  if constexpr (MODE == 1) {
    __syncthreads();
    acc = *(const u32x4 *)(smem + t * 16);
  }
  out[blockIdx.x * 256 + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

template <int LDS>
void lds_offsets(int rows, int *offsets) {
  using T = RsCfg<256, 256, 2, 2, LDS>;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < 8; ++c) offsets[r * 8 + c] = r * T::ROWB + chunk_pos<LDS>(r, c) * 16;
}

// hipGetLastError() also reports earlier runtime calls on this thread: each
// launching probe clears it first (clear_error), then checks its own launch.
void clear_error() { (void)hipGetLastError(); }

hgemm_status_t launched() {
  return hipGetLastError() == hipSuccess ? HGEMM_OK : HGEMM_ERR_HIP;
}

}  // namespace

extern "C" {

hgemm_status_t hgemm_probe_mfma(int dtype, const void *x, const void *y, float *d, void *stream) {
  clear_error();
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

hgemm_status_t hgemm_probe_mfma16(int dtype, const void *x, const void *y, float *d,
                                  void *stream) {
  clear_error();
  if (dtype != HGEMM_F16 && dtype != HGEMM_BF16) return HGEMM_ERR_INVALID_ARG;
  if (!x || !y || !d) return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)d) & 15) return HGEMM_ERR_UNSUPPORTED;
  if (dtype == HGEMM_F16)
    hipLaunchKernelGGL(probe_mfma16_kernel<kF16>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (const u32x4 *)y, d);
  else
    hipLaunchKernelGGL(probe_mfma16_kernel<kBF16>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (const u32x4 *)y, d);
  return launched();
}

hgemm_status_t hgemm_probe_fragments(int mn_major, int bx, const void *src, int64_t ld,
                                     void *dst, void *stream) {
  clear_error();
  if (!src || !dst || (mn_major != 0 && mn_major != 1)) return HGEMM_ERR_INVALID_ARG;
  if (bx != 64 && bx != 128 && bx != 192 && bx != 256) return HGEMM_ERR_INVALID_ARG;
  if (ld < (mn_major ? bx : 64) || ld % 8 != 0 || ld > (1 << 20)) return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return HGEMM_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t *p = (const uint16_t *)src;
  u32x4 *q = (u32x4 *)dst;
  const int l = (int)ld;
  if (mn_major) {
    if (bx == 64) hipLaunchKernelGGL((probe_fragments_kernel<1, 64>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 128) hipLaunchKernelGGL((probe_fragments_kernel<1, 128>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 192) hipLaunchKernelGGL((probe_fragments_kernel<1, 192>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 256) hipLaunchKernelGGL((probe_fragments_kernel<1, 256>), dim3(1), dim3(64), 0, s, p, l, q);
  } else {
    if (bx == 64) hipLaunchKernelGGL((probe_fragments_kernel<0, 64>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 128) hipLaunchKernelGGL((probe_fragments_kernel<0, 128>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 192) hipLaunchKernelGGL((probe_fragments_kernel<0, 192>), dim3(1), dim3(64), 0, s, p, l, q);
    if (bx == 256) hipLaunchKernelGGL((probe_fragments_kernel<0, 256>), dim3(1), dim3(64), 0, s, p, l, q);
  }
  return launched();
}

hgemm_status_t hgemm_probe_operand_offsets(int mn_major, int bx, int *load_row, int *load_chunk,
                                           int *read_off) {
  if (!load_row || !load_chunk || !read_off || (mn_major != 0 && mn_major != 1))
    return HGEMM_ERR_INVALID_ARG;
  if (bx != 64 && bx != 128 && bx != 192 && bx != 256) return HGEMM_ERR_INVALID_ARG;
  const int rowb = 2 * bx;
  for (int seg = 0; seg < bx / 8; ++seg)
    for (int l = 0; l < 64; ++l) {
      int chunk;
      if (mn_major) {
        // k-row of the lane's chunk: the offset is k*ld + chunk*8 elements; with ld = 1 << 16
        // the k-row is recovered from the offset
        const uint32_t off = mnmajor_load_offset<kLdsXor>(seg, l, 1 << 16, rowb, 0, bx, chunk);
        load_row[seg * 64 + l] = (int)((off / 2u) >> 16);
      } else {
        const uint32_t off = kmajor_load_offset<kLdsXor>(seg, l, 1 << 16, chunk);
        load_row[seg * 64 + l] = (int)((off / 2u) >> 16);
      }
      load_chunk[seg * 64 + l] = chunk;
    }
  const int reads = mn_major ? 2 : 1;
  for (int f = 0; f < bx / 16; ++f)
    for (int sl = 0; sl < 2; ++sl)
      for (int r = 0; r < reads; ++r)
        for (int l = 0; l < 64; ++l) {
          const int o = mn_major ? (int)mnmajor_frag_offset<kLdsXor>(l, 16 * f, rowb) +
                                       (32 * sl + 4 * r) * rowb
                                 : f * 16 * 128 + (int)kmajor_frag_offset<kLdsXor>(l, sl);
          read_off[((f * 2 + sl) * reads + r) * 64 + l] = o;
        }
  return HGEMM_OK;
}

hgemm_status_t hgemm_probe_lds_roundtrip(int lds_layout, const void *src, void *dst,
                                         void *stream) {
  clear_error();
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
    case kLdsXorRow:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsXorRow>, dim3(1), dim3(256), 0, s,
                         (const u32x4 *)src, (u32x4 *)dst);
      break;
    default:
      return HGEMM_ERR_INVALID_ARG;
  }
  return launched();
}

hgemm_status_t hgemm_probe_mfma_peak(int waves, int iters, float *out, uint64_t *clocks,
                                     void *stream) {
  clear_error();
  if (waves <= 0 || waves % 4 != 0 || iters <= 0 || !out) return HGEMM_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_mfma_peak_kernel, dim3(waves / 4), dim3(256), 0, (hipStream_t)stream,
                     iters, out, clocks);
  return launched();
}

hgemm_status_t hgemm_probe_mfma_rate(int shape, int random, int waves, int iters, float *out,
                                     uint64_t *clocks, void *stream) {
  clear_error();
  if ((shape != 0 && shape != 1) || (random != 0 && random != 1)) return HGEMM_ERR_INVALID_ARG;
  if (waves <= 0 || waves % 4 != 0 || iters <= 0 || iters % 8 != 0 || !out)
    return HGEMM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g(waves / 4), b(256);
  if (shape == 0 && !random) hipLaunchKernelGGL((probe_mfma_rate_kernel<0, false>), g, b, 0, s, iters, out, clocks);
  if (shape == 0 && random) hipLaunchKernelGGL((probe_mfma_rate_kernel<0, true>), g, b, 0, s, iters, out, clocks);
  if (shape == 1 && !random) hipLaunchKernelGGL((probe_mfma_rate_kernel<1, false>), g, b, 0, s, iters, out, clocks);
  if (shape == 1 && random) hipLaunchKernelGGL((probe_mfma_rate_kernel<1, true>), g, b, 0, s, iters, out, clocks);
  return launched();
}

hgemm_status_t hgemm_probe_lds_read(int workgroups, int iters, int pattern, float *out,
                                    void *stream) {
  clear_error();
  if (workgroups <= 0 || iters <= 0 || !out) return HGEMM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  switch (pattern) {
    case 0: hipLaunchKernelGGL(probe_lds_read_kernel<0>, dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(probe_lds_read_kernel<1>, dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL(probe_lds_read_kernel<2>, dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL(probe_lds_read_kernel<3>, dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 4: hipLaunchKernelGGL((probe_lds_frag_kernel<false, true>), dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 5: hipLaunchKernelGGL((probe_lds_frag_kernel<false, false>), dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 6: hipLaunchKernelGGL((probe_lds_frag_kernel<true, true>), dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 7: hipLaunchKernelGGL((probe_lds_frag_kernel<true, false>), dim3(workgroups), dim3(256), 0, s, iters, out); break;
    case 8: hipLaunchKernelGGL(probe_lds_half_row_kernel, dim3(workgroups), dim3(256), 0, s, iters, out); break;
    default: return HGEMM_ERR_INVALID_ARG;
  }
  return launched();
}

hgemm_status_t hgemm_probe_lds_lanes(int workgroups, int iters, const uint32_t *lane_offsets,
                                     float *out, void *stream) {
  clear_error();
  if (workgroups <= 0 || iters <= 0 || !lane_offsets || !out) return HGEMM_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_lds_lanes_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     iters, lane_offsets, out);
  return launched();
}

hgemm_status_t hgemm_probe_l2_read(int workgroups, int iters, int mode, const void *buf,
                                   uint32_t window_bytes, uint32_t row_stride, float *out,
                                   void *stream) {
  clear_error();
  if (workgroups <= 0 || iters <= 0 || !buf || !out) return HGEMM_ERR_INVALID_ARG;
  if (row_stride < 128u || (row_stride & 15u)) return HGEMM_ERR_INVALID_ARG;
  if (window_bytes < 65536u || window_bytes > (1u << 30) || (window_bytes & (window_bytes - 1)))
    return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)buf) & 15) return HGEMM_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t *b = (const uint16_t *)buf;
  switch (mode) {
    case 0: hipLaunchKernelGGL((probe_l2_kernel<0, 16>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    case 1: hipLaunchKernelGGL((probe_l2_kernel<1, 16>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    case 2: hipLaunchKernelGGL((probe_l2_kernel<0, 8>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    case 3: hipLaunchKernelGGL((probe_l2_kernel<1, 8>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    case 4: hipLaunchKernelGGL((probe_l2_kernel<0, 16, true>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    case 5: hipLaunchKernelGGL((probe_l2_kernel<1, 16, true>), dim3(workgroups), dim3(256), 0, s, b, window_bytes, row_stride, iters, out); break;
    default: return HGEMM_ERR_INVALID_ARG;
  }
  return launched();
}


hgemm_status_t hgemm_probe_mix(int kind, int nload, int nread, int workgroups, int iters,
                               const void *buf, uint32_t window_bytes, float *out,
                               uint64_t *clocks, void *stream) {
  clear_error();
  if (workgroups <= 0 || iters <= 0 || !buf || !out || !clocks) return HGEMM_ERR_INVALID_ARG;
  if (window_bytes < 65536u || window_bytes > (1u << 30) || (window_bytes & (window_bytes - 1)))
    return HGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)buf) & 15) return HGEMM_ERR_UNSUPPORTED;
  MixFn fn = nullptr;
  if (nread == 0) {
    fn = kind == 0 ? mix_fn<0, 0>(nload) : kind == 1 ? mix_fn<1, 0>(nload)
         : kind == 2 ? mix_fn<2, 0>(nload) : nullptr;
  } else if (nread == 16) {
    fn = kind == 0 ? mix_fn<0, 16>(nload) : kind == 1 ? mix_fn<1, 16>(nload)
         : kind == 2 ? mix_fn<2, 16>(nload) : nullptr;
  } else if (nread == 16 + 256) {  // with a workgroup barrier every 128 MFMAs
    fn = kind == 0 ? mix_fn<0, 16, true>(nload) : nullptr;
  } else if (nread == 256) {
    fn = kind == 0 ? mix_fn<0, 0, true>(nload) : nullptr;
  }
  if (fn == nullptr) return HGEMM_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fn, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t *)buf, window_bytes, iters, out, clocks);
  return launched();
}

hgemm_status_t hgemm_probe_lds_offsets(int lds_layout, int rows, int *offsets) {
  if (rows <= 0 || !offsets) return HGEMM_ERR_INVALID_ARG;
  switch (lds_layout) {
    case kLdsXor: lds_offsets<kLdsXor>(rows, offsets); break;
    case kLdsPlain: lds_offsets<kLdsPlain>(rows, offsets); break;
    case kLdsPad: lds_offsets<kLdsPad>(rows, offsets); break;
    case kLdsXorRow: lds_offsets<kLdsXorRow>(rows, offsets); break;
    default: return HGEMM_ERR_INVALID_ARG;
  }
  return HGEMM_OK;
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
