// hgemm_api.hip -- C ABI of libhgemm.so (declared in include/hgemm.h):
// argument validation, the kernel table, the per-shape choice and the launch
// on the caller's stream.  Nothing here allocates device memory or
// synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "hgemm.h"
#include "gemm_kernel.hpp"
#include "gemm_regstage.hpp"
#include "gemm_ws_kernel.hpp"
#include "gemm_pp_kernel.hpp"

namespace {

using namespace hgemm;

thread_local int g_last_hip_error = 0;

typedef void (*kernel_fn)(GemmArgs);

struct KernelEntry {
  const char *name;
  int layout, dtype, bm, bn, bk, lds, default_group_m;
  bool production;  // candidate of the automatic choice
  bool general;     // honours leading dimensions, alpha, beta and K splits
  kernel_fn fn;
  kernel_fn split_fn;  // K segments of the tail tiles only (general kernels)
  kernel_fn mixed_fn;  // K segments, then whole tiles, in one launch (general kernels)
  kernel_fn fixup;     // adds the K segments of split tiles (general kernels)
  int threads = 256;   // workgroup size of fn, split_fn and mixed_fn
  int nsb = 2;         // B stages of the LDS ring (A has one more)
  bool persistent = false;  // fn runs one workgroup per CU over all tiles
  bool timed = false;       // fn writes per-workgroup clock counters to the workspace
  int counter_bytes = 32;   // ... this many bytes of them per workgroup
};
constexpr int kFixupThreads = 256;  // gemm_sk_fixup's workgroup size

template <class T, int LAYOUT, int DT>
constexpr KernelEntry entry(const char *name, int group_m, bool production) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, production, true,
                     &gemm_kernel<T, LAYOUT, DT, kWhole>, &gemm_kernel<T, LAYOUT, DT, kSegments>,
                     &gemm_kernel<T, LAYOUT, DT, kMixed>, &gemm_sk_fixup<T, DT>, T::NT, T::NSB};
}
// persistent: one workgroup per CU loops over the tiles (whole K)
template <class T, int LAYOUT, int DT>
constexpr KernelEntry persistent_entry(const char *name, int group_m, bool production) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, production, true,
                     &gemm_kernel<T, LAYOUT, DT, kPersistent>, nullptr, nullptr, nullptr, T::NT,
                     T::NSB, true};
}
// the production kernel with per-workgroup clock counters (launch mode
// kTimed): measures the engine clock a shape runs at; never chosen
// automatically
template <class T, int LAYOUT, int DT>
constexpr KernelEntry timed_entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, false, true,
                     &gemm_kernel<T, LAYOUT, DT, kTimed>, nullptr, nullptr, nullptr, T::NT,
                     T::NSB, false, true};
}
// whole-K tiles only (no K-split instantiations)
template <class T, int LAYOUT, int DT>
constexpr KernelEntry dp_entry(const char *name, int group_m, bool production) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, production, true,
                     &gemm_kernel<T, LAYOUT, DT, kWhole>, nullptr, nullptr, nullptr, T::NT,
                     T::NSB};
}
// producer/consumer wave specialisation: leading dimensions, alpha and beta,
// no K split; an ablation, never chosen automatically
template <class T, int DT>
constexpr KernelEntry ws_entry(const char *name, int group_m) {
  return KernelEntry{name, kTN, DT, T::BM, T::BN, T::BK, T::LDS, group_m, false, true,
                     &gemm_ws_kernel<T, DT>, nullptr, nullptr, nullptr, T::NT};
}
// two alternating wave groups on the 256 x 256 tile: leading dimensions, alpha
// and beta, no K split; an ablation, never chosen automatically
template <int DT>
constexpr KernelEntry pp_entry(const char *name, int group_m) {
  return KernelEntry{name, kTN, DT, PpCfg::BM, PpCfg::BN, PpCfg::BK, PpCfg::LDS, group_m, false,
                     true, &gemm_pp_kernel<DT>, nullptr, nullptr, nullptr, PpCfg::NT};
}
// the 128 x 128 tile on eight waves in two groups that split K: leading
// dimensions, alpha and beta, no K split; an ablation, never chosen
// automatically
template <int DT>
constexpr KernelEntry ppk_entry(const char *name, int group_m) {
  return KernelEntry{name, kTN, DT, PpkCfg::BM, PpkCfg::BN, PpkCfg::BK, PpkCfg::LDS, group_m,
                     false, true, &gemm_ppk_kernel<DT>, nullptr, nullptr, nullptr, PpkCfg::NT};
}
// the production kernel with per-wave main-loop phase clocks (launch mode
// kPhases): a measurement copy; never chosen automatically
template <class T, int LAYOUT, int DT>
constexpr KernelEntry phases_entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, false, true,
                     &gemm_kernel<T, LAYOUT, DT, kPhases>, nullptr, nullptr, nullptr, T::NT,
                     T::NSB, false, true, 64 * T::NW};
}
template <int DT>
constexpr KernelEntry pp_timed_entry(const char *name, int group_m) {
  return KernelEntry{name, kTN, DT, PpCfg::BM, PpCfg::BN, PpCfg::BK, PpCfg::LDS, group_m, false,
                     true, &gemm_pp_kernel<DT, true>, nullptr, nullptr, nullptr, PpCfg::NT,
                     PpCfg::NSB, false, true};
}
// the register-staged baseline assumes packed TN/NN operands, alpha 1, beta 0
template <class T, int LAYOUT, int DT>
constexpr KernelEntry rs_entry(const char *name, int group_m) {
  return KernelEntry{name, LAYOUT, DT, T::BM, T::BN, T::BK, T::LDS, group_m, false, false,
                     &regstage_kernel<T, LAYOUT, DT>, nullptr, nullptr, nullptr};
}

using T256 = TileCfg<256, 256>;
using T128 = TileCfg<128, 128>;
using T64 = TileCfg<64, 64>;
using T128x256 = TileCfg<128, 256>;
using W128x256 = WsCfg<128, 256>;
using T256W2x4 = TileCfg<256, 256, kLdsXor, 1, 2, 4>;  // eight waves, two per SIMD
using T128R3 = TileCfg<128, 128, kLdsXor, 1, 2, 2, 3>;  // 4 A + 3 B stages, 112 KiB
// loads spread over the step: 4 A + 4 B stages (128 KiB), 5 A + 5 B (160 KiB)
using T128S4 = TileCfg<128, 128, kLdsXor, 1, 2, 2, 4, 1>;
using T128S5 = TileCfg<128, 128, kLdsXor, 1, 2, 2, 5, 1>;
using T256x128 = TileCfg<256, 128>;  // 3 A + 2 B stages, 128 KiB
using T192x256 = TileCfg<192, 256>;  // 3 A + 2 B stages, 136 KiB
using T64R4 = TileCfg<64, 64, kLdsXor, 1, 2, 2, 4>;  // 5 A + 4 B stages, 72 KiB
using T256x192 = TileCfg<256, 192>;  // 3 A + 2 B stages, 144 KiB
using T192x192 = TileCfg<192, 192>;  // 3 A + 2 B stages, 120 KiB
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
    // wave specialisation: 4 loader + 4 MFMA waves on a 128 x 256 tile, and the
    // single-role pipeline on the same tile for comparison
    ws_entry<W128x256, kF16>("ws_tn_f16_128x256x64", 4),
    ws_entry<W128x256, kBF16>("ws_tn_bf16_128x256x64", 4),
    entry<T128x256, kTN, kF16>("tn_f16_128x256x64", 4, false),
    entry<T128x256, kTN, kBF16>("tn_bf16_128x256x64", 4, false),
    // the 256 x 256 tile on eight waves (two per SIMD)
    entry<T256W2x4, kTN, kF16>("tn_f16_256x256x64_w2x4", 4, false),
    entry<T256W2x4, kTN, kBF16>("tn_bf16_256x256x64_w2x4", 4, false),
    // the 128 x 128 tile with a deeper LDS ring, for a single round of tiles
    dp_entry<T128R3, kTN, kF16>("tn_f16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kTN, kBF16>("tn_bf16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kNN, kF16>("nn_f16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kNN, kBF16>("nn_bf16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kAtTN, kF16>("at_tn_f16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kAtTN, kBF16>("at_tn_bf16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kAtNN, kF16>("at_nn_f16_128x128x64_r3", 4, true),
    dp_entry<T128R3, kAtNN, kBF16>("at_nn_bf16_128x128x64_r3", 4, true),
    // the 256 x 256 kernel as a persistent launch
    persistent_entry<T256, kTN, kF16>("tn_f16_256x256x64_persist", 4, false),
    persistent_entry<T256, kTN, kBF16>("tn_bf16_256x256x64_persist", 4, false),
    persistent_entry<T256, kNN, kBF16>("nn_bf16_256x256x64_persist", 4, false),
    // the 256 x 256 tile on eight waves in two alternating groups (memory phase /
    // MFMA phase), TN
    pp_entry<kF16>("tn_f16_256x256x64_pp", 4),
    pp_entry<kBF16>("tn_bf16_256x256x64_pp", 4),
    // production kernels with per-workgroup clock counters (measurement copies)
    timed_entry<T256, kTN, kF16>("tn_f16_256x256x64_clk", 4),
    timed_entry<T256, kNN, kBF16>("nn_bf16_256x256x64_clk", 4),
    timed_entry<T128R3, kTN, kF16>("tn_f16_128x128x64_r3_clk", 4),
    timed_entry<T64, kTN, kF16>("tn_f16_64x64x64_clk", 4),
    pp_timed_entry<kF16>("tn_f16_256x256x64_pp_clk", 4),
    pp_timed_entry<kBF16>("tn_bf16_256x256x64_pp_clk", 4),
    // production kernels with main-loop phase clocks (measurement copies)
    phases_entry<T256, kTN, kF16>("tn_f16_256x256x64_ph", 4),
    phases_entry<T256, kNN, kBF16>("nn_bf16_256x256x64_ph", 4),
    phases_entry<T128R3, kTN, kF16>("tn_f16_128x128x64_r3_ph", 4),
    // the 128 x 128 tile on eight waves in two groups that split K (TN)
    ppk_entry<kF16>("tn_f16_128x128x64_ppk", 4),
    ppk_entry<kBF16>("tn_bf16_128x128x64_ppk", 4),
    // the 128 x 128 tile with its loads spread evenly over the step's MFMAs
    // before the barrier (A and B rings of equal depth): measured level with
    // the deeper-ring kernel, an ablation
    dp_entry<T128S4, kTN, kF16>("tn_f16_128x128x64_s4", 4, false),
    dp_entry<T128S4, kNN, kBF16>("nn_bf16_128x128x64_s4", 4, false),
    dp_entry<T128S5, kTN, kF16>("tn_f16_128x128x64_s5", 4, false),
    // 256 x 128 tiles: one round where 128 x 128 tiles would need two
    dp_entry<T256x128, kTN, kF16>("tn_f16_256x128x64", 4, true),
    dp_entry<T256x128, kTN, kBF16>("tn_bf16_256x128x64", 4, true),
    dp_entry<T256x128, kNN, kF16>("nn_f16_256x128x64", 4, true),
    dp_entry<T256x128, kNN, kBF16>("nn_bf16_256x128x64", 4, true),
    dp_entry<T256x128, kAtTN, kF16>("at_tn_f16_256x128x64", 4, true),
    dp_entry<T256x128, kAtTN, kBF16>("at_tn_bf16_256x128x64", 4, true),
    dp_entry<T256x128, kAtNN, kF16>("at_nn_f16_256x128x64", 4, true),
    dp_entry<T256x128, kAtNN, kBF16>("at_nn_bf16_256x128x64", 4, true),
    // 192 x 256 tiles (the transposed-A forms further down)
    dp_entry<T192x256, kTN, kF16>("tn_f16_192x256x64", 4, true),
    dp_entry<T192x256, kTN, kBF16>("tn_bf16_192x256x64", 4, true),
    dp_entry<T192x256, kNN, kF16>("nn_f16_192x256x64", 4, true),
    dp_entry<T192x256, kNN, kBF16>("nn_bf16_192x256x64", 4, true),
    // the 64 x 64 tile with a deeper LDS ring, for a single round of tiles
    // whose operands do not stay in the L2
    dp_entry<T64R4, kTN, kF16>("tn_f16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kTN, kBF16>("tn_bf16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kNN, kF16>("nn_f16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kNN, kBF16>("nn_bf16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kAtTN, kF16>("at_tn_f16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kAtTN, kBF16>("at_tn_bf16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kAtNN, kF16>("at_nn_f16_64x64x64_r4", 4, true),
    dp_entry<T64R4, kAtNN, kBF16>("at_nn_bf16_64x64x64_r4", 4, true),
    // 256 x 192 and 192 x 192 tiles
    dp_entry<T256x192, kTN, kF16>("tn_f16_256x192x64", 4, true),
    dp_entry<T256x192, kTN, kBF16>("tn_bf16_256x192x64", 4, true),
    dp_entry<T256x192, kAtTN, kF16>("at_tn_f16_256x192x64", 4, true),
    dp_entry<T256x192, kAtTN, kBF16>("at_tn_bf16_256x192x64", 4, true),
    dp_entry<T192x192, kTN, kF16>("tn_f16_192x192x64", 4, true),
    dp_entry<T192x192, kTN, kBF16>("tn_bf16_192x192x64", 4, true),
    // 192-wide m/n-contiguous operand tiles: 384-byte k-rows laid end to end
    // over the 1 KiB load segments
    dp_entry<T256x192, kNN, kF16>("nn_f16_256x192x64", 4, true),
    dp_entry<T256x192, kNN, kBF16>("nn_bf16_256x192x64", 4, true),
    dp_entry<T192x192, kNN, kF16>("nn_f16_192x192x64", 4, true),
    dp_entry<T192x192, kNN, kBF16>("nn_bf16_192x192x64", 4, true),
    dp_entry<T192x256, kAtTN, kF16>("at_tn_f16_192x256x64", 4, true),
    dp_entry<T192x256, kAtTN, kBF16>("at_tn_bf16_192x256x64", 4, true),
    dp_entry<T192x192, kAtTN, kF16>("at_tn_f16_192x192x64", 4, true),
    dp_entry<T192x192, kAtTN, kBF16>("at_tn_bf16_192x192x64", 4, true),
    dp_entry<T192x256, kAtNN, kF16>("at_nn_f16_192x256x64", 4, true),
    dp_entry<T192x256, kAtNN, kBF16>("at_nn_bf16_192x256x64", 4, true),
    dp_entry<T256x192, kAtNN, kF16>("at_nn_f16_256x192x64", 4, true),
    dp_entry<T256x192, kAtNN, kBF16>("at_nn_bf16_256x192x64", 4, true),
    dp_entry<T192x192, kAtNN, kF16>("at_nn_f16_192x192x64", 4, true),
    dp_entry<T192x192, kAtNN, kBF16>("at_nn_bf16_192x192x64", 4, true),
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

int find_kernel(int layout, int dtype, int bm, int bn, int nsb = 2) {
  for (int i = 0; i < kTableSize; ++i)
    if (kTable[i].production && kTable[i].layout == layout && kTable[i].dtype == dtype &&
        kTable[i].bm == bm && kTable[i].bn == bn && kTable[i].nsb == nsb)
      return i;
  return -1;
}

// Cost model of the automatic choice, in units of one K step of a 256 x 256
// tile on every CU at once (about 1.3 us on MI355X).  A launch of BM x BN
// tiles runs ceil(tiles / 256 CUs) rounds, each tile taking
// (KT + kTileFixed) * (BM*BN / 256^2) / rate units, rate the per-CU
// throughput of that tile relative to the 256 x 256 kernel.  The 128 x 128
// and 64 x 64 kernels have two rates each: one workgroup per CU (a single
// round), and several sharing a CU when there are more tiles than CUs (two of
// 128 x 128, four of 64 x 64, as their LDS allows), which also share the
// fixed cost.  The other tiles take one workgroup per CU.  Tiles 192 or 128
// wide fill the CUs where square tiles leave a partial round: 256 x 128
// covers in one round what takes the 128 tile two (1024 x 8192 x 8192: 1327
// against 1196 TFLOPS), and 192 x 256, 256 x 192 and 192 x 192 fill rounds
// that 256 x 256 tiles leave part empty (3072^3: 256 tiles of 192 x 192
// against 144 of 256 x 256, 21 % faster).  The rates were fitted on measured
// times of every production kernel over four sets of 133 shapes (square,
// skinny, long-K, 60 drawn at random, and single rounds of 64 x 64 tiles; TN
// f16 and NN bf16): the choice is 0.36 % behind the fastest kernel on
// average, 124 of 133 within 2 %.  Each rate sits inside a range that gives
// the same choices (192 x 256: 0.78-0.82; 192 x 192: 0.64-0.72; 256 x 128:
// 0.66-0.82).  With single-round rates where CUs are shared, the choice took
// the 128 tile where the 256 tile was 14-24 % faster (3072^3,
// 6000 x 6000 x 3000).  Where workgroups share a CU they overlap each other's
// prologue and epilogue: four 64 x 64 tiles share the fixed cost (rate 0.37,
// measured at 0.25-0.45); for two 128 x 128 tiles the time per round was
// refitted on eight sets (298 shapes, two of 60 random ones measured after
// the other constants were set) as (KT - 1) steps at rate 0.56: of 298
// choices six change, all to faster kernels (4-18 %; NN 1152 x 7168 x 9664
// now takes one round of 192 x 192 tiles, 4096 x 4096 x 256 the 128 tile),
// and in leave-one-set-out fits the choice is 0.43 % behind the fastest kernel
// on average against 0.55 % before, worst 10 % against 18 %.
constexpr int64_t kCUs = 256;
constexpr double kTileFixed = 3.0;        // prologue and epilogue of a tile, in K steps
struct TileCand {
  int bm, bn;
  double rate;          // sustained rate relative to the 256 x 256 tile
  double rate_shared;   // ... with more tiles than CUs
  double fixed_shared;  // fixed K steps of a tile then (workgroups sharing a CU overlap theirs)
};
// in order of preference on equal estimates
const TileCand kCand[7] = {{256, 256, 1.0, 1.0, kTileFixed},   {192, 256, 0.80, 0.80, kTileFixed},
                           {256, 192, 0.83, 0.83, kTileFixed}, {192, 192, 0.68, 0.68, kTileFixed},
                           {256, 128, 0.76, 0.76, kTileFixed}, {128, 128, 0.8, 0.56, -1.0},
                           {64, 64, 0.5, 0.37, kTileFixed / 4}};
constexpr int kNumCand = 7;
constexpr double kSplitFixed = 6.9;       // the fixup launch and the wait for it
constexpr double kSlotCost = 0.055;       // one 256 KiB partial sum written and read back
constexpr int kMaxAutoSplit = 64;
// The split runs only where its estimate is below kSplitMargin times the best
// unsplit one.  On the 32 shapes of three sweeps (49 tuning and check shapes,
// 60 drawn at random) where a workspace allows it, every split estimated
// below 0.86 of the unsplit tiles measured faster (3-36 %; 6x for
// 512 x 512 x 65536), while those estimated at 0.86-0.97 ranged from 13 %
// slower to 8 % faster, half of them slower: the estimate leaves out costs
// that the 192 x 256 and 256 x 128 tiles do not have.
constexpr double kSplitMargin = 0.86;
constexpr int64_t kMaxSlots = 1024;       // 256 MiB of partial sums at most

int64_t tile_count(const TileCand &c, int64_t M, int64_t N) {
  return ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
}

// Workgroups that share a CU overlap each other's prologue and epilogue, so
// there the fixed cost of a tile is smaller (for the 64 x 64 tile a quarter:
// on the measured sweeps this moves one choice of 133, TN 1152 x 1664 x 1472,
// from the 128 x 128 tile to the 14 % faster 64 x 64 one).  A tile costs at
// least one step.
double dp_cost(int i, int64_t M, int64_t N, int64_t KT) {
  const TileCand &c = kCand[i];
  const int64_t tiles = tile_count(c, M, N);
  const bool shared = tiles > kCUs;
  const double rate = shared ? c.rate_shared : c.rate;
  const double steps = std::max((double)KT + (shared ? c.fixed_shared : kTileFixed), 1.0);
  return (double)((tiles + kCUs - 1) / kCUs) * steps * (double)(c.bm * c.bn) / 65536.0 / rate;
}

// Automatic choice without a K split: the tile with the least estimated
// time; ties go to the earlier candidate.  A single round of 128 x 128 tiles
// over at least kDeepRingSteps K steps takes the ring with one more stage per
// operand: one workgroup per CU either way, and the deeper prefetch hides the
// load latency (measured 3-17 % faster there).  With more than one round two
// workgroups share a CU, which the deeper ring's LDS would forbid.
constexpr int64_t kDeepRingSteps = 24;
// A single round of 64 x 64 tiles takes the ring with 5 A + 4 B stages once A
// and B together pass kDeepRing64Bytes: the default ring loads two steps
// ahead, which at this tile's short steps (8 MFMAs a wave) no longer covers
// the load latency once the operands stop staying in the L2.  Measured on 24
// single-round TN shapes (512^2 to 1024^2, K 1024 to 16384): 1.5-1.8x faster
// on all 16 whose A and B pass 7 MiB, 1-4 % slower on the 8 that stay at or
// under 8 MiB (two of them, at 8 MiB, on the wrong side of the threshold).
constexpr int64_t kDeepRing64Bytes = int64_t(6) << 20;
// Candidates without a kernel for the layout and dtype are skipped.
bool has_cand(int i, int layout, int dtype) {
  return find_kernel(layout, dtype, kCand[i].bm, kCand[i].bn) >= 0;
}
int auto_kernel(int layout, int dtype, int64_t M, int64_t N, int64_t K) {
  const int64_t KT = K > 0 ? (K + 63) / 64 : 1;
  int best = 0;
  for (int i = 1; i < kNumCand; ++i)
    if (has_cand(i, layout, dtype) && dp_cost(i, M, N, KT) < dp_cost(best, M, N, KT)) best = i;
  const TileCand &c = kCand[best];
  if (c.bm == 128 && c.bn == 128 && tile_count(c, M, N) <= kCUs && KT >= kDeepRingSteps)
    return find_kernel(layout, dtype, 128, 128, 3);
  if (c.bm == 64 && c.bn == 64 && tile_count(c, M, N) <= kCUs && 2 * (M + N) * K > kDeepRing64Bytes)
    return find_kernel(layout, dtype, 64, 64, 4);
  return find_kernel(layout, dtype, c.bm, c.bn);
}

// K split of the last, partial round of 256 x 256 tiles (the tail): the
// tiles that do not fill a round of the 256 CUs are each cut into S K
// segments run side by side, whose FP32 partial sums (BM*BN*4 bytes a
// segment) a second kernel adds in order.
struct Plan {
  int kidx = -1;
  int split = 0;         // 0: no split
  int64_t dp_tiles = 0;  // tiles of the whole rounds, computed without a split
  int64_t sk_tiles = 0;  // tail tiles, each split into `split` segments
  size_t ws_bytes = 0;
  double cost = 0.0;
};

double split_cost(int64_t full_rounds, int64_t tail, int64_t KT, int64_t S) {
  const int64_t waves = (tail * S + kCUs - 1) / kCUs;
  return (double)full_rounds * ((double)KT + kTileFixed) +
         (double)waves * ((double)((KT + S - 1) / S) + kTileFixed) + kSplitFixed +
         kSlotCost * (double)(tail * S);
}

// split > 0: that many segments; split == 0: the number with the least
// estimated time.  No plan (split 0) when there is no tail or too few K steps.
Plan split_plan(int layout, int dtype, int64_t M, int64_t N, int64_t K, int split) {
  Plan p;
  const int64_t KT = (K + 63) / 64;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t tail = tiles % kCUs, full = tiles / kCUs;
  if (tail == 0 || KT < 2) return p;
  int64_t S = split;
  if (split <= 0) {
    S = 0;
    double best = 0.0;
    for (int64_t s = 2; s <= std::min<int64_t>(KT, kMaxAutoSplit) && tail * s <= kMaxSlots; ++s) {
      const double c = split_cost(full, tail, KT, s);
      if (S == 0 || c < best) S = s, best = c;
    }
  }
  if (S < 2 || S > KT || tail * S > (int64_t(1) << 20)) return p;
  p.kidx = find_kernel(layout, dtype, 256, 256);
  p.split = (int)S;
  p.sk_tiles = tail;
  p.dp_tiles = tiles - tail;
  p.ws_bytes = (size_t)tail * (size_t)S * 256 * 256 * 4;
  p.cost = split_cost(full, tail, KT, S);
  return p;
}

// The plan of a call: the automatic tile choice, or the split schedule when a
// large enough workspace is given and it is estimated faster (or forced).
Plan choose(int layout, int dtype, int64_t M, int64_t N, int64_t K, int split, size_t ws_bytes) {
  Plan dp;
  dp.kidx = auto_kernel(layout, dtype, M, N, K);
  if (split < 0 || ws_bytes == 0) return dp;
  const Plan sk = split_plan(layout, dtype, M, N, K, split);
  if (sk.split == 0 || sk.ws_bytes > ws_bytes) return dp;
  if (split > 0) return sk;
  const int64_t KT = (K + 63) / 64;
  double best = dp_cost(0, M, N, KT);
  for (int i = 1; i < kNumCand; ++i)
    if (has_cand(i, layout, dtype)) best = std::min(best, dp_cost(i, M, N, KT));
  return sk.cost < kSplitMargin * best ? sk : dp;
}

struct Call {
  int layout;  // kTN, kNN, kAtTN, kAtNN
  int64_t M, N, K;
  int dtype;
  float alpha, beta;
  const void *A, *B;
  void *C;
  int64_t lda, ldb, ldc;
  void *ws = nullptr;  // workspace for a K split (none: no split)
  size_t ws_bytes = 0;
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

hgemm_status_t launch(kernel_fn fn, int64_t grid, const GemmArgs &a, void *stream, int threads) {
  // hipGetLastError() reports the last error of any earlier runtime call on
  // this thread too: clear it so that only the launch's own result is seen
  (void)hipGetLastError();
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3((unsigned)threads), 0, (hipStream_t)stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return HGEMM_ERR_HIP;
  }
  return HGEMM_OK;
}

hgemm_status_t run(const Call &c, void *stream, const hgemm_config_t *cfg) {
  hgemm_status_t st = validate(c);
  if (st != HGEMM_OK) return st;
  int kidx = -1, group_m = 0, xcd = 1, split = 0;
  if (cfg != nullptr) {
    if (cfg->split < -1 || cfg->split == 1 || cfg->group_m < 0 || cfg->xcd_remap < -1 ||
        cfg->xcd_remap > 1 || cfg->kernel < -1 || cfg->kernel >= kTableSize)
      return HGEMM_ERR_INVALID_ARG;
    kidx = cfg->kernel;
    group_m = cfg->group_m;
    if (cfg->xcd_remap >= 0) xcd = cfg->xcd_remap;
    split = cfg->split;
  }
  if (split > 0 && c.ws == nullptr) return HGEMM_ERR_INVALID_ARG;  // a split needs a workspace
  if (c.ws != nullptr && (reinterpret_cast<uintptr_t>(c.ws) & 15) != 0)
    return HGEMM_ERR_UNSUPPORTED;
  if (kidx >= 0 && (kTable[kidx].layout != c.layout || kTable[kidx].dtype != c.dtype))
    return HGEMM_ERR_INVALID_ARG;
  if (c.M == 0 || c.N == 0) return HGEMM_OK;
  Plan plan;
  if (kidx < 0) {
    plan = choose(c.layout, c.dtype, c.M, c.N, c.K, split, c.ws != nullptr ? c.ws_bytes : 0);
  } else {
    plan.kidx = kidx;
    if (split > 0) {
      if (kTable[kidx].bm != 256 || kTable[kidx].split_fn == nullptr) return HGEMM_ERR_UNSUPPORTED;
      plan = split_plan(c.layout, c.dtype, c.M, c.N, c.K, split);
      plan.kidx = kidx;
    }
  }
  if (split > 0 && (plan.split == 0 || plan.ws_bytes > c.ws_bytes))
    return HGEMM_ERR_UNSUPPORTED;  // no tail to split, or the workspace is too small
  if (plan.kidx < 0) return HGEMM_ERR_UNSUPPORTED;
  const KernelEntry &e = kTable[plan.kidx];
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
  a.tile_begin = 0;
  a.grid = (int)tiles;
  a.sk_split = 0;
  a.sk_tiles = 0;
  a.ws = nullptr;
  if (e.timed) {  // clock counters in the workspace, counter_bytes per workgroup
    if (c.ws == nullptr || c.ws_bytes < (size_t)tiles * e.counter_bytes)
      return HGEMM_ERR_UNSUPPORTED;
    a.ws = static_cast<float *>(c.ws);
  }
  if (plan.split == 0)
    return launch(e.fn, e.persistent ? std::min<int64_t>(tiles, kCUs) : tiles, a, stream,
                  e.threads);
  // the whole rounds' tiles and the tail's K segments in one launch (the
  // segments alone when there is no whole round), then the sums
  a.tile_begin = (int)plan.dp_tiles;
  a.sk_split = plan.split;
  a.sk_tiles = (int)plan.sk_tiles;
  a.ws = static_cast<float *>(c.ws);
  const int64_t nseg = plan.sk_tiles * plan.split;
  if (plan.dp_tiles > 0) {
    a.grid = (int)plan.dp_tiles;
    st = launch(e.mixed_fn, plan.dp_tiles + nseg, a, stream, e.threads);
  } else {
    a.grid = (int)nseg;
    st = launch(e.split_fn, nseg, a, stream, e.threads);
  }
  if (st != HGEMM_OK) return st;
  a.grid = (int)plan.sk_tiles * fixup_parts(e.bm, e.bn);
  return launch(e.fixup, a.grid, a, stream, kFixupThreads);
}

// ---- the no-allocation variant of hgemm_gemm_ws ----------------------------
// The K split's FP32 partial sums go to this file-scope array instead of a
// caller workspace.  Each device that runs the library holds its own copy,
// kNoAllocScratchBytes, from the code object's load until the process ends.
// Its device address differs per device and is not the host-side name's
// address: it is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that pointer is handed to kernels.  No kernel
// expects it to start at zero (every partial sum is written before the fixup
// reads it), so calls never clear it; calls that overlap in time on one device
// share it and race.
constexpr size_t kNoAllocScratchBytes = HGEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
static_assert(kNoAllocScratchBytes % 256 == 0, "whole 256 KiB slots");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there); nullptr with the status in *st on failure.
void *scratch_on_current_device(hgemm_status_t *st) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    *st = HGEMM_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = HGEMM_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
      g_last_hip_error = (int)(err != hipSuccess ? err : hipErrorInvalidSymbol);
      *st = HGEMM_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
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

hgemm_status_t hgemm_tn(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype, const void *A,
                        const void *Bt, void *C, void *stream) {
  return run(packed(kTN, M, N, K, dtype, A, Bt, C), stream, nullptr);
}

hgemm_status_t hgemm_nn(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype, const void *A,
                        const void *B, void *C, void *stream) {
  return run(packed(kNN, M, N, K, dtype, A, B, C), stream, nullptr);
}

hgemm_status_t hgemm_tn_ex(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype, const void *A,
                           const void *Bt, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(packed(kTN, M, N, K, dtype, A, Bt, C), stream, cfg);
}

hgemm_status_t hgemm_nn_ex(int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype, const void *A,
                           const void *B, void *C, void *stream, const hgemm_config_t *cfg) {
  return run(packed(kNN, M, N, K, dtype, A, B, C), stream, cfg);
}

hgemm_status_t hgemm_gemm_ex(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                             float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                             float beta, void *C, int64_t ldc, void *stream,
                             const hgemm_config_t *cfg) {
  const int layout = layout_of(opA, opB);
  if (layout < 0) return HGEMM_ERR_INVALID_ARG;
  return run(Call{layout, M, N, K, dtype, alpha, beta, A, B, C, lda, ldb, ldc}, stream, cfg);
}

hgemm_status_t hgemm_gemm(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                          float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                          float beta, void *C, int64_t ldc, void *stream) {
  return hgemm_gemm_ex(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                       nullptr);
}

size_t hgemm_gemm_ws_size(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype) {
  const int layout = layout_of(opA, opB);
  if (layout < 0 || M <= 0 || N <= 0 || K <= 0 || (dtype != HGEMM_F16 && dtype != HGEMM_BF16))
    return 0;
  return choose(layout, dtype, M, N, K, 0, SIZE_MAX).ws_bytes;
}

hgemm_status_t hgemm_gemm_ws_ex(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                                float alpha, const void *A, int64_t lda, const void *B,
                                int64_t ldb, float beta, void *C, int64_t ldc, void *workspace,
                                size_t ws_bytes, void *stream, const hgemm_config_t *cfg) {
  const int layout = layout_of(opA, opB);
  if (layout < 0) return HGEMM_ERR_INVALID_ARG;
  Call c{layout, M, N, K, dtype, alpha, beta, A, B, C, lda, ldb, ldc};
  c.ws = workspace;
  c.ws_bytes = workspace != nullptr ? ws_bytes : 0;
  return run(c, stream, cfg);
}

hgemm_status_t hgemm_gemm_ws(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N, int64_t K, hgemm_dtype_t dtype,
                             float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                             float beta, void *C, int64_t ldc, void *workspace, size_t ws_bytes,
                             void *stream) {
  return hgemm_gemm_ws_ex(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc,
                          workspace, ws_bytes, stream, nullptr);
}

hgemm_status_t hgemm_gemm_noalloc(hgemm_op_t opA, hgemm_op_t opB, int64_t M, int64_t N,
                                  int64_t K, hgemm_dtype_t dtype, float alpha, const void *A,
                                  int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                                  int64_t ldc, void *stream) {
  const int layout = layout_of(opA, opB);
  if (layout < 0) return HGEMM_ERR_INVALID_ARG;
  Call c{layout, M, N, K, dtype, alpha, beta, A, B, C, lda, ldb, ldc};
  hgemm_status_t st = validate(c);
  if (st != HGEMM_OK || c.M == 0 || c.N == 0) return st;
  // the plan hgemm_gemm_ws would take with an unlimited workspace
  const size_t need = choose(layout, dtype, M, N, K, 0, SIZE_MAX).ws_bytes;
  if (need > kNoAllocScratchBytes) return HGEMM_ERR_SCRATCH;
  if (need > 0) {
    c.ws = scratch_on_current_device(&st);
    if (c.ws == nullptr) return st;
    c.ws_bytes = kNoAllocScratchBytes;
  }
  return run(c, stream, nullptr);
}

const char *hgemm_status_string(hgemm_status_t status) {
  switch ((int)status) {
    case HGEMM_OK: return "ok";
    case HGEMM_ERR_INVALID_ARG: return "invalid argument";
    case HGEMM_ERR_UNSUPPORTED: return "unsupported shape, alignment or config";
    case HGEMM_ERR_HIP: return "HIP runtime error";
    case HGEMM_ERR_SCRATCH:
      return "the K split would need more than the library's static scratch "
             "(HGEMM_NOALLOC_SCRATCH_BYTES); call hgemm_gemm_ws with a workspace";
    default: return "unknown status";
  }
}

int hgemm_last_hip_error(void) { return g_last_hip_error; }

const char *hgemm_version(void) { return "hgemm-gfx950 1.5"; }

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

int hgemm_auto_kernel(int layout, hgemm_dtype_t dtype, int64_t M, int64_t N, int64_t K) {
  if (layout < kTN || layout > kAtNN || (dtype != HGEMM_F16 && dtype != HGEMM_BF16) || M <= 0 ||
      N <= 0)
    return -1;
  return auto_kernel(layout, dtype, M, N, K);
}

}  // extern "C"
