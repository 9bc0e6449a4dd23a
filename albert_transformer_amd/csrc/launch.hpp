// Host-side launch helpers for the GEMM kernel, shared by the encoder and
// the text path.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "gemm.hpp"
#include "host.hpp"
#include "splitk.hpp"

namespace albert {

// Kernel timing without marker packets.  A caller that wants one launch
// timed arms a pair of events here; the next launch_kernel() hands them to
// hipExtLaunchKernel, which stamps them from that kernel's own dispatch,
// so a timed kernel is not separated from its neighbours by extra gaps.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline thread_local LaunchEvents g_launch_events;

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                          Args... args) {
  const LaunchEvents ev = g_launch_events;
  g_launch_events = LaunchEvents{};
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
}

// Persistent launch: one block per CU at most (a multiple of 8, so that the
// kernel's XCD-aware tile numbering is a bijection), each walking its tiles.
template <typename T, bool F8, int BM, int BN, int WGM, int WGN, int RB, int STAGES, int EPI,
          bool DEFER, int KR = 0>
void launch_gemm(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  g.n_tiles = g.N / BN;
  const int64_t tiles = (max_rows + BM - 1) / BM * g.n_tiles;
  const int64_t grid = std::min<int64_t>((tiles + 7) / 8 * 8, grid_cap);
  launch_kernel(gemm_kernel<T, F8, BM, BN, WGM, WGN, RB, STAGES, EPI, DEFER, KR>,
                dim3((unsigned)grid), dim3(WGM * WGN * 64), s, g);
}

// Split-K product for very small batches (split_factor() > 0): S partial
// products over 64 x 256 tiles of 4 waves (one per SIMD), walked by at most
// grid_cap workgroups, then the reduce kernel with the product's epilogue.
// A caller timing the launch gets the start of the first kernel and the end
// of the second.
template <typename T, bool F8, int EPI>
void launch_split(GemmArgs g, SplitArgs r, int S, int64_t max_rows, int grid_cap, hipStream_t s) {
  constexpr int RB = F8 ? 64 : 128;
  g.ksplit = S;
  g.ldp = max_rows;
  g.n_tiles = g.N / 256;
  r.part = g.part;
  r.S = S;
  r.ldp = max_rows;
  r.N = g.N;
  const int64_t tiles = (max_rows + 63) / 64 * g.n_tiles * S;
  const int64_t grid = std::min<int64_t>((tiles + 7) / 8 * 8, grid_cap);
  const LaunchEvents ev = g_launch_events;
  g_launch_events = LaunchEvents{};
  hipExtLaunchKernelGGL(gemm_kernel<T, F8, 64, 256, 1, 4, RB, 2, EPI_PART, false>, dim3((unsigned)grid),
                        dim3(256), 0, s, ev.start, nullptr, 0, g);
  hipExtLaunchKernelGGL(splitk_reduce_kernel<T, F8, EPI>, dim3((unsigned)max_rows), dim3(256), 0, s,
                        nullptr, ev.stop, 0, r);
}
// K slices of the split-K tile for a product of depth K
template <typename T, bool F8>
constexpr int split_slices(int K) {
  return F8 ? K / 64 : K * (int)sizeof(T) / 128;
}

// Large tiles for plain and GELU epilogues; full-row tiles for LayerNorm.
// bf16 tiles use 8 waves (two per SIMD, so one wave's LDS waits hide
// behind the other's matrix-core work): the bias GEMMs with at least 12
// (an even number of) K slices as 2 x 4 waves keeping each tile's outputs
// in registers to store them during the next tile, the GELU GEMM, the
// short-K bias GEMM and the fp32 output projections as 4 x 2 waves storing
// directly (the faster pair on the encoder's shapes).  E4M3
// operands stage 64-byte rows (one 64-deep MFMA step per slice); their
// bias/GELU GEMMs run as 4 x 2 waves with deferred stores.
template <typename T, bool F8, int EPI>
void gemm_big(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  constexpr bool bf = std::is_same<T, bf16>::value && !F8;
  constexpr int RB = F8 ? 64 : 128;
  const int slices = g.K * (F8 ? 1 : (int)sizeof(T)) / RB;
  if constexpr (bf && EPI == EPI_GELU) {
    launch_gemm<T, F8, 256, 256, 4, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  } else if constexpr (bf && EPI == EPI_BIAS) {
    if (slices >= 12 && slices % 2 == 0 && !g.Y8)
      launch_gemm<T, F8, 256, 256, 2, 4, RB, 2, EPI, true>(g, max_rows, grid_cap, s);
    else  // short K (the input projection): 4 x 2 waves, stored directly
      launch_gemm<T, F8, 256, 256, 4, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  } else if constexpr (F8 && (EPI == EPI_BIAS || EPI == EPI_GELU)) {
    if (slices >= 12 && slices % 2 == 0 && !g.Y8)
      launch_gemm<T, F8, 256, 256, 4, 2, RB, 2, EPI, true>(g, max_rows, grid_cap, s);
    else
      launch_gemm<T, F8, 256, 256, 2, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  } else if constexpr (bf && EPI == EPI_OUT) {  // output projections: 4 x 2 waves
    launch_gemm<T, F8, 256, 256, 4, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  } else {
    launch_gemm<T, F8, 256, 256, 2, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  }
}
// 128-row tiles need at least a full wave of them; smaller batches use
// 64-row tiles (4 waves, one per SIMD) to spread over more CUs.
// (E4M3 fragments are too wide for the 8-wave tile's register budget, so the
// low-precision variant always uses the 4-wave one.)
// The tile spans the whole row of N (768 for the encoder, 512 for the text
// path's convolutions).
// The text path's convolutions (bf16, EPI_LN_ACT, K = 2560) run the
// 128-row tile three stages deep (32-deep slices, the kernel instantiated
// per K slices mod 3): 10 % faster than two.
template <typename T, bool F8, int N, int EPI>
void gemm_ln_n(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  if constexpr (!F8) {
    if ((max_rows + 127) / 128 >= grid_cap) {
      if constexpr (EPI == EPI_LN_ACT && std::is_same<T, bf16>::value) {
        if (g.K % 32 == 0 && g.K / 32 >= 5) {
          const int kr = (g.K / 32) % 3;
          if (kr == 0)
            launch_gemm<T, F8, 128, N, 2, 4, 64, 3, EPI, false, 0>(g, max_rows, grid_cap, s);
          else if (kr == 1)
            launch_gemm<T, F8, 128, N, 2, 4, 64, 3, EPI, false, 1>(g, max_rows, grid_cap, s);
          else
            launch_gemm<T, F8, 128, N, 2, 4, 64, 3, EPI, false, 2>(g, max_rows, grid_cap, s);
          return;
        }
      }
      launch_gemm<T, F8, 128, N, 2, 4, 64, 2, EPI, false>(g, max_rows, grid_cap, s);
      return;
    }
  }
  launch_gemm<T, F8, 64, N, 1, 4, 64, 2, EPI, false>(g, max_rows, grid_cap, s);
}
template <typename T, bool F8>
void gemm_ln(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  gemm_ln_n<T, F8, 768, EPI_LN>(g, max_rows, grid_cap, s);
}

// LayerNorm over rows of 768 split between two blocks of 384 features
// (EPI_LN_PAIR, bf16 storage).  bf16 operands: 256-row tiles (4 x 2 waves
// of 64 x 192) when they fill the chip, else 128-row tiles (2 x 4 waves of
// 64 x 96), three stages of 32-deep K slices, the kernel instantiated per
// K slices mod 3.  E4M3 operands: 128-row tiles of 2 x 2 waves of 64 x 192
// (one wave per SIMD: each wave may hold 512 registers), two stages of
// 64-deep slices; with eight waves, or three stages, they spill.  At most
// grid_cap blocks rounded down to a multiple of 16, so that the two halves
// of a row tile normally run at the same time on one XCD (a half whose
// partner is late hands its rows over instead of waiting).  The caller
// clears g.xch before the first launch and gives each launch since then
// its own g.xtag.
template <int BM, int KR>
constexpr auto ln_pair_kernel =
    gemm_kernel<bf16, false, BM, 384, BM == 64 ? 1 : BM / 64, BM == 64 ? 4 : 8 / (BM / 64), 64, 3,
                EPI_LN_PAIR, false, KR>;
// threads of the bf16 pair kernel with BM-row tiles
constexpr unsigned ln_pair_threads(int BM) { return BM == 64 ? 256 : 512; }
constexpr auto ln_pair_kernel_f8 = gemm_kernel<bf16, true, 128, 384, 2, 2, 64, 2, EPI_LN_PAIR, false, 0>;
template <int BM>
inline const void* ln_pair_pick(int kr) {
  return kr == 0   ? reinterpret_cast<const void*>(ln_pair_kernel<BM, 0>)
         : kr == 1 ? reinterpret_cast<const void*>(ln_pair_kernel<BM, 1>)
                   : reinterpret_cast<const void*>(ln_pair_kernel<BM, 2>);
}
// Polls of the partner's row statistics before a half is handed over
// (each poll is a device-scope load plus a short sleep, about a
// microsecond: the halves of a tile normally finish within a few).
constexpr int kPairPolls = 64;
// Tile height: the tallest whose tiles (two per row tile) fill grid_cap
// CUs; 64-row tiles (4 waves of 64 x 96) below that: smaller batches spread
// over more CUs.
inline int ln_pair_rows(int64_t max_rows, int grid_cap, bool f8) {
  if (f8) return 128;
  if ((max_rows + 255) / 256 * 2 >= grid_cap) return 256;
  if ((max_rows + 127) / 128 * 2 >= grid_cap) return 128;
  return 64;
}
// K the pair kernels accept: bf16, whole 32-deep slices, at least 3 + 2 of
// them; E4M3, an even number of 64-deep slices
inline bool ln_pair_k_ok(int K, bool f8) {
  return f8 ? K % 128 == 0 && K > 0 : K % 32 == 0 && K / 32 >= 5;
}
template <bool F8>
inline hipError_t gemm_ln_pair(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  if (!ln_pair_k_ok(g.K, F8) || g.N != 768) return hipErrorInvalidValue;
  const int BM = ln_pair_rows(max_rows, grid_cap, F8);
  g.n_tiles = 2;
  const int64_t tiles = (max_rows + BM - 1) / BM * 2;
  const int64_t grid = std::min<int64_t>((tiles + 15) / 16 * 16, grid_cap / 16 * 16);
  const void* k = F8 ? reinterpret_cast<const void*>(ln_pair_kernel_f8)
                     : BM == 256 ? ln_pair_pick<256>((g.K / 32) % 3)
                     : BM == 128 ? ln_pair_pick<128>((g.K / 32) % 3) : ln_pair_pick<64>((g.K / 32) % 3);
  const unsigned threads = F8 ? 256 : ln_pair_threads(BM);
  const LaunchEvents ev = g_launch_events;
  g_launch_events = LaunchEvents{};
  void* args[] = {&g};
  const hipError_t e = hipExtLaunchKernel(k, dim3((unsigned)grid), dim3(threads), args, 0, s,
                                          ev.start, ev.stop, 0);
  return e;
}

}  // namespace albert
