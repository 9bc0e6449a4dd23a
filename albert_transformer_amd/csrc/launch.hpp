// Host-side launch helpers for the GEMM kernel, shared by the encoder and
// the text path.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "gemm.hpp"

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
          bool DEFER>
void launch_gemm(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  g.n_tiles = g.N / BN;
  const int64_t tiles = (max_rows + BM - 1) / BM * g.n_tiles;
  const int64_t grid = std::min<int64_t>((tiles + 7) / 8 * 8, grid_cap);
  launch_kernel(gemm_kernel<T, F8, BM, BN, WGM, WGN, RB, STAGES, EPI, DEFER>,
                dim3((unsigned)grid), dim3(WGM * WGN * 64), s, g);
}

// Large tiles for plain and GELU epilogues; full-row tiles for LayerNorm.
// bf16 tiles use 8 waves (two per SIMD, so one wave's LDS waits hide
// behind the other's matrix-core work): the bias GEMMs with at least 12
// (an even number of) K slices as 2 x 4 waves keeping each tile's outputs
// in registers to store them during the next tile, the GELU GEMM as 4 x 2
// waves storing directly (the faster pair on the encoder's shapes).  E4M3
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
    else
      launch_gemm<T, F8, 256, 256, 2, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
  } else if constexpr (F8 && (EPI == EPI_BIAS || EPI == EPI_GELU)) {
    if (slices >= 12 && slices % 2 == 0 && !g.Y8)
      launch_gemm<T, F8, 256, 256, 4, 2, RB, 2, EPI, true>(g, max_rows, grid_cap, s);
    else
      launch_gemm<T, F8, 256, 256, 2, 2, RB, 2, EPI, false>(g, max_rows, grid_cap, s);
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
template <typename T, bool F8, int N, int EPI>
void gemm_ln_n(GemmArgs g, int64_t max_rows, int grid_cap, hipStream_t s) {
  if constexpr (!F8) {
    if ((max_rows + 127) / 128 >= grid_cap) {
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

}  // namespace albert
