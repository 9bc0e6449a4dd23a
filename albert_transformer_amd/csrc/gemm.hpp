// Token-row GEMM on the matrix cores with fused epilogues.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k] + b[n]      (weights [out, in], the
//   biased projection of contract A in "Qwen3-TTS and Kokoro: Two Routes
//   from Text to Speech")
//
// followed by one of:
//   EPI_BIAS  store Y
//   EPI_GELU  store gelu_tanh(Y)                    (FFN 768->2048)
//   EPI_LN    store LN(Y + R) * g + beta over the full row of N (output
//             projection + residual + LayerNorm, and FFN 2048->768 +
//             residual + LayerNorm: steps 5 and 6 of "Inside One Real ALBERT
//             Layer"); the block tile spans the whole row so the row
//             statistics never leave the chip
//   EPI_OUT   store Y as fp32 into the caller's output, packed row m going to
//             out row seq(m) * T + pos(m) (padded) or m (packed)
//
// Tiling: a block computes BM token rows x BN output features with WGM x WGN
// waves; each wave owns a (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA
// tiles.  Weights are the MFMA A operand and tokens the B operand, so each
// lane ends up owning one token and runs of 4 consecutive features: stores
// are 4-wide and LayerNorm row statistics reduce inside a lane, then across
// the two half-waves, then across the WGN waves through LDS.
// The K loop stages BK-wide slices of X and W in LDS (rows padded by 16
// bytes so that the fragment reads are bank-conflict free), double-buffered
// through registers: the next slice is fetched from global memory while the
// matrix cores work on the current one.
#pragma once

#include "common.hpp"

namespace albert {

enum Epi { EPI_BIAS = 0, EPI_GELU = 1, EPI_LN = 2, EPI_OUT = 3 };

struct GemmArgs {
  const void* X;       // [M, K] activations, row stride ldx (elements)
  int64_t ldx;
  const void* W;       // [N, K] weights, row stride K
  const float* bias;   // [N]
  void* Y;             // [M, N] output (EPI_BIAS / EPI_GELU / EPI_LN), stride ldy
  int64_t ldy;
  const void* R;       // [M, N] residual (EPI_LN), stride ldr
  int64_t ldr;
  const float* ln_g;   // [N] (EPI_LN)
  const float* ln_b;
  float eps;
  float* out;          // EPI_OUT: fp32 output rows of N
  const int* row_seq;  // EPI_OUT padded mapping
  const int* row_pos;
  int out_T;           // EPI_OUT: padded T, or 0 for packed rows
  const int* status;
  const int* m_ptr;    // device: number of valid rows M
  int N, K;
  int n_tiles;         // N / BN
};

template <typename T, int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_kernel(GemmArgs g) {
  typedef Tr<T> TR;
  constexpr int NT = WGM * WGN * 64;
  constexpr int BK = TR::BK;
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = BK / VEC;         // chunks per staged row
  constexpr int LDK = BK + VEC;         // padded LDS row (elements)
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int XCH = BM * CPR / NT;
  constexpr int WCH = BN * CPR / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "load split");
  static_assert(BK % 16 == 0, "BK");

  __shared__ __attribute__((aligned(16))) T lds[2 * (BM + BN) * LDK];

  if (*g.status != 0) return;
  const int M = *g.m_ptr;
  const int tile = blockIdx.x;
  const int tn = tile % g.n_tiles, tm = tile / g.n_tiles;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hh = lane >> 5;

  const T* __restrict__ X = static_cast<const T*>(g.X);
  const T* __restrict__ W = static_cast<const T*>(g.W);

  uint4 rx[XCH], rw[WCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      const int m = m0 + r;
      if (m < M)
        rx[i] = *reinterpret_cast<const uint4*>(X + (int64_t)m * g.ldx + k0 + cc * VEC);
      else
        rx[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      rw[i] = *reinterpret_cast<const uint4*>(W + (int64_t)(n0 + r) * g.K + k0 + cc * VEC);
    }
  };
  auto sstore = [&](int buf) {
    T* sx = lds + buf * (BM + BN) * LDK;
    T* sw = sx + BM * LDK;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      *reinterpret_cast<uint4*>(sx + r * LDK + cc * VEC) = rx[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      *reinterpret_cast<uint4*>(sw + r * LDK + cc * VEC) = rw[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const T* sx = lds + cur * (BM + BN) * LDK + (wm * WTM + l32) * LDK + hh * 8;
    const T* sw = lds + cur * (BM + BN) * LDK + BM * LDK + (wn * WTN + l32) * LDK + hh * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      typename TR::frag fx[TM], fw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fx[i] = TR::load(sx + i * 32 * LDK + kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) fw[j] = TR::load(sw + j * 32 * LDK + kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) TR::mma(acc[i][j], fw[j], fx[i]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4q+e] holds token m0 + wm*WTM + i*32 + l32 and feature
  // n0 + wn*WTN + j*32 + 8q + 4hh + e.
  if constexpr (EPI == EPI_LN) {
    static_assert(BN * 1 > 0, "");
    float* red = reinterpret_cast<float*>(lds);  // [WGN][BM], reused twice
    const int N = g.N;
    const T* __restrict__ R = static_cast<const T*>(g.R);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WTM + i * 32 + l32;
      const int mr = m < M ? m : M - 1;  // rows past M compute on a valid row, never stored
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * hh;
          const f32x4 rv = TR::load4f(R + (int64_t)mr * g.ldr + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[i][j][4 * q + e] + g.bias[n + e] + rv[e];
            acc[i][j][4 * q + e] = v;
            s += v;
          }
        }
      s += wave_xor(s, 32);
      if (hh == 0) red[wn * BM + wm * WTM + i * 32 + l32] = s;
    }
    __syncthreads();
    float mean[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WGN; ++w) s += red[w * BM + wm * WTM + i * 32 + l32];
      mean[i] = s * (1.0f / N);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = acc[i][j][r] - mean[i];
          s += d * d;
        }
      s += wave_xor(s, 32);
      if (hh == 0) red[wn * BM + wm * WTM + i * 32 + l32] = s;
    }
    __syncthreads();
    T* __restrict__ Y = static_cast<T*>(g.Y);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WGN; ++w) s += red[w * BM + wm * WTM + i * 32 + l32];
      const float rstd = 1.0f / sqrtf(s * (1.0f / N) + g.eps);
      const int m = m0 + wm * WTM + i * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * hh;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (acc[i][j][4 * q + e] - mean[i]) * rstd * g.ln_g[n + e] + g.ln_b[n + e];
          TR::store4(Y + (int64_t)m * g.ldy + n, o[0], o[1], o[2], o[3]);
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WTM + i * 32 + l32;
      if (m >= M) continue;
      int64_t orow = m;
      if constexpr (EPI == EPI_OUT) {
        if (g.out_T) orow = (int64_t)g.row_seq[m] * g.out_T + g.row_pos[m];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * hh;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[i][j][4 * q + e] + g.bias[n + e];
            if constexpr (EPI == EPI_GELU) o[e] = gelu_tanh(o[e]);
          }
          if constexpr (EPI == EPI_OUT) {
            *reinterpret_cast<f32x4*>(g.out + orow * g.N + n) = f32x4{o[0], o[1], o[2], o[3]};
          } else {
            TR::store4(static_cast<T*>(g.Y) + orow * g.ldy + n, o[0], o[1], o[2], o[3]);
          }
        }
    }
  }
}

}  // namespace albert
