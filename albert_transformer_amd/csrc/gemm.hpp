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
// Tiling.  A block computes BM token rows x BN output features with WGM x WGN
// waves; each wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA tiles.
// Weights are the MFMA A operand and tokens the B operand, so each lane ends
// up owning one token and runs of 4 consecutive features: stores are 4-wide,
// and LayerNorm row statistics reduce inside a lane, then across the two
// half-waves, then across the WGN waves through LDS.
//
// Staging.  Each K slice of RB bytes per row (X rows then W rows) goes from
// global memory straight into LDS with gfx950's global_load_lds_dwordx4: one
// wave instruction fills 1 KB of LDS, 16 bytes per lane in lane order, with
// no register round trip.  Because the DMA fixes where each lane's 16 bytes
// land, bank conflicts of the fragment reads are avoided by choosing which
// 16-byte chunk each lane fetches: physical chunk p of row r holds logical
// chunk p ^ key(r), key(r) = (r / (256/RB)) % (RB/16), so the 8 rows read
// by 8 consecutive lanes fall on distinct banks.  Two LDS buffers alternate
// (the loop is unrolled by two so each half names its buffers statically):
// while the matrix cores consume one slice, the DMA fills the other.
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

typedef __attribute__((address_space(3))) void lds_ptr_t;

// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format, no swizzle, out-of-range reads return zero.
constexpr int kRsrcWord3 = 0x00020000;

template <int RB>
__device__ __forceinline__ int swz_key(int row) {
  return (row / (256 / RB)) % (RB / 16);
}

template <typename T, int BM, int BN, int WGM, int WGN, int RB, int EPI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_kernel(GemmArgs g) {
  typedef Tr<T> TR;
  constexpr int NW = WGM * WGN;
  constexpr int CH = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = RB / 16;                // chunks per staged row
  constexpr int BK = RB / sizeof(T);          // K elements per slice
  constexpr int RPI = 1024 / RB;              // rows one DMA instruction fills
  constexpr int NINST = (BM + BN) / RPI;      // DMA instructions per slice
  constexpr int IPW = NINST / NW;             // ... per wave
  constexpr int STAGE = (BM + BN) * RB;       // bytes per slice
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KSTEPS = BK / 16;             // MFMA k-steps per slice
  constexpr int FCH = 8 / CH;                 // chunks per fragment (1 bf16, 2 fp32)
  static_assert(NINST % NW == 0, "DMA split");
  static_assert((BM / RPI) % NW == 0, "each DMA slot must be all-X or all-W");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(RB == 64 || RB == 128, "row bytes");

  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];

  if (*g.status != 0) return;
  const int M = *g.m_ptr;
  const int tile = blockIdx.x;
  const int tn = tile % g.n_tiles, tm = tile / g.n_tiles;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hh = lane >> 5;

  const char* Xt = static_cast<const char*>(g.X) + (int64_t)m0 * g.ldx * (int64_t)sizeof(T);
  const char* Wt = static_cast<const char*>(g.W) + (int64_t)n0 * g.K * (int64_t)sizeof(T);
  // Buffer resources over the tile's rows: the hardware range check turns
  // reads of X rows at or past M into zeros (their results are never stored).
  const int64_t xbytes = (int64_t)(M - m0) * g.ldx * (int64_t)sizeof(T);
  const int64_t wbytes = (int64_t)(g.N - n0) * g.K * (int64_t)sizeof(T);
  const int xrec = __builtin_amdgcn_readfirstlane((int)(xbytes > 0x7fffffff ? 0x7fffffff : xbytes));
  const int wrec = __builtin_amdgcn_readfirstlane((int)(wbytes > 0x7fffffff ? 0x7fffffff : wbytes));
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Xt), (short)0, xrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Wt), (short)0, wrec, kRsrcWord3);

  // DMA sources.  Instruction i of this wave fills rows q*RPI .. q*RPI+RPI-1
  // of the slice, q = wave + i*NW (X rows first, then W rows); lane t takes
  // row q*RPI + t/CPR and logical chunk (t%CPR) ^ key(row).  For the tile
  // shapes used here the key does not depend on i, so one 32-bit per-lane
  // byte offset (VGPR) plus a uniform per-instruction offset (SGPR) address
  // every load.
  static_assert(CPR == 8 ? (NW % 2 == 0) : true, "swizzle key must not depend on i");
  const int lrow = lane / CPR;
  const int lchunk = (lane % CPR) ^ swz_key<RB>(wave * RPI + lrow);
  const int xoff = lrow * (int)g.ldx * (int)sizeof(T) + lchunk * 16;
  const int woff = lrow * g.K * (int)sizeof(T) + lchunk * 16;
  const int xrow_b = (int)g.ldx * (int)sizeof(T);  // bytes per X row
  const int wrow_b = g.K * (int)sizeof(T);
  auto issue = [&](char* buf, int k0) __attribute__((always_inline)) {
    const int kb = k0 * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave + i * NW;
      char* dst = buf + q * RPI * RB;
      if (i * NW * RPI < BM)  // compile-time per i (static_assert above)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t*)dst, 16, xoff,
                                                 kb + q * RPI * xrow_b, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t*)dst, 16, woff,
                                                 kb + (q * RPI - BM) * wrow_b, 0, 0);
    }
  };

  // Fragment read offsets: row part and swizzled chunk part per k-step.
  const int key = swz_key<RB>(l32);
  const int xrow = (wm * WTM + l32) * RB;
  const int wrow = (BM + wn * WTN + l32) * RB;
  int coff[KSTEPS][FCH];
#pragma unroll
  for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
    for (int f = 0; f < FCH; ++f) coff[j][f] = (((j * 16 + hh * 8) / CH + f) ^ key) * 16;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      typename TR::frag fx[TM], fw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const char* p = buf + xrow + i * 32 * RB;
        fx[i] = TR::load2(reinterpret_cast<const T*>(p + coff[j][0]),
                          reinterpret_cast<const T*>(p + coff[j][FCH - 1]));
      }
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) {
        const char* p = buf + wrow + jj * 32 * RB;
        fw[jj] = TR::load2(reinterpret_cast<const T*>(p + coff[j][0]),
                           reinterpret_cast<const T*>(p + coff[j][FCH - 1]));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) TR::mma(acc[i][jj], fw[jj], fx[i]);
    }
  };

  const int KT = g.K / BK;  // even: the host checks K % (2*BK) == 0
  issue(lds0, 0);
  for (int kt = 0; kt < KT; kt += 2) {
    __syncthreads();  // slice kt is in lds0 everywhere; lds1 is free
    issue(lds1, (kt + 1) * BK);
    compute(lds0);
    __syncthreads();  // slice kt+1 is in lds1 everywhere; lds0 is free
    if (kt + 2 < KT) issue(lds0, (kt + 2) * BK);
    compute(lds1);
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4q+e] holds token m0 + wm*WTM + i*32 + l32 and feature
  // n0 + wn*WTN + j*32 + 8q + 4hh + e.
  if constexpr (EPI == EPI_LN) {
    __syncthreads();  // every wave is done with the staging buffers
    float* red = reinterpret_cast<float*>(lds0);  // [WGN][BM]
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
          const f32x4 bv = *reinterpret_cast<const f32x4*>(g.bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[i][j][4 * q + e] + bv[e] + rv[e];
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
          const f32x4 gv = *reinterpret_cast<const f32x4*>(g.ln_g + n);
          const f32x4 bv = *reinterpret_cast<const f32x4*>(g.ln_b + n);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (acc[i][j][4 * q + e] - mean[i]) * rstd * gv[e] + bv[e];
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
          const f32x4 bv = *reinterpret_cast<const f32x4*>(g.bias + n);
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[i][j][4 * q + e] + bv[e];
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
