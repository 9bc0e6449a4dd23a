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

template <typename T, int BM, int BN, int WGM, int WGN, int RB, int STAGES, int EPI>
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
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(IPW * (STAGES - 2) <= 63, "vmcnt range");

  // One LDS array per stage, so that alias analysis sees that the DMA into
  // one stage never touches the stage being read.
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds2[STAGES > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char lds3[STAGES > 3 ? STAGE : 16];

  if (*g.status != 0) return;
  const int M = *g.m_ptr;
  // XCD-aware tile order: consecutive workgroups are dealt round-robin to the
  // 8 XCDs, so renumber them so that each XCD works on a contiguous range of
  // tiles (row-major, features fastest): the blocks running together on one
  // XCD then share their X rows and weight columns in that XCD's L2.
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xq = nb / 8, xrem = nb % 8, xcd = bid % 8, xl = bid / 8;
  const int tile = xcd < xrem ? xcd * (xq + 1) + xl : xrem * (xq + 1) + (xcd - xrem) * xq + xl;
  const int tn = tile % g.n_tiles, tm = tile / g.n_tiles;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;

  // Per-feature epilogue vectors (bias; LayerNorm gain and shift) are staged
  // in LDS up front: their load latency hides behind the K loop, and the
  // epilogue then reads them without waiting on global memory (on gfx9 a
  // wait for a load also waits for every earlier store).
  constexpr int NVEC = EPI == EPI_LN ? 3 : 1;
  __shared__ float vecs[NVEC][BN];
  for (int c = threadIdx.x; c < BN; c += WGM * WGN * 64) {
    vecs[0][c] = g.bias[n0 + c];
    if constexpr (EPI == EPI_LN) {
      vecs[1 % NVEC][c] = g.ln_g[n0 + c];
      vecs[2 % NVEC][c] = g.ln_b[n0 + c];
    }
  }

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

  // One slice: fragments of k-step j+1 are read while the matrix cores
  // work on k-step j, and the scheduler is asked to alternate MFMAs with
  // LDS reads so the reads hide behind the 32-cycle MFMAs.
  auto compute = [&](const char* buf) __attribute__((always_inline)) {
    typename TR::frag fx[2][TM], fw[2][TN];
    auto ld = [&](int j, int b) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const char* p = buf + xrow + i * 32 * RB;
        fx[b][i] = TR::load2(reinterpret_cast<const T*>(p + coff[j][0]),
                             reinterpret_cast<const T*>(p + coff[j][FCH - 1]));
      }
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) {
        const char* p = buf + wrow + jj * 32 * RB;
        fw[b][jj] = TR::load2(reinterpret_cast<const T*>(p + coff[j][0]),
                              reinterpret_cast<const T*>(p + coff[j][FCH - 1]));
      }
    };
    ld(0, 0);
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      if (j + 1 < KSTEPS) ld(j + 1, (j + 1) & 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          TR::mma(acc[i][jj], fw[j & 1][jj], fx[j & 1][i]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // then one LDS read
        }
    }
  };

  // STAGES-deep pipeline: slices t+1 .. t+STAGES-2 stay in flight while
  // slice t is consumed.  Before the barrier of slice t each wave waits only
  // for its own DMA of slice t (later slices may still be in flight); the
  // barrier then makes every wave's part visible and frees the buffer
  // consumed at t-1, which receives slice t+STAGES-1.  The slice count is a
  // multiple of STAGES (checked by the host), so the main loop is
  // branch-free and the last STAGES slices are peeled with static waits.
  const int KT = g.K / BK;
#define ALBERT_BUF(i) ((i) == 0 ? lds0 : (i) == 1 ? lds1 : (i) == 2 ? lds2 : lds3)
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(ALBERT_BUF(s), s * BK);
  for (int kt = 0; kt < KT - STAGES; kt += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(IPW * (STAGES - 2)) : "memory");
      issue(ALBERT_BUF((s + STAGES - 1) % STAGES), (kt + s + STAGES - 1) * BK);
      compute(ALBERT_BUF(s));
    }
  }
  {
    const int kt = KT - STAGES;
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      // slices issued after slice kt+s: min(STAGES-2, STAGES-1-s)
      if constexpr (true) {
        if (s + 1 < STAGES - 1 || s == 0)
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(IPW * (STAGES - 2)) : "memory");
        else if (s == STAGES - 2)
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(IPW * (STAGES > 2 ? 1 : 0)) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
      if (s == 0) issue(ALBERT_BUF(STAGES - 1), (kt + STAGES - 1) * BK);
      compute(ALBERT_BUF(s));
    }
  }
#undef ALBERT_BUF

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4q+e] holds token m0 + wm*WTM + i*32 + l32 and feature
  // n0 + wn*WTN + j*32 + 8q + 4hh + e.  (The K loop's barriers ordered the
  // LDS vectors written above.)
  const float* __restrict__ bias_s = vecs[0];
  if constexpr (EPI == EPI_LN) {
    const float* __restrict__ g_s = vecs[1 % NVEC];
    const float* __restrict__ b_s = vecs[2 % NVEC];
    __syncthreads();  // every wave is done with the staging buffers
    float* red = reinterpret_cast<float*>(lds0);  // [WGN][BM]
    const int N = g.N;
    const T* __restrict__ R = static_cast<const T*>(g.R);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WTM + i * 32 + l32;
      const int mr = m < M ? m : M - 1;  // rows past M compute on a valid row, never stored
      const T* __restrict__ rrow = R + (int64_t)mr * g.ldr + n0 + wn * WTN + 4 * hh;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        f32x4 rv[4];  // this column group's residual loads first, then one wait
#pragma unroll
        for (int q = 0; q < 4; ++q) rv[q] = TR::load4f(rrow + j * 32 + 8 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[i][j][4 * q + e] + bias_s[nl + e] + rv[q][e];
            acc[i][j][4 * q + e] = v;
            s += v;
          }
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
          const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (acc[i][j][4 * q + e] - mean[i]) * rstd * g_s[nl + e] + b_s[nl + e];
          TR::store4(Y + (int64_t)m * g.ldy + n0 + nl, o[0], o[1], o[2], o[3]);
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
          const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[i][j][4 * q + e] + bias_s[nl + e];
            if constexpr (EPI == EPI_GELU) o[e] = gelu_tanh(o[e]);
          }
          if constexpr (EPI == EPI_OUT) {
            *reinterpret_cast<f32x4*>(g.out + orow * g.N + n0 + nl) = f32x4{o[0], o[1], o[2], o[3]};
          } else {
            TR::store4(static_cast<T*>(g.Y) + orow * g.ldy + n0 + nl, o[0], o[1], o[2], o[3]);
          }
        }
    }
  }
}

}  // namespace albert
