// Second half of a split-K product (EPI_PART in gemm.hpp): the S partial
// sums of each output row are added in order, the bias added, and the
// epilogue of the product applied -- the same epilogues as the one-pass
// products: store (EPI_BIAS), GELU (EPI_GELU), residual + LayerNorm over the
// row (EPI_LN, steps 5 and 6 of "Inside One Real ALBERT Layer"), or the fp32
// output rows (EPI_OUT).
//
// Used when a batch is so small that even 64-row tiles would occupy a few
// CUs (a single utterance has 36 rows): splitting K over S workgroups per
// tile spreads the products over the chip, and this pass costs a read of
// S x M x N fp32 values, a few hundred kilobytes there.  One workgroup per
// row, each thread over N / 256 columns; LayerNorm statistics are reduced in
// the workgroup in a fixed order, so the result does not depend on timing.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace albert {

struct SplitArgs {
  const float* part;   // [S][ldp][N] partial sums
  int S;
  int64_t ldp;
  int N;
  const float* bias;   // [N]
  void* Y;             // [M, N] (EPI_BIAS / EPI_GELU / EPI_LN), stride ldy
  int64_t ldy;
  void* Y8;            // E4M3 copy of Y (EPI_BIAS / EPI_LN), or null
  int64_t ldy8;
  const void* R;       // [M, N] residual (EPI_LN), stride ldr
  int64_t ldr;
  const float* ln_g;
  const float* ln_b;
  float eps;
  float* out;          // EPI_OUT: fp32 rows of N
  const int* row_seq;
  const int* row_pos;
  int out_T;
  const int* status;
  const int* m_ptr;
};

// T: storage type of Y and R; F8: E4M3 operands (an EPI_GELU output, whose
// one consumer is the next product, is stored as E4M3 codes).
template <typename T, bool F8, int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(SplitArgs r) {
  constexpr int NT = 256, MAXC = 9;  // N <= 2304
  if (*r.status != 0) return;
  const int m = blockIdx.x;
  if (m >= *r.m_ptr) return;
  const int tid = threadIdx.x;
  const int nc = r.N / NT;  // columns per thread (N is a multiple of 256)
  float v[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c < nc) {
      const int n = tid + c * NT;
      float acc = 0.f;
      for (int s = 0; s < r.S; ++s) acc += r.part[((int64_t)s * r.ldp + m) * r.N + n];
      v[c] = acc + r.bias[n];
    }
  }
  if constexpr (EPI == EPI_LN) {
    __shared__ float red[NT / 64];
    const T* R = static_cast<const T*>(r.R) + (int64_t)m * r.ldr;
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nc) {
        v[c] += (float)R[tid + c * NT];
        sum += v[c];
      }
    auto block_sum = [&](float x) __attribute__((always_inline)) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
      __syncthreads();
      if ((tid & 63) == 0) red[tid >> 6] = x;
      __syncthreads();
      return (red[0] + red[1]) + (red[2] + red[3]);
    };
    const float mean = block_sum(sum) / r.N;
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nc) sq += (v[c] - mean) * (v[c] - mean);
    const float rstd = 1.0f / sqrtf(block_sum(sq) / r.N + r.eps);
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nc) {
        const int n = tid + c * NT;
        const float o = ln_out(v[c], mean, rstd, r.ln_g[n], r.ln_b[n]);
        static_cast<T*>(r.Y)[(int64_t)m * r.ldy + n] = (T)o;
        if constexpr (F8) {
          if (r.Y8) static_cast<fp8*>(r.Y8)[(int64_t)m * r.ldy8 + n] = (fp8)(pack_e4m3x4(o, 0.f, 0.f, 0.f) & 0xFFu);
        }
      }
  } else if constexpr (EPI == EPI_OUT) {
    const int64_t orow = r.out_T ? (int64_t)r.row_seq[m] * r.out_T + r.row_pos[m] : m;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nc) r.out[orow * r.N + tid + c * NT] = v[c];
  } else {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nc) {
        const int n = tid + c * NT;
        float o = v[c];
        if constexpr (EPI == EPI_GELU) o = gelu_tanh(o);
        if constexpr (F8 && EPI == EPI_GELU) {
          static_cast<fp8*>(r.Y)[(int64_t)m * r.ldy + n] = (fp8)(pack_e4m3x4(o, 0.f, 0.f, 0.f) & 0xFFu);
        } else {
          static_cast<T*>(r.Y)[(int64_t)m * r.ldy + n] = (T)o;
          if constexpr (F8 && EPI == EPI_BIAS) {
            if (r.Y8) static_cast<fp8*>(r.Y8)[(int64_t)m * r.ldy8 + n] = (fp8)(pack_e4m3x4(o, 0.f, 0.f, 0.f) & 0xFFu);
          }
        }
      }
  }
}

}  // namespace albert
