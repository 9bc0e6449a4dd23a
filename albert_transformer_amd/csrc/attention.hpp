// Fused masked-softmax bidirectional attention over packed sequences.
//
// Per sequence s and head h: C = softmax(Q K^T / sqrt(64)) V over the
// sequence's own keys only ("Inside One Real ALBERT Layer", step 4; the
// shorthand softmax(QK^T/sqrt(d) + mask) V of "How Kokoro TTS Works and Where
// CKE Stands", section "What ALBERT does here": keys beyond the length get no
// weight).  The 1/8 scale is already folded into the stored query weights.
//
// Two grids.  Per sequence (long sequences): (sequences, 12 heads, query
// tiles of 128 from the sequence's start).  Packed blocks (many short
// sequences): (blocks of 128 packed query rows, 12 heads); a block may hold
// the tail of one sequence, several whole short ones and the head of
// another.  Each wave owns 32 queries.  The workgroup walks the sequences
// of its queries in order, staging each one's keys and values in LDS in
// chunks of 128 keys (K row-major, V transposed), zero-filled past its
// length, and a lane takes only the chunks of its own sequence (for the
// others its scores are masked, which leaves its running softmax exactly
// unchanged).  Every lane therefore sees its sequence's keys in the same
// blocks, from the sequence's start, whichever grid and packing.
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// and 16 keys of every 32-key block: the running max and sum of the online
// softmax need only the partner half-wave, and the probabilities feed the
// second MFMA (O^T = V^T P^T) directly from registers, with V^T read from
// LDS in the matching key order.  With F8 the context is written as E4M3
// codes (its one consumer is the output projection's matrix product).
#pragma once

#include "attend.hpp"
#include "common.hpp"

namespace albert {

struct AttnArgs {
  const void* qkv;    // [M, 3H]: q*(1/8) | k | v, head h at h*64
  void* ctx;          // [M, H] (T, or E4M3 codes)
  const int* cu;      // [n_seq + 1]
  const int* row_seq; // [M] sequence of each packed row
  const int* m_ptr;   // device: M
  const int* status;
  int packed;         // 1: packed-block grid, 0: per-sequence grid
};

template <typename T, bool F8>
// At least three waves per SIMD (168 VGPRs): the staging of each chunk is
// latency-bound, and with two the kernel ran 28 % slower; four spill.
__global__ void __launch_bounds__(256, 3)
attention_kernel(AttnArgs a) {
  typedef Tr<T> TR;
  constexpr int H = 768, D = 64, LDQKV = 3 * H;
  constexpr int KC = 128;                 // keys per staged chunk
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDKS = D + VEC;           // K rows, padded
  constexpr int LDVT = KC + 4;            // V^T rows, padded (66 words for bf16)
  __shared__ __attribute__((aligned(16))) T Ks[KC * LDKS];
  __shared__ __attribute__((aligned(16))) T Vt[D * LDVT];

  if (*a.status != 0) return;
  const int h = blockIdx.y;
  int q0, q1, s_first, s_last;  // query rows [q0, q1), their sequences
  if (a.packed) {
    const int M = *a.m_ptr;
    q0 = blockIdx.x * 128;
    if (q0 >= M) return;
    q1 = min(q0 + 128, M);
    s_first = a.row_seq[q0];
    s_last = a.row_seq[q1 - 1];
  } else {
    const int sq = blockIdx.x, start = a.cu[sq];
    q0 = start + blockIdx.z * 128;
    q1 = min(q0 + 128, a.cu[sq + 1]);
    if (q0 >= q1) return;
    s_first = s_last = sq;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qi = q0 + wave * 32 + l32;  // this lane's query row (column of S^T)
  const bool qv = qi < q1;
  const int my_seq = qv ? a.row_seq[qi] : -1;

  const T* __restrict__ qkv = static_cast<const T*>(a.qkv);
  typename TR::frag fq[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    fq[kk] = qv ? TR::load(qkv + (int64_t)qi * LDQKV + h * D + kk * 16 + hh * 8) : TR::zero();

  f32x16 o[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { o[0][r] = 0.f; o[1][r] = 0.f; }
  float mrun = kNegInf, lrun = 0.f;

  for (int sq = s_first; sq <= s_last; ++sq) {
    const int start = a.cu[sq], L = a.cu[sq + 1] - start;
    const bool mine = my_seq == sq;
    const T* __restrict__ base = qkv + (int64_t)start * LDQKV;
    for (int c0 = 0; c0 < L; c0 += KC) {
      const int nk = min(KC, L - c0);
      const int nk32 = (nk + 31) / 32 * 32;  // rows the 32-key blocks below read
      __syncthreads();  // the previous chunk is fully consumed
      // K chunk, row-major [key][dim]
      for (int idx = tid; idx < nk32 * (D / VEC); idx += 256) {
        const int j = idx / (D / VEC), cc = idx % (D / VEC);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < nk) v = *reinterpret_cast<const uint4*>(base + (int64_t)(c0 + j) * LDQKV + H + h * D + cc * VEC);
        *reinterpret_cast<uint4*>(Ks + j * LDKS + cc * VEC) = v;
      }
      // V chunk, transposed [dim][key]: a task reads one 16-byte chunk of two
      // consecutive key rows (coalesced along the rows) and writes words that
      // each hold one dim for both keys.
      for (int idx = tid; idx < (nk32 / 2) * (D / VEC); idx += 256) {
        const int cc = idx % (D / VEC), p = idx / (D / VEC);
        const int j = 2 * p;
        T t0[VEC], t1[VEC];
        uint4 u0 = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
        if (j < nk) u0 = *reinterpret_cast<const uint4*>(base + (int64_t)(c0 + j) * LDQKV + 2 * H + h * D + cc * VEC);
        if (j + 1 < nk) u1 = *reinterpret_cast<const uint4*>(base + (int64_t)(c0 + j + 1) * LDQKV + 2 * H + h * D + cc * VEC);
        *reinterpret_cast<uint4*>(t0) = u0;
        *reinterpret_cast<uint4*>(t1) = u1;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T* dst = Vt + (cc * VEC + e) * LDVT + j;
          dst[0] = t0[e];
          dst[1] = t1[e];
        }
      }
      __syncthreads();

      // this lane's keys in the chunk: all of it up to the sequence's end,
      // or none when the lane's query belongs to another sequence (a pass
      // with none leaves the lane's state exactly unchanged, so a wave
      // whose queries all belong to other sequences skips it)
      const int nkb = (nk + 31) / 32;
      if (__any(mine)) {
        attend_pass<T>(o, mrun, lrun, fq, nkb, 0, mine ? L - c0 : 0, hh,
                       [&](int b, int kk) { return TR::load(Ks + (b * 32 + l32) * LDKS + hh * 8 + kk * 16); },
                       [&](int b, int c, int dt) {
                         const T* vp = Vt + (dt * 32 + l32) * LDVT + b * 32 + 16 * c + 4 * hh;
                         return TR::load2x4(vp, vp + 8);
                       });
      }
    }
  }
  lrun += wave_xor(lrun, 32);
  if (!qv) return;
  const float inv = 1.0f / lrun;
  const int64_t orow = (int64_t)qi * H + h * D;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = dt * 32 + 8 * q + 4 * hh;
      store4_as<T, F8>(a.ctx, orow + d, o[dt][4 * q + 0] * inv, o[dt][4 * q + 1] * inv,
                       o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv);
    }
}

}  // namespace albert
