// One step of the masked-softmax attention of one query per lane, shared by
// the fused and the separate attention kernels.
//
// softmax(q K^T) V over a sequence's keys ("Inside One Real ALBERT Layer",
// step 4) is accumulated over passes of up to four 32-key blocks.  Within
// a pass every score is computed first (S^T = K Q^T on the matrix cores,
// lane = query, 16 keys of each block per lane), then one maximum, one
// rescale of the running sum and output, and the probabilities feed
// O^T += V^T P^T straight from registers.  Across passes the running
// maximum makes it the usual online softmax, so the result does not depend
// on how the keys are cut into passes beyond rounding; two kernels that cut
// them the same way (passes from the sequence's start) produce the same
// bits.  Keys outside [lo, hi) of the pass are masked per lane; the mask is
// skipped when every lane of the wave keeps every key of the pass.
#pragma once

#include "common.hpp"

namespace albert {

// kfrag(b, kk): K fragment of block b, k-step kk (dims 16kk..16kk+15) for
// this lane (key 32b + l32 of the pass).  vfrag(b, c, dt): V^T fragment of
// dims 32dt + l32, keys 32b + 16c + 4hh + {0..3, 8..11} of the pass, in the
// order of the probabilities that from_f32(p + 8c) packs.
template <typename T, typename KFrag, typename VFrag>
__device__ __forceinline__ void attend_pass(f32x16 (&o)[2], float& mrun, float& lrun,
                                            const typename Tr<T>::frag (&fq)[4], int nb, int lo,
                                            int hi, int hh, KFrag&& kfrag, VFrag&& vfrag) {
  typedef Tr<T> TR;
  constexpr int NB = 4;
  const bool masked = !__all(lo <= 0 && hi >= 32 * nb);
  f32x16 s[NB];
  float mx = kNegInf;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) TR::mma(s[b], kfrag(b, kk), fq[kk]);
      // s[b][r]: key 32b + 8(r/4) + 4hh + r%4 of the pass
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * b + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < lo || key >= hi) s[b][r] = kNegInf;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    }
  }
  mx = fmaxf(mx, wave_xor(mx, 32));
  const float mnew = fmaxf(mrun, mx);
  // a lane that has met none of its keys yet keeps a zero state
  const float alpha = mnew == kNegInf ? 1.f : fast_exp2((mrun - mnew) * kLog2e);
  const float mb = mnew == kNegInf ? 0.f : mnew * kLog2e;
  mrun = mnew;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    o[0][r] *= alpha;
    o[1][r] *= alpha;
  }
  float psum = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < nb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(s[b][r] * kLog2e - mb);
        psum += p[r];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const typename TR::frag fp = TR::from_f32(p + 8 * c);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) TR::mma(o[dt], vfrag(b, c, dt), fp);
      }
    }
  }
  lrun = lrun * alpha + psum;
}

}  // namespace albert
