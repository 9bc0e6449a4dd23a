// Length regulation: token features -> audio-aligned frames.
//
// Durations d[t] are integers >= 1; the aligned stream repeats row t of the
// token features d[t] times, in token order, so the frame count is
// A = sum d ("How Kokoro TTS Works and Where CKE Stands", section "The time
// axis is where a circuit becomes difficult"; the [p1,p2,p3], d=[2,1,3] ->
// [p1,p1,p2,p3,p3,p3] example of "Qwen3-TTS and Kokoro: Two Routes from Text
// to Speech", section "Path one").  The durations themselves come from the
// rule on the same page: sigmoid of each duration channel, summed, divided
// by the speed, rounded and clamped to at least one frame.
//
// Tokens are packed (sequence s at rows cu[s] .. cu[s+1]-1), so one global
// exclusive scan of d gives every token's first frame, and sequence s's
// frames start at the scan value of its first token.  The path is bound by
// HBM bytes: each token row is read once and written d[t] times.
#pragma once

#include "common.hpp"

namespace albert {

enum DurStatus { DST_OK = 0, DST_LENGTH = 3 };

__global__ void set_status_kernel(int* status) { *status = DST_OK; }

// d[t] = max(1, rint(sum_k sigmoid(logits[t, k]) / speed)), fp32 arithmetic,
// round half to even.  One wave per token, lanes over channels.
__global__ void __launch_bounds__(256)
durations_kernel(const float* __restrict__ logits, int total, int K, float inv_speed,
                 int* __restrict__ dur) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= total) return;  // whole waves leave together
  float s = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float x = logits[(int64_t)t * K + k];
    s += 1.0f / (1.0f + fast_exp2(-x * kLog2e));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) dur[t] = max(1, (int)rintf(s * inv_speed));
}

// Block-local scan of durations (1024 tokens per block): writes each
// token's exclusive prefix within its block and the block total; flags any
// duration < 1.
__global__ void __launch_bounds__(1024)
dur_scan_local_kernel(const int* __restrict__ dur, int total, int64_t* __restrict__ excl,
                      int64_t* __restrict__ block_sum, int* __restrict__ status) {
  __shared__ int64_t sh[1024];
  const int t = blockIdx.x * 1024 + threadIdx.x;
  int64_t d = 0;
  if (t < total) {
    const int v = dur[t];
    if (v < 1) atomicOr(status, (int)DST_LENGTH);
    d = v < 1 ? 0 : v;
  }
  sh[threadIdx.x] = d;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t add = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
    __syncthreads();
    sh[threadIdx.x] += add;
    __syncthreads();
  }
  if (t < total) excl[t] = sh[threadIdx.x] - d;
  if (threadIdx.x == 1023) block_sum[blockIdx.x] = sh[1023];
}

// One block: checks the token offsets (cu[0] = 0, cu[n] = total, every
// sequence non-empty), scans the block totals, checks that the frames fit
// the caller's output, and only then writes the sequences' frame offsets.
__global__ void __launch_bounds__(1024)
dur_scan_blocks_kernel(int64_t* __restrict__ block_sum, int nblocks, const int64_t* __restrict__ excl,
                       const int* __restrict__ cu_tok, int n_seq, int total, int64_t max_frames,
                       int* __restrict__ cu_frames, int* __restrict__ status) {
  __shared__ int64_t sh[1024];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) {
    carry = 0;
    if (cu_tok[0] != 0 || cu_tok[n_seq] != total) atomicOr(status, (int)DST_LENGTH);
  }
  for (int s = threadIdx.x; s < n_seq; s += 1024)
    if (cu_tok[s + 1] - cu_tok[s] < 1) atomicOr(status, (int)DST_LENGTH);
  __syncthreads();
  for (int base = 0; base < nblocks; base += 1024) {
    const int i = base + threadIdx.x;
    const int64_t v = i < nblocks ? block_sum[i] : 0;
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int64_t add = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
      __syncthreads();
      sh[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < nblocks) block_sum[i] = carry + sh[threadIdx.x] - v;  // exclusive
    __syncthreads();
    if (threadIdx.x == 1023) carry += sh[1023];
    __syncthreads();
  }
  const int64_t frames = carry;
  if (threadIdx.x == 0 && frames > max_frames) atomicOr(status, (int)DST_LENGTH);
  __syncthreads();
  if (*status != DST_OK) return;
  // cu_frames[s] = first frame of sequence s (its first token's offset)
  for (int s = threadIdx.x; s <= n_seq; s += 1024) {
    const int t = cu_tok[s];
    const int64_t f = t < total ? block_sum[t / 1024] + excl[t] : frames;
    cu_frames[s] = (int)f;
  }
}

// Scatter: one wave per token writes its row to frames
// [start, start + d).  Rows are C floats, written 16 bytes per lane, as
// non-temporal stores (the frames are not read again here; 79 % instead of
// 65 % of HBM bandwidth).
__global__ void __launch_bounds__(256)
expand_kernel(const float* __restrict__ feat, const int* __restrict__ dur,
              const int64_t* __restrict__ excl, const int64_t* __restrict__ block_off, int total,
              int C, float* __restrict__ out, const int* __restrict__ status) {
  if (*status != DST_OK) return;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= total) return;
  const int64_t f0 = block_off[t / 1024] + excl[t];
  const int d = dur[t];
  const f32x4* src = reinterpret_cast<const f32x4*>(feat + (int64_t)t * C);
  const int c4 = C / 4;
  for (int c = lane; c < c4; c += 64) {
    const f32x4 v = src[c];
    for (int r = 0; r < d; ++r)
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (f0 + r) * C) + c);
  }
}

}  // namespace albert
