// Request validation, packed-row bookkeeping, the three-table embedding with
// its LayerNorm, and the zeroing of padded output rows.
//
// The non-template kernels have internal linkage: each translation unit of
// the library (encoder, text path) gets its own copy.
//
// Every kernel reads the device status word first and does nothing when a
// previous step has rejected the request, so that a rejected request never
// writes the caller's output (the validate-before-write contract of the page
// "ALBERT: How Kokoro's Phoneme Encoder Works", section "How CKE Represents
// It"; the header ID check of "How Kokoro TTS Works and Where CKE Stands",
// section "How I want CKE to stitch it").
#pragma once

#include "common.hpp"

namespace albert {

enum DevStatus { ST_OK = 0, ST_LENGTH = 3, ST_ID = 4 };

// Inclusive prefix sum over one 1024-thread block (Hillis-Steele in LDS).
__device__ __forceinline__ int block_incl_scan_1024(int v, int* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int add = (t >= off) ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  int r = sh[t];
  __syncthreads();
  return r;
}

// Greedy grouping of consecutive sequences for the fused Q|K|V + attention
// kernel: each group takes sequences in order while their rows fit 256.
// groups[0] = number of groups g, groups[1 + i] = first row of group i
// (the row offset of its first sequence), groups[1 + g] = the rows in all.  Called by the whole block after this block has
// written cu[0..n]; `bad` is the block's rejection flag in LDS.  Every
// sequence has at most 256 rows (checked on the host), n <=
// kGreedyMaxSeqs.  The offsets go to LDS, each thread finds by binary
// search where a group starting at its sequences must end (nxt) and where
// the group after it ends (nxt2), and one thread walks that chain from
// sequence 0 two groups per dependent LDS load.  cu is written by this same block, so
// it must not be declared __restrict__ (nor the caller's copy be read
// through one): the compiler could then move its loads above the barrier.
constexpr int kGreedyMaxSeqs = 8192;
__device__ void greedy_groups(const int* cu, int n, int* groups, const int* bad) {
  __shared__ int scu[kGreedyMaxSeqs + 1];
  __shared__ short nxt[kGreedyMaxSeqs + 1];
  __shared__ short nxt2[kGreedyMaxSeqs];
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's cu[] stores are done
  __syncthreads();                     // every wave's cu[] and the flag are written
  if (*bad) {
    if (threadIdx.x == 0) groups[0] = 0;
    return;
  }
  for (int i = threadIdx.x; i <= n; i += blockDim.x) scu[i] = cu[i];
  __syncthreads();
  for (int s = threadIdx.x; s < n; s += blockDim.x) {
    // largest t in (s, n] with scu[t] - scu[s] <= 256
    int lo = s + 1, hi = n;
    const int lim = scu[s] + 256;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (scu[mid] <= lim) lo = mid;
      else hi = mid - 1;
    }
    nxt[s] = (short)lo;
  }
  if (threadIdx.x == 0) nxt[n] = (short)n;
  __syncthreads();
  for (int s = threadIdx.x; s < n; s += blockDim.x) nxt2[s] = nxt[nxt[s]];
  __syncthreads();
  if (threadIdx.x == 0) {
    int g = 0, s = 0;
    while (s < n) {
      const int t = nxt[s], u = nxt2[s];  // independent loads
      groups[1 + g++] = scu[s];
      if (t < n) groups[1 + g++] = scu[t];
      s = u;
    }
    groups[1 + g] = scu[n];
    groups[0] = g;
  }
}

// Padded batch: check every length in [1, T], write cu[0..B] (prefix sums)
// and the status word (and, with groups, the greedy groups).  One block of
// 1024 threads.
static __global__ void __launch_bounds__(1024)
derive_padded_kernel(const int* __restrict__ lengths, int B, int T, int* cu,
                     int* __restrict__ status, int* __restrict__ groups) {
  __shared__ int sh[1024];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < B; base += 1024) {
    const int i = base + threadIdx.x;
    int len = 0;
    if (i < B) {
      len = lengths[i];
      if (len < 1 || len > T) { bad = 1; len = 0; }
    }
    const int incl = block_incl_scan_1024(len, sh);
    if (i < B) cu[i + 1] = carry + incl;
    // the last thread's inclusive sum is this chunk's total
    if (threadIdx.x == 1023) sh[0] = incl;
    __syncthreads();
    carry += sh[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    cu[0] = 0;
    *status = bad ? ST_LENGTH : ST_OK;
  }
  if (groups) greedy_groups(cu, B, groups, &bad);
}

// Packed batch: cu_in[0] = 0, cu_in[n] = total, every length in
// [1, max_len]; copy the offsets into the workspace (and, with groups, the
// greedy groups).  One block.
static __global__ void __launch_bounds__(1024)
derive_packed_kernel(const int* __restrict__ cu_in, int n, int total, int max_len,
                     int* cu, int* __restrict__ status, int* __restrict__ groups) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (cu_in[0] != 0 || cu_in[n] != total) ? 1 : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int d = cu_in[i + 1] - cu_in[i];
    if (d < 1 || d > max_len) bad = 1;
  }
  for (int i = threadIdx.x; i <= n; i += 1024) cu[i] = cu_in[i];
  __syncthreads();
  if (threadIdx.x == 0) *status = bad ? ST_LENGTH : ST_OK;
  if (groups) greedy_groups(cu, n, groups, &bad);
}

// One block per sequence: write each valid row's sequence index and
// position, and check the ID at that slot.  Pad slots are never read.
// pad_T > 0: ids is [B, pad_T]; pad_T == 0: ids is packed [total].
static __global__ void __launch_bounds__(256)
rows_ids_kernel(const int* __restrict__ ids, const int* __restrict__ cu, int pad_T, int vocab,
                int* __restrict__ row_seq, int* __restrict__ row_pos, int* __restrict__ status) {
  if (*status != ST_OK) return;
  const int b = blockIdx.x;
  const int start = cu[b], L = cu[b + 1] - start;
  int bad = 0;
  for (int t = threadIdx.x; t < L; t += blockDim.x) {
    const int r = start + t;
    row_seq[r] = b;
    row_pos[r] = t;
    if (ids) {  // null for the LayerNorm-output entry, which has no IDs
      const int id = pad_T ? ids[(int64_t)b * pad_T + t] : ids[r];
      bad |= (id < 0 || id >= vocab);
    }
  }
  if (bad) atomicOr(status, (int)ST_ID);
}

// Three-table embedding + LayerNorm over E = 128 ("Inside One Real ALBERT
// Layer", step 1): e = word[id] + pos[t] + type[0]; LN with the given eps.
// 16 lanes per row, 8 channels per lane; fp32 arithmetic, output in T (or
// as E4M3 codes when F8: the output only feeds the projection's product).
template <typename T, bool F8>
__global__ void __launch_bounds__(256)
embed_ln_kernel(const int* __restrict__ ids, int pad_T, const int* __restrict__ row_seq,
                const int* __restrict__ row_pos, const int* __restrict__ m_ptr,
                const T* __restrict__ word, const T* __restrict__ pos, const T* __restrict__ type,
                const float* __restrict__ g, const float* __restrict__ bta, float eps,
                void* __restrict__ out, const int* __restrict__ status) {
  constexpr int E = 128;
  if (*status != ST_OK) return;
  const int M = *m_ptr;
  const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (r >= M) return;  // whole 16-lane groups leave together
  const int p = row_pos[r];
  const int id = pad_T ? ids[(int64_t)row_seq[r] * pad_T + p] : ids[r];
  float v[8];
  const int c0 = sub * 8;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    f32x4 a = Tr<T>::load4f(word + (int64_t)id * E + c0 + 4 * q);
    f32x4 b = Tr<T>::load4f(pos + (int64_t)p * E + c0 + 4 * q);
    f32x4 c = Tr<T>::load4f(type + c0 + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q + e] = a[e] + b[e] + c[e];
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += v[e];
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
  const float mean = s * (1.0f / E);
  float s2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) { v[e] -= mean; s2 += v[e] * v[e]; }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s2 += __shfl_xor(s2, m, 16);
  const float rstd = 1.0f / sqrtf(s2 * (1.0f / E) + eps);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = c0 + 4 * q;
    store4_as<T, F8>(out, (int64_t)r * E + c,
                     v[4 * q + 0] * rstd * g[c + 0] + bta[c + 0],
                     v[4 * q + 1] * rstd * g[c + 1] + bta[c + 1],
                     v[4 * q + 2] * rstd * g[c + 2] + bta[c + 2],
                     v[4 * q + 3] * rstd * g[c + 3] + bta[c + 3]);
  }
}

// Caller-supplied embedding LayerNorm output (fp32 [M, 128], packed rows)
// converted to the projection's operand type: the split in which the
// embedding runs elsewhere and the encoder block starts at the projection
// ("Kokoro-82M-encoder-hailo10h", "What this is not").  Four channels per
// thread.
template <typename T, bool F8>
__global__ void __launch_bounds__(256)
features_in_kernel(const float* __restrict__ x, const int* __restrict__ m_ptr,
                   void* __restrict__ out, const int* __restrict__ status) {
  constexpr int E = 128;
  if (*status != ST_OK) return;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)(*m_ptr) * E) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + i);
  store4_as<T, F8>(out, i, v[0], v[1], v[2], v[3]);
}

// Padded output: rows t >= lengths[b] of out[B, T, n_out] are set to 0.
static __global__ void __launch_bounds__(256)
zero_pad_rows_kernel(float* __restrict__ out, const int* __restrict__ cu, int T, int n_out,
                     const int* __restrict__ status) {
  if (*status != ST_OK) return;
  const int b = blockIdx.x;
  const int L = cu[b + 1] - cu[b];
  const int per_row = n_out / 4;
  const int64_t n4 = (int64_t)(T - L) * per_row;
  f32x4* o = reinterpret_cast<f32x4*>(out + ((int64_t)b * T + L) * n_out);
  for (int64_t i = threadIdx.x; i < n4; i += blockDim.x) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace albert
