// Kokoro's parallel text path on the GPU: embedding, convolution blocks,
// bidirectional LSTM ("How Kokoro TTS Works and Where CKE Stands": a small
// separate path of an embedding, three weight-normalized convolutions and a
// bidirectional LSTM beside the ALBERT; [512, T] features).
//
// Rows are packed tokens (sequence s at rows cu[s] .. cu[s+1]-1), as in the
// encoder.  A convolution of width K over a sequence is one GEMM over the
// unfolded input col[m, j*C + c] = x[m + j - K/2, c] (zero where that row
// is outside m's sequence), so zero padding happens at every sequence's own
// ends and neighbours in the pack never mix.  The unfolded input is never
// built: the GEMM's DMA reads the shifted rows of x directly, guided by a
// per-row mask of the taps inside the row's sequence; its LayerNorm and
// LeakyReLU run in the GEMM's full-row epilogue.  The LSTM input projection (both
// directions, both biases) is a second GEMM into fp32 gate pre-activations;
// the recurrence below then only adds W_hh h_{t-1}.
#pragma once

#include "common.hpp"

namespace albert {

constexpr int kLstmH = 256;   // units per direction
constexpr int kLstmSeq = 32;  // sequences per recurrence workgroup

// x[m, :] = emb[id(m), :] for the M valid rows; C a multiple of 8.
__global__ void __launch_bounds__(256)
text_embed_kernel(const int* __restrict__ ids, int pad_T, const int* __restrict__ row_seq,
                  const int* __restrict__ row_pos, const int* __restrict__ m_ptr,
                  const bf16* __restrict__ emb, int C, bf16* __restrict__ out,
                  const int* __restrict__ status) {
  if (*status != 0) return;
  const int cpr = C / 8;  // 16-byte chunks per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)(*m_ptr) * cpr) return;
  const int m = (int)(i / cpr), c = (int)(i % cpr);
  const int id = pad_T ? ids[(int64_t)row_seq[m] * pad_T + row_pos[m]] : ids[m];
  reinterpret_cast<uint4*>(out + (int64_t)m * C)[c] =
      reinterpret_cast<const uint4*>(emb + (int64_t)id * C)[c];
}

// The convolution taps of each packed row: bit j of taps[m] is set when
// input row m + j - K/2 belongs to m's sequence (the convolution GEMM reads
// that row for tap j, and zeros otherwise: zero padding at each sequence's
// own ends).  One thread per row.
__global__ void __launch_bounds__(256)
conv_taps_kernel(const int* __restrict__ row_seq, const int* __restrict__ row_pos,
                 const int* __restrict__ cu, const int* __restrict__ m_ptr, int K,
                 unsigned char* __restrict__ taps, const int* __restrict__ status) {
  if (*status != 0) return;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= *m_ptr) return;
  const int s = row_seq[m], p = row_pos[m], L = cu[s + 1] - cu[s];
  unsigned v = 0;
  for (int j = 0; j < K; ++j) {
    const int q = p + j - K / 2;
    if (q >= 0 && q < L) v |= 1u << j;
  }
  taps[m] = (unsigned char)v;
}

struct LstmArgs {
  const float* xg;   // [M, 2*4H] fp32: W_ih x + b_ih + b_hh, direction d at column d*4H
  const bf16* whh;   // W_hh of both directions in fragment order (see lstm_kernel)
  float* out;        // output rows of 2H fp32, direction d at column d*H
  int out_T;         // padded T (row = seq*T + t), or 0 for packed rows (cu[seq] + t)
  const int* cu;     // [n_seq + 1]
  int n_seq;
  const int* status;
};

__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}
__device__ __forceinline__ float tanh_f(float x) {
  return __builtin_fmaf(2.0f, sigmoid_f(2.0f * x), -1.0f);
}
// One cell update: c <- sigmoid(f) c + sigmoid(i) tanh(g); returns
// sigmoid(o) tanh(c).  The multiply-adds are explicit so that both
// recurrence kernels round every step alike.
__device__ __forceinline__ float lstm_cell(float zi, float zf, float zg, float zo, float& c) {
  const float cn = __builtin_fmaf(sigmoid_f(zf), c, sigmoid_f(zi) * tanh_f(zg));
  c = cn;
  return sigmoid_f(zo) * tanh_f(cn);
}

// LSTM recurrence.  Grid (ceil(n_seq / 32), 2 directions), 8 waves.  The
// workgroup carries 32 sequences of one direction through their own
// lengths: the forward direction visits t = 0 .. L-1, the backward one
// t = L-1 .. 0, so padding never enters either scan (the masking that the
// "Kokoro-82M-LiteRT" card warns about).  Each step is G^T = W_hh h^T on
// the matrix cores: wave w owns units [32w, 32w+32) of all four gates (A
// = those W_hh rows, streamed from L2), the B operand is h_{t-1} of the 32
// sequences, kept in LDS as bf16; so every lane holds the i, f, g, o
// pre-activations of the same 16 (unit, sequence) pairs and updates their
// cell state (fp32, in registers) without any exchange.
// W_hh is stored in fragment order -- [d][wave][k-step][gate][lane][8] --
// so that each wave-wide fragment load reads one contiguous kilobyte.
__global__ void __launch_bounds__(512)
lstm_kernel(LstmArgs a) {
  constexpr int H = kLstmH, LDH = H + 8;  // padded rows: conflict-free fragment reads
  __shared__ __attribute__((aligned(16))) bf16 hs[2][kLstmSeq * LDH];
  if (*a.status != 0) return;
  const int d = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int seq = blockIdx.x * kLstmSeq + l32;  // this lane's sequence (MFMA column)
  const bool sv = seq < a.n_seq;
  const int start = sv ? a.cu[seq] : 0;
  const int L = sv ? a.cu[seq + 1] - start : 0;
  int Lmax = L;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) Lmax = max(Lmax, __shfl_xor(Lmax, off, 64));

  for (int i = tid; i < kLstmSeq * LDH; i += 512) hs[0][i] = (bf16)0.0f;
  float c[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
  const bf16* __restrict__ W = a.whh + ((int64_t)d * 8 + wave) * (H / 16) * 4 * 64 * 8;
  const int ubase = 32 * wave + 4 * hh;  // unit of register r: ubase + 8*(r/4) + r%4
  __syncthreads();

  // W_hh fragment of k-step kk for gate g (rows g*H + 32*wave + l32,
  // columns kk*16 + hh*8 ..): one contiguous kilobyte per wave.
  auto wload = [&](int kk, int g) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(W + ((kk * 4 + g) * 64 + lane) * 8);
  };
  constexpr int KS = H / 16;  // 16 k-steps
  // W_hh prefetch distance (k-steps).  One k-step ahead keeps the kernel
  // within its 256 registers; three ahead spilled in the step loop and ran
  // 16 % slower on MI355X.
  constexpr int PD = 1;
  static_assert(KS % (PD + 1) == 0, "the fragment ring must wrap at a step boundary");

  // Gate inputs of step tau as the accumulators' starting value (the MFMA
  // adds into them).
  f32x16 acc[4];
  auto xload = [&](int tau) __attribute__((always_inline)) {
    const bool act = tau < L;
    const int t = d == 0 ? tau : L - 1 - tau;
    const float* xr = a.xg + ((int64_t)start + t) * (8 * H) + d * 4 * H + ubase;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = act ? *reinterpret_cast<const f32x4*>(xr + g * H + 8 * q)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[g][4 * q + e] = v[e];
      }
  };
  // W_hh streams from L2 through a ring of PD+1 k-steps, PD k-steps of
  // loads in flight behind the matrix cores; the stream runs on across step
  // boundaries (W_hh is the same for every step), so no step starts cold.
  bf16x8 wr[PD + 1][4];
  xload(0);
#pragma unroll
  for (int kk = 0; kk < PD; ++kk)
#pragma unroll
    for (int g = 0; g < 4; ++g) wr[kk][g] = wload(kk, g);

  for (int tau = 0; tau < Lmax; ++tau) {
    const int cur = tau & 1;
    const bool act = tau < L;
    const int t = d == 0 ? tau : L - 1 - tau;
    const int64_t row = (int64_t)start + t;
    const bf16* hb = hs[cur] + l32 * LDH + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int g = 0; g < 4; ++g) wr[(kk + PD) % (PD + 1)][g] = wload((kk + PD) % KS, g);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(hb + kk * 16);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[kk % (PD + 1)][g], b, acc[g], 0, 0, 0);
      // keep each k-step's loads in place: hoisting them all would hold
      // every W_hh fragment of the step in registers at once
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16* hn = hs[cur ^ 1] + l32 * LDH;
    const int64_t orow = a.out_T ? (int64_t)seq * a.out_T + t : row;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e;
        hv[e] = lstm_cell(acc[0][r], acc[1][r], acc[2][r], acc[3][r], c[r]);
      }
      const int u = ubase + 8 * q;
      Tr<bf16>::store4(hn + u, hv[0], hv[1], hv[2], hv[3]);
      if (act)
        *reinterpret_cast<f32x4*>(a.out + orow * (2 * H) + d * H + u) =
            f32x4{hv[0], hv[1], hv[2], hv[3]};
    }
    xload(tau + 1);   // next step's gate inputs, in flight across the barrier
    __syncthreads();  // h_t complete in hs[cur^1]; hs[cur] free for step tau+1's writes
  }
}

// Multi-workgroup recurrence.  Each direction of a group of 32 sequences
// is carried by a quad of workgroups; member m owns units [64m, 64m+64) and
// keeps their W_hh rows (4 gates x 64 units x 256 inputs, 128 KB) in
// registers for the whole scan, so no weight bytes move per step.  Wave w
// of member m owns the 32 gate rows of units 64m + 8w .. +7 as one MFMA
// tile, rows ordered so that lane (l32, hh) receives the four gates of
// units 64m + 8w + 4hh + j (j = 0..3) for sequence l32: acc[4j + g] is gate
// g of unit j.  After each step a member publishes its 64 units of h_t
// (bf16) and a step flag; once all four flags reach the step, every member
// reads the full h_t into LDS for the next step.  The quad must be resident
// at once (the host uses a cooperative launch); every wait is bounded, and a
// wait that runs out sets the status word to ALBERT_E_SYNC and ends the
// workgroup, after which its partners' waits run out too.
constexpr int kMcMembers = 4;
constexpr int kMcSpin = 1 << 20;  // polls (each after a short sleep) before giving up

__global__ void zero_ints_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

struct LstmMcArgs {
  const float* xg;   // as LstmArgs
  const bf16* whh;   // [d][member][wave][k-step 16][lane 64][8], rows permuted as above
  float* out;
  int out_T;
  const int* cu;
  int n_seq;
  int seq0;          // first sequence of this launch
  int n_quads;       // (groups of 32 sequences in this launch) x 2 directions
  bf16* hx;          // exchange, [quad][parity 2][32 sequences][256 units]
  int* flags;        // [quad][member], zero before the launch
  int* status;
};

__global__ void __launch_bounds__(512)
lstm_mc_kernel(LstmMcArgs a) {
  constexpr int H = kLstmH, LDH = H + 8, KS = H / 16;
  __shared__ __attribute__((aligned(16))) bf16 hs[kLstmSeq * LDH];
  __shared__ int ok_s;
  // workgroup b -> quad q, member m: the four members of a quad are b, b+8,
  // b+16, b+24 (workgroups are dealt to the 8 XCDs round-robin, so a quad
  // shares one XCD)
  const int b = blockIdx.x;
  const int q = (b / 32) * 8 + b % 8, m = (b / 8) % kMcMembers;
  if (q >= a.n_quads || *a.status != 0) return;
  const int d = q % 2, grp = q / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int seq = a.seq0 + grp * kLstmSeq + l32;
  const bool sv = seq < a.n_seq;
  const int start = sv ? a.cu[seq] : 0;
  const int L = sv ? a.cu[seq + 1] - start : 0;
  int Lmax = L;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) Lmax = max(Lmax, __shfl_xor(Lmax, off, 64));
  const int ub = 64 * m + 8 * wave + 4 * hh;  // this lane's units ub .. ub+3

  bf16x8 wf[KS];
  const bf16* __restrict__ W = a.whh + ((((int64_t)d * kMcMembers + m) * 8 + wave) * KS) * 64 * 8;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) wf[kk] = *reinterpret_cast<const bf16x8*>(W + (kk * 64 + lane) * 8);
  for (int i = tid; i < kLstmSeq * LDH; i += 512) hs[i] = (bf16)0.0f;
  float c[4] = {0.f, 0.f, 0.f, 0.f};

  // gate inputs of step tau for this lane's 4 units: one 16-byte load per gate
  f32x4 xv[4];
  auto xload = [&](int tau) __attribute__((always_inline)) {
    const bool act = tau < L;
    const int t = d == 0 ? tau : L - 1 - tau;
    const float* xr = a.xg + ((int64_t)start + t) * (8 * H) + d * 4 * H + ub;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      xv[g] = act ? *reinterpret_cast<const f32x4*>(xr + g * H) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  xload(0);
  bf16* const hxq = a.hx + (int64_t)q * 2 * kLstmSeq * H;
  int* const fq = a.flags + q * kMcMembers;
  // the weight registers have arrived before the step loop (otherwise the
  // loop's waits for them would also wait for each step's gate-input loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int tau = 0; tau < Lmax; ++tau) {
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[4 * j + g] = xv[g][j];
    xload(tau + 1);  // in flight across the step
    const bf16* hb = hs + l32 * LDH + hh * 8;
    bf16x8 hf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) hf[kk] = *reinterpret_cast<const bf16x8*>(hb + kk * 16);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk], hf[kk], acc, 0, 0, 0);
    float hv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[j] = lstm_cell(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3], c[j]);
    }
    if (tau < L) {
      const int t = d == 0 ? tau : L - 1 - tau;
      const int64_t orow = a.out_T ? (int64_t)seq * a.out_T + t : (int64_t)start + t;
      *reinterpret_cast<f32x4*>(a.out + orow * (2 * H) + d * H + ub) = f32x4{hv[0], hv[1], hv[2], hv[3]};
    }
    if (tau + 1 == Lmax) break;
    // publish this member's h_t, then meet the other members
    bf16* const hxp = hxq + (tau & 1) * kLstmSeq * H;
    Tr<bf16>::store4(hxp + l32 * H + ub, hv[0], hv[1], hv[2], hv[3]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have reached L2
    __syncthreads();                                   // every wave is done with hs
    if (wave == 0) {  // lane 0 publishes; lanes 0..3 watch one member each
      if (lane == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(fq + m, tau + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      bool ok = true;
      for (int polls = 0;; ++polls) {
        const int v = lane < kMcMembers
                          ? __hip_atomic_load(fq + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : tau + 1;
        if (__all(v >= tau + 1)) break;
        if (polls >= kMcSpin) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (lane == 0) {
        if (!ok) __hip_atomic_store(a.status, kStatusSync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok_s = ok;
      }
    }
    __syncthreads();
    if (!ok_s) return;
    {  // h_t of all 256 units -> LDS: 32 bytes per thread
      const int sq = tid / 16, ch = tid % 16;
      const uint4* src = reinterpret_cast<const uint4*>(hxp + sq * H + ch * 16);
      uint4* dst = reinterpret_cast<uint4*>(hs + sq * LDH + ch * 16);
      dst[0] = src[0];
      dst[1] = src[1];
    }
    __syncthreads();
  }
}

}  // namespace albert
