// Device-side building blocks shared by the encoder's HIP kernels (gfx950).
//
// Storage types: __bf16 (the production path) or float (the fp32 debug
// path); the low-precision variant keeps bf16 storage and feeds the matrix
// products OCP FP8 E4M3 operands.  All arithmetic outside the matrix cores
// is fp32.
//
// Matrix-core conventions used by every kernel here (CDNA 32x32 MFMA):
//   D[32x32] += A[32xK] * B[Kx32], wave64.
//   Lane l supplies row (l % 32) of A and column (l % 32) of B, each as 8
//   consecutive elements of a 16-wide K step; half-wave h = l / 32 supplies
//   elements h*8 .. h*8+7 of that step.  Because A and B use the same
//   (lane, element) -> k assignment, any permutation of k inside a step is
//   harmless; the kernels exploit this to feed softmax probabilities straight
//   from accumulator registers.
//   Lane l holds D column (l % 32); register r holds D row
//   8*(r/4) + 4*h + (r%4).
//   bf16: one v_mfma_f32_32x32x16_bf16 per K step of 16.
//   fp32: eight v_mfma_f32_32x32x2_f32, element s of each lane in the s-th.
//   E4M3: one v_mfma_scale_f32_32x32x64_f8f6f4 per K step of 64, each lane
//   supplying 32 consecutive elements (again any k permutation shared by A
//   and B is harmless); A's per-lane E8M0 scale multiplies its row by a
//   power of two.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace albert {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned char fp8;  // one OCP FP8 E4M3 code
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kStatusSync = 7;  // ALBERT_E_SYNC: cooperating workgroups never met

template <typename T> struct Tr;

template <> struct Tr<bf16> {
  typedef bf16x8 frag;
  static constexpr int BK = 32;  // GEMM K tile: 64 bytes per row
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  // one fragment stored as 16-byte chunks at p0 (and p1 when a fragment
  // spans two chunks; bf16 fragments are a single chunk)
  static __device__ __forceinline__ frag load2(const bf16* p0, const bf16*) { return load(p0); }
  // two groups of 4 consecutive elements
  static __device__ __forceinline__ frag load2x4(const bf16* p0, const bf16* p1) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    frag f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
  static __device__ __forceinline__ frag from_f32(const float* v) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)v[e];
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)0.0f;
    return f;
  }
  static __device__ __forceinline__ void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
  }
  static __device__ __forceinline__ f32x4 load4f(const bf16* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    f32x4 r;
    r[0] = (float)v[0]; r[1] = (float)v[1]; r[2] = (float)v[2]; r[3] = (float)v[3];
    return r;
  }
};

template <> struct Tr<float> {
  struct frag { f32x4 lo, hi; };
  static constexpr int BK = 16;  // 64 bytes per row
  static __device__ __forceinline__ frag load(const float* p) {
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
  }
  static __device__ __forceinline__ frag load2(const float* p0, const float* p1) {
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p0);
    f.hi = *reinterpret_cast<const f32x4*>(p1);
    return f;
  }
  static __device__ __forceinline__ frag load2x4(const float* p0, const float* p1) {
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p0);
    f.hi = *reinterpret_cast<const f32x4*>(p1);
    return f;
  }
  static __device__ __forceinline__ frag from_f32(const float* v) {
    frag f;
    f.lo[0] = v[0]; f.lo[1] = v[1]; f.lo[2] = v[2]; f.lo[3] = v[3];
    f.hi[0] = v[4]; f.hi[1] = v[5]; f.hi[2] = v[6]; f.hi[3] = v[7];
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
    f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
    return f;
  }
  static __device__ __forceinline__ void mma(f32x16& c, const frag& a, const frag& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[s], b.lo[s], c, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[s], b.hi[s], c, 0, 0, 0);
  }
  static __device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
  static __device__ __forceinline__ f32x4 load4f(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
  }
};

template <> struct Tr<fp8> {
  typedef i32x8 frag;  // 32 E4M3 codes: one lane's share of a 64-deep K step
  static __device__ __forceinline__ frag load2(const fp8* p0, const fp8* p1) {
    const int4 a = *reinterpret_cast<const int4*>(p0);
    const int4 b = *reinterpret_cast<const int4*>(p1);
    frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return f;
  }
  // c += (A * 2^(sa - 127)) * B with E4M3 A and B (format code 0 for both);
  // sa is the E8M0 exponent of this lane's A row, B is unscaled (127).
  static __device__ __forceinline__ void mma_s(f32x16& c, const frag& a, const frag& b, int sa) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127);
  }
};

// Four fp32 values -> four E4M3 codes in memory order, rounding to nearest
// even; magnitudes beyond 448 (the largest finite code) saturate first.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const float lo = -448.f, hi = 448.f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, lo), hi), fminf(fmaxf(b, lo), hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, lo), hi), fminf(fmaxf(d, lo), hi), w, true);
  return (uint32_t)w;
}

// Store four values at element idx of an array of T, or of E4M3 codes.
template <typename T, bool F8>
__device__ __forceinline__ void store4_as(void* base, int64_t idx, float a, float b, float c, float d) {
  if constexpr (F8)
    *reinterpret_cast<uint32_t*>(static_cast<fp8*>(base) + idx) = pack_e4m3x4(a, b, c, d);
  else
    Tr<T>::store4(static_cast<T*>(base) + idx, a, b, c, d);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU, tanh approximation: x/2 (1 + tanh(a)), a = sqrt(2/pi) (x + 0.044715 x^3).
// Uses 1/2 (1 + tanh(a)) = 1 / (1 + e^(-2a)); for large |a| the exponential
// saturates to +inf or 0 and the result to 0 or x without special cases.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float a = c * (x + 0.044715f * (x * x * x));
  const float e = fast_exp2(-2.0f * kLog2e * a);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float wave_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// 16-byte row pieces of a 32x32 accumulator tile.
//
// In the MFMA result layout, lane (l32, hh) holds row l32 of the tile at
// columns 8q + 4hh + e (q, e = 0..3): four runs of 4 columns, so a store or
// load of one run covers 8 bytes (bf16) and one instruction touches 32 rows
// with 16 bytes each.  Lanes l and l + 32 can swap whole runs with
// v_permlane32_swap (lanes 32..63 of its first operand trade places with
// lanes 0..31 of its second): after swapping lane l's run q = 1 with lane
// l + 32's run q = 0 (and likewise runs 3 and 2), lane (l32, hh) holds
// columns 8hh .. 8hh + 7 and 16 + 8hh .. 16 + 8hh + 7, two 16-byte pieces, so
// one instruction covers 32 contiguous bytes of each of 32 rows and the
// tile's traffic takes half the memory instructions.  The same swap maps
// 16-byte pieces read from memory back to the accumulator layout.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Runs q = 0..3 of a tile row as bf16 pairs (w[q][0] = columns 0-1 of the
// run, w[q][1] = columns 2-3) -> the lane's two 16-byte pieces (columns
// 8hh.. and 16 + 8hh..).
__device__ __forceinline__ void swap_runs_to_pieces(const uint32_t (&w)[4][2], uint4& p0, uint4& p1) {
  const u32x2 a = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
  const u32x2 c = __builtin_amdgcn_permlane32_swap(w[2][0], w[3][0], false, false);
  const u32x2 d = __builtin_amdgcn_permlane32_swap(w[2][1], w[3][1], false, false);
  p0 = uint4{a[0], b[0], a[1], b[1]};
  p1 = uint4{c[0], d[0], c[1], d[1]};
}

// The inverse: the lane's two 16-byte pieces of bf16 -> runs q = 0..3 as fp32.
__device__ __forceinline__ void pieces_to_runs(const uint4& p0, const uint4& p1, f32x4 (&r)[4]) {
  const u32x2 a = __builtin_amdgcn_permlane32_swap(p0.x, p0.z, false, false);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(p0.y, p0.w, false, false);
  const u32x2 c = __builtin_amdgcn_permlane32_swap(p1.x, p1.z, false, false);
  const u32x2 d = __builtin_amdgcn_permlane32_swap(p1.y, p1.w, false, false);
  const uint32_t w[4][2] = {{a[0], b[0]}, {a[1], b[1]}, {c[0], d[0]}, {c[1], d[1]}};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[q][0] = __uint_as_float(w[q][0] << 16);
    r[q][1] = __uint_as_float(w[q][0] & 0xFFFF0000u);
    r[q][2] = __uint_as_float(w[q][1] << 16);
    r[q][3] = __uint_as_float(w[q][1] & 0xFFFF0000u);
  }
}

// Two fp32 values as one bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

}  // namespace albert
