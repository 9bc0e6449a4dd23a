// Fused Q|K|V projection and attention for one head of a group of whole
// sequences (bf16 storage; bf16 or E4M3 matrix-product operands).
//
// The layer's q, k, v projections ("Inside One Real ALBERT Layer", step 3)
// and the masked-softmax attention (step 4; "How Kokoro TTS Works and Where
// CKE Stands", "What ALBERT does here") computed in one workgroup, so q, k
// and v of the group never leave the chip: the workgroup owns head h and a
// group of consecutive whole sequences of at most 256 rows in all (packed
// greedily on the device, or S = 256 / longest per group, chosen on the
// host, for very large batches), computes the 192 projected features of head
// h (q/8 | k | v, the query scale folded into the weights) for those rows on
// the matrix cores, stores them in LDS as bf16 (the same storage point as
// the unfused path) and runs the attention of every query against the keys
// of its own sequence.  Only the context leaves the workgroup.
//
// GEMM phase: 256 rows x 192 features, K = 768 in slices of 128 bytes per
// row (64 bf16 or 128 E4M3 elements) staged in LDS by buffer_load ... lds
// DMA (two stages), 8 waves as 4 (rows) x 2 (features) of 64 x 96; weights
// are the MFMA A operand, tokens B (lane = token), as in gemm.hpp.  E4M3
// weight rows carry an E8M0 exponent that the matrix core applies as A's
// scale; Q, K and V are stored as bf16 either way.  Rows of the tile past
// the group belong to the next group, or lie past M: the DMA's row offset is
// in the scalar offset, which the buffer range check does not cover, so
// those rows read whatever the workspace holds there.  Their queries are
// never stored, their keys are masked (the score is replaced, not added
// to), and their V^T columns are written as zeros.
//
// Attention phase: the stage buffers are reused for Q and K (row-major) and
// V^T; wave w owns queries 32w .. 32w+31 of the tile, one per lane, as in
// attention.hpp (S^T = K Q^T, online softmax per lane with the partner
// half-wave, O^T = V^T P^T); a lane's keys are those of its own sequence,
// so key blocks outside it are masked per lane.  With E4M3 operands the
// context is written as E4M3 codes (its one consumer is the output
// projection's matrix product).
#pragma once

#include <type_traits>

#include "attend.hpp"
#include "common.hpp"
#include "gemm.hpp"

namespace albert {

struct QkvAttnArgs {
  const void* X;        // [M, 768] layer input (row stride 768), bf16 or E4M3 codes
  const void* Wh;       // [12][192][768]: per head q/8 | k | v weight rows, bf16 or E4M3 codes
  const unsigned char* Eh;  // E4M3: [12][192] E8M0 exponents of those rows
  const float* bh;      // [12][192]: their biases
  void* ctx;            // [M, 768] attention context, bf16 or E4M3 codes
  const int* cu;        // [n_seq + 1] packed row offsets
  const int* row_seq;   // [M] sequence of each row
  const int* status;
  const int* groups;    // greedy groups (count, first rows, rows in all), or null:
  int n_seq;
  int S;                //   then groups of S consecutive sequences
  int n_pairs;          // groups (an upper bound with greedy groups) * 12
};

template <bool F8>
__global__ void __launch_bounds__(512)
qkv_attention_kernel(QkvAttnArgs a) {
  typedef typename std::conditional<F8, fp8, bf16>::type TO;  // operand codes
  typedef Tr<TO> TRO;                                         // operand fragments
  typedef Tr<bf16> TR;                                        // attention
  constexpr int ES = sizeof(TO);
  constexpr int H = 768, D = 64, NH = 12, BM = 256, BN = 3 * D;
  constexpr int WGN = 2, NW = 8, NT = NW * 64;
  constexpr int WTM = 64, WTN = 96, TM = 2, TN = 3;
  constexpr int RB = 128, CPR = RB / 16, BK = RB / ES, RPI = 1024 / RB;
  constexpr int KS = F8 ? 64 : 16;         // K per MFMA step
  constexpr int FE = F8 ? 32 : 8;          // elements per lane per step
  constexpr int CH = 16 / ES, FCH = FE / CH;  // chunks per fragment
  constexpr int NINST = (BM + BN) / RPI, IPW = NINST / NW;
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int KSTEPS = BK / KS, KT = H / BK;
  constexpr int LDQ = D + 8;       // Q and K rows (144 bytes)
  constexpr int LDV = BM + 8;      // V^T rows (528 bytes)
  static_assert(NINST % NW == 0 && (BM / RPI) % NW == 0 && NW % 2 == 0, "DMA split");
  static_assert(KT % 2 == 0 && KSTEPS >= 1, "two stages of whole MFMA steps");
  static_assert(BM * LDQ * 2 + 32 * LDV * 2 <= STAGE, "attention buffers fit a stage");
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];
  __shared__ float bias_s[BN];

  if (*a.status != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hh = lane >> 5;
  const int M = a.cu[a.n_seq];

  // One (group, head) pair: the GEMM phase, then the attention phase.
  auto one = [&](int grp, int h) __attribute__((always_inline)) {
    int r0, r1;  // the group's rows
    if (a.groups) {
      r0 = a.groups[1 + grp];
      r1 = a.groups[2 + grp];
    } else {
      const int s0 = grp * a.S;
      r0 = a.cu[s0];
      r1 = a.cu[min(s0 + a.S, a.n_seq)];
    }
    const int nrows = r1 - r0;                        // <= 256 by the grouping
    if (r0 < 0 || r1 > M || nrows <= 0 || nrows > BM) return;  // never, with well-formed groups

    if (tid < BN) bias_s[tid] = a.bh[h * BN + tid];

    // ---------------------------------------------------------- GEMM phase
    const char* Xt = static_cast<const char*>(a.X) + (int64_t)r0 * H * ES;
    const char* Wt = static_cast<const char*>(a.Wh) + (int64_t)h * BN * H * ES;
    const int64_t xbytes = (int64_t)(M - r0) * H * ES;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(Xt), (short)0,
        __builtin_amdgcn_readfirstlane((int)(xbytes > 0x7fffffff ? 0x7fffffff : xbytes)),
        kRsrcWord3);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Wt), (short)0, BN * H * ES, kRsrcWord3);
    const int lrow = lane / CPR;
    const int lchunk = (lane % CPR) ^ swz_key<RB>(wave * RPI + lrow);
    const int loff = lrow * H * ES + lchunk * 16;
    auto issue = [&](char* buf, int k0) __attribute__((always_inline)) {
      int kb = k0 * ES;
      asm volatile("" : "+s"(kb));
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int q = wave + i * NW;
        char* dst = buf + q * RPI * RB;
        if (i * NW * RPI < BM)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t*)dst, 16, loff,
                                                   kb + q * RPI * H * ES, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t*)dst, 16, loff,
                                                   kb + (q * RPI - BM) * H * ES, 0, 0);
      }
    };
    const int key = swz_key<RB>(l32);
    const int xrow = (wm * WTM + l32) * RB;
    const int wrow = (BM + wn * WTN + l32) * RB;
    int coff[KSTEPS][FCH];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
      for (int f = 0; f < FCH; ++f) coff[j][f] = (((j * KS + hh * FE) / CH + f) ^ key) * 16;
    int sc[TN];  // E4M3: E8M0 exponents of this lane's weight rows
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) sc[jj] = F8 ? a.Eh[h * BN + wn * WTN + jj * 32 + l32] : 127;

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
        typename TRO::frag fx[TM], fw[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const char* p = buf + xrow + i * 32 * RB;
          fx[i] = TRO::load2(reinterpret_cast<const TO*>(p + coff[j][0]),
                             reinterpret_cast<const TO*>(p + coff[j][FCH - 1]));
        }
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          const char* p = buf + wrow + jj * 32 * RB;
          fw[jj] = TRO::load2(reinterpret_cast<const TO*>(p + coff[j][0]),
                              reinterpret_cast<const TO*>(p + coff[j][FCH - 1]));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int jj = 0; jj < TN; ++jj) {
            if constexpr (F8)
              TRO::mma_s(acc[i][jj], fw[jj], fx[i], sc[jj]);
            else
              TRO::mma(acc[i][jj], fw[jj], fx[i]);
            if constexpr (!F8) {  // MFMA / LDS-read alternation: bf16 only
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // (3 % slower with E4M3
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  //  fragments, 6 % faster here)
            }
          }
      }
    };
  #define ALBERT_QA_WAIT_BARRIER() asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory")
    issue(lds0, 0);
    // kept as a loop: unrolled (six E4M3 slices), loads hoisted across
    // iterations spill
  #pragma unroll 1
    for (int kt = 0; kt < KT; kt += 2) {
      ALBERT_QA_WAIT_BARRIER();
      issue(lds1, (kt + 1) * BK);
      compute(lds0);
      ALBERT_QA_WAIT_BARRIER();
      if (kt + 2 < KT) issue(lds0, (kt + 2) * BK);
      compute(lds1);
    }
  #undef ALBERT_QA_WAIT_BARRIER
    __syncthreads();  // every wave is done with the stage buffers

    // Q and K rows [token][dim] at the start of lds0 / lds1, V^T [dim][token]
    // after them, dims 0..31 in lds0 and 32..63 in lds1.
    bf16* Qs = reinterpret_cast<bf16*>(lds0);
    bf16* Ks = reinterpret_cast<bf16*>(lds1);
    bf16* Vt0 = reinterpret_cast<bf16*>(lds0 + BM * LDQ * 2);
    bf16* Vt1 = reinterpret_cast<bf16*>(lds1 + BM * LDQ * 2);
    // acc[i][j][4q+e]: token wm*64 + 32i + l32, feature wn*96 + 32j + 8q + 4hh + e
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int tok = wm * WTM + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f0 = wn * WTN + j * 32 + 8 * q + 4 * hh;  // 4 consecutive features
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * q + e] + bias_s[f0 + e];
          if (f0 < D) {
            TR::store4(Qs + tok * LDQ + f0, o[0], o[1], o[2], o[3]);
          } else if (f0 < 2 * D) {
            TR::store4(Ks + tok * LDQ + (f0 - D), o[0], o[1], o[2], o[3]);
          } else {
            // V^T columns of rows past the group are zero: their keys get
            // probability 0, and 0 times a stale non-finite value would not
            // be 0 (rows past M hold whatever the workspace held)
            const int d0 = f0 - 2 * D;
            bf16* vt = d0 < 32 ? Vt0 + d0 * LDV : Vt1 + (d0 - 32) * LDV;
#pragma unroll
            for (int e = 0; e < 4; ++e) vt[e * LDV + tok] = tok < nrows ? (bf16)o[e] : (bf16)0.0f;
          }
        }
    }
    __syncthreads();

    // ----------------------------------------------------- attention phase
    const int qr = wave * 32 + l32;  // this lane's query (tile row)
    int ks = 0, ke = 0;              // its keys: tile rows [ks, ke)
    if (qr < nrows) {
      const int s = a.row_seq[r0 + qr];
      ks = a.cu[s] - r0;
      ke = a.cu[s + 1] - r0;
    }
    int kmin = qr < nrows ? ks : BM, kmax = ke;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, off, 64));
      kmax = max(kmax, __shfl_xor(kmax, off, 64));
    }
    const int kb0 = kmin / 32 * 32;  // wave-uniform key-block range
    const int kb1 = (kmax + 31) / 32 * 32;

    bf16x8 fq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fq[kk] = TR::load(Qs + qr * LDQ + kk * 16 + hh * 8);
    f32x16 o[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) { o[0][r] = 0.f; o[1][r] = 0.f; }
    float mrun = kNegInf, lrun = 0.f;
    // passes of up to 128 keys from the wave's first key block (for a wave
    // whose queries share one sequence, its start, as in the separate kernel)
    for (int kc = kb0; kc < kb1; kc += 128) {
      attend_pass<bf16>(o, mrun, lrun, fq, min(4, (kb1 - kc) / 32), ks - kc, ke - kc, hh,
                        [&](int b, int kk) { return TR::load(Ks + (kc + b * 32 + l32) * LDQ + hh * 8 + kk * 16); },
                        [&](int b, int c, int dt) {
                          const bf16* vp = (dt == 0 ? Vt0 : Vt1) + l32 * LDV + kc + b * 32 + 16 * c + 4 * hh;
                          return TR::load2x4(vp, vp + 8);
                        });
    }
    lrun += wave_xor(lrun, 32);
    // (every lane takes part in the swap of 16-byte pieces; only lanes with
    // a query of the group store)
    const float inv = qr < nrows ? 1.0f / lrun : 0.f;
    const int64_t orow = ((int64_t)r0 + qr) * H + h * D;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      if constexpr (F8) {
        if (qr < nrows) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = dt * 32 + 8 * q + 4 * hh;
            store4_as<bf16, F8>(a.ctx, orow + d, o[dt][4 * q + 0] * inv, o[dt][4 * q + 1] * inv,
                                o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv);
          }
        }
      } else {
        uint32_t pk[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pk[q][0] = pack_bf16x2(o[dt][4 * q + 0] * inv, o[dt][4 * q + 1] * inv);
          pk[q][1] = pack_bf16x2(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv);
        }
        uint4 p0, p1;
        swap_runs_to_pieces(pk, p0, p1);
        if (qr < nrows) {
          bf16* cp = static_cast<bf16*>(a.ctx) + orow + dt * 32 + 8 * hh;
          *reinterpret_cast<uint4*>(cp) = p0;
          *reinterpret_cast<uint4*>(cp + 16) = p1;
        }
      }
    }
  };

  // One pair per block.  Workgroups are dealt to the 8 XCDs round-robin,
  // so block b runs on XCD b % 8 as its (b / 8)-th block there.  The pairs
  // that exist (with greedy groups their count is known on the device only;
  // the grid covers the S-grouping count, never fewer) are cut into 8
  // contiguous ranges, one per XCD, taken by that XCD's first blocks: the
  // 12 heads of a group share one XCD (or two at a range boundary), so its
  // rows of X are read from that XCD's L2 after the first head, and every
  // XCD gets the same number of pairs.  (A persistent loop over pairs made
  // the compiler hold addresses across it, spilling with E4M3 fragments,
  // and slowed the next kernels.)
  const int npairs = a.groups ? min(a.groups[0] * NH, a.n_pairs) : a.n_pairs;
  const int xcd = (int)blockIdx.x % 8;
  const int plo = (int)((int64_t)npairs * xcd / 8), phi = (int)((int64_t)npairs * (xcd + 1) / 8);
  const int pair = plo + (int)blockIdx.x / 8;
  if (pair < phi) one(pair / NH, pair % NH);
}

}  // namespace albert
