// Fused Q|K|V projection and attention for one head of a group of whole
// sequences (bf16 storage; bf16 or E4M3 matrix-product operands).
//
// The layer's q, k, v projections ("Inside One Real ALBERT Layer", step 3)
// and the masked-softmax attention (step 4; "How Kokoro TTS Works and Where
// CKE Stands", "What ALBERT does here") computed in one workgroup, so q, k
// and v of the group never leave the chip.  A (group, head) pair is a group
// of consecutive whole sequences of at most 256 rows in all (packed greedily
// on the device, or S = 256 / longest per group, chosen on the host, for
// very large batches) and one head h: the workgroup computes the 192
// projected features of head h (q/8 | k | v, the query scale folded into
// the weights) for those rows on the matrix cores, stores them in LDS as
// bf16 (the same storage point as the unfused path) and runs the attention
// of every query against the keys of its own sequence.  Only the context
// leaves the workgroup.
//
// Persistence (bf16 operands).  One workgroup per CU walks its share of
// the pairs (E4M3 operands: one workgroup per pair, see PERSIST).  Its
// last K slice consumed, a pair's Q, K and V^T go to LDS (region A, which
// also holds the odd K slices), and the DMA of the next pair's first K slice
// (region B, the even slices) is issued before the attention phase, so that
// slice's latency hides behind the attention instead of starting the next
// pair's products cold.  Nothing else touches global memory during the
// attention phase (each lane's key range is read before the prefetch, the
// next bias arrives by DMA with the slice), and the context is written with
// buffer stores whose range check drops rows past the group, so every wave
// issues the same stores and the next wait can leave exactly those in
// flight.
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
// Attention phase: Q and K are row-major [token][64] with 16-byte chunks
// XOR-swizzled by row (conflict-free fragment reads without padding), V^T
// is [dim][token]; wave w owns queries 32w .. 32w+31 of the tile, one per
// lane, as in attention.hpp (S^T = K Q^T, online softmax per lane with the
// partner half-wave, O^T = V^T P^T); a lane's keys are those of its own
// sequence, so key blocks outside it are masked per lane.  With E4M3
// operands the context is written as E4M3 codes (its one consumer is the
// output projection's matrix product).
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
  constexpr int WGN = 2, NW = 8;
  constexpr int WTM = 64, WTN = 96, TM = 2, TN = 3;
  constexpr int RB = 128, CPR = RB / 16, BK = RB / ES, RPI = 1024 / RB;
  constexpr int KS = F8 ? 64 : 16;         // K per MFMA step
  constexpr int FE = F8 ? 32 : 8;          // elements per lane per step
  constexpr int CH = 16 / ES, FCH = FE / CH;  // chunks per fragment
  constexpr int NINST = (BM + BN) / RPI, IPW = NINST / NW;
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int KSTEPS = BK / KS, KT = H / BK;
  constexpr int LDV = BM + 4;              // V^T rows (520 bytes: 8-byte aligned, conflict-free)
  constexpr int QK_BYTES = BM * D * 2;     // Q (or K): 256 rows of 128 bytes
  constexpr int VT_BYTES = 32 * LDV * 2;   // one half of V^T (32 dims)
  constexpr int ATT = 2 * QK_BYTES + 2 * VT_BYTES;
  constexpr int NST = F8 ? 8 : 4;          // context stores per lane and pair
  // E4M3 fragments are twice as wide: carried around the pair loop they
  // spill (and a spill reload waits for the prefetch), so with E4M3
  // operands every workgroup takes one pair and the host launches one
  // workgroup per pair
  constexpr bool PERSIST = !F8;
  static_assert(NINST % NW == 0 && (BM / RPI) % NW == 0 && NW % 2 == 0, "DMA split");
  static_assert(KT % 2 == 0 && KSTEPS >= 1, "two stages of whole MFMA steps");
  static_assert(ATT >= STAGE, "region A holds a stage");
  // region A: odd K slices, then Q | K | V^T (dims 0-31) | V^T (dims 32-63);
  // region B: even K slices (the next pair's first slice during attention)
  __shared__ __attribute__((aligned(1024))) char lds_a[ATT];
  __shared__ __attribute__((aligned(1024))) char lds_b[STAGE];
  __shared__ __attribute__((aligned(16))) float bias_s[2][256];  // this pair's and the next pair's biases
  __shared__ unsigned char exp_s[F8 ? NH * BN : 4];              // E4M3: every head's row exponents

  if (*a.status != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hh = lane >> 5;
  const int M = a.cu[a.n_seq];

  // The pairs that exist (with greedy groups their count is known on the
  // device only; the grid covers at most the S-grouping count) are cut into
  // 8 contiguous ranges, one per XCD (workgroups are dealt to the XCDs
  // round-robin): the 12 heads of a group share one XCD (two at a range
  // boundary), so its rows of X are read from that XCD's L2 after the first
  // head.  Block b walks pairs lo + b/8, lo + b/8 + per, ... of its XCD's
  // range.
  const int npairs = a.groups ? min(a.groups[0] * NH, a.n_pairs) : a.n_pairs;
  const int xcd = (int)blockIdx.x % 8, per = (int)gridDim.x / 8;
  const int plo = (int)((int64_t)npairs * xcd / 8), phi = (int)((int64_t)npairs * (xcd + 1) / 8);
  int pair = plo + (int)blockIdx.x / 8;
  if (pair >= phi) return;

  // rows [r0, r1) of group grp
  auto group_rows = [&](int grp, int& g0, int& g1) __attribute__((always_inline)) {
    if (a.groups) {
      g0 = a.groups[1 + grp];
      g1 = a.groups[2 + grp];
    } else {
      const int s0 = grp * a.S;
      g0 = a.cu[s0];
      g1 = a.cu[min(s0 + a.S, a.n_seq)];
    }
  };

  if constexpr (F8) {
    for (int i = tid; i < NH * BN; i += NW * 64) exp_s[i] = a.Eh[i];
    __syncthreads();
  }

  // DMA of one K slice of the current pair's rows and head into buf; the
  // bias of head h into bias_s[bsel] (wave 0, one 1 KB instruction whose
  // lanes past the 192 floats read zeros)
  const int lrow = lane / CPR;
  const int lchunk = (lane % CPR) ^ swz_key<RB>(wave * RPI + lrow);
  const int loff = lrow * H * ES + lchunk * 16;
  __amdgpu_buffer_rsrc_t xr, wr;
  auto set_pair = [&](int g0, int hd) __attribute__((always_inline)) {
    const char* Xt = static_cast<const char*>(a.X) + (int64_t)g0 * H * ES;
    const char* Wt = static_cast<const char*>(a.Wh) + (int64_t)hd * BN * H * ES;
    const int64_t xbytes = (int64_t)(M - g0) * H * ES;
    xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(Xt), (short)0,
        __builtin_amdgcn_readfirstlane((int)(xbytes > 0x7fffffff ? 0x7fffffff : xbytes)), kRsrcWord3);
    wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Wt), (short)0, BN * H * ES, kRsrcWord3);
  };
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
  auto issue_bias = [&](int hd, int sel) __attribute__((always_inline)) {
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.bh + hd * BN), (short)0, BN * 4, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_ptr_t*)&bias_s[sel][0], 16, lane * 16, 0, 0, 0);
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

  // Q and K: row t at t * 128 bytes, 16-byte chunk c of it at chunk c ^ (t % 8)
  bf16* Qs = reinterpret_cast<bf16*>(lds_a);
  bf16* Ks = reinterpret_cast<bf16*>(lds_a + QK_BYTES);
  bf16* Vt0 = reinterpret_cast<bf16*>(lds_a + 2 * QK_BYTES);
  bf16* Vt1 = reinterpret_cast<bf16*>(lds_a + 2 * QK_BYTES + VT_BYTES);
  auto qk_at = [](int t, int d) __attribute__((always_inline)) {  // element offset of (t, d)
    return t * D + ((((d >> 3) ^ (t & 7)) << 3) | (d & 7));
  };

  // rows of a group from the device's grouping: checked before any DMA
  // addresses them (never false with well-formed groups)
  auto rows_ok = [&](int g0, int g1) __attribute__((always_inline)) {
    return g0 >= 0 && g1 <= M && g1 - g0 > 0 && g1 - g0 <= BM;
  };

  // the first pair: its first slice and bias
  int r0, r1;
  group_rows(pair / NH, r0, r1);
  if (!rows_ok(r0, r1)) return;
  int h = pair % NH;
  set_pair(r0, h);
  issue(lds_b, 0);
  issue_bias(h, 0);
  int bsel = 0;
  bool first = true;

#define ALBERT_QA_WAIT_BARRIER(N) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory")
  // kept as loops: unrolled (six E4M3 slices), loads hoisted across
  // iterations spill
#pragma unroll 1
  for (;;) {
    const int nrows = r1 - r0;  // <= 256 by the grouping
    int sc[TN];                 // E4M3: E8M0 exponents of this lane's weight rows
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      if constexpr (F8)
        sc[jj] = exp_s[h * BN + wn * WTN + jj * 32 + l32];
      else
        sc[jj] = 127;
    }

    // ---------------------------------------------------------- GEMM phase
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
    // even slices in region B, odd slices in region A; the first wait of a
    // pair after the first leaves the previous pair's context stores (the
    // youngest NST operations of every wave) in flight
#pragma unroll 1
    for (int kt = 0; kt < KT; kt += 2) {
      if (kt == 0 && !first)
        ALBERT_QA_WAIT_BARRIER(NST);
      else
        ALBERT_QA_WAIT_BARRIER(0);
      issue(lds_a, (kt + 1) * BK);
      compute(lds_b);
      ALBERT_QA_WAIT_BARRIER(0);
      if (kt + 2 < KT) issue(lds_b, (kt + 2) * BK);
      compute(lds_a);
    }

    // each lane's keys: tile rows [ks, ke) of its query's sequence (read
    // now, before the next pair's DMA, so that no global load is waited for
    // while that DMA is in flight)
    const int qr = wave * 32 + l32;  // this lane's query (tile row)
    int ks = 0, ke = 0;
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
    const int kb0 = __builtin_amdgcn_readfirstlane(kmin / 32 * 32);  // wave-uniform key-block range
    const int kb1 = __builtin_amdgcn_readfirstlane((kmax + 31) / 32 * 32);
    __syncthreads();  // every wave is done with both stage buffers

    // Q, K, V^T of the pair into region A
    // acc[i][j][4q+e]: token wm*64 + 32i + l32, feature wn*96 + 32j + 8q + 4hh + e;
    // the 32-feature tile j of wave column wn is q (wn 0, j 0-1), k (wn 0,
    // j 2; wn 1, j 0) or v (wn 1, j 1-2): two static paths per wave column
    const float* bias = bias_s[bsel];
    auto put = [&](int i, int j, int part, int c0) __attribute__((always_inline)) {
      // tile (i, j) holds features c0 .. c0+31 of part (0 q, 1 k, 2 v)
      const int tok = wm * WTM + i * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int fl = 8 * q + 4 * hh;  // 4 consecutive features c0 + fl ..
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * q + e] + bias[part * D + c0 + fl + e];
        if (part < 2) {
          // the swizzled address is recomputed at each store (an opaque copy
          // of the row): precomputed for every (i, q) they would be spilled
          int t = tok;
          asm volatile("" : "+v"(t));
          TR::store4((part == 0 ? Qs : Ks) + qk_at(t, c0 + fl), o[0], o[1], o[2], o[3]);
        } else {
          // V^T columns of rows past the group are zero: their keys get
          // probability 0, and 0 times a stale non-finite value would not
          // be 0 (rows past M hold whatever the workspace held)
          bf16* vt = (c0 == 0 ? Vt0 : Vt1) + fl * LDV + tok;
#pragma unroll
          for (int e = 0; e < 4; ++e) vt[e * LDV] = tok < nrows ? (bf16)o[e] : (bf16)0.0f;
        }
      }
    };
    // weight tile by weight tile: both token tiles of a weight tile share
    // its bias reads
    if (wn == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 1, 0, 32);
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 2, 1, 0);
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 0, 1, 32);
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 1, 2, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) put(i, 2, 2, 32);
    }

    // the next pair: its first slice and bias, in flight during the attention
    // (issued after the stores above: no spill reload may follow it)
    __builtin_amdgcn_sched_barrier(0);
    const int nxt = pair + per;
    const int cr0 = r0, ch = h;
    bool more = false;
    if (PERSIST && nxt < phi) {
      int n0, n1;
      group_rows(nxt / NH, n0, n1);
      more = rows_ok(n0, n1);
      if (more) {
        r0 = n0;
        r1 = n1;
        h = nxt % NH;
        set_pair(r0, h);
        issue_bias(h, bsel ^ 1);
        issue(lds_b, 0);
      }
    }
    // Q, K and V^T are written (a plain barrier: the DMA just issued into
    // region B is not waited for)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ----------------------------------------------------- attention phase
    bf16x8 fq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fq[kk] = TR::load(Qs + qk_at(qr, kk * 16 + hh * 8));
    f32x16 o[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) { o[0][r] = 0.f; o[1][r] = 0.f; }
    float mrun = kNegInf, lrun = 0.f;
    // passes of up to 128 keys from the wave's first key block (for a wave
    // whose queries share one sequence, its start, as in the separate kernel)
    for (int kc = kb0; kc < kb1; kc += 128) {
      attend_pass<bf16>(o, mrun, lrun, fq, min(4, (kb1 - kc) / 32), ks - kc, ke - kc, hh,
                        [&](int b, int kk) { return TR::load(Ks + qk_at(kc + b * 32 + l32, hh * 8 + kk * 16)); },
                        [&](int b, int c, int dt) {
                          const bf16* vp = (dt == 0 ? Vt0 : Vt1) + l32 * LDV + kc + b * 32 + 16 * c + 4 * hh;
                          return TR::load2x4(vp, vp + 8);
                        });
    }
    lrun += wave_xor(lrun, 32);

    // the context: NST buffer stores per lane, over the group's rows only
    // (rows past it fall outside the resource and are dropped)
    const float inv = qr < nrows ? 1.0f / lrun : 0.f;
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(a.ctx) + (int64_t)cr0 * H * ES, (short)0,
        __builtin_amdgcn_readfirstlane(nrows * H * ES), kRsrcWord3);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      if constexpr (F8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = dt * 32 + 8 * q + 4 * hh;
          __builtin_amdgcn_raw_buffer_store_b32(
              pack_e4m3x4(o[dt][4 * q + 0] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                          o[dt][4 * q + 3] * inv),
              cr, qr * H + ch * D + d, 0, 0);
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
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const int off = (qr * H + ch * D + dt * 32 + 8 * hh) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{p0.x, p0.y, p0.z, p0.w}, cr, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{p1.x, p1.y, p1.z, p1.w}, cr, off + 32, 0, 0);
      }
    }
    if (!PERSIST || !more) break;
    pair = nxt;
    bsel ^= 1;
    first = false;
  }
#undef ALBERT_QA_WAIT_BARRIER
}

}  // namespace albert
