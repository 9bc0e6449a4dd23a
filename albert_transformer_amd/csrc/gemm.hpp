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
//   EPI_LN_ACT  store LeakyReLU(LN(Y) * g + beta), no residual (the text
//             path's convolution blocks).  X is then the layer input [M, C]
//             read as the convolution's unfolded input: K = taps * C, and
//             column j*C + c of row m is channel c of input row
//             m + j - taps/2 when that row is in m's sequence (bit j of
//             taps[m]), else zero.  The DMA reads the shifted rows directly
//             (an absent tap reads past the buffer's range, which returns
//             zeros), so no unfolded copy is made.
//   EPI_LN_PAIR as EPI_LN, with the row split over two blocks of BN = N/2
//             features that run at the same time: each reduces its half of
//             every row to a mean and a sum of squared deviations, the two
//             blocks swap these through device memory, and both combine
//             them the same way (Chan, Golub and LeVeque's pairwise update),
//             so the row statistics are identical in both halves
//   EPI_OUT   store Y as fp32 into the caller's output, packed row m going to
//             out row seq(m) * T + pos(m) (padded) or m (packed)
//   EPI_PART  split K: tile (s, m, n) sums K slices [s*K/S, (s+1)*K/S) and
//             stores the fp32 sum, without bias, at part[s][m][n]; a second
//             kernel (splitk.hpp) adds the S partial sums in order and applies
//             the epilogue.  For very small batches, whose tiles would
//             otherwise occupy a few CUs.
//
// Tiling.  A block computes BM token rows x BN output features with WGM x WGN
// waves; each wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA tiles.
// Weights are the MFMA A operand and tokens the B operand, so each lane ends
// up owning one token and runs of 4 consecutive features: stores are 4-wide,
// and LayerNorm row statistics reduce inside a lane, then across the two
// half-waves, then across the WGN waves through LDS.
//
// Staging.  Each K slice of RB bytes per row (X rows then W rows) goes from
// global memory straight into LDS with gfx950's buffer_load ... lds DMA: one
// wave instruction fills 1 KB of LDS, 16 bytes per lane in lane order, with
// no register round trip.  Because the DMA fixes where each lane's 16 bytes
// land, bank conflicts of the fragment reads are avoided by choosing which
// 16-byte chunk each lane fetches: physical chunk p of row r holds logical
// chunk p ^ key(r), key(r) = (r / (256/RB)) % (RB/16), so the 8 rows read
// by 8 consecutive lanes fall on distinct banks.  Each stage has its own LDS
// array (the loop is unrolled so each step names its buffers statically):
// while the matrix cores consume one slice, the DMA fills the others.
//
// Persistence.  The grid holds at most one block per CU (a multiple of 8);
// each block walks tiles slot, slot + G, slot + 2G, ...  Once the last slice
// of a tile has been read out of LDS, the block issues the DMA of the next
// tile's first slices and loads the next tile's epilogue vectors, and only
// then runs the current tile's epilogue: the next tile's fill latency hides
// behind the epilogue's arithmetic and stores.  Tiles of one round are
// numbered so that each XCD (workgroups are dealt to the 8 XCDs
// round-robin) gets a contiguous range, features fastest, so blocks running
// together on one XCD share X rows and weight columns in that XCD's L2.
//
// Low precision (F8).  X and W are OCP FP8 E4M3 codes and each weight row
// carries a power-of-two scale (an E8M0 exponent, applied by the matrix
// core as A's per-row scale, so the product is exact up to accumulation).
// Outputs keep the storage type T except the GELU output, whose only
// consumer is the next product (E4M3); the bias and LayerNorm epilogues can
// also write an E4M3 copy of their output (Y8) for the next product while Y
// stays the bf16 residual stream.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace albert {

enum Epi { EPI_BIAS = 0, EPI_GELU = 1, EPI_LN = 2, EPI_OUT = 3, EPI_LN_ACT = 4, EPI_LN_PAIR = 5,
           EPI_PART = 6 };

struct GemmArgs {
  const void* X;       // [M, K] activations, row stride ldx (elements)
  int64_t ldx;
  const void* W;       // [N, K] weights, row stride K
  const unsigned char* wexp;  // F8: [N] E8M0 exponent of each weight row
  const unsigned char* taps;  // EPI_LN_ACT: [M] the convolution taps inside each row's sequence
  const float* bias;   // [N]
  void* Y;             // [M, N] output (EPI_BIAS / EPI_GELU / EPI_LN), stride ldy
  int64_t ldy;
  void* Y8;            // F8, EPI_BIAS (not deferred) / EPI_LN: E4M3 copy of Y, or null
  int64_t ldy8;
  const void* R;       // [M, N] residual (EPI_LN), stride ldr
  int64_t ldr;
  const float* ln_g;   // [N] (EPI_LN, EPI_LN_ACT)
  const float* ln_b;
  float eps;
  float slope;         // EPI_LN_ACT: LeakyReLU negative slope
  float* out;          // EPI_OUT: fp32 output rows of N
  const int* row_seq;  // EPI_OUT padded mapping
  const int* row_pos;
  int out_T;           // EPI_OUT: padded T, or 0 for packed rows
  const int* status;
  const int* m_ptr;    // device: number of valid rows M
  int N, K;
  int n_tiles;         // N / BN
  // EPI_LN_PAIR: per row tile 4*BM + 8 words (see the epilogue), cleared
  // before the first launch that uses them; this launch's tag (1..4095,
  // distinct among the launches since the clear); polls of the partner's
  // statistics before handing this half over
  unsigned long long* xch;
  int xtag;
  int pair_spin;
  // EPI_LN_PAIR: [M, 2, BN] fp32, where a half that hands its rows over
  // leaves its values before normalisation (row m, half h at (2m + h) * BN;
  // both halves may try to hand over, and only one of them wins), so that
  // the partner normalises exactly the values the half itself would have
  float* hand;
  // EPI_PART: S splits of K; partial sums [S][ldp][N] fp32
  int ksplit;
  float* part;
  int64_t ldp;
};

// LayerNorm output of one value: (v - mean) * rstd * gain + shift, written
// once here so that every path that normalises a value (a block's own
// columns, or a partner's handed-over columns) rounds it the same way.
__device__ __forceinline__ float ln_out(float v, float mean, float rstd, float gain, float shift) {
  return __builtin_fmaf((v - mean) * rstd, gain, shift);
}

// Polls (each after a short sleep) of a block that is known to be running
// before giving up and reporting ALBERT_E_SYNC.
constexpr int kPairSpin = 1 << 20;


typedef __attribute__((address_space(3))) void lds_ptr_t;

// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format, no swizzle, out-of-range reads return zero.
constexpr int kRsrcWord3 = 0x00020000;

template <int RB>
__device__ __forceinline__ int swz_key(int row) {
  return (row / (256 / RB)) % (RB / 16);
}

// Wait until this wave has at most N vector-memory operations outstanding,
// then meet the other waves of the block.
#define ALBERT_WAIT_BARRIER(N) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory")

template <typename T, bool F8, int BM, int BN, int WGM, int WGN, int RB, int STAGES, int EPI,
          bool DEFER, int KR = 0>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_kernel(GemmArgs g) {
  typedef typename std::conditional<F8, fp8, T>::type TO;  // operand codes
  typedef Tr<TO> TR;                                         // operand fragments
  typedef Tr<T> TS;                                          // storage
  constexpr int ES = sizeof(TO);
  constexpr int NW = WGM * WGN;
  constexpr int NT = NW * 64;
  constexpr int CH = 16 / ES;                 // elements per 16-byte chunk
  constexpr int CPR = RB / 16;                // chunks per staged row
  constexpr int BK = RB / ES;                 // K elements per slice
  constexpr int KS = F8 ? 64 : 16;            // K per MFMA step
  constexpr int FE = F8 ? 32 : 8;             // elements per lane per step
  constexpr bool YF8 = F8 && EPI == EPI_GELU; // output stored as E4M3 codes
  constexpr int YES = YF8 ? 1 : (int)sizeof(T);
  constexpr int RPI = 1024 / RB;              // rows one DMA instruction fills
  constexpr int NINST = (BM + BN) / RPI;      // DMA instructions per slice
  constexpr int IPW = NINST / NW;             // ... per wave
  constexpr int STAGE = (BM + BN) * RB;       // bytes per slice
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KSTEPS = BK / KS;             // MFMA k-steps per slice
  constexpr int FCH = FE / CH;                // chunks per fragment (1 bf16, 2 fp32 / E4M3)
  constexpr bool PAIR = EPI == EPI_LN_PAIR;                // LayerNorm row split over two blocks
  constexpr bool LNE = EPI == EPI_LN || EPI == EPI_LN_ACT || PAIR;  // LayerNorm epilogue
  constexpr bool RES = EPI == EPI_LN || PAIR;              // with a residual
  constexpr bool CONV = EPI == EPI_LN_ACT;                 // convolution taps from shifted rows
  // bf16 rows are read and written as 16-byte pieces (swap_runs_to_pieces);
  // E4M3 outputs keep one 4-byte store per run
  constexpr bool P16 = std::is_same<T, bf16>::value;
  constexpr int kMaxTaps = 7;
  constexpr int NVEC = LNE ? 3 : 1;          // bias (+ LayerNorm gain, shift)
  constexpr int VPT = (BN + NT - 1) / NT;     // vector elements per thread
  static_assert(NINST % NW == 0, "DMA split");
  static_assert((BM / RPI) % NW == 0, "each DMA slot must be all-X or all-W");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(RB == 64 || RB == 128, "row bytes");
  static_assert(KSTEPS >= 1, "slice shorter than one MFMA step");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(KR >= 0 && KR < STAGES, "K slices past the last whole round");
  static_assert(EPI != EPI_LN_PAIR || 2 * BM <= NT, "one thread per row statistic");
  static_assert(!CONV || BM / RPI == NW, "convolution: one input row per lane and slice");
  static_assert(IPW * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(CPR == 8 ? (NW % 2 == 0) : true, "swizzle key must not depend on i");
  // Deferred stores: bf16 (or E4M3) outputs of tile i are kept in registers
  // and written in NB batches of SB stores during the first NB K-slices of
  // tile i+1.
  // bf16 outputs are held as 16-byte pieces (swap_runs_to_pieces, two per
  // 32x32 tile); E4M3 outputs as one 4-byte word per run of 4
  constexpr bool DP16 = DEFER && !YF8;
  constexpr int NST = TM * TN * (DP16 ? 2 : 4);  // stores per lane per tile
  constexpr int NB = 8, SB = NST / NB;
  constexpr int HW = YF8 ? 1 : 2;             // 32-bit words per store
  // LayerNorm residual rows by LDS DMA (bf16 storage): between the K loop
  // and the next tile's prologue the staging buffers are free, and each wave
  // loads its own 16-byte residual pieces into a private region of them (one
  // 1 KB instruction per 32-column tile and piece, each lane's piece at its
  // own slot) and reads back its own slots.  So every residual load of the
  // region is in flight at once and holds no registers while it is; loaded
  // into registers, the compiler (at its register limit with the LayerNorm
  // tile's accumulators) waited for each 16 bytes in turn.  Both 32-row
  // halves of a wave's rows at once when the regions fit, else one half
  // after the other.
  constexpr int RWB = TN * 2 * 1024;                       // one half's pieces per wave
  constexpr bool RBOTH = STAGE / (TM * RWB) >= 1 && NW <= STAGES * (STAGE / (TM * RWB));
  constexpr int RREG = RBOTH ? TM * RWB : RWB;             // bytes of a wave's region
  constexpr int WPA = STAGE / RREG;                        // regions per staging buffer
  constexpr bool RDMA = RES && P16 && WPA >= 1 && NW <= STAGES * WPA;
  static_assert(!DEFER || (std::is_same<T, bf16>::value && STAGES == 2 &&
                           (EPI == EPI_BIAS || EPI == EPI_GELU) && NST % NB == 0 &&
                           SB <= 63 && TN % (NB / TM) == 0),
                "deferred stores: bf16, two stages, bias/GELU epilogues");

  // One LDS array per stage, so that alias analysis sees that the DMA into
  // one stage never touches the stage being read.
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds2[STAGES > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char lds3[STAGES > 3 ? STAGE : 16];
  // Epilogue vectors, double-buffered across consecutive tiles, and the
  // LayerNorm cross-wave row reduction.
  __shared__ __attribute__((aligned(16))) float vecs[2][NVEC][BN];
  __shared__ float red[LNE ? (PAIR ? 2 : 1) * WGN * BM : 1];
  // EPI_LN_PAIR: per row, mean and squared deviations of the first half of
  // the features, then of the second
  __shared__ float pst[PAIR ? 4 * BM : 1];
  __shared__ int pflag;

  if (*g.status != 0) return;
  const int M = *g.m_ptr;
  constexpr bool PART = EPI == EPI_PART;
  const int S = PART ? g.ksplit : 1;
  const int mn_tiles = ((M + BM - 1) / BM) * g.n_tiles;
  const int ntiles = mn_tiles * S;
  const int G = gridDim.x;  // the host launches a multiple of 8 blocks (EPI_LN_PAIR: of 16)
  int tile = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  if (tile >= ntiles) return;
  // EPI_LN_PAIR: n_tiles = 2 and G / 8 is even, so the block 8 away (on
  // the same XCD) holds tile ^ 1, the other half of the same rows, in the
  // same round

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hh = lane >> 5;

  // ------------------------------------------------------- per-tile state
  int m0 = 0, n0 = 0;
  int ks0 = 0;  // EPI_PART: this tile's split of K, and its first K element
  int kbase = 0;
  int xb0 = 0;  // CONV: first input row of the X resource (taps/2 above the tile)
  __amdgpu_buffer_rsrc_t xr, wr;
  int sc[TN];  // F8: E8M0 exponents of this lane's weight rows
#pragma unroll
  for (int j = 0; j < TN; ++j) sc[j] = 127;
  // Buffer resources over the tile's rows.  The range check covers only the
  // per-lane offset (the row offset of a DMA instruction is in its scalar
  // offset), so X rows at or past M read whatever the buffer holds there;
  // each token is one column of the product, and those columns are never
  // stored.
  auto setup = [&](int t) __attribute__((always_inline)) {
    ks0 = PART ? t / mn_tiles : 0;
    kbase = PART ? ks0 * (g.K / S) : 0;
    t = PART ? t % mn_tiles : t;
    m0 = (t / g.n_tiles) * BM;
    n0 = (t % g.n_tiles) * BN;
    xb0 = CONV ? max(m0 - (g.K / (int)g.ldx) / 2, 0) : m0;
    const char* Xt = static_cast<const char*>(g.X) + (int64_t)xb0 * g.ldx * (int64_t)ES;
    const char* Wt = static_cast<const char*>(g.W) + (int64_t)n0 * g.K * (int64_t)ES;
    const int64_t xbytes = (int64_t)(M - xb0) * g.ldx * (int64_t)ES;
    const int64_t wbytes = (int64_t)(g.N - n0) * g.K * (int64_t)ES;
    const int xrec = __builtin_amdgcn_readfirstlane((int)(xbytes > 0x7fffffff ? 0x7fffffff : xbytes));
    const int wrec = __builtin_amdgcn_readfirstlane((int)(wbytes > 0x7fffffff ? 0x7fffffff : wbytes));
    xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Xt), (short)0, xrec, kRsrcWord3);
    wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Wt), (short)0, wrec, kRsrcWord3);
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < TN; ++j) sc[j] = g.wexp[n0 + wn * WTN + j * 32 + l32];
    }
  };

  // DMA sources.  Instruction i of this wave fills rows q*RPI .. q*RPI+RPI-1
  // of the slice, q = wave + i*NW (X rows first, then W rows); lane t takes
  // row q*RPI + t/CPR and logical chunk (t%CPR) ^ key(row).  For the tile
  // shapes used here the key does not depend on i, so one 32-bit per-lane
  // byte offset (VGPR) plus a uniform per-instruction offset (SGPR) address
  // every load.
  const int lrow = lane / CPR;
  const int lchunk = (lane % CPR) ^ swz_key<RB>(wave * RPI + lrow);
  const int xoff = lrow * (int)g.ldx * ES + lchunk * 16;
  const int woff = lrow * g.K * ES + lchunk * 16;
  const int xrow_b = (int)g.ldx * ES;  // bytes per X row
  const int wrow_b = g.K * ES;
  // CONV: this lane's input-row offset for each tap (its X row is
  // m0 + wave*RPI + lrow), or one past any buffer range for an absent tap
  int xo[CONV ? kMaxTaps : 1];
  auto conv_offsets = [&]() __attribute__((always_inline)) {
    if constexpr (CONV) {
      const int half = (g.K / (int)g.ldx) / 2;
      const int r = m0 + wave * RPI + lrow;
      const unsigned mask = r < M ? (unsigned)g.taps[r] : 0u;
#pragma unroll
      for (int j = 0; j < kMaxTaps; ++j)
        xo[j] = ((mask >> j) & 1u) ? (r + j - half - xb0) * xrow_b + lchunk * 16 : 0x7FFFFFF0;
    }
  };
  auto issue = [&](char* buf, int k0) __attribute__((always_inline)) {
    k0 += kbase;
    int kb = k0 * ES;
    // keep the per-slice offset opaque so the compiler does not precompute
    // (and keep live) every slice's per-instruction offsets
    asm volatile("" : "+s"(kb));
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave + i * NW;
      char* dst = buf + q * RPI * RB;
      if (i * NW * RPI < BM) {  // compile-time per i (static_assert above)
        if constexpr (CONV) {  // tap j = k0 / C, channels from k0 - j*C (a slice holds one tap)
          const int C = (int)g.ldx, j = k0 / C;
          const int vo = j == 0 ? xo[0] : j == 1 ? xo[1] : j == 2 ? xo[2] : j == 3 ? xo[3]
                       : j == 4 ? xo[4] : j == 5 ? xo[5] : xo[6];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t*)dst, 16, vo, (k0 - j * C) * ES,
                                                   0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t*)dst, 16, xoff,
                                                   kb + q * RPI * xrow_b, 0, 0);
        }
      } else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t*)dst, 16, woff,
                                                 kb + (q * RPI - BM) * wrow_b, 0, 0);
    }
  };
#define ALBERT_BUF(i) ((i) == 0 ? lds0 : (i) == 1 ? lds1 : (i) == 2 ? lds2 : lds3)
  auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(ALBERT_BUF(s), s * BK);
  };

  // Epilogue vectors go through registers into LDS; loading them for the
  // next tile before the current epilogue hides their latency, and the
  // epilogue then reads LDS only (on gfx9 a wait for a global load also
  // waits for every earlier store).
  float vreg[NVEC][VPT];
  auto vload = [&](int nb0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = tid + k * NT;
      if (c < BN) {
        vreg[0][k] = g.bias[nb0 + c];
        if constexpr (LNE) {
          vreg[1 % NVEC][k] = g.ln_g[nb0 + c];
          vreg[2 % NVEC][k] = g.ln_b[nb0 + c];
        }
      }
    }
  };
  auto vstore = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = tid + k * NT;
      if (c < BN) {
#pragma unroll
        for (int v = 0; v < NVEC; ++v) vecs[b][v][c] = vreg[v][k];
      }
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
    for (int f = 0; f < FCH; ++f) coff[j][f] = (((j * KS + hh * FE) / CH + f) ^ key) * 16;

  f32x16 acc[TM][TN];

  // Deferred-store state: packed bf16 pairs, the output resource of the tile
  // they belong to (rows at or past M fall outside it and are dropped by the
  // hardware range check, so every batch issues the same number of stores),
  // and per-row byte offsets.  Before the first tile the resource is empty.
  uint32_t held[DEFER && !DP16 ? TM : 1][DEFER && !DP16 ? TN : 1][4][HW];
  uint4 hp[DP16 ? TM : 1][DP16 ? TN : 1][2];
  __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(g.Y, (short)0, 0, kRsrcWord3);
  int hoff[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) hoff[i] = 0;
  if constexpr (DP16) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) hp[i][j][0] = hp[i][j][1] = uint4{0u, 0u, 0u, 0u};
  } else if constexpr (DEFER) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int w = 0; w < HW; ++w) held[i][j][q][w] = 0u;
  }
  // batch b: token tile i = b / (NB/TM), column tiles j in [jb, jb + TN/(NB/TM))
  auto store_batch = [&](int b) __attribute__((always_inline)) {
    if constexpr (DP16) {
      constexpr int JPB = TN / (NB / TM);
      const int i = b / (NB / TM), jb = (b % (NB / TM)) * JPB;
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int jj = 0; jj < JPB; ++jj) {
        const int off = hoff[i] + (jb + jj) * 32 * YES;
        const uint4 a = hp[i][jb + jj][0], c = hp[i][jb + jj][1];
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{a.x, a.y, a.z, a.w}, yr, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{c.x, c.y, c.z, c.w}, yr, off + 16 * YES, 0, 0);
      }
    } else if constexpr (DEFER) {
      constexpr int JPB = TN / (NB / TM);
      const int i = b / (NB / TM), jb = (b % (NB / TM)) * JPB;
#pragma unroll
      for (int jj = 0; jj < JPB; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int off = hoff[i] + ((jb + jj) * 32 + 8 * q) * YES;
          if constexpr (HW == 2) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            u32x2 v = {held[i][jb + jj][q][0], held[i][jb + jj][q][1]};
            __builtin_amdgcn_raw_buffer_store_b64(v, yr, off, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(held[i][jb + jj][q][0], yr, off, 0, 0);
          }
        }
    }
  };

  // One slice: fragments of k-step j+1 are read while the matrix cores
  // work on k-step j, and the scheduler is asked to alternate MFMAs with
  // LDS reads so the reads hide behind the 32-cycle MFMAs.  Blocks with two
  // waves per SIMD (8 waves) have half the registers per wave, so they read
  // each k-step's fragments right before use instead.
  constexpr int PF = (NW <= 4 && !DEFER) ? 2 : 1;
  // E4M3 fragments are twice as wide (8 VGPRs): a slice is one 64-deep
  // step; the fragments of the shorter side (token or weight tiles) stay in
  // registers while those of the longer side stream through two register
  // sets.
  auto compute_f8 = [&](const char* buf) __attribute__((always_inline)) {
    constexpr bool ROWS_RESIDENT = TM <= TN;  // stream weight fragments
    constexpr int NR = ROWS_RESIDENT ? TM : TN, NS = ROWS_RESIDENT ? TN : TM;
    typename TR::frag fr[NR], fs[2];
    auto ldf = [&](bool tok, int t) __attribute__((always_inline)) {
      const char* p = buf + (tok ? xrow : wrow) + t * 32 * RB;
      return TR::load2(reinterpret_cast<const TO*>(p + coff[0][0]),
                       reinterpret_cast<const TO*>(p + coff[0][FCH - 1]));
    };
#pragma unroll
    for (int r = 0; r < NR; ++r) fr[r] = ldf(ROWS_RESIDENT, r);
    fs[0] = ldf(!ROWS_RESIDENT, 0);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (t + 1 < NS) fs[(t + 1) & 1] = ldf(!ROWS_RESIDENT, t + 1);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int i = ROWS_RESIDENT ? r : t, jj = ROWS_RESIDENT ? t : r;
        const typename TR::frag& fx = ROWS_RESIDENT ? fr[r] : fs[t & 1];
        const typename TR::frag& fw = ROWS_RESIDENT ? fs[t & 1] : fr[r];
        if constexpr (F8) TR::mma_s(acc[i][jj], fw, fx, sc[jj]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // then one LDS read
      }
    }
  };
  auto compute_slice = [&](const char* buf) __attribute__((always_inline)) {
    if constexpr (F8) {
      static_assert(KSTEPS == 1, "E4M3 slices hold one MFMA step");
      compute_f8(buf);
    } else {
      typename TR::frag fx[PF][TM], fw[PF][TN];
      auto ld = [&](int j, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const char* p = buf + xrow + i * 32 * RB;
          fx[b][i] = TR::load2(reinterpret_cast<const TO*>(p + coff[j][0]),
                               reinterpret_cast<const TO*>(p + coff[j][FCH - 1]));
        }
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          const char* p = buf + wrow + jj * 32 * RB;
          fw[b][jj] = TR::load2(reinterpret_cast<const TO*>(p + coff[j][0]),
                                reinterpret_cast<const TO*>(p + coff[j][FCH - 1]));
        }
      };
      if constexpr (PF == 2) ld(0, 0);
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        if constexpr (PF == 2) {
          if (j + 1 < KSTEPS) ld(j + 1, (j + 1) & 1);
        } else {
          ld(j, 0);
        }
        if constexpr (PF == 1 && LNE) {
          // LayerNorm tiles (six weight fragments a step): every read of the
          // step first, then its MFMAs weight tile by weight tile, so that
          // one LDS latency per step is exposed instead of one per MFMA
          // (3 % on FFN2+LN; the bias/GELU tiles do better alternating)
          __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
          for (int jj = 0; jj < TN; ++jj)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              TR::mma(acc[i][jj], fw[0][jj], fx[0][i]);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        } else {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
              TR::mma(acc[i][jj], fw[j % PF][jj], fx[j % PF][i]);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // then one LDS read
            }
        }
      }
    }
  };

  // A wave consuming a slice runs at raised priority: when both waves of a
  // SIMD can issue, the one feeding the matrix core goes first (the DMA
  // issue, the waits and the epilogue run at the normal priority).  About
  // 1 % end to end on the encoder's products.
  auto compute = [&](const char* buf) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    compute_slice(buf);
    __builtin_amdgcn_s_setprio(0);
  };

  // ------------------------------------------------------------ epilogue
  // acc[i][j][4q+e] holds token m0 + wm*WTM + i*32 + l32 and feature
  // n0 + wn*WTN + j*32 + 8q + 4hh + e.
  auto epilogue = [&](int em0, int en0, int eks, int vb, auto&& next_prologue)
                      __attribute__((always_inline)) -> bool {
    const float* __restrict__ bias_s = vecs[vb][0];
    if constexpr (PART) {
      // runs of 4 fp32 sums: 16-byte stores, 32 bytes of a row per instruction
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = em0 + wm * WTM + i * 32 + l32;
        if (m >= M) continue;
        float* prow = g.part + ((int64_t)eks * g.ldp + m) * g.N + en0;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
            *reinterpret_cast<f32x4*>(prow + nl) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
      }
    } else if constexpr (LNE) {
      const float* __restrict__ g_s = vecs[vb][1 % NVEC];
      const float* __restrict__ b_s = vecs[vb][2 % NVEC];
      const int N = g.N;
      const T* __restrict__ R = static_cast<const T*>(g.R);
      // RDMA: this wave's region, and the DMA of the residual pieces of its
      // rows of half i (rows past M read row M - 1: computed, never stored)
      char* rreg = nullptr;
      __amdgpu_buffer_rsrc_t rr;
      auto res_issue = [&](int i) __attribute__((always_inline)) {
        if constexpr (RDMA) {
          const int m = em0 + wm * WTM + i * 32 + l32;
          const int mr = m < M ? m : M - 1;
          const int vo = ((mr - em0) * (int)g.ldr + wn * WTN + 8 * hh) * (int)sizeof(T);
          char* dst = rreg + (RBOTH ? i * RWB : 0);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int pc = 0; pc < 2; ++pc)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t*)(dst + (2 * j + pc) * 1024), 16, vo,
                                                       (j * 32 + pc * 16) * (int)sizeof(T), 0, 0);
        }
      };
      if constexpr (RDMA) {
        const int a = wave / WPA;
        rreg = (a == 0 ? lds0 : a == 1 ? lds1 : a == 2 ? lds2 : lds3) + (wave % WPA) * RREG;
        const int64_t rbytes = ((int64_t)(M - em0) * g.ldr - en0) * (int64_t)sizeof(T);
        rr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(R + (int64_t)em0 * g.ldr + en0), (short)0,
            __builtin_amdgcn_readfirstlane((int)(rbytes > 0x7fffffff ? 0x7fffffff : rbytes)), kRsrcWord3);
#pragma unroll
        for (int i = 0; i < (RBOTH ? TM : 1); ++i) res_issue(i);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's pieces have landed
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = em0 + wm * WTM + i * 32 + l32;
        const int mr = m < M ? m : M - 1;  // rows past M compute on a valid row, never stored
        const int64_t roff = (int64_t)mr * g.ldr + en0 + wn * WTN;
        float s = 0.f;
        if constexpr (RDMA && !RBOTH) {
          if (i > 0) {  // the region's previous half has been read
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            res_issue(i);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          f32x4 rv[4];  // this column group's residual loads first, then one wait
          if constexpr (RDMA) {
            const char* sp = rreg + (RBOTH ? i * RWB : 0) + 2 * j * 1024 + lane * 16;
            pieces_to_runs(*reinterpret_cast<const uint4*>(sp), *reinterpret_cast<const uint4*>(sp + 1024), rv);
          } else if constexpr (RES && P16) {
            const T* rp = R + roff + j * 32 + 8 * hh;
            pieces_to_runs(*reinterpret_cast<const uint4*>(rp), *reinterpret_cast<const uint4*>(rp + 16), rv);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if constexpr (RES)
                rv[q] = TS::load4f(R + roff + j * 32 + 8 * q + 4 * hh);
              else
                rv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = acc[i][j][4 * q + e] + rv[q][e];  // acc started at the bias
              acc[i][j][4 * q + e] = v;
              s += v;
            }
          }
        }
        s += wave_xor(s, 32);
        if (hh == 0) red[wn * BM + wm * WTM + i * 32 + l32] = s;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // every wave has read its residual region: the next tile's first
      // slices may land in the staging buffers
      if constexpr (RDMA) next_prologue();
      constexpr float inv_cols = 1.0f / (PAIR ? BN : 1);  // the block's share of the row (PAIR)
      constexpr int R2 = PAIR ? WGN * BM : 0;             // where the squared deviations go
      float mean[TM], rstd[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WGN; ++w) s += red[w * BM + wm * WTM + i * 32 + l32];
        mean[i] = PAIR ? s * inv_cols : s * (1.0f / N);
      }
      if constexpr (!PAIR) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
        if (hh == 0) red[R2 + wn * BM + wm * WTM + i * 32 + l32] = s;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      T* __restrict__ Y = static_cast<T*>(g.Y);
      // This block's columns: normalised from registers, or (raw, EPI_LN_PAIR
      // handing its half over) the fp32 values before normalisation, into
      // the handoff rows.
      auto store_own = [&](bool raw) __attribute__((always_inline)) {
        uint32_t pk[4][2];  // P16: one tile row's runs as bf16 pairs
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = em0 + wm * WTM + i * 32 + l32;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
              if constexpr (PAIR) {
                if (raw) {
                  *reinterpret_cast<f32x4*>(g.hand + ((int64_t)m * 2 + en0 / BN) * BN + nl) =
                      f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]};
                  continue;
                }
              }
              float o[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                o[e] = ln_out(acc[i][j][4 * q + e], mean[i], rstd[i], g_s[nl + e], b_s[nl + e]);
                if constexpr (EPI == EPI_LN_ACT) o[e] = o[e] >= 0.f ? o[e] : o[e] * g.slope;
              }
              if constexpr (P16) {
                pk[q][0] = pack_bf16x2(o[0], o[1]);
                pk[q][1] = pack_bf16x2(o[2], o[3]);
              } else {
                TS::store4(Y + (int64_t)m * g.ldy + en0 + nl, o[0], o[1], o[2], o[3]);
              }
              if constexpr (F8) store4_as<T, true>(g.Y8, (int64_t)m * g.ldy8 + en0 + nl, o[0], o[1], o[2], o[3]);
              if constexpr (P16) {
                if (q == 3) {
                  uint4 p0, p1;
                  swap_runs_to_pieces(pk, p0, p1);
                  T* yp = Y + (int64_t)m * g.ldy + en0 + wn * WTN + j * 32 + 8 * hh;
                  *reinterpret_cast<uint4*>(yp) = p0;
                  *reinterpret_cast<uint4*>(yp + 16) = p1;
                }
              }
            }
        }
      };
      // EPI_LN_PAIR.  Per row tile the exchange holds each half's 2*BM
      // statistic words, one word per half saying that the half normalises
      // itself, and one handoff word; every word carries the launch's tag
      // in its upper 32 bits (tags start at 1, so cleared words never match).
      // A block publishes its statistics and polls the partner's for a short
      // while.  If they all came, it normalises its own half and then learns
      // whether the partner does the same or handed its half over.  If not
      // (the partner is late, or not resident), it leaves its fp32 values
      // before normalisation in the handoff rows and claims the handoff word
      // (the partner then normalises those very values with the same
      // statistics and the same ln_out, so the output bits do not depend on
      // which block normalised them): the partner, whenever
      // it runs, normalises both halves.  If the partner claimed first, this
      // block normalises both.  Each remaining wait is for a block that has
      // already published its statistics, so it is running and ends.
      const int half = en0 / BN;
      const size_t xbase = (size_t)(em0 / BM) * (4 * BM + 8);
      // word i of this row tile: statistics [half][2*BM], decisions at 4*BM
      // + half, the handoff word at 4*BM + 2
      auto xw = [&](int i) __attribute__((always_inline)) { return g.xch + xbase + i; };
      const unsigned long long tag = (unsigned long long)(unsigned)g.xtag << 32;
      constexpr unsigned long long kTagMask = ~0xFFFFFFFFull;
      // poll word p up to `spin` times for this launch's tag; its value to *dst
      auto poll = [&](unsigned long long* p, int spin, float* dst) __attribute__((always_inline)) {
        unsigned long long u = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int polls = 0; (u & kTagMask) != tag; ++polls) {
          if (polls >= spin) return false;
          __builtin_amdgcn_s_sleep(1);
          u = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *dst = __uint_as_float((unsigned)u);
        return true;
      };
      bool help = false;  // this block also normalises the partner's half
      if constexpr (PAIR) {
        // thread t < 2*BM: statistic t / BM (0: mean, 1: squared
        // deviations) of row t % BM
        unsigned long long* const theirs = xw((half ^ 1) * 2 * BM + tid);
        float* const pdst = pst + (half ^ 1) * 2 * BM + tid;
        bool found = true;
        if (tid < 2 * BM) {
          const int kind = tid / BM, row = tid % BM;
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < WGN; ++w) v += red[kind * R2 + w * BM + row];
          if (kind == 0) v *= inv_cols;
          __hip_atomic_store(xw(half * 2 * BM + tid), tag | __float_as_uint(v), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          pst[half * 2 * BM + tid] = v;
          found = poll(theirs, g.pair_spin, pdst);
        }
        if (__syncthreads_and(found)) {
          if (tid == 0)
            __hip_atomic_store(xw(4 * BM + half), tag | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          store_own(true);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's rows have left
          __syncthreads();
          if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            unsigned long long cur = __hip_atomic_load(xw(4 * BM + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool won = false;
            if ((cur & kTagMask) != tag)  // not claimed in this launch yet
              won = __hip_atomic_compare_exchange_strong(xw(4 * BM + 2), &cur, tag | (unsigned)(half + 1),
                                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            pflag = won ? 1 : 0;
          }
          __syncthreads();
          if (pflag) return true;  // the partner normalises both halves
          // the partner handed over first, after publishing its statistics
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          bool ok = true;
          if (tid < 2 * BM) ok = poll(theirs, kPairSpin, pdst);
          if (!__syncthreads_and(ok)) return false;
          help = true;
        }
        // both halves combine the same four numbers in the same order
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WTM + i * 32 + l32;
          const float ma = pst[row], qa = pst[BM + row], mb = pst[2 * BM + row], qb = pst[3 * BM + row];
          const float d = ma - mb;
          mean[i] = (ma + mb) * 0.5f;
          const float m2 = (qa + qb) + d * d * (0.5f * BN);
          rstd[i] = 1.0f / sqrtf(m2 * (1.0f / N) + g.eps);
        }
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < WGN; ++w) s += red[w * BM + wm * WTM + i * 32 + l32];
          rstd[i] = 1.0f / sqrtf(s * (1.0f / N) + g.eps);
        }
      }
      store_own(false);
      if constexpr (PAIR) {
        if (!help) {  // does the partner normalise its own half?
          if (tid == 0) {
            int r = 2;  // 0: yes, 1: handed over, 2: no answer
            const unsigned long long handed = tag | (unsigned)((half ^ 1) + 1);
            for (int polls = 0;; ++polls) {
              const unsigned long long d =
                  __hip_atomic_load(xw(4 * BM + (half ^ 1)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if ((d & kTagMask) == tag) { r = 0; break; }
              if (__hip_atomic_load(xw(4 * BM + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == handed) {
                r = 1;
                break;
              }
              if (polls >= kPairSpin) break;
              __builtin_amdgcn_s_sleep(1);
            }
            pflag = r;
          }
          __syncthreads();
          const int r = pflag;
          if (r == 2) return false;
          if (r == 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            help = true;
          }
        }
        if (help) {  // the partner's values before normalisation are in the handoff rows
          const int n0p = (half ^ 1) * BN;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int m = em0 + wm * WTM + i * 32 + l32;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
                const int c = n0p + nl;
                T* const y = Y + (int64_t)m * g.ldy + c;
                const f32x4 pv =
                    *reinterpret_cast<const f32x4*>(g.hand + ((int64_t)m * 2 + (half ^ 1)) * BN + nl);
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = ln_out(pv[e], mean[i], rstd[i], g.ln_g[c + e], g.ln_b[c + e]);
                TS::store4(y, o[0], o[1], o[2], o[3]);
                if constexpr (F8)
                  store4_as<T, true>(g.Y8, (int64_t)m * g.ldy8 + c, o[0], o[1], o[2], o[3]);
              }
          }
        }
      }
      // the next tile's epilogue reuses `red` and `pst`: everyone has read them
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else if constexpr (DEFER) {
      // pack into registers; stored during the next tile's K loop
      char* ybase = static_cast<char*>(g.Y) + ((int64_t)em0 * g.ldy + en0) * (int64_t)YES;
      const int64_t ybytes = (int64_t)(M - em0) * g.ldy * (int64_t)YES;
      yr = __builtin_amdgcn_make_buffer_rsrc(
          ybase, (short)0,
          __builtin_amdgcn_readfirstlane((int)(ybytes > 0x7fffffff ? 0x7fffffff : ybytes)), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        hoff[i] = ((wm * WTM + i * 32 + l32) * (int)g.ldy + wn * WTN + (DP16 ? 8 : 4) * hh) * YES;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          uint32_t pk[4][2];  // DP16: the tile row's runs as bf16 pairs
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + j * 32 + 8 * q + 4 * hh;
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = acc[i][j][4 * q + e] + bias_s[nl + e];
              if constexpr (EPI == EPI_GELU) o[e] = gelu_tanh(o[e]);
            }
            if constexpr (DP16) {
              pk[q][0] = pack_bf16x2(o[0], o[1]);
              pk[q][1] = pack_bf16x2(o[2], o[3]);
            } else {
              held[i][j][q][0] = pack_e4m3x4(o[0], o[1], o[2], o[3]);
            }
          }
          if constexpr (DP16) swap_runs_to_pieces(pk, hp[i][j][0], hp[i][j][1]);
        }
      }
    } else {
      uint32_t pk[4][2];  // P16: one tile row's runs as bf16 pairs
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = em0 + wm * WTM + i * 32 + l32;
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
              *reinterpret_cast<f32x4*>(g.out + orow * g.N + en0 + nl) = f32x4{o[0], o[1], o[2], o[3]};
            } else if constexpr (P16 && !F8) {
              pk[q][0] = pack_bf16x2(o[0], o[1]);
              pk[q][1] = pack_bf16x2(o[2], o[3]);
              if (q == 3) {
                uint4 p0, p1;
                swap_runs_to_pieces(pk, p0, p1);
                T* yp = static_cast<T*>(g.Y) + orow * g.ldy + en0 + wn * WTN + j * 32 + 8 * hh;
                *reinterpret_cast<uint4*>(yp) = p0;
                *reinterpret_cast<uint4*>(yp + 16) = p1;
              }
            } else {
              store4_as<T, YF8>(g.Y, orow * g.ldy + en0 + nl, o[0], o[1], o[2], o[3]);
              if constexpr (F8 && EPI == EPI_BIAS) {
                if (g.Y8) store4_as<T, true>(g.Y8, orow * g.ldy8 + en0 + nl, o[0], o[1], o[2], o[3]);
              }
            }
          }
      }
    }
    return true;
  };

  // --------------------------------------------------------- tile loop
  setup(tile);
  conv_offsets();
  vload(n0);
  vstore(0);
  prologue();
  int vb = 0;
  const int KT = g.K / S / BK;  // KR more than a multiple of STAGES, at least STAGES + KR (host)
  for (;;) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if constexpr (LNE) {
      // LayerNorm tiles start their accumulators at the bias: their
      // epilogue, which holds every accumulator and waits for each LDS read
      // in turn, then reads no bias, and these reads overlap the first
      // slice's DMA (about 1 % on both LayerNorm products)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // this tile's vectors are in LDS
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(&vecs[vb][0][wn * WTN + j * 32 + 8 * q + 4 * hh]);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = b4[e];
        }
    }

    if constexpr (DEFER) {
      // Two stages; step t waits for slice t, issues slice t+1, then (t < NB)
      // the previous tile's store batch t, then computes slice t.  The only
      // vector-memory operations younger than slice t's DMA at step t are the
      // SB stores of batch t-1, so the wait lets them stay in flight.
      // Steps 0..NB+1 are unrolled, then pairs, then the last two peeled
      // (the host guarantees KT >= NB + 4 and KT even).
#pragma unroll
      for (int t = 0; t < NB + 2; ++t) {
        if (t >= 1 && t <= NB) ALBERT_WAIT_BARRIER(SB);
        else ALBERT_WAIT_BARRIER(0);
        issue(ALBERT_BUF((t + 1) % 2), (t + 1) * BK);
        // all of slice t+1's DMA must be issued before the stores: the next
        // step's wait counts only the stores as younger operations
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (t < NB) store_batch(t);
        __builtin_amdgcn_sched_barrier(0);
        compute(ALBERT_BUF(t % 2));
      }
      for (int kt = NB + 2; kt < KT - 2; kt += 2) {
        ALBERT_WAIT_BARRIER(0);
        issue(lds1, (kt + 1) * BK);
        compute(lds0);
        ALBERT_WAIT_BARRIER(0);
        issue(lds0, (kt + 2) * BK);
        compute(lds1);
      }
      ALBERT_WAIT_BARRIER(0);
      issue(lds1, (KT - 1) * BK);
      compute(lds0);
      ALBERT_WAIT_BARRIER(0);
      compute(lds1);
    } else {
      // STAGES-deep pipeline: slices t+1 .. t+STAGES-2 stay in flight while
      // slice t is consumed.  Before the barrier of slice t each wave waits
      // only for its own DMA of slice t (later slices may still be in flight);
      // the barrier then makes every wave's part visible and frees the buffer
      // consumed at t-1, which receives slice t+STAGES-1.  The main loop is
      // branch-free; the last STAGES + KR slices (KR = KT mod STAGES, fixed
      // per instantiation) are peeled with static buffers and waits.
      for (int kt = 0; kt < KT - STAGES - KR; kt += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
          ALBERT_WAIT_BARRIER(IPW * (STAGES - 2));
          issue(ALBERT_BUF((s + STAGES - 1) % STAGES), (kt + s + STAGES - 1) * BK);
          compute(ALBERT_BUF(s));
        }
      }
      // kt0 is a multiple of STAGES, so slice kt0 + s sits in buffer
      // s % STAGES; after slice kt0 + s, min(STAGES-2, NS-1-s) younger
      // slices are in flight
      auto tail = [&](auto rc) __attribute__((always_inline)) {
        constexpr int NS = STAGES + decltype(rc)::value;
        const int kt0 = KT - NS;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int pend = STAGES - 2 < NS - 1 - s ? STAGES - 2 : NS - 1 - s;
          if (pend >= 2)
            ALBERT_WAIT_BARRIER(2 * IPW);
          else if (pend == 1)
            ALBERT_WAIT_BARRIER(IPW);
          else
            ALBERT_WAIT_BARRIER(0);
          if (s + STAGES - 1 < NS)
            issue(ALBERT_BUF((s + STAGES - 1) % STAGES), (kt0 + s + STAGES - 1) * BK);
          compute(ALBERT_BUF(s % STAGES));
        }
      };
      tail(std::integral_constant<int, KR>{});
    }

    const int next = tile + G;
    const bool more = next < ntiles;
    const int em0 = m0, en0 = n0, eks = ks0;
    if (more) {
      setup(next);
      conv_offsets();
      vload(n0);
    }
    // every wave has finished reading the staging buffers (their reads fed
    // the MFMAs above), so the next tile's first slices may land there
    asm volatile("s_barrier" ::: "memory");
    auto next_prologue = [&]() __attribute__((always_inline)) {
      if (more) prologue();
    };
    // (the LayerNorm epilogue reading its residual through the staging
    // buffers issues the prologue itself, once it has read them)
    if constexpr (!RDMA) next_prologue();
    if (!epilogue(em0, en0, eks, vb, next_prologue)) {
      // EPI_LN_PAIR: the partner never delivered its statistics; report it
      // and stop (nothing of this tile is stored)
      if (tid == 0) __hip_atomic_store(const_cast<int*>(g.status), kStatusSync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next tile's DMA has landed
      return;
    }
    if (!more) {
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) store_batch(bt);  // last tile: write everything now
      break;
    }
    vstore(vb ^ 1);  // read only after the next tile's K-loop barriers
    vb ^= 1;
    tile = next;
  }
#undef ALBERT_BUF
}

#undef ALBERT_WAIT_BARRIER

}  // namespace albert
