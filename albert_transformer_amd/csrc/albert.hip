// Host side of the encoder library: the C ABI declared in include/albert.h,
// weight packing, workspace planning and the launch sequence.
//
// Launch sequence of one request (all on the caller's stream):
//   derive (lengths -> offsets, status) -> rows/IDs check -> embedding + LN
//   -> 128->768 projection -> n_iter x [QKV GEMM -> attention -> out-proj +
//   residual + LN -> FFN1 + GELU -> FFN2 + residual + LN] -> 768->512
//   projection into `out` (+ zeroing of padded rows).
// The same weight pointers serve every execution of the shared layer (page
// "ALBERT: How Kokoro's Phoneme Encoder Works", "Cross-layer parameter
// sharing"); only the activations change.  With intermediate grouping (G
// weight sets) execution i takes set floor(i * G / n_iter).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "albert.h"
#include "attention.hpp"
#include "duration.hpp"
#include "gemm.hpp"
#include "host.hpp"
#include "launch.hpp"
#include "prologue.hpp"
#include "qkv_attention.hpp"

using namespace albert;

// Device pointers of one layer weight set (matrices in dtype -- E4M3 codes
// plus per-row E8M0 exponents under ALBERT_FP8 -- vectors fp32).
struct LayerW {
  const void *qkv_w, *o_w, *ffn1_w, *ffn2_w;
  const void* qkv_wh;  // bf16 / E4M3: [12][192][768] per head q/8 | k | v rows
  const unsigned char* qkv_eh;  // E4M3: their E8M0 exponents [12][192]
  const float* qkv_bh; // [12][192]
  const unsigned char *qkv_e, *o_e, *ffn1_e, *ffn2_e;
  const float *qkv_b, *o_b, *ln1_g, *ln1_b, *ffn1_b, *ffn2_b, *ln2_g, *ln2_b;
};

// Scratch of albert_encode_noalloc: the workspace of a request, in the
// library's own device memory, for callers that cannot allocate.  Every GPU
// the library runs on holds one copy of it until the process ends.  In host
// code its name is only a stand-in: the device address of each GPU's copy is
// taken once per device (scratch_address) and used everywhere instead.
static __device__ __align__(256) unsigned char scratch[ALBERT_SCRATCH_BYTES];

struct albert_ctx {
  albert_config cfg;
  int dtype;
  int device;
  void* scratch = nullptr;  // this device's copy of `scratch`
  int grid_cap;  // persistent GEMM grid: CUs rounded down to a multiple of 8
  bool ln_pair = false;  // LayerNorm GEMMs on block pairs (bf16 storage)
  void* mem;
  // device pointers (tables/matrices in dtype, vectors fp32)
  const void *word, *pos, *type, *proj_w, *out_w;
  const unsigned char *proj_e, *out_e;
  const float *emb_g, *emb_b, *proj_b, *out_b;
  std::vector<LayerW> layers;  // n_groups weight sets
  // optional kernel timing (albert_time_kernel)
  int time_kind = -1;
  int n_timed = 0;
  std::vector<hipEvent_t> ev;  // start/stop pairs
};

namespace {

__global__ void clear_u64_kernel(unsigned long long* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// Device address of `scratch` on `device` (the current device), looked up
// once per device and kept; null if the lookup fails.
void* scratch_address(int device) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) addr[device] = p;
  }
  return addr[device];
}

__global__ void copy_status_kernel(const int* __restrict__ src, int* __restrict__ dst) { *dst = *src; }


// Launch `fn` on stream s; when `kind` is the kernel kind selected with
// albert_time_kernel(), its kernel carries a pair of timing events.
template <typename Fn>
void timed(albert_ctx* c, int kind, hipStream_t s, Fn&& fn) {
  const bool on = c->time_kind == kind && 2 * (c->n_timed + 1) <= (int)c->ev.size();
  if (on) g_launch_events = LaunchEvents{c->ev[2 * c->n_timed], c->ev[2 * c->n_timed + 1]};
  fn();  // launches exactly one kernel through launch_kernel(), which takes the events
  if (on) {
    if (g_launch_events.start == nullptr) ++c->n_timed;
    g_launch_events = LaunchEvents{};
  }
}

// One request.  T is the storage type; F8 selects E4M3 matrix-product
// operands (ALBERT_FP8).  feats != null: packed rows of embedding LayerNorm
// output replace the IDs and the embedding.
template <typename T, bool F8>
int run(albert_ctx* c, const int32_t* ids, const int32_t* lens_or_cu, int n_seq, int pad_T,
        int64_t max_rows, int max_len, float* out, void* ws, hipStream_t s,
        const float* feats, unsigned flags) {
  const albert_config& cf = c->cfg;
  const Layout L = plan(c->cfg, c->dtype, n_seq, max_rows);
  char* w = static_cast<char*>(ws);
  int* status = reinterpret_cast<int*>(w + L.status);
  int* cu = reinterpret_cast<int*>(w + L.cu);
  int* row_seq = reinterpret_cast<int*>(w + L.row_seq);
  int* row_pos = reinterpret_cast<int*>(w + L.row_pos);
  void* emb = w + L.emb;          // operand of the input projection
  T* X = reinterpret_cast<T*>(w + L.x);
  T* X1 = reinterpret_cast<T*>(w + L.x1);
  T* QKV = reinterpret_cast<T*>(w + L.qkv);
  void* CTX = w + L.ctx;          // operand of the output projection
  void* G = w + L.g;              // operand of FFN2
  // operands of the Q|K|V and FFN1 products, and their E4M3 copies
  void* X8 = F8 ? static_cast<void*>(w + L.x8) : static_cast<void*>(X);
  void* X18 = F8 ? static_cast<void*>(w + L.x18) : static_cast<void*>(X1);
  void* Y8 = F8 ? X8 : nullptr;
  void* Y18 = F8 ? X18 : nullptr;
  const int H = cf.hidden, F = cf.ffn;
  const int* m_ptr = cu + n_seq;

  // Q|K|V and attention in one kernel when every sequence fits a 256-row
  // tile: groups of consecutive whole sequences, packed greedily on the
  // device (up to kGreedyMaxSeqs sequences), else S = 256 / longest per
  // group, chosen on the host; the separate kernels otherwise.
  constexpr bool can_fuse = std::is_same<T, bf16>::value;
  const bool fuse = can_fuse && max_len <= 256 && !(flags & ALBERT_UNFUSED);
  const bool greedy = fuse && n_seq <= kGreedyMaxSeqs;
  int* groups = greedy ? reinterpret_cast<int*>(w + L.groups) : nullptr;
  if (pad_T)
    hipLaunchKernelGGL(derive_padded_kernel, dim3(1), dim3(1024), 0, s, lens_or_cu, n_seq, pad_T,
                       cu, status, groups);
  else
    hipLaunchKernelGGL(derive_packed_kernel, dim3(1), dim3(1024), 0, s, lens_or_cu, n_seq,
                       (int)max_rows, max_len, cu, status, groups);
  if (feats) {
    // row -> sequence map for the attention's packed query blocks
    hipLaunchKernelGGL(rows_ids_kernel, dim3(n_seq), dim3(256), 0, s, nullptr, cu, 0, cf.vocab,
                       row_seq, row_pos, status);
    timed(c, ALBERT_K_EMBED, s, [&] {
      launch_kernel(features_in_kernel<T, F8>,
                    dim3((unsigned)((max_rows * cf.emb / 4 + 255) / 256)), dim3(256), s, feats,
                    m_ptr, emb, status);
    });
  } else {
    hipLaunchKernelGGL(rows_ids_kernel, dim3(n_seq), dim3(256), 0, s, ids, cu, pad_T, cf.vocab,
                       row_seq, row_pos, status);
    timed(c, ALBERT_K_EMBED, s, [&] {
      launch_kernel(embed_ln_kernel<T, F8>, dim3((unsigned)((max_rows + 15) / 16)), dim3(256),
                    s, ids, pad_T, row_seq, row_pos, m_ptr, (const T*)c->word, (const T*)c->pos,
                    (const T*)c->type, c->emb_g, c->emb_b, cf.ln_eps, emb, status);
    });
  }

  GemmArgs base{};
  base.status = status;
  base.m_ptr = m_ptr;
  base.eps = cf.ln_eps;

  // A product of the request: over K splits for very small batches (the
  // partial sums in the workspace, then a reduce kernel with the epilogue),
  // else the one-pass kernels one_pass() launches.
  float* part = reinterpret_cast<float*>(w + L.part);
  auto product = [&](auto epi, GemmArgs& ga, int kind, auto&& one_pass) {
    constexpr int EPI = decltype(epi)::value;
    const int S = split_factor(max_rows, ga.N, split_slices<T, F8>(ga.K));
    if (S > 0) {
      ga.part = part;
      SplitArgs r{};
      r.bias = ga.bias; r.Y = ga.Y; r.ldy = ga.ldy; r.Y8 = ga.Y8; r.ldy8 = ga.ldy8;
      r.R = ga.R; r.ldr = ga.ldr; r.ln_g = ga.ln_g; r.ln_b = ga.ln_b; r.eps = ga.eps;
      r.out = ga.out; r.row_seq = ga.row_seq; r.row_pos = ga.row_pos; r.out_T = ga.out_T;
      r.status = status; r.m_ptr = m_ptr;
      timed(c, kind, s, [&] { launch_split<T, F8, EPI>(ga, r, S, max_rows, c->grid_cap, s); });
    } else {
      one_pass();
    }
  };
  using Bias = std::integral_constant<int, EPI_BIAS>;
  using Gelu = std::integral_constant<int, EPI_GELU>;
  using Ln = std::integral_constant<int, EPI_LN>;
  using Out = std::integral_constant<int, EPI_OUT>;

  GemmArgs g = base;  // input projection E -> H
  g.X = emb; g.ldx = cf.emb; g.W = c->proj_w; g.wexp = c->proj_e; g.bias = c->proj_b;
  g.Y = X; g.ldy = H; g.Y8 = Y8; g.ldy8 = H; g.N = H; g.K = cf.emb;
  product(Bias{}, g, ALBERT_K_PROJ, [&] {
    timed(c, ALBERT_K_PROJ, s, [&] { gemm_big<T, F8, EPI_BIAS>(g, max_rows, c->grid_cap, s); });
  });

  // LayerNorm GEMMs: bf16 rows (bf16 or E4M3 operands) split over two
  // blocks that swap row statistics (full rows in one block otherwise).
  // Their exchange words are cleared once per request and whenever the
  // launch tags wrap.
  constexpr bool can_pair = std::is_same<T, bf16>::value;
  const bool pair = can_pair && c->ln_pair;
  unsigned long long* xch = reinterpret_cast<unsigned long long*>(w + L.xch);
  const int64_t xwords = (int64_t)ln_pair_words(max_rows);
  int xtag = 0;
  bool launch_failed = false;
  auto clear_xch = [&] {
    hipLaunchKernelGGL(clear_u64_kernel, dim3((unsigned)((xwords + 255) / 256)), dim3(256), 0, s,
                       xch, xwords);
  };
  if (pair) clear_xch();
  auto gemm_layernorm = [&](GemmArgs& ga, int kind) {
    if (pair) {
      if (++xtag > 4095) {
        clear_xch();
        xtag = 1;
      }
      ga.xch = xch;
      ga.hand = reinterpret_cast<float*>(w + L.hand);
      ga.xtag = xtag;
      ga.pair_spin = (flags & ALBERT_LN_HANDOFF) ? 0 : kPairPolls;
      timed(c, kind, s, [&] {
        if (gemm_ln_pair<F8>(ga, max_rows, c->grid_cap, s) != hipSuccess) launch_failed = true;
      });
    } else {
      timed(c, kind, s, [&] { gemm_ln<T, F8>(ga, max_rows, c->grid_cap, s); });
    }
  };

  // Any S consecutive sequences fit 256 rows, so greedy groups take at
  // least S sequences each (the last one aside): there are never more of
  // them than S-groups, whose count sizes the grid.
  const int S = fuse ? 256 / max_len : 0;  // >= 1 when fused
  const int64_t pairs = fuse ? (int64_t)((n_seq + S - 1) / S) * cf.heads : 0;
  for (int it = 0; it < cf.n_iter; ++it) {
    const LayerW& lw = c->layers[(size_t)((int64_t)it * cf.n_groups / cf.n_iter)];
    if (fuse) {
      QkvAttnArgs qa{X8, lw.qkv_wh, lw.qkv_eh, lw.qkv_bh, CTX, cu, row_seq, status, groups, n_seq,
                     S, (int)pairs};
      timed(c, ALBERT_K_QKV_ATTN, s, [&] {
        if constexpr (can_fuse)
          launch_kernel(qkv_attention_kernel<F8>,  // persistent with bf16 operands
                        dim3((unsigned)(F8 ? (pairs + 7) / 8 * 8
                                           : std::min<int64_t>((pairs + 7) / 8 * 8, c->grid_cap))),
                        dim3(512), s, qa);
      });
    } else {
      g = base;  // fused Q|K|V projection
      g.X = X8; g.ldx = H; g.W = lw.qkv_w; g.wexp = lw.qkv_e; g.bias = lw.qkv_b; g.Y = QKV;
      g.ldy = 3 * H; g.N = 3 * H; g.K = H;
      product(Bias{}, g, ALBERT_K_QKV, [&] {
        timed(c, ALBERT_K_QKV, s, [&] { gemm_big<T, F8, EPI_BIAS>(g, max_rows, c->grid_cap, s); });
      });

      // short sequences on average (many per 128 rows): packed query blocks;
      // otherwise query tiles aligned to each sequence
      const bool packed = max_rows < (int64_t)n_seq * 128;
      AttnArgs a{QKV, CTX, cu, row_seq, m_ptr, status, packed ? 1 : 0};
      const dim3 grid = packed ? dim3((unsigned)((max_rows + 127) / 128), cf.heads)
                               : dim3(n_seq, cf.heads, (max_len + 127) / 128);
      timed(c, ALBERT_K_ATTN, s, [&] { launch_kernel(attention_kernel<T, F8>, grid, dim3(256), s, a); });
    }

    g = base;  // output projection + residual + LayerNorm
    g.X = CTX; g.ldx = H; g.W = lw.o_w; g.wexp = lw.o_e; g.bias = lw.o_b; g.R = X; g.ldr = H;
    g.ln_g = lw.ln1_g; g.ln_b = lw.ln1_b; g.Y = X1; g.ldy = H; g.Y8 = Y18; g.ldy8 = H;
    g.N = H; g.K = H;
    product(Ln{}, g, ALBERT_K_ATTN_OUT_LN, [&] { gemm_layernorm(g, ALBERT_K_ATTN_OUT_LN); });

    g = base;  // FFN 768 -> 2048 + GELU
    g.X = X18; g.ldx = H; g.W = lw.ffn1_w; g.wexp = lw.ffn1_e; g.bias = lw.ffn1_b; g.Y = G;
    g.ldy = F; g.N = F; g.K = H;
    product(Gelu{}, g, ALBERT_K_FFN1_GELU, [&] {
      timed(c, ALBERT_K_FFN1_GELU, s, [&] { gemm_big<T, F8, EPI_GELU>(g, max_rows, c->grid_cap, s); });
    });

    g = base;  // FFN 2048 -> 768 + residual + LayerNorm
    g.X = G; g.ldx = F; g.W = lw.ffn2_w; g.wexp = lw.ffn2_e; g.bias = lw.ffn2_b; g.R = X1;
    g.ldr = H; g.ln_g = lw.ln2_g; g.ln_b = lw.ln2_b; g.Y = X; g.ldy = H; g.Y8 = Y8; g.ldy8 = H;
    g.N = H; g.K = F;
    product(Ln{}, g, ALBERT_K_FFN2_LN, [&] { gemm_layernorm(g, ALBERT_K_FFN2_LN); });
  }

  g = base;  // output projection H -> 512, fp32, into the caller's rows
  g.X = X8; g.ldx = H; g.W = c->out_w; g.wexp = c->out_e; g.bias = c->out_b; g.out = out;
  g.row_seq = row_seq; g.row_pos = row_pos; g.out_T = pad_T; g.N = cf.out_dim; g.K = H;
  product(Out{}, g, ALBERT_K_OUT, [&] {
    timed(c, ALBERT_K_OUT, s, [&] { gemm_big<T, F8, EPI_OUT>(g, max_rows, c->grid_cap, s); });
  });
  if (pad_T)
    hipLaunchKernelGGL(zero_pad_rows_kernel, dim3(n_seq), dim3(256), 0, s, out, cu, pad_T,
                       cf.out_dim, status);
  return hipGetLastError() == hipSuccess && !launch_failed ? ALBERT_OK : ALBERT_E_HIP;
}

// Dispatch on the context's dtype.
template <typename... A>
int run_any(albert_ctx* c, A... args) {  // args end with (feats, flags)
  switch (c->dtype) {
    case ALBERT_BF16: return run<bf16, false>(c, args...);
    case ALBERT_FP8: return run<bf16, true>(c, args...);
    default: return run<float, false>(c, args...);
  }
}

int finish(int rc, const void* ws, hipStream_t s, unsigned flags) {
  if (rc != ALBERT_OK || (flags & ALBERT_ASYNC)) return rc;
  return albert_read_status(ws, s);
}

bool device_matches(const albert_ctx* c) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == c->device;
}

}  // namespace

extern "C" {

int albert_default_config(albert_config* cfg) {
  if (!cfg) return ALBERT_E_ARG;
  *cfg = kokoro_config();
  return ALBERT_OK;
}

int albert_n_tensors(const albert_config* cfg) {
  if (!cfg || !config_ok(*cfg)) return -1;
  return 9 + ALBERT_LAYER_TENSORS * cfg->n_groups;
}

const char* albert_tensor_name(const albert_config* cfg, int index) {
  if (!cfg || !config_ok(*cfg)) return nullptr;
  const int r = role_of(*cfg, index);
  return r < 0 ? nullptr : kNames[r];
}

int albert_tensor_shape(const albert_config* cfg, int index, int64_t* rows, int64_t* cols) {
  if (!cfg || !rows || !cols || !config_ok(*cfg)) return ALBERT_E_ARG;
  return shape_of(*cfg, index, rows, cols) ? ALBERT_OK : ALBERT_E_ARG;
}

int albert_load_weights(albert_ctx** out_ctx, const albert_config* cfg,
                        const float* const* host, int dtype, void* stream) {
  if (!out_ctx) return ALBERT_E_ARG;
  *out_ctx = nullptr;
  if (!cfg || !host || !config_ok(*cfg) ||
      (dtype != ALBERT_F32 && dtype != ALBERT_BF16 && dtype != ALBERT_FP8))
    return ALBERT_E_ARG;
  const albert_config c = *cfg;
  const bool f8 = dtype == ALBERT_FP8;
  const int G = c.n_groups;
  Image im;
  if (const int rc = build_image(c, host, dtype, &im); rc != ALBERT_OK) return rc;
  const std::vector<Seg>& seg = im.seg;
  const size_t off = im.bytes.size();
  albert_ctx* ctx = new (std::nothrow) albert_ctx();
  if (!ctx) return ALBERT_E_ARG;
  ctx->cfg = c;
  ctx->dtype = dtype;
  int n_cu = 0;
  if (hipGetDevice(&ctx->device) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, ctx->device) !=
          hipSuccess ||
      hipMalloc(&ctx->mem, off) != hipSuccess) {
    delete ctx;
    return ALBERT_E_HIP;
  }
  ctx->scratch = scratch_address(ctx->device);
  if (!ctx->scratch) {
    (void)hipFree(ctx->mem);
    delete ctx;
    return ALBERT_E_HIP;
  }
  ctx->grid_cap = std::max(8, n_cu / 8 * 8);
  {  // paired LayerNorm blocks: shapes they take, and one block per CU fits
    const bool f8 = dtype == ALBERT_FP8;
    bool ok = dtype != ALBERT_F32 && ctx->grid_cap >= 16 && c.hidden == 768 &&
              ln_pair_k_ok(c.hidden, f8) && ln_pair_k_ok(c.ffn, f8);
    std::vector<const void*> ks;
    if (f8) ks.push_back(reinterpret_cast<const void*>(ln_pair_kernel_f8));
    else
      for (int kr = 0; kr < 3; ++kr) {
        ks.push_back(ln_pair_pick<256>(kr));
        ks.push_back(ln_pair_pick<128>(kr));
        ks.push_back(ln_pair_pick<64>(kr));
      }
    for (size_t i = 0; i < ks.size(); ++i) {
      const unsigned threads = f8 ? 256 : ln_pair_threads(i % 3 == 2 ? 64 : 128);
      int per_cu = 0;
      ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ks[i], threads, 0) ==
                     hipSuccess &&
           per_cu >= 1;
    }
    ctx->ln_pair = ok;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(ctx->mem, im.bytes.data(), off, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipFree(ctx->mem);
    delete ctx;
    return ALBERT_E_HIP;
  }
  char* m = static_cast<char*>(ctx->mem);
  auto P = [&](int sidx) { return (const void*)(m + seg[sidx].off); };
  auto Pf = [&](int sidx) { return (const float*)(m + seg[sidx].off); };
  ctx->word = P(S_WORD); ctx->pos = P(S_POS); ctx->type = P(S_TYPE);
  ctx->emb_g = Pf(S_EMB_G); ctx->emb_b = Pf(S_EMB_B);
  ctx->proj_w = P(S_PROJ_W); ctx->proj_b = Pf(S_PROJ_B);
  ctx->out_w = P(S_OUT_W); ctx->out_b = Pf(S_OUT_B);
  auto Pe = [&](int sidx) { return (const unsigned char*)(m + seg[sidx].off); };
  ctx->proj_e = Pe(S_PROJ_E); ctx->out_e = Pe(S_OUT_E);
  ctx->layers.resize(G);
  for (int g = 0; g < G; ++g) {
    const int s0 = S_LAYER0 + L_SEGS * g;
    LayerW& lw = ctx->layers[g];
    lw.qkv_w = P(s0 + L_QKV_W); lw.qkv_b = Pf(s0 + L_QKV_B);
    lw.o_w = P(s0 + L_O_W); lw.o_b = Pf(s0 + L_O_B);
    lw.ln1_g = Pf(s0 + L_LN1_G); lw.ln1_b = Pf(s0 + L_LN1_B);
    lw.ffn1_w = P(s0 + L_F1_W); lw.ffn1_b = Pf(s0 + L_F1_B);
    lw.ffn2_w = P(s0 + L_F2_W); lw.ffn2_b = Pf(s0 + L_F2_B);
    lw.ln2_g = Pf(s0 + L_LN2_G); lw.ln2_b = Pf(s0 + L_LN2_B);
    lw.qkv_e = Pe(s0 + L_QKV_E); lw.o_e = Pe(s0 + L_O_E);
    lw.qkv_wh = P(s0 + L_QKV_WH);
    lw.qkv_eh = Pe(s0 + L_QKV_EH);
    lw.qkv_bh = Pf(s0 + L_QKV_BH);
    lw.ffn1_e = Pe(s0 + L_F1_E); lw.ffn2_e = Pe(s0 + L_F2_E);
  }
  *out_ctx = ctx;
  return ALBERT_OK;
}

size_t albert_workspace_bytes(const albert_ctx* ctx, int n_seq, int64_t max_rows) {
  if (!ctx || n_seq < 1 || max_rows < 1) return 0;
  return plan(ctx->cfg, ctx->dtype, n_seq, max_rows).total;
}

int albert_encode(albert_ctx* ctx, const int32_t* ids, const int32_t* lengths, int B, int T,
                  float* out, void* ws, size_t ws_bytes, void* stream, unsigned flags) {
  if (ctx && B == 0) return ALBERT_OK;  // empty batch: nothing to do
  if (!ctx || !ids || !lengths || !out || !ws || B < 1 || T < 1 || T > ctx->cfg.max_pos ||
      ((uintptr_t)ws % kAlign) != 0 || (int64_t)B * T > INT32_MAX || !device_matches(ctx))
    return ALBERT_E_ARG;
  const int64_t rows = (int64_t)B * T;
  const size_t need = plan(ctx->cfg, ctx->dtype, B, rows).total;
  if (ws_bytes < need) return ALBERT_E_WORKSPACE;
  const size_t out_bytes = (size_t)rows * ctx->cfg.out_dim * 4;
  if (overlaps(out, out_bytes, ids, (size_t)rows * 4) ||
      overlaps(out, out_bytes, lengths, (size_t)B * 4) || overlaps(out, out_bytes, ws, need))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rc = run_any(ctx, ids, lengths, B, T, rows, T, out, ws, s, (const float*)nullptr,
                         flags);
  return finish(rc, ws, s, flags);
}

int albert_encode_noalloc(albert_ctx* ctx, const int32_t* ids, const int32_t* lengths, int B,
                          int T, float* out, int32_t* status, void* stream, unsigned flags) {
  if (ctx && B == 0) return ALBERT_OK;  // empty batch: nothing to do
  if (!ctx || !ids || !lengths || !out || !status || B < 1 || T < 1 || T > ctx->cfg.max_pos ||
      (int64_t)B * T > INT32_MAX || !ctx->scratch || !device_matches(ctx))
    return ALBERT_E_ARG;
  const int64_t rows = (int64_t)B * T;
  const Layout L = plan(ctx->cfg, ctx->dtype, B, rows);
  if (L.total > (size_t)ALBERT_SCRATCH_BYTES) return ALBERT_E_SCRATCH;
  const size_t out_bytes = (size_t)rows * ctx->cfg.out_dim * 4;
  if (overlaps(out, out_bytes, ids, (size_t)rows * 4) ||
      overlaps(out, out_bytes, lengths, (size_t)B * 4) ||
      overlaps(out, out_bytes, status, 4) || overlaps(status, 4, ids, (size_t)rows * 4) ||
      overlaps(status, 4, lengths, (size_t)B * 4))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the same launch sequence as albert_encode, on this device's scratch
  int rc = run_any(ctx, ids, lengths, B, T, rows, T, out, ctx->scratch, s, (const float*)nullptr,
                   flags);
  if (rc == ALBERT_OK) {
    hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(1), 0, s,
                       reinterpret_cast<const int*>(static_cast<char*>(ctx->scratch) + L.status),
                       status);
    if (hipGetLastError() != hipSuccess) rc = ALBERT_E_HIP;
  }
  return rc;
}

int albert_encode_varlen(albert_ctx* ctx, const int32_t* ids, const int32_t* cu_seqlens, int n,
                         int total, int max_len, float* out, void* ws, size_t ws_bytes,
                         void* stream, unsigned flags) {
  if (ctx && n == 0 && total == 0) return ALBERT_OK;  // empty batch
  if (!ctx || !ids || !cu_seqlens || !out || !ws || n < 1 || total < 1 || max_len < 1 ||
      max_len > ctx->cfg.max_pos || ((uintptr_t)ws % kAlign) != 0 || !device_matches(ctx))
    return ALBERT_E_ARG;
  const size_t need = plan(ctx->cfg, ctx->dtype, n, total).total;
  if (ws_bytes < need) return ALBERT_E_WORKSPACE;
  const size_t out_bytes = (size_t)total * ctx->cfg.out_dim * 4;
  if (overlaps(out, out_bytes, ids, (size_t)total * 4) ||
      overlaps(out, out_bytes, cu_seqlens, (size_t)(n + 1) * 4) ||
      overlaps(out, out_bytes, ws, need))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rc = run_any(ctx, ids, cu_seqlens, n, 0, (int64_t)total, max_len, out, ws, s,
                         (const float*)nullptr, flags);
  return finish(rc, ws, s, flags);
}

int albert_encode_features(albert_ctx* ctx, const float* x, const int32_t* cu_seqlens, int n,
                           int total, int max_len, float* out, void* ws, size_t ws_bytes,
                           void* stream, unsigned flags) {
  if (ctx && n == 0 && total == 0) return ALBERT_OK;  // empty batch
  if (!ctx || !x || !cu_seqlens || !out || !ws || n < 1 || total < 1 || max_len < 1 ||
      max_len > ctx->cfg.max_pos || ((uintptr_t)ws % kAlign) != 0 || ((uintptr_t)x % 16) != 0 ||
      !device_matches(ctx))
    return ALBERT_E_ARG;
  const size_t need = plan(ctx->cfg, ctx->dtype, n, total).total;
  if (ws_bytes < need) return ALBERT_E_WORKSPACE;
  const size_t out_bytes = (size_t)total * ctx->cfg.out_dim * 4;
  if (overlaps(out, out_bytes, x, (size_t)total * ctx->cfg.emb * 4) ||
      overlaps(out, out_bytes, cu_seqlens, (size_t)(n + 1) * 4) ||
      overlaps(out, out_bytes, ws, need))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rc = run_any(ctx, (const int32_t*)nullptr, cu_seqlens, n, 0, (int64_t)total, max_len,
                         out, ws, s, x, flags);
  return finish(rc, ws, s, flags);
}

int albert_read_status(const void* ws, void* stream) {
  if (!ws) return ALBERT_E_ARG;
  int st = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&st, ws, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return ALBERT_E_HIP;
  return st;
}

int albert_tap(const albert_ctx* ctx, int n_seq, int64_t max_rows, int tap, size_t* offset,
               size_t* bytes, int64_t* row_stride) {
  if (!ctx || !offset || !bytes || !row_stride || n_seq < 1 || max_rows < 1) return ALBERT_E_ARG;
  const Layout L = plan(ctx->cfg, ctx->dtype, n_seq, max_rows);
  const size_t es = store_bytes(ctx->dtype), eo = operand_bytes(ctx->dtype);
  const albert_config& c = ctx->cfg;
  const size_t R = (size_t)max_rows;
  if ((tap == ALBERT_TAP_X8 || tap == ALBERT_TAP_X1_8) && ctx->dtype != ALBERT_FP8)
    return ALBERT_E_ARG;
  switch (tap) {
    case ALBERT_TAP_STATUS: *offset = L.status; *bytes = 4; *row_stride = 0; break;
    case ALBERT_TAP_CU: *offset = L.cu; *bytes = (size_t)(n_seq + 1) * 4; *row_stride = 0; break;
    case ALBERT_TAP_ROW_SEQ: *offset = L.row_seq; *bytes = R * 4; *row_stride = 0; break;
    case ALBERT_TAP_ROW_POS: *offset = L.row_pos; *bytes = R * 4; *row_stride = 0; break;
    case ALBERT_TAP_EMB: *offset = L.emb; *bytes = R * c.emb * eo; *row_stride = c.emb; break;
    case ALBERT_TAP_X: *offset = L.x; *bytes = R * c.hidden * es; *row_stride = c.hidden; break;
    case ALBERT_TAP_QKV:
      *offset = L.qkv; *bytes = R * 3 * c.hidden * es; *row_stride = 3 * c.hidden; break;
    case ALBERT_TAP_CTX: *offset = L.ctx; *bytes = R * c.hidden * eo; *row_stride = c.hidden; break;
    case ALBERT_TAP_X1: *offset = L.x1; *bytes = R * c.hidden * es; *row_stride = c.hidden; break;
    case ALBERT_TAP_G: *offset = L.g; *bytes = R * c.ffn * eo; *row_stride = c.ffn; break;
    case ALBERT_TAP_X8: *offset = L.x8; *bytes = R * c.hidden; *row_stride = c.hidden; break;
    case ALBERT_TAP_X1_8: *offset = L.x18; *bytes = R * c.hidden; *row_stride = c.hidden; break;
    default: return ALBERT_E_ARG;
  }
  return ALBERT_OK;
}

static void drop_events(albert_ctx* ctx) {
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  ctx->ev.clear();
  ctx->time_kind = -1;
  ctx->n_timed = 0;
}

int albert_time_kernel(albert_ctx* ctx, int kind, int max_launches) {
  if (!ctx || kind < -1 || kind >= ALBERT_K_COUNT || (kind >= 0 && max_launches < 1))
    return ALBERT_E_ARG;
  drop_events(ctx);
  if (kind < 0) return ALBERT_OK;
  ctx->ev.resize((size_t)2 * max_launches);
  for (auto& e : ctx->ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      drop_events(ctx);
      return ALBERT_E_HIP;
    }
  }
  ctx->time_kind = kind;
  return ALBERT_OK;
}

int albert_kernel_time(albert_ctx* ctx, int* launches, double* total_ms) {
  if (!ctx || !launches || !total_ms) return ALBERT_E_ARG;
  double sum = 0.0;
  for (int i = 0; i < ctx->n_timed; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(ctx->ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, ctx->ev[2 * i], ctx->ev[2 * i + 1]) != hipSuccess)
      return ALBERT_E_HIP;
    sum += ms;
  }
  *launches = ctx->n_timed;
  *total_ms = sum;
  return ALBERT_OK;
}

int albert_durations(const float* logits, int total, int K, float speed, int32_t* dur,
                     void* stream) {
  if (!logits || !dur || total < 1 || K < 1 || !std::isfinite(speed) || speed <= 0.f)
    return ALBERT_E_ARG;
  if (overlaps(dur, (size_t)total * 4, logits, (size_t)total * K * 4)) return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(durations_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, logits,
                     total, K, 1.0f / speed, dur);
  return hipGetLastError() == hipSuccess ? ALBERT_OK : ALBERT_E_HIP;
}

namespace {
struct ExpandLayout {
  size_t status, excl, block_sum, total;
  int nblocks;
};
ExpandLayout expand_plan(int total) {
  ExpandLayout L{};
  L.nblocks = (total + 1023) / 1024;
  size_t off = 0;
  L.status = off; off += kAlign;
  L.excl = off; off += align_up((size_t)total * 8, kAlign);
  L.block_sum = off; off += align_up((size_t)L.nblocks * 8, kAlign);
  L.total = off;
  return L;
}
}  // namespace

size_t albert_expand_workspace_bytes(int total) {
  return total < 1 ? 0 : expand_plan(total).total;
}

int albert_expand(const float* feat, const int32_t* dur, const int32_t* cu_tok, int n, int total,
                  int C, float* out, int64_t max_frames, int32_t* cu_frames, void* ws,
                  size_t ws_bytes, void* stream, unsigned flags) {
  if (!feat || !dur || !cu_tok || !out || !cu_frames || !ws || n < 1 || total < 1 || C < 4 ||
      C % 4 != 0 || max_frames < 1 || max_frames > INT32_MAX || ((uintptr_t)ws % kAlign) != 0)
    return ALBERT_E_ARG;
  const ExpandLayout L = expand_plan(total);
  if (ws_bytes < L.total) return ALBERT_E_WORKSPACE;
  const size_t out_b = (size_t)max_frames * C * 4, cuf_b = (size_t)(n + 1) * 4;
  const size_t feat_b = (size_t)total * C * 4, dur_b = (size_t)total * 4;
  if (overlaps(out, out_b, feat, feat_b) || overlaps(out, out_b, dur, dur_b) ||
      overlaps(out, out_b, cu_tok, cuf_b) || overlaps(out, out_b, ws, L.total) ||
      overlaps(out, out_b, cu_frames, cuf_b) || overlaps(cu_frames, cuf_b, feat, feat_b) ||
      overlaps(cu_frames, cuf_b, dur, dur_b) || overlaps(cu_frames, cuf_b, cu_tok, cuf_b) ||
      overlaps(cu_frames, cuf_b, ws, L.total))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int* status = reinterpret_cast<int*>(w + L.status);
  int64_t* excl = reinterpret_cast<int64_t*>(w + L.excl);
  int64_t* bsum = reinterpret_cast<int64_t*>(w + L.block_sum);
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, s, status);
  hipLaunchKernelGGL(dur_scan_local_kernel, dim3(L.nblocks), dim3(1024), 0, s, dur, total, excl,
                     bsum, status);
  hipLaunchKernelGGL(dur_scan_blocks_kernel, dim3(1), dim3(1024), 0, s, bsum, L.nblocks, excl,
                     cu_tok, n, total, max_frames, cu_frames, status);
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, feat, dur,
                     excl, bsum, total, C, out, status);
  const int rc = hipGetLastError() == hipSuccess ? ALBERT_OK : ALBERT_E_HIP;
  return finish(rc, ws, s, flags);
}

void albert_free(albert_ctx* ctx) {
  if (!ctx) return;
  drop_events(ctx);
  if (ctx->mem) (void)hipFree(ctx->mem);
  delete ctx;
}

const char* albert_status_str(int status) {
  switch (status) {
    case ALBERT_OK: return "ok";
    case ALBERT_E_ARG: return "invalid argument";
    case ALBERT_E_WORKSPACE: return "workspace too small";
    case ALBERT_E_LENGTH: return "sequence length out of range or bad offsets";
    case ALBERT_E_ID: return "phoneme id outside the vocabulary";
    case ALBERT_E_ALIAS: return "output overlaps an input or the workspace";
    case ALBERT_E_HIP: return "HIP runtime error";
    case ALBERT_E_SCRATCH: return "request larger than the static scratch (ALBERT_SCRATCH_BYTES)";
    case ALBERT_E_SYNC:
      return "cooperating workgroups did not meet (LayerNorm row halves or LSTM quad not co-resident)";
    default: return "unknown status";
  }
}

}  // extern "C"
