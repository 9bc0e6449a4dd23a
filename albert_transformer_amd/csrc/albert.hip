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
#include <new>
#include <type_traits>
#include <vector>

#include "albert.h"
#include "attention.hpp"
#include "duration.hpp"
#include "gemm.hpp"
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

struct albert_ctx {
  albert_config cfg;
  int dtype;
  int device;
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

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

const char* const kNames[ALBERT_N_TENSORS] = {
    "emb.word", "emb.pos", "emb.type", "emb.ln.g", "emb.ln.b", "proj.w", "proj.b",
    "q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "o.w", "o.b", "attn_ln.g", "attn_ln.b",
    "ffn1.w", "ffn1.b", "ffn2.w", "ffn2.b", "ffn_ln.g", "ffn_ln.b", "out.w", "out.b"};

// Role (index into kNames) of tensor i under c's number of weight sets.
int role_of(const albert_config& c, int i) {
  const int G = c.n_groups;
  if (i < 0) return -1;
  if (i < 7) return i;
  if (i < 7 + ALBERT_LAYER_TENSORS * G) return 7 + (i - 7) % ALBERT_LAYER_TENSORS;
  if (i < 9 + ALBERT_LAYER_TENSORS * G) return 23 + (i - 7 - ALBERT_LAYER_TENSORS * G);
  return -1;
}

bool shape_of(const albert_config& c, int i, int64_t* r, int64_t* k) {
  const int64_t E = c.emb, H = c.hidden, F = c.ffn, O = c.out_dim;
  int64_t rows = 0, cols = 1;
  switch (role_of(c, i)) {
    case 0: rows = c.vocab; cols = E; break;
    case 1: rows = c.max_pos; cols = E; break;
    case 2: rows = c.n_types; cols = E; break;
    case 3: case 4: rows = E; break;
    case 5: rows = H; cols = E; break;
    case 6: rows = H; break;
    case 7: case 9: case 11: case 13: rows = H; cols = H; break;
    case 8: case 10: case 12: case 14: case 15: case 16: rows = H; break;
    case 17: rows = F; cols = H; break;
    case 18: rows = F; break;
    case 19: rows = H; cols = F; break;
    case 20: case 21: case 22: rows = H; break;
    case 23: rows = O; cols = H; break;
    case 24: rows = O; break;
    default: return false;
  }
  *r = rows;
  *k = cols;
  return true;
}

// The kernels are specialised for Kokoro's geometry; sizes that only change
// loop counts or table extents are free within tile multiples.
// (The GEMM K loop runs an even number of 128-byte slices: every K here --
// 128, 768 and ffn -- is a multiple of 128 elements.)
bool config_ok(const albert_config& c) {
  return c.emb == 128 && c.hidden == 768 && c.heads == 12 && c.head_dim == 64 &&
         c.vocab >= 1 && c.max_pos >= 1 && c.max_pos <= 512 && c.n_types >= 1 &&
         c.ffn >= 256 && c.ffn % 256 == 0 && c.out_dim >= 256 && c.out_dim % 256 == 0 &&
         c.n_iter >= 0 && c.n_groups >= 1 && c.n_groups <= std::max(c.n_iter, 1) &&
         std::isfinite(c.ln_eps) && c.ln_eps > 0.f;
}

uint16_t f32_to_bf16_bits(float f) {
  // round to nearest, ties to even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3 code of a finite value: round to nearest even on the 3-bit
// mantissa grid of the value's binade (subnormals share the 2^-6 binade),
// magnitudes of 448 and beyond saturate to 448 (0x7E; 0x7F is NaN).
uint8_t f32_to_e4m3(double v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  const double a = std::fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  int e = 0;
  std::frexp(a, &e);                 // a = f * 2^e, 0.5 <= f < 1
  int E = std::max(e - 1, -6);
  double q = std::nearbyint(std::ldexp(a, 3 - E));  // ties to even
  if (q >= 16.0) { q *= 0.5; E += 1; }              // rounded up into the next binade
  if (q < 8.0) return sign | (uint8_t)q;            // subnormal (E == -6) or zero
  return sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8));
}

// Largest k with max|row| * 2^k <= 448 (0 for a zero row), within the
// E8M0 range used here.
int e4m3_row_exp(const float* row, int64_t n, float scale) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) m = std::max(m, std::fabs((double)row[i] * scale));
  if (m == 0.0) return 0;
  int k = (int)std::floor(std::log2(448.0 / m));
  while (m * std::ldexp(1.0, k + 1) <= 448.0) ++k;
  while (m * std::ldexp(1.0, k) > 448.0) --k;
  return std::min(k, 127);
}

__global__ void clear_u64_kernel(unsigned long long* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

struct Layout {
  size_t status, cu, groups, row_seq, row_pos, emb, x, x1, x8, x18, qkv, ctx, g, xch, total;
  int64_t rows_cap;
};

// Bytes per stored element / per matrix-product operand element.
size_t store_bytes(int dtype) { return dtype == ALBERT_F32 ? 4 : 2; }
size_t operand_bytes(int dtype) { return dtype == ALBERT_FP8 ? 1 : store_bytes(dtype); }

Layout plan(const albert_ctx* c, int n_seq, int64_t max_rows) {
  Layout L{};
  const size_t es = store_bytes(c->dtype), eo = operand_bytes(c->dtype);
  const bool f8 = c->dtype == ALBERT_FP8;
  const int64_t rows = (int64_t)align_up((size_t)max_rows, 256);
  const size_t H = (size_t)c->cfg.hidden;
  size_t off = 0;
  L.rows_cap = rows;
  L.status = off; off += kAlign;
  L.cu = off; off += align_up((size_t)(n_seq + 1) * 4, kAlign);
  L.row_seq = off; off += align_up((size_t)rows * 4, kAlign);
  L.row_pos = off; off += align_up((size_t)rows * 4, kAlign);
  L.emb = off; off += align_up((size_t)rows * c->cfg.emb * eo, kAlign);
  L.x = off; off += align_up((size_t)rows * H * es, kAlign);
  L.x1 = off; off += align_up((size_t)rows * H * es, kAlign);
  L.x8 = off; off += f8 ? align_up((size_t)rows * H, kAlign) : 0;
  L.x18 = off; off += f8 ? align_up((size_t)rows * H, kAlign) : 0;
  L.qkv = off; off += align_up((size_t)rows * 3 * H * es, kAlign);
  L.ctx = off; off += align_up((size_t)rows * H * eo, kAlign);
  L.g = off; off += align_up((size_t)rows * c->cfg.ffn * eo, kAlign);
  // row statistics swapped by the paired LayerNorm GEMMs (bf16)
  L.xch = off; off += c->dtype != ALBERT_F32 ? align_up(ln_pair_words(rows) * 8, kAlign) : 0;
  // the fused kernel's sequence groups (last: the activations keep the
  // offsets they have without it)
  L.groups = off; off += align_up((size_t)(n_seq + 2) * 4, kAlign);
  L.total = off;
  return L;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

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
  const Layout L = plan(c, n_seq, max_rows);
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

  GemmArgs g = base;  // input projection E -> H
  g.X = emb; g.ldx = cf.emb; g.W = c->proj_w; g.wexp = c->proj_e; g.bias = c->proj_b;
  g.Y = X; g.ldy = H; g.Y8 = Y8; g.ldy8 = H; g.N = H; g.K = cf.emb;
  timed(c, ALBERT_K_PROJ, s, [&] { gemm_big<T, F8, EPI_BIAS>(g, max_rows, c->grid_cap, s); });

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
          launch_kernel(qkv_attention_kernel<F8>, dim3((unsigned)((pairs + 7) / 8 * 8)),
                        dim3(512), s, qa);
      });
    } else {
      g = base;  // fused Q|K|V projection
      g.X = X8; g.ldx = H; g.W = lw.qkv_w; g.wexp = lw.qkv_e; g.bias = lw.qkv_b; g.Y = QKV;
      g.ldy = 3 * H; g.N = 3 * H; g.K = H;
      timed(c, ALBERT_K_QKV, s, [&] { gemm_big<T, F8, EPI_BIAS>(g, max_rows, c->grid_cap, s); });

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
    gemm_layernorm(g, ALBERT_K_ATTN_OUT_LN);

    g = base;  // FFN 768 -> 2048 + GELU
    g.X = X18; g.ldx = H; g.W = lw.ffn1_w; g.wexp = lw.ffn1_e; g.bias = lw.ffn1_b; g.Y = G;
    g.ldy = F; g.N = F; g.K = H;
    timed(c, ALBERT_K_FFN1_GELU, s, [&] { gemm_big<T, F8, EPI_GELU>(g, max_rows, c->grid_cap, s); });

    g = base;  // FFN 2048 -> 768 + residual + LayerNorm
    g.X = G; g.ldx = F; g.W = lw.ffn2_w; g.wexp = lw.ffn2_e; g.bias = lw.ffn2_b; g.R = X1;
    g.ldr = H; g.ln_g = lw.ln2_g; g.ln_b = lw.ln2_b; g.Y = X; g.ldy = H; g.Y8 = Y8; g.ldy8 = H;
    g.N = H; g.K = F;
    gemm_layernorm(g, ALBERT_K_FFN2_LN);
  }

  g = base;  // output projection H -> 512, fp32, into the caller's rows
  g.X = X8; g.ldx = H; g.W = c->out_w; g.wexp = c->out_e; g.bias = c->out_b; g.out = out;
  g.row_seq = row_seq; g.row_pos = row_pos; g.out_T = pad_T; g.N = cf.out_dim; g.K = H;
  timed(c, ALBERT_K_OUT, s, [&] { gemm_big<T, F8, EPI_OUT>(g, max_rows, c->grid_cap, s); });
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
  *cfg = albert_config{178, 512, 2, 128, 768, 12, 64, 2048, 12, 1, 512, 1e-12f};
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
  const size_t es = store_bytes(dtype);   // tables
  const size_t em = operand_bytes(dtype); // weight matrices
  const int G = c.n_groups, NT = 9 + ALBERT_LAYER_TENSORS * G;
  std::vector<int64_t> rows(NT), cols(NT);
  for (int i = 0; i < NT; ++i) {
    if (!host[i]) return ALBERT_E_ARG;
    shape_of(c, i, &rows[i], &cols[i]);
    for (int64_t e = 0; e < rows[i] * cols[i]; ++e)
      if (!std::isfinite(host[i][e])) return ALBERT_E_ARG;
  }
  const int64_t H = c.hidden;

  // Device image: segments in the order below, each 256-byte aligned.
  // Per weight set: Q|K|V packed into one [3H, H] matrix (queries scaled)
  // and one [3H] bias, then o, attn LN, ffn1, ffn2, ffn LN.  Under
  // ALBERT_FP8 every matrix also has a segment of per-row E8M0 exponents
  // (empty otherwise).
  enum { S_WORD, S_POS, S_TYPE, S_EMB_G, S_EMB_B, S_PROJ_W, S_PROJ_B, S_OUT_W, S_OUT_B,
         S_PROJ_E, S_OUT_E, S_LAYER0 };
  enum { L_QKV_W, L_QKV_B, L_O_W, L_O_B, L_LN1_G, L_LN1_B, L_F1_W, L_F1_B, L_F2_W, L_F2_B,
         L_LN2_G, L_LN2_B, L_QKV_E, L_O_E, L_F1_E, L_F2_E, L_QKV_WH, L_QKV_BH, L_QKV_EH, L_SEGS };
  const bool hm = dtype != ALBERT_F32;  // head-major Q|K|V copy for the fused kernel
  struct Seg { size_t off, bytes; };
  std::vector<Seg> seg;
  size_t off = 0;
  auto add = [&](size_t bytes) { seg.push_back({off, bytes}); off += align_up(bytes, kAlign); };
  add((size_t)c.vocab * c.emb * es);       // word
  add((size_t)c.max_pos * c.emb * es);     // pos
  add((size_t)c.n_types * c.emb * es);     // type
  add((size_t)c.emb * 4);                  // emb g
  add((size_t)c.emb * 4);                  // emb b
  add((size_t)H * c.emb * em);             // proj w
  add((size_t)H * 4);                      // proj b
  add((size_t)c.out_dim * H * em);         // out w
  add((size_t)c.out_dim * 4);              // out b
  add(f8 ? (size_t)H : 0);                 // proj exponents
  add(f8 ? (size_t)c.out_dim : 0);         // out exponents
  for (int g = 0; g < G; ++g) {
    add((size_t)3 * H * H * em);           // qkv w
    add((size_t)3 * H * 4);                // qkv b
    add((size_t)H * H * em);               // o w
    add((size_t)H * 4);                    // o b
    add((size_t)H * 4);                    // ln1 g
    add((size_t)H * 4);                    // ln1 b
    add((size_t)c.ffn * H * em);           // ffn1 w
    add((size_t)c.ffn * 4);                // ffn1 b
    add((size_t)H * c.ffn * em);           // ffn2 w
    add((size_t)H * 4);                    // ffn2 b
    add((size_t)H * 4);                    // ln2 g
    add((size_t)H * 4);                    // ln2 b
    add(f8 ? (size_t)3 * H : 0);           // qkv exponents
    add(f8 ? (size_t)H : 0);               // o exponents
    add(f8 ? (size_t)c.ffn : 0);           // ffn1 exponents
    add(f8 ? (size_t)H : 0);               // ffn2 exponents
    add(hm ? (size_t)3 * H * H * em : 0);  // head-major q/8 | k | v
    add(hm ? (size_t)3 * H * 4 : 0);       // their biases
    add(hm && f8 ? (size_t)3 * H : 0);     // their exponents
  }
  std::vector<unsigned char> img(off, 0);

  auto put_mat = [&](int s, const float* src, int64_t n, float scale, size_t elem_off) {
    unsigned char* d = img.data() + seg[s].off + elem_off * es;
    for (int64_t e = 0; e < n; ++e) {
      const float v = src[e] * scale;  // scale is 1 or a power of two: exact
      if (es == 2) {
        const uint16_t bits = f32_to_bf16_bits(v);
        std::memcpy(d + e * 2, &bits, 2);
      } else {
        std::memcpy(d + e * 4, &v, 4);
      }
    }
  };
  auto put_vec = [&](int s, const float* src, int64_t n, float scale, size_t elem_off) {
    float* d = reinterpret_cast<float*>(img.data() + seg[s].off) + elem_off;
    for (int64_t e = 0; e < n; ++e) d[e] = src[e] * scale;
  };
  // A weight matrix [rows, cols] placed at row row_off of segment s: in the
  // storage dtype, or (ALBERT_FP8) as E4M3 codes of each row times 2^k with
  // the exponent 127 - k in segment se.
  auto put_w = [&](int s, int se, const float* src, int64_t rows, int64_t cols, float scale,
                   int64_t row_off) {
    if (!f8) {
      put_mat(s, src, rows * cols, scale, (size_t)(row_off * cols));
      return;
    }
    unsigned char* d = img.data() + seg[s].off + row_off * cols;
    unsigned char* ex = img.data() + seg[se].off + row_off;
    for (int64_t r = 0; r < rows; ++r) {
      const float* row = src + r * cols;
      const int k = e4m3_row_exp(row, cols, scale);
      ex[r] = (unsigned char)(127 - k);
      for (int64_t i = 0; i < cols; ++i)
        d[r * cols + i] = f32_to_e4m3(std::ldexp((double)(row[i] * scale), k));
    }
  };
  const float qscale = 1.0f / std::sqrt((float)c.head_dim);  // 1/8 for head_dim 64
  put_mat(S_WORD, host[0], rows[0] * cols[0], 1.f, 0);
  put_mat(S_POS, host[1], rows[1] * cols[1], 1.f, 0);
  put_mat(S_TYPE, host[2], rows[2] * cols[2], 1.f, 0);
  put_vec(S_EMB_G, host[3], c.emb, 1.f, 0);
  put_vec(S_EMB_B, host[4], c.emb, 1.f, 0);
  put_w(S_PROJ_W, S_PROJ_E, host[5], H, c.emb, 1.f, 0);
  put_vec(S_PROJ_B, host[6], H, 1.f, 0);
  const int out_i = 7 + ALBERT_LAYER_TENSORS * G;
  put_w(S_OUT_W, S_OUT_E, host[out_i], c.out_dim, H, 1.f, 0);
  put_vec(S_OUT_B, host[out_i + 1], c.out_dim, 1.f, 0);
  for (int g = 0; g < G; ++g) {
    const float* const* t = host + 7 + ALBERT_LAYER_TENSORS * g;  // q.w .. ffn_ln.b
    const int s0 = S_LAYER0 + L_SEGS * g;
    put_w(s0 + L_QKV_W, s0 + L_QKV_E, t[0], H, H, qscale, 0);
    put_w(s0 + L_QKV_W, s0 + L_QKV_E, t[2], H, H, 1.f, H);
    put_w(s0 + L_QKV_W, s0 + L_QKV_E, t[4], H, H, 1.f, 2 * H);
    put_vec(s0 + L_QKV_B, t[1], H, qscale, 0);
    put_vec(s0 + L_QKV_B, t[3], H, 1.f, (size_t)H);
    put_vec(s0 + L_QKV_B, t[5], H, 1.f, (size_t)(2 * H));
    put_w(s0 + L_O_W, s0 + L_O_E, t[6], H, H, 1.f, 0);
    put_vec(s0 + L_O_B, t[7], H, 1.f, 0);
    put_vec(s0 + L_LN1_G, t[8], H, 1.f, 0);
    put_vec(s0 + L_LN1_B, t[9], H, 1.f, 0);
    put_w(s0 + L_F1_W, s0 + L_F1_E, t[10], c.ffn, H, 1.f, 0);
    put_vec(s0 + L_F1_B, t[11], c.ffn, 1.f, 0);
    put_w(s0 + L_F2_W, s0 + L_F2_E, t[12], H, c.ffn, 1.f, 0);
    put_vec(s0 + L_F2_B, t[13], H, 1.f, 0);
    put_vec(s0 + L_LN2_G, t[14], H, 1.f, 0);
    put_vec(s0 + L_LN2_B, t[15], H, 1.f, 0);
    if (hm) {  // head h: rows h*64.. of q (scaled), then of k, then of v
      const int64_t D = c.head_dim, NH = c.heads;
      unsigned char* wd = img.data() + seg[s0 + L_QKV_WH].off;
      float* bd = reinterpret_cast<float*>(img.data() + seg[s0 + L_QKV_BH].off);
      const unsigned char* wq = img.data() + seg[s0 + L_QKV_W].off;  // packed rows, as stored
      const unsigned char* eq = img.data() + seg[s0 + L_QKV_E].off;
      unsigned char* ed = img.data() + seg[s0 + L_QKV_EH].off;
      for (int64_t hd = 0; hd < NH; ++hd)
        for (int64_t part = 0; part < 3; ++part)
          for (int64_t dd = 0; dd < D; ++dd) {
            const int64_t src_row = hd * D + dd, dst_row = (hd * 3 + part) * D + dd;
            const float sc = part == 0 ? qscale : 1.f;
            // the same stored row (bf16 values or E4M3 codes), moved
            std::memcpy(wd + dst_row * H * em, wq + (part * H + src_row) * H * em, (size_t)(H * em));
            if (f8) ed[dst_row] = eq[part * H + src_row];
            bd[dst_row] = t[2 * part + 1][src_row] * sc;
          }
    }
  }

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
      }
    for (const void* k : ks) {
      int per_cu = 0;
      ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, f8 ? 256 : 512, 0) ==
                     hipSuccess &&
           per_cu >= 1;
    }
    ctx->ln_pair = ok;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(ctx->mem, img.data(), off, hipMemcpyHostToDevice, s) != hipSuccess ||
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
  return plan(ctx, n_seq, max_rows).total;
}

int albert_encode(albert_ctx* ctx, const int32_t* ids, const int32_t* lengths, int B, int T,
                  float* out, void* ws, size_t ws_bytes, void* stream, unsigned flags) {
  if (ctx && B == 0) return ALBERT_OK;  // empty batch: nothing to do
  if (!ctx || !ids || !lengths || !out || !ws || B < 1 || T < 1 || T > ctx->cfg.max_pos ||
      ((uintptr_t)ws % kAlign) != 0 || (int64_t)B * T > INT32_MAX || !device_matches(ctx))
    return ALBERT_E_ARG;
  const int64_t rows = (int64_t)B * T;
  const size_t need = plan(ctx, B, rows).total;
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

int albert_encode_varlen(albert_ctx* ctx, const int32_t* ids, const int32_t* cu_seqlens, int n,
                         int total, int max_len, float* out, void* ws, size_t ws_bytes,
                         void* stream, unsigned flags) {
  if (ctx && n == 0 && total == 0) return ALBERT_OK;  // empty batch
  if (!ctx || !ids || !cu_seqlens || !out || !ws || n < 1 || total < 1 || max_len < 1 ||
      max_len > ctx->cfg.max_pos || ((uintptr_t)ws % kAlign) != 0 || !device_matches(ctx))
    return ALBERT_E_ARG;
  const size_t need = plan(ctx, n, total).total;
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
  const size_t need = plan(ctx, n, total).total;
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
  const Layout L = plan(ctx, n_seq, max_rows);
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
    case ALBERT_E_SYNC:
      return "cooperating workgroups did not meet (LayerNorm row halves or LSTM quad not co-resident)";
    default: return "unknown status";
  }
}

}  // extern "C"
