// Host-side parts of the encoder library that touch no GPU: configuration
// checks and the canonical tensor table, the weight repacking into the
// device image (bf16 rounding, E4M3 codes with per-row exponents, the
// head-major Q|K|V copy), the workspace plan and the aliasing test.  Plain
// C++ (no HIP): albert.hip includes it, and a sanitizer build of the host
// checks compiles it with g++ alone.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "albert.h"

namespace albert {

// Kokoro's encoder configuration.
inline albert_config kokoro_config() {
  return albert_config{178, 512, 2, 128, 768, 12, 64, 2048, 12, 1, 512, 1e-12f};
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline const char* const kNames[ALBERT_N_TENSORS] = {
    "emb.word", "emb.pos", "emb.type", "emb.ln.g", "emb.ln.b", "proj.w", "proj.b",
    "q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "o.w", "o.b", "attn_ln.g", "attn_ln.b",
    "ffn1.w", "ffn1.b", "ffn2.w", "ffn2.b", "ffn_ln.g", "ffn_ln.b", "out.w", "out.b"};

// Role (index into kNames) of tensor i under c's number of weight sets.
inline int role_of(const albert_config& c, int i) {
  const int G = c.n_groups;
  if (i < 0) return -1;
  if (i < 7) return i;
  if (i < 7 + ALBERT_LAYER_TENSORS * G) return 7 + (i - 7) % ALBERT_LAYER_TENSORS;
  if (i < 9 + ALBERT_LAYER_TENSORS * G) return 23 + (i - 7 - ALBERT_LAYER_TENSORS * G);
  return -1;
}

inline bool shape_of(const albert_config& c, int i, int64_t* r, int64_t* k) {
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
inline bool config_ok(const albert_config& c) {
  return c.emb == 128 && c.hidden == 768 && c.heads == 12 && c.head_dim == 64 &&
         c.vocab >= 1 && c.max_pos >= 1 && c.max_pos <= 512 && c.n_types >= 1 &&
         c.ffn >= 256 && c.ffn % 256 == 0 && c.out_dim >= 256 && c.out_dim % 256 == 0 &&
         c.n_iter >= 0 && c.n_groups >= 1 && c.n_groups <= std::max(c.n_iter, 1) &&
         std::isfinite(c.ln_eps) && c.ln_eps > 0.f;
}

inline uint16_t f32_to_bf16_bits(float f) {
  // round to nearest, ties to even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3 code of a finite value: round to nearest even on the 3-bit
// mantissa grid of the value's binade (subnormals share the 2^-6 binade),
// magnitudes of 448 and beyond saturate to 448 (0x7E; 0x7F is NaN).
inline uint8_t f32_to_e4m3(double v) {
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
inline int e4m3_row_exp(const float* row, int64_t n, float scale) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) m = std::max(m, std::fabs((double)row[i] * scale));
  if (m == 0.0) return 0;
  int k = (int)std::floor(std::log2(448.0 / m));
  while (m * std::ldexp(1.0, k + 1) <= 448.0) ++k;
  while (m * std::ldexp(1.0, k) > 448.0) --k;
  return std::min(k, 127);
}

// Exchange words the paired LayerNorm launches need for up to max_rows rows:
// 4*BM + 8 per row tile, for any tile height (64, 128 or 256 rows).
inline size_t ln_pair_words(int64_t max_rows) {
  return (size_t)std::max({(max_rows + 63) / 64 * (4 * 64 + 8), (max_rows + 127) / 128 * (4 * 128 + 8),
                           (max_rows + 255) / 256 * (4 * 256 + 8)});
}

// Split K (very small batches): requests of at most kSplitRows token rows
// (one utterance, or a few short ones) run their products as S partial
// products over 64-row tiles, whose fp32 partial sums [S][rows][N] take at
// most kSplitRows x kSplitCols x 4 bytes of the workspace.  S depends on the
// product alone (never on the batch), so two requests in this regime give
// every row the same bits, padded or packed.
constexpr int64_t kSplitRows = 256;
constexpr int64_t kSplitCols = 32768;  // S x N

// Splits of K for a product of max_rows x N x K over 64 x 256 tiles whose K
// slices number kslices, or 0 for the one-pass product: the largest S of a
// fixed ladder that divides the slices into an even number (at least 2) per
// split, with S x N <= kSplitCols.
inline int split_factor(int64_t max_rows, int N, int kslices) {
  if (max_rows > kSplitRows || N % 256 != 0) return 0;
  int best = 0;
  for (int S : {2, 3, 4, 6, 8, 12, 16}) {
    if (kslices % S != 0 || (kslices / S) % 2 != 0 || (int64_t)S * N > kSplitCols) continue;
    best = S;
  }
  return best;
}

// Byte offsets of a request's buffers in its workspace.
struct Layout {
  size_t status, cu, groups, row_seq, row_pos, emb, x, x1, x8, x18, qkv, ctx, g, xch, hand, part, total;
  int64_t rows_cap;
};

// Bytes per stored element / per matrix-product operand element.
inline size_t store_bytes(int dtype) { return dtype == ALBERT_F32 ? 4 : 2; }
inline size_t operand_bytes(int dtype) { return dtype == ALBERT_FP8 ? 1 : store_bytes(dtype); }

inline Layout plan(const albert_config& cfg, int dtype, int n_seq, int64_t max_rows) {
  Layout L{};
  const size_t es = store_bytes(dtype), eo = operand_bytes(dtype);
  const bool f8 = dtype == ALBERT_FP8;
  const int64_t rows = (int64_t)align_up((size_t)max_rows, 256);
  const size_t H = (size_t)cfg.hidden;
  size_t off = 0;
  L.rows_cap = rows;
  L.status = off; off += kAlign;
  L.cu = off; off += align_up((size_t)(n_seq + 1) * 4, kAlign);
  L.row_seq = off; off += align_up((size_t)rows * 4, kAlign);
  L.row_pos = off; off += align_up((size_t)rows * 4, kAlign);
  L.emb = off; off += align_up((size_t)rows * cfg.emb * eo, kAlign);
  L.x = off; off += align_up((size_t)rows * H * es, kAlign);
  L.x1 = off; off += align_up((size_t)rows * H * es, kAlign);
  L.x8 = off; off += f8 ? align_up((size_t)rows * H, kAlign) : 0;
  L.x18 = off; off += f8 ? align_up((size_t)rows * H, kAlign) : 0;
  L.qkv = off; off += align_up((size_t)rows * 3 * H * es, kAlign);
  L.ctx = off; off += align_up((size_t)rows * H * eo, kAlign);
  L.g = off; off += align_up((size_t)rows * cfg.ffn * eo, kAlign);
  // row statistics swapped by the paired LayerNorm GEMMs (bf16)
  L.xch = off; off += dtype != ALBERT_F32 ? align_up(ln_pair_words(rows) * 8, kAlign) : 0;
  // fp32 values a LayerNorm half hands to its partner (per row, a slot for
  // each half)
  L.hand = off; off += dtype != ALBERT_F32 ? align_up((size_t)rows * H * 4, kAlign) : 0;
  // partial sums of split-K products (very small batches)
  L.part = off; off += rows <= kSplitRows ? (size_t)rows * kSplitCols * 4 : 0;
  // the fused kernel's sequence groups (last: the activations keep the
  // offsets they have without it)
  L.groups = off; off += align_up((size_t)(n_seq + 2) * 4, kAlign);
  L.total = off;
  return L;
}

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Segments of the device weight image.  Globals first, then L_SEGS segments
// per layer weight set.  Under ALBERT_FP8 every matrix has a segment of
// per-row E8M0 exponents (empty otherwise); the head-major Q|K|V copy feeds
// the fused Q|K|V + attention kernel (bf16 and FP8; empty for fp32).
enum { S_WORD, S_POS, S_TYPE, S_EMB_G, S_EMB_B, S_PROJ_W, S_PROJ_B, S_OUT_W, S_OUT_B,
       S_PROJ_E, S_OUT_E, S_LAYER0 };
enum { L_QKV_W, L_QKV_B, L_O_W, L_O_B, L_LN1_G, L_LN1_B, L_F1_W, L_F1_B, L_F2_W, L_F2_B,
       L_LN2_G, L_LN2_B, L_QKV_E, L_O_E, L_F1_E, L_F2_E, L_QKV_WH, L_QKV_BH, L_QKV_EH, L_SEGS };
struct Seg { size_t off, bytes; };
struct Image {
  std::vector<unsigned char> bytes;
  std::vector<Seg> seg;
};

// The device image of a weight set: every tensor in its storage form, in
// segments (each 256-byte aligned) in the order of the S_ and L_ indices
// above.  host: albert_n_tensors(c) fp32 arrays in canonical order.
// Returns ALBERT_E_ARG for a null tensor or a non-finite value.
inline int build_image(const albert_config& c, const float* const* host, int dtype, Image* im) {
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
  const bool hm = dtype != ALBERT_F32;  // head-major Q|K|V copy for the fused kernel
  std::vector<Seg>& seg = im->seg;
  seg.clear();
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
  std::vector<unsigned char>& img = im->bytes;
  img.assign(off, 0);

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

  return ALBERT_OK;
}

}  // namespace albert
