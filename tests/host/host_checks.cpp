// Host-side checks of the encoder library's C++ that touches no GPU (the
// weight repacking, the E4M3 and bf16 encoders, the workspace plan and the
// aliasing test), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.
//
// Each check compares against a definition written independently here:
// E4M3 by the nearest of the 254 finite code values (decoded from their
// bit fields), bf16 by the two neighbouring bf16 values, the plan by
// disjointness and alignment of every buffer, the image by reading every
// stored tensor back.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "host.hpp"

using namespace albert;

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// Value of an E4M3 code from its fields: sign, 4-bit exponent (bias 7), 3-bit
// mantissa; exponent field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN.
static double e4m3_value(int code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  const double mag = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, e - 10);
  return s ? -mag : mag;
}

static void check_e4m3() {
  std::vector<double> grid;  // the non-negative finite values, ascending
  for (int c = 0; c < 0x7F; ++c) grid.push_back(e4m3_value(c));
  for (int c = 0; c < 0x7F; ++c) CHECK(f32_to_e4m3(e4m3_value(c)) == c);          // exact codes
  for (int c = 1; c < 0x7F; ++c) CHECK(f32_to_e4m3(-e4m3_value(c)) == (0x80 | c));
  auto nearest = [&](double a) {  // ties to the even code (its mantissa's last bit 0)
    if (a >= 448.0) return 0x7E;
    int best = 0;
    for (int c = 1; c < 0x7F; ++c) {
      const double d = std::fabs(grid[c] - a), db = std::fabs(grid[best] - a);
      if (d < db || (d == db && (c & 1) == 0)) best = c;
    }
    return best;
  };
  for (int c = 0; c + 1 < 0x7F; ++c) {  // midpoints and their neighbours
    const double mid = 0.5 * (grid[c] + grid[c + 1]);
    for (double v : {mid, std::nextafter(mid, 0.0), std::nextafter(mid, 1e9)}) {
      CHECK(f32_to_e4m3(v) == nearest(v));
      CHECK(f32_to_e4m3(-v) == (0x80 | nearest(v)) || nearest(v) == 0);
    }
  }
  std::mt19937_64 rng(7);
  std::uniform_real_distribution<double> ex(-14.0, 10.0);
  for (int i = 0; i < 200000; ++i) {
    const double v = std::ldexp(1.0, 0) * std::exp2(ex(rng));
    CHECK(f32_to_e4m3(v) == nearest(v));
  }
  CHECK(f32_to_e4m3(1e30) == 0x7E && f32_to_e4m3(-1e30) == 0xFE);  // saturation
}

static void check_bf16() {
  std::mt19937 rng(11);
  std::uniform_int_distribution<uint32_t> bits;
  for (int i = 0; i < 500000; ++i) {
    uint32_t u = bits(rng);
    if (((u >> 23) & 0xFF) == 0xFF) continue;  // finite inputs only
    float f;
    std::memcpy(&f, &u, 4);
    const uint16_t b = f32_to_bf16_bits(f);
    const uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;  // the two bf16 neighbours
    float flo, fhi, fb;
    std::memcpy(&flo, &lo, 4);
    std::memcpy(&fhi, &hi, 4);
    const uint32_t ub = (uint32_t)b << 16;
    std::memcpy(&fb, &ub, 4);
    const double dlo = std::fabs((double)f - flo), dhi = std::fabs((double)fhi - f);
    if (((hi >> 23) & 0xFF) == 0xFF) {  // the upper neighbour overflows
      CHECK(ub == lo || std::isinf(fb));
      continue;
    }
    const uint32_t want = dlo < dhi ? lo : dhi < dlo ? hi : (((lo >> 16) & 1) ? hi : lo);
    CHECK(ub == want);
  }
}

static void check_plan() {
  albert_config c = kokoro_config();
  for (int dtype : {ALBERT_F32, ALBERT_BF16, ALBERT_FP8})
    for (int n : {1, 2, 7, 256, 1024, 9000})
      for (int64_t rows : {(int64_t)1, (int64_t)36, (int64_t)255, (int64_t)256, (int64_t)4425,
                           (int64_t)32768, (int64_t)61876}) {
        if (rows < n) continue;
        const Layout L = plan(c, dtype, n, rows);
        const int64_t R = L.rows_cap;
        CHECK(R >= rows && R % 256 == 0 && R - rows < 256);
        const size_t es = store_bytes(dtype), eo = operand_bytes(dtype);
        const bool pair = dtype != ALBERT_F32, f8 = dtype == ALBERT_FP8;
        struct B { size_t off, bytes; };
        const std::vector<B> bufs = {
            {L.status, 4}, {L.cu, (size_t)(n + 1) * 4}, {L.row_seq, (size_t)R * 4},
            {L.row_pos, (size_t)R * 4}, {L.emb, (size_t)R * c.emb * eo},
            {L.x, (size_t)R * c.hidden * es}, {L.x1, (size_t)R * c.hidden * es},
            {L.x8, f8 ? (size_t)R * c.hidden : 0}, {L.x18, f8 ? (size_t)R * c.hidden : 0},
            {L.qkv, (size_t)R * 3 * c.hidden * es}, {L.ctx, (size_t)R * c.hidden * eo},
            {L.g, (size_t)R * c.ffn * eo}, {L.xch, pair ? ln_pair_words(R) * 8 : 0},
            {L.hand, pair ? (size_t)R * c.hidden * 4 : 0}, {L.groups, (size_t)(n + 2) * 4},
            {L.part, R <= kSplitRows ? (size_t)R * kSplitCols * 4 : 0}};
        for (size_t i = 0; i < bufs.size(); ++i) {
          CHECK(bufs[i].off % 256 == 0);
          CHECK(bufs[i].off + bufs[i].bytes <= L.total);
          for (size_t j = i + 1; j < bufs.size(); ++j)
            CHECK(bufs[i].bytes == 0 || bufs[j].bytes == 0 ||
                  bufs[i].off + bufs[i].bytes <= bufs[j].off || bufs[j].off + bufs[j].bytes <= bufs[i].off);
        }
      }
}

static void check_split_factor() {
  // every split leaves whole, even slice counts within the partial-sum bytes,
  // and depends on the product only
  for (int N : {512, 768, 2048, 2304})
    for (int ks : {4, 12, 24, 32, 64}) {
      const int S = split_factor(36, N, ks);
      for (int64_t rows : {(int64_t)1, (int64_t)200, (int64_t)256})
        CHECK(split_factor(rows, N, ks) == S);
      CHECK(split_factor(257, N, ks) == 0 && split_factor(32768, N, ks) == 0);
      if (S == 0) continue;
      CHECK(S >= 2 && ks % S == 0 && (ks / S) % 2 == 0 && (int64_t)S * N <= kSplitCols);
    }
  CHECK(split_factor(36, 768, 64) == 16);   // fp32 2048-deep: 16 splits of 4 slices
  CHECK(split_factor(36, 2304, 24) == 12);  // fp32 Q|K|V: 12 splits of 2 slices
  CHECK(split_factor(36, 2048, 12) == 6);   // bf16 FFN1: 6 splits of 2 slices
}

static void check_overlaps() {
  static char buf[64];
  CHECK(overlaps(buf, 8, buf + 4, 8) && overlaps(buf + 4, 8, buf, 8));
  CHECK(!overlaps(buf, 8, buf + 8, 8) && !overlaps(buf + 8, 8, buf, 8));
  CHECK(overlaps(buf, 64, buf + 10, 1) && overlaps(buf + 10, 1, buf, 64));
  CHECK(!overlaps(buf, 0, buf, 8) && !overlaps(nullptr, 8, buf, 8) && !overlaps(buf, 8, nullptr, 8));
}

// Read a bf16 bit pattern back as a float.
static float bf(const unsigned char* p) {
  uint16_t b;
  std::memcpy(&b, p, 2);
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

static void check_image(int G, int dtype) {
  albert_config c = kokoro_config();
  c.n_groups = G;
  const int NT = 9 + ALBERT_LAYER_TENSORS * G;
  std::vector<std::vector<float>> t(NT);
  std::vector<const float*> ptr(NT);
  std::mt19937 rng(100 + G + 10 * dtype);
  std::normal_distribution<float> nd(0.f, 0.02f);
  for (int i = 0; i < NT; ++i) {
    int64_t r, k;
    CHECK(shape_of(c, i, &r, &k));
    t[i].resize((size_t)(r * k));
    for (float& v : t[i]) v = nd(rng);
    ptr[i] = t[i].data();
  }
  Image im;
  CHECK(build_image(c, ptr.data(), dtype, &im) == ALBERT_OK);
  const size_t es = store_bytes(dtype), em = operand_bytes(dtype);
  const int64_t H = c.hidden;
  for (size_t s = 0; s < im.seg.size(); ++s) {
    CHECK(im.seg[s].off % 256 == 0);
    CHECK(im.seg[s].off + im.seg[s].bytes <= im.bytes.size());
    if (s + 1 < im.seg.size()) CHECK(im.seg[s].off + im.seg[s].bytes <= im.seg[s + 1].off);
  }
  // a matrix element as stored, as the value the products use
  auto wval = [&](int seg_w, int seg_e, int64_t row, int64_t col, int64_t cols) -> double {
    const unsigned char* base = im.bytes.data() + im.seg[seg_w].off;
    if (dtype == ALBERT_FP8) {
      const int e = im.bytes[im.seg[seg_e].off + row];
      return e4m3_value(base[row * cols + col]) * std::ldexp(1.0, e - 127);
    }
    if (dtype == ALBERT_BF16) return bf(base + (row * cols + col) * 2);
    float f;
    std::memcpy(&f, base + (row * cols + col) * 4, 4);
    return f;
  };
  // within the storage format's rounding: half a unit in the last place (an
  // E4M3 value below 2^-6 in the row's scaled units is subnormal: half a
  // step of 2^-9 there); k is the row's E8M0 exponent under FP8
  auto near = [&](double got, double want, int e = 127) {
    const double tol = dtype == ALBERT_F32    ? 0.0
                       : dtype == ALBERT_BF16 ? std::ldexp(std::fabs(want), -8)
                                              : std::max(std::ldexp(std::fabs(want), -4), std::ldexp(1.0, -10 + e - 127));
    return std::fabs(got - want) <= tol;
  };
  auto rexp = [&](int seg_e, int64_t row) {
    return dtype == ALBERT_FP8 ? (int)im.bytes[im.seg[seg_e].off + row] : 127;
  };
  // tables in the storage type
  for (int64_t e = 0; e < (int64_t)c.vocab * c.emb; e += 37) {
    const unsigned char* b = im.bytes.data() + im.seg[S_WORD].off + e * es;
    float f;
    if (es == 2) f = bf(b); else std::memcpy(&f, b, 4);
    CHECK(near(f, t[0][e]));
  }
  for (int g = 0; g < G; ++g) {
    const int s0 = S_LAYER0 + L_SEGS * g;
    const float* const* lt = ptr.data() + 7 + ALBERT_LAYER_TENSORS * g;  // q.w ..
    for (int64_t r = 0; r < 3 * H; r += 7)
      for (int64_t k = 0; k < H; k += 11) {
        const int part = (int)(r / H);
        const double want = lt[2 * part][(r % H) * H + k] * (part == 0 ? 0.125 : 1.0);
        CHECK(near(wval(s0 + L_QKV_W, s0 + L_QKV_E, r, k, H), want, rexp(s0 + L_QKV_E, r)));
      }
    const float* qb = reinterpret_cast<const float*>(im.bytes.data() + im.seg[s0 + L_QKV_B].off);
    for (int64_t r = 0; r < 3 * H; ++r) {
      const int part = (int)(r / H);
      CHECK(qb[r] == lt[2 * part + 1][r % H] * (part == 0 ? 0.125f : 1.0f));
    }
    if (dtype != ALBERT_F32) {  // head-major copy: the same stored rows, moved
      const unsigned char* wh = im.bytes.data() + im.seg[s0 + L_QKV_WH].off;
      const unsigned char* wp = im.bytes.data() + im.seg[s0 + L_QKV_W].off;
      const float* bh = reinterpret_cast<const float*>(im.bytes.data() + im.seg[s0 + L_QKV_BH].off);
      for (int64_t hd = 0; hd < c.heads; ++hd)
        for (int part = 0; part < 3; ++part)
          for (int64_t d = 0; d < c.head_dim; ++d) {
            const int64_t dst = (hd * 3 + part) * c.head_dim + d, src = part * H + hd * c.head_dim + d;
            CHECK(std::memcmp(wh + dst * H * em, wp + src * H * em, (size_t)(H * em)) == 0);
            CHECK(bh[dst] == qb[src]);
            if (dtype == ALBERT_FP8)
              CHECK(im.bytes[im.seg[s0 + L_QKV_EH].off + dst] == im.bytes[im.seg[s0 + L_QKV_E].off + src]);
          }
    }
    for (int64_t r = 0; r < c.ffn; r += 13)
      for (int64_t k = 0; k < H; k += 17)
        CHECK(near(wval(s0 + L_F1_W, s0 + L_F1_E, r, k, H), lt[10][r * H + k], rexp(s0 + L_F1_E, r)));
    for (int64_t r = 0; r < H; r += 13)
      for (int64_t k = 0; k < c.ffn; k += 17)
        CHECK(near(wval(s0 + L_F2_W, s0 + L_F2_E, r, k, c.ffn), lt[12][r * c.ffn + k], rexp(s0 + L_F2_E, r)));
    const float* g2 = reinterpret_cast<const float*>(im.bytes.data() + im.seg[s0 + L_LN2_G].off);
    for (int64_t r = 0; r < H; ++r) CHECK(g2[r] == lt[14][r]);  // vectors exactly
    if (dtype == ALBERT_FP8) {  // each row's largest magnitude times 2^k is at most 448
      for (int64_t r = 0; r < c.ffn; r += 5) {
        const int e = im.bytes[im.seg[s0 + L_F1_E].off + r];
        double m = 0;
        for (int64_t k = 0; k < H; ++k) m = std::max(m, std::fabs((double)lt[10][r * H + k]));
        const int k2 = 127 - e;
        CHECK(m * std::ldexp(1.0, k2) <= 448.0 && m * std::ldexp(1.0, k2 + 1) > 448.0);
      }
    }
  }
  // a non-finite weight is refused
  t[5][3] = NAN;
  CHECK(build_image(c, ptr.data(), dtype, &im) == ALBERT_E_ARG);
  ptr[5] = nullptr;
  CHECK(build_image(c, ptr.data(), dtype, &im) == ALBERT_E_ARG);
}

int main() {
  check_e4m3();
  check_bf16();
  check_plan();
  check_split_factor();
  check_overlaps();
  for (int dtype : {ALBERT_F32, ALBERT_BF16, ALBERT_FP8})
    for (int G : {1, 3}) check_image(G, dtype);
  std::printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
