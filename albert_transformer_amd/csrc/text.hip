// Host side of Kokoro's parallel text encoder: the albert_text_* part of the
// C ABI in include/albert.h.
//
// Launch sequence of one request (all on the caller's stream):
//   derive (lengths -> offsets, status) -> rows/IDs check -> embedding ->
//   convolution taps of each row -> n_conv x [convolution GEMM (shifted
//   rows read directly) + LayerNorm + LeakyReLU] ->
//   LSTM input projection GEMM (both directions, fp32) -> LSTM recurrence
//   -> zeroing of padded rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "albert.h"
#include "gemm.hpp"
#include "launch.hpp"
#include "prologue.hpp"
#include "text_encoder.hpp"

using namespace albert;

struct albert_text_ctx {
  albert_text_config cfg;
  int device;
  int grid_cap;
  void* mem;
  const bf16* emb;
  std::vector<const bf16*> conv_w;  // [C, K*C], column j*C + c is tap j, input channel c
  std::vector<const float*> conv_b, ln_g, ln_b;
  const bf16* w_ih;                 // [8H, C]: forward gates, then backward gates
  const float* b_gates;             // [8H]: b_ih + b_hh
  const bf16* w_hh;                 // both directions, in the recurrence's fragment order
  const bf16* w_hh_mc;              // the same, in the four-workgroup recurrence's order
  int mc_groups = 0;                // groups of 32 sequences per cooperative launch (0: none)
  int time_kind = -1;
  int n_timed = 0;
  std::vector<hipEvent_t> ev;
};

namespace {

bool text_config_ok(const albert_text_config& c) {
  return c.vocab >= 1 && c.channels == 512 && c.kernel >= 1 && c.kernel <= 7 &&
         c.kernel % 2 == 1 && c.n_conv >= 1 && c.n_conv <= 8 && c.hidden == kLstmH && std::isfinite(c.ln_eps) &&
         c.ln_eps > 0.f && std::isfinite(c.slope);
}

// Canonical names for up to 8 convolution blocks.
const std::vector<std::string>& all_names() {
  static const std::vector<std::string> names = [] {
    std::vector<std::string> v{"emb"};
    for (int i = 0; i < 8; ++i)
      for (const char* k : {".v", ".g", ".b", ".ln.g", ".ln.b"})
        v.push_back("conv" + std::to_string(i) + k);
    for (const char* d : {"fwd", "bwd"})
      for (const char* k : {".w_ih", ".w_hh", ".b_ih", ".b_hh"})
        v.push_back(std::string("lstm.") + d + k);
    return v;
  }();
  return names;
}

// Index into all_names() of tensor `index` under c, or -1.
int name_slot(const albert_text_config& c, int index) {
  const int nc = 5 * c.n_conv;
  if (index < 0 || index >= 1 + nc + 8) return -1;
  if (index <= nc) return index;
  return 1 + 5 * 8 + (index - 1 - nc);
}

bool text_shape(const albert_text_config& c, int index, int64_t* r, int64_t* k) {
  const int slot = name_slot(c, index);
  if (slot < 0) return false;
  const int64_t C = c.channels, H = c.hidden;
  if (slot == 0) { *r = c.vocab; *k = C; return true; }
  if (slot <= 40) {
    const int part = (slot - 1) % 5;
    *r = C;
    *k = part == 0 ? C * c.kernel : 1;
    return true;
  }
  const int part = (slot - 41) % 4;  // w_ih, w_hh, b_ih, b_hh
  *r = 4 * H;
  *k = part == 0 ? C : part == 1 ? H : 1;
  return true;
}

uint16_t bf16_bits(double v) {
  const float f = (float)v;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite values)
  return (uint16_t)(u >> 16);
}

struct TextLayout {
  size_t status, cu, row_seq, row_pos, emb, x1, x2, taps, xg, hx, flags, total;
  int mc_groups;  // groups of 32 sequences per launch of the four-workgroup recurrence
};

TextLayout text_plan(const albert_text_ctx* c, int n_seq, int64_t max_rows) {
  TextLayout L{};
  const size_t rows = align_up((size_t)max_rows, 256);
  const size_t C = (size_t)c->cfg.channels, K = (size_t)c->cfg.kernel, H = (size_t)c->cfg.hidden;
  size_t off = 0;
  L.status = off; off += kAlign;
  L.cu = off; off += align_up((size_t)(n_seq + 1) * 4, kAlign);
  L.row_seq = off; off += align_up(rows * 4, kAlign);
  L.row_pos = off; off += align_up(rows * 4, kAlign);
  L.emb = off; off += align_up(rows * C * 2, kAlign);
  L.x1 = off; off += align_up(rows * C * 2, kAlign);
  L.x2 = off; off += align_up(rows * C * 2, kAlign);
  L.taps = off; off += align_up(rows, kAlign);  // the convolution taps of each row
  L.xg = off; off += align_up(rows * 8 * H * 4, kAlign);
  // exchange buffers of the four-workgroup recurrence: per launch up to
  // mc_groups groups x 2 directions, each h_t twice (parity) as bf16
  L.mc_groups = std::min((n_seq + kLstmSeq - 1) / kLstmSeq, c->mc_groups);
  L.hx = off; off += align_up((size_t)L.mc_groups * 2 * 2 * kLstmSeq * H * 2, kAlign);
  L.flags = off; off += align_up((size_t)L.mc_groups * 2 * kMcMembers * 4, kAlign);
  L.total = off;
  return L;
}


template <typename Fn>
void ttimed(albert_text_ctx* c, int kind, hipStream_t s, Fn&& fn) {
  const bool on = c->time_kind == kind && 2 * (c->n_timed + 1) <= (int)c->ev.size();
  if (on) g_launch_events = LaunchEvents{c->ev[2 * c->n_timed], c->ev[2 * c->n_timed + 1]};
  fn();  // launches exactly one kernel through launch_kernel(), which takes the events
  if (on) {
    if (g_launch_events.start == nullptr) ++c->n_timed;
    g_launch_events = LaunchEvents{};
  }
}

int text_run(albert_text_ctx* c, const int32_t* ids, const int32_t* lens_or_cu, int n_seq,
             int pad_T, int64_t max_rows, int max_len, float* out, void* ws, hipStream_t s,
             unsigned flags) {
  const albert_text_config& cf = c->cfg;
  const TextLayout L = text_plan(c, n_seq, max_rows);
  char* w = static_cast<char*>(ws);
  int* status = reinterpret_cast<int*>(w + L.status);
  int* cu = reinterpret_cast<int*>(w + L.cu);
  int* row_seq = reinterpret_cast<int*>(w + L.row_seq);
  int* row_pos = reinterpret_cast<int*>(w + L.row_pos);
  // embedding rows, then the blocks alternate x1 <- emb, x2 <- x1, x1 <- x2, ...
  bf16* X[3] = {reinterpret_cast<bf16*>(w + L.emb), reinterpret_cast<bf16*>(w + L.x1),
                reinterpret_cast<bf16*>(w + L.x2)};
  unsigned char* taps = reinterpret_cast<unsigned char*>(w + L.taps);
  float* XG = reinterpret_cast<float*>(w + L.xg);
  const int C = cf.channels, K = cf.kernel, H = cf.hidden;
  const int* m_ptr = cu + n_seq;

  if (pad_T)
    hipLaunchKernelGGL(derive_padded_kernel, dim3(1), dim3(1024), 0, s, lens_or_cu, n_seq, pad_T,
                       cu, status, (int*)nullptr);
  else
    hipLaunchKernelGGL(derive_packed_kernel, dim3(1), dim3(1024), 0, s, lens_or_cu, n_seq,
                       (int)max_rows, max_len, cu, status, (int*)nullptr);
  hipLaunchKernelGGL(rows_ids_kernel, dim3(n_seq), dim3(256), 0, s, ids, cu, pad_T, cf.vocab,
                     row_seq, row_pos, status);
  ttimed(c, ALBERT_TK_EMBED, s, [&] {
    launch_kernel(text_embed_kernel, dim3((unsigned)((max_rows * (C / 8) + 255) / 256)),
                  dim3(256), s, ids, pad_T, row_seq, row_pos, m_ptr, c->emb, C, X[0], status);
  });

  GemmArgs base{};
  base.status = status;
  base.m_ptr = m_ptr;
  ttimed(c, ALBERT_TK_TAPS, s, [&] {
    launch_kernel(conv_taps_kernel, dim3((unsigned)((max_rows + 255) / 256)), dim3(256), s,
                  row_seq, row_pos, cu, m_ptr, K, taps, status);
  });
  int cur = 0;
  for (int i = 0; i < cf.n_conv; ++i) {
    const int nxt = cur == 1 ? 2 : 1;
    GemmArgs g = base;  // convolution as one GEMM over the (virtually) unfolded input
    g.X = X[cur]; g.ldx = C; g.taps = taps; g.W = c->conv_w[i]; g.bias = c->conv_b[i];
    g.ln_g = c->ln_g[i]; g.ln_b = c->ln_b[i]; g.eps = cf.ln_eps; g.slope = cf.slope;
    g.Y = X[nxt]; g.ldy = C; g.N = C; g.K = K * C;
    ttimed(c, ALBERT_TK_CONV, s, [&] {
      gemm_ln_n<bf16, false, 512, EPI_LN_ACT>(g, max_rows, c->grid_cap, s);
    });
    cur = nxt;
  }

  GemmArgs g = base;  // LSTM input projection, both directions, fp32 out
  g.X = X[cur]; g.ldx = C; g.W = c->w_ih; g.bias = c->b_gates; g.out = XG; g.out_T = 0;
  g.N = 8 * H; g.K = C;
  ttimed(c, ALBERT_TK_LSTM_IN, s, [&] {
    gemm_big<bf16, false, EPI_OUT>(g, max_rows, c->grid_cap, s);
  });

  bool launch_failed = false;
  if (L.mc_groups > 0 && !(flags & ALBERT_UNFUSED)) {
    // four cooperating workgroups per direction and group of 32 sequences,
    // at most mc_groups groups per launch (all resident together)
    ttimed(c, ALBERT_TK_LSTM, s, [&] {
      const LaunchEvents ev = g_launch_events;
      g_launch_events = LaunchEvents{};
      if (ev.start) (void)hipEventRecord(ev.start, s);
      for (int seq0 = 0; seq0 < n_seq; seq0 += L.mc_groups * kLstmSeq) {
        const int groups = std::min(L.mc_groups, (n_seq - seq0 + kLstmSeq - 1) / kLstmSeq);
        const int quads = 2 * groups;
        int* fl = reinterpret_cast<int*>(w + L.flags);
        hipLaunchKernelGGL(zero_ints_kernel, dim3((quads * kMcMembers + 255) / 256), dim3(256),
                           0, s, fl, quads * kMcMembers);
        LstmMcArgs ma{XG, c->w_hh_mc, out, pad_T, cu, n_seq, seq0, quads,
                      reinterpret_cast<bf16*>(w + L.hx), fl, status};
        void* args[] = {&ma};
        // quads padded to a multiple of 8, 4 workgroups each (see the kernel)
        const unsigned grid = (unsigned)((quads + 7) / 8 * 32);
        if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(lstm_mc_kernel), dim3(grid),
                                       dim3(512), args, 0, s) != hipSuccess)
          launch_failed = true;
      }
      if (ev.stop) (void)hipEventRecord(ev.stop, s);
      g_launch_events = LaunchEvents{};  // consumed
    });
  } else {
    LstmArgs la{XG, c->w_hh, out, pad_T, cu, n_seq, status};
    ttimed(c, ALBERT_TK_LSTM, s, [&] {
      launch_kernel(lstm_kernel, dim3((unsigned)((n_seq + kLstmSeq - 1) / kLstmSeq), 2),
                    dim3(512), s, la);
    });
  }
  if (pad_T)
    hipLaunchKernelGGL(zero_pad_rows_kernel, dim3(n_seq), dim3(256), 0, s, out, cu, pad_T, 2 * H,
                       status);
  return hipGetLastError() == hipSuccess && !launch_failed ? ALBERT_OK : ALBERT_E_HIP;
}

int text_finish(int rc, const void* ws, hipStream_t s, unsigned flags) {
  if (rc != ALBERT_OK || (flags & ALBERT_ASYNC)) return rc;
  return albert_read_status(ws, s);
}

bool text_device_ok(const albert_text_ctx* c) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == c->device;
}

void text_drop_events(albert_text_ctx* ctx) {
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  ctx->ev.clear();
  ctx->time_kind = -1;
  ctx->n_timed = 0;
}

}  // namespace

extern "C" {

int albert_text_default_config(albert_text_config* cfg) {
  if (!cfg) return ALBERT_E_ARG;
  *cfg = albert_text_config{178, 512, 5, 3, kLstmH, 1e-5f, 0.2f};
  return ALBERT_OK;
}

int albert_text_n_tensors(const albert_text_config* cfg) {
  if (!cfg || !text_config_ok(*cfg)) return -1;
  return 1 + 5 * cfg->n_conv + 8;
}

const char* albert_text_tensor_name(const albert_text_config* cfg, int index) {
  if (!cfg || !text_config_ok(*cfg)) return nullptr;
  const int slot = name_slot(*cfg, index);
  return slot < 0 ? nullptr : all_names()[slot].c_str();
}

int albert_text_tensor_shape(const albert_text_config* cfg, int index, int64_t* rows,
                             int64_t* cols) {
  if (!cfg || !rows || !cols || !text_config_ok(*cfg)) return ALBERT_E_ARG;
  return text_shape(*cfg, index, rows, cols) ? ALBERT_OK : ALBERT_E_ARG;
}

int albert_text_load_weights(albert_text_ctx** out_ctx, const albert_text_config* cfg,
                             const float* const* host, void* stream) {
  if (!out_ctx) return ALBERT_E_ARG;
  *out_ctx = nullptr;
  if (!cfg || !host || !text_config_ok(*cfg)) return ALBERT_E_ARG;
  const albert_text_config c = *cfg;
  const int NT = 1 + 5 * c.n_conv + 8;
  for (int i = 0; i < NT; ++i) {
    if (!host[i]) return ALBERT_E_ARG;
    int64_t r = 0, k = 0;
    text_shape(c, i, &r, &k);
    for (int64_t e = 0; e < r * k; ++e)
      if (!std::isfinite(host[i][e])) return ALBERT_E_ARG;
  }
  const int64_t C = c.channels, K = c.kernel, H = c.hidden;

  struct Seg { size_t off, bytes; };
  std::vector<Seg> seg;
  size_t off = 0;
  auto add = [&](size_t bytes) { seg.push_back({off, bytes}); off += align_up(bytes, kAlign); };
  add((size_t)c.vocab * C * 2);                 // 0 emb
  for (int i = 0; i < c.n_conv; ++i) {
    add((size_t)C * K * C * 2);                 // conv w (GEMM layout)
    add((size_t)C * 4);                         // conv b
    add((size_t)C * 4);                         // ln g
    add((size_t)C * 4);                         // ln b
  }
  const int s_wih = (int)seg.size();
  add((size_t)8 * H * C * 2);                   // w_ih, both directions
  add((size_t)8 * H * 4);                       // b_ih + b_hh
  add((size_t)2 * 4 * H * H * 2);               // w_hh, both directions
  add((size_t)2 * 4 * H * H * 2);               // w_hh again, four-workgroup order
  std::vector<unsigned char> img(off, 0);
  auto bf = [&](int s) { return reinterpret_cast<uint16_t*>(img.data() + seg[s].off); };
  auto fp = [&](int s) { return reinterpret_cast<float*>(img.data() + seg[s].off); };

  for (int64_t e = 0; e < (int64_t)c.vocab * C; ++e) bf(0)[e] = bf16_bits(host[0][e]);
  for (int i = 0; i < c.n_conv; ++i) {
    const float* v = host[1 + 5 * i];
    const float* gn = host[2 + 5 * i];
    uint16_t* wd = bf(1 + 4 * i);
    for (int64_t o = 0; o < C; ++o) {
      double nrm = 0.0;
      for (int64_t e = 0; e < C * K; ++e) nrm += (double)v[o * C * K + e] * v[o * C * K + e];
      if (!(nrm > 0.0)) return ALBERT_E_ARG;
      const double sc = (double)gn[o] / std::sqrt(nrm);
      for (int64_t ci = 0; ci < C; ++ci)
        for (int64_t j = 0; j < K; ++j)  // input [o][ci][j] -> GEMM column j*C + ci
          wd[o * K * C + j * C + ci] = bf16_bits((double)(float)(sc * v[(o * C + ci) * K + j]));
    }
    std::memcpy(fp(2 + 4 * i), host[3 + 5 * i], (size_t)C * 4);
    std::memcpy(fp(3 + 4 * i), host[4 + 5 * i], (size_t)C * 4);
    std::memcpy(fp(4 + 4 * i), host[5 + 5 * i], (size_t)C * 4);
  }
  const int l0 = 1 + 5 * c.n_conv;  // lstm.fwd.w_ih
  for (int d = 0; d < 2; ++d) {
    const float* wih = host[l0 + 4 * d];
    const float* whh = host[l0 + 4 * d + 1];
    const float* bih = host[l0 + 4 * d + 2];
    const float* bhh = host[l0 + 4 * d + 3];
    for (int64_t e = 0; e < 4 * H * C; ++e) bf(s_wih)[d * 4 * H * C + e] = bf16_bits(wih[e]);
    for (int64_t e = 0; e < 4 * H; ++e)
      fp(s_wih + 1)[d * 4 * H + e] = (float)((double)bih[e] + bhh[e]);
    // fragment order [d][wave 8][k-step H/16][gate 4][lane 64][8]: lane
    // (l32, hh) of wave w holds row g*H + 32w + l32, columns kk*16 + hh*8 ..
    uint16_t* wd = bf(s_wih + 2) + d * 4 * H * H;
    for (int64_t wv = 0; wv < 8; ++wv)
      for (int64_t kk = 0; kk < H / 16; ++kk)
        for (int64_t g = 0; g < 4; ++g)
          for (int64_t ln = 0; ln < 64; ++ln)
            for (int64_t e = 0; e < 8; ++e) {
              const int64_t r = g * H + 32 * wv + (ln & 31);
              const int64_t k = kk * 16 + (ln >> 5) * 8 + e;
              wd[(((wv * (H / 16) + kk) * 4 + g) * 64 + ln) * 8 + e] = bf16_bits(whh[r * H + k]);
            }
    // four-workgroup order [d][member 4][wave 8][k-step H/16][lane 64][8]:
    // row l32 of wave w's tile in member m is gate l32 % 4 of unit
    // 64m + 8w + u/2 + 4(u%2), u = l32 / 4, so that MFMA lane (l32, hh)
    // ends up with the four gates of units 64m + 8w + 4hh .. +3
    uint16_t* wm = bf(s_wih + 3) + d * 4 * H * H;
    for (int64_t mb = 0; mb < kMcMembers; ++mb)
      for (int64_t wv = 0; wv < 8; ++wv)
        for (int64_t kk = 0; kk < H / 16; ++kk)
          for (int64_t ln = 0; ln < 64; ++ln)
            for (int64_t e = 0; e < 8; ++e) {
              const int64_t tr = ln & 31, u = tr / 4, g = tr % 4;
              const int64_t unit = 64 * mb + 8 * wv + u / 2 + 4 * (u % 2);
              const int64_t k = kk * 16 + (ln >> 5) * 8 + e;
              wm[((((mb * 8 + wv) * (H / 16) + kk) * 64) + ln) * 8 + e] =
                  bf16_bits(whh[(g * H + unit) * H + k]);
            }
  }

  albert_text_ctx* ctx = new (std::nothrow) albert_text_ctx();
  if (!ctx) return ALBERT_E_ARG;
  ctx->cfg = c;
  int n_cu = 0;
  if (hipGetDevice(&ctx->device) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, ctx->device) !=
          hipSuccess ||
      hipMalloc(&ctx->mem, off) != hipSuccess) {
    delete ctx;
    return ALBERT_E_HIP;
  }
  ctx->grid_cap = std::max(8, n_cu / 8 * 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(ctx->mem, img.data(), off, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipFree(ctx->mem);
    delete ctx;
    return ALBERT_E_HIP;
  }
  char* m = static_cast<char*>(ctx->mem);
  ctx->emb = reinterpret_cast<const bf16*>(m + seg[0].off);
  for (int i = 0; i < c.n_conv; ++i) {
    ctx->conv_w.push_back(reinterpret_cast<const bf16*>(m + seg[1 + 4 * i].off));
    ctx->conv_b.push_back(reinterpret_cast<const float*>(m + seg[2 + 4 * i].off));
    ctx->ln_g.push_back(reinterpret_cast<const float*>(m + seg[3 + 4 * i].off));
    ctx->ln_b.push_back(reinterpret_cast<const float*>(m + seg[4 + 4 * i].off));
  }
  ctx->w_ih = reinterpret_cast<const bf16*>(m + seg[s_wih].off);
  ctx->b_gates = reinterpret_cast<const float*>(m + seg[s_wih + 1].off);
  ctx->w_hh = reinterpret_cast<const bf16*>(m + seg[s_wih + 2].off);
  ctx->w_hh_mc = reinterpret_cast<const bf16*>(m + seg[s_wih + 3].off);
  // the four-workgroup recurrence needs a cooperative launch: all of its
  // workgroups resident at once; groups per launch in multiples of 4 (a
  // launch is a multiple of 32 workgroups)
  int coop = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, ctx->device) ==
          hipSuccess &&
      coop &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lstm_mc_kernel, 512, 0) ==
          hipSuccess &&
      per_cu >= 1)
    ctx->mc_groups = std::min(64, (per_cu * n_cu) / 32 * 4);
  *out_ctx = ctx;
  return ALBERT_OK;
}

size_t albert_text_workspace_bytes(const albert_text_ctx* ctx, int n_seq, int64_t max_rows) {
  if (!ctx || n_seq < 1 || max_rows < 1) return 0;
  return text_plan(ctx, n_seq, max_rows).total;
}

int albert_text_encode(albert_text_ctx* ctx, const int32_t* ids, const int32_t* lengths, int B,
                       int T, float* out, void* ws, size_t ws_bytes, void* stream,
                       unsigned flags) {
  if (ctx && B == 0) return ALBERT_OK;
  if (!ctx || !ids || !lengths || !out || !ws || B < 1 || T < 1 ||
      ((uintptr_t)ws % kAlign) != 0 || (int64_t)B * T > INT32_MAX || !text_device_ok(ctx))
    return ALBERT_E_ARG;
  const int64_t rows = (int64_t)B * T;
  const size_t need = text_plan(ctx, B, rows).total;
  if (ws_bytes < need) return ALBERT_E_WORKSPACE;
  const size_t out_bytes = (size_t)rows * 2 * ctx->cfg.hidden * 4;
  if (overlaps(out, out_bytes, ids, (size_t)rows * 4) ||
      overlaps(out, out_bytes, lengths, (size_t)B * 4) || overlaps(out, out_bytes, ws, need))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return text_finish(text_run(ctx, ids, lengths, B, T, rows, T, out, ws, s, flags), ws, s, flags);
}

int albert_text_encode_varlen(albert_text_ctx* ctx, const int32_t* ids, const int32_t* cu_seqlens,
                              int n, int total, int max_len, float* out, void* ws,
                              size_t ws_bytes, void* stream, unsigned flags) {
  if (ctx && n == 0 && total == 0) return ALBERT_OK;
  if (!ctx || !ids || !cu_seqlens || !out || !ws || n < 1 || total < 1 || max_len < 1 ||
      ((uintptr_t)ws % kAlign) != 0 || !text_device_ok(ctx))
    return ALBERT_E_ARG;
  const size_t need = text_plan(ctx, n, total).total;
  if (ws_bytes < need) return ALBERT_E_WORKSPACE;
  const size_t out_bytes = (size_t)total * 2 * ctx->cfg.hidden * 4;
  if (overlaps(out, out_bytes, ids, (size_t)total * 4) ||
      overlaps(out, out_bytes, cu_seqlens, (size_t)(n + 1) * 4) ||
      overlaps(out, out_bytes, ws, need))
    return ALBERT_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return text_finish(text_run(ctx, ids, cu_seqlens, n, 0, total, max_len, out, ws, s, flags), ws,
                     s, flags);
}

int albert_text_tap(const albert_text_ctx* ctx, int n_seq, int64_t max_rows, int tap,
                    size_t* offset, size_t* bytes, int64_t* row_stride) {
  if (!ctx || !offset || !bytes || !row_stride || n_seq < 1 || max_rows < 1) return ALBERT_E_ARG;
  const TextLayout L = text_plan(ctx, n_seq, max_rows);
  const size_t R = (size_t)max_rows, C = (size_t)ctx->cfg.channels, H = (size_t)ctx->cfg.hidden;
  switch (tap) {
    case ALBERT_TT_STATUS: *offset = L.status; *bytes = 4; *row_stride = 0; break;
    case ALBERT_TT_CU: *offset = L.cu; *bytes = (size_t)(n_seq + 1) * 4; *row_stride = 0; break;
    case ALBERT_TT_EMB: *offset = L.emb; *bytes = R * C * 2; *row_stride = (int64_t)C; break;
    case ALBERT_TT_CONV:  // blocks alternate x1, x2, x1, ...
      *offset = ctx->cfg.n_conv % 2 ? L.x1 : L.x2; *bytes = R * C * 2; *row_stride = (int64_t)C;
      break;
    case ALBERT_TT_XG:
      *offset = L.xg; *bytes = R * 8 * H * 4; *row_stride = (int64_t)(8 * H);
      break;
    default: return ALBERT_E_ARG;
  }
  return ALBERT_OK;
}

int albert_text_time_kernel(albert_text_ctx* ctx, int kind, int max_launches) {
  if (!ctx || kind < -1 || kind >= ALBERT_TK_COUNT || (kind >= 0 && max_launches < 1))
    return ALBERT_E_ARG;
  text_drop_events(ctx);
  if (kind < 0) return ALBERT_OK;
  ctx->ev.resize((size_t)2 * max_launches);
  for (auto& e : ctx->ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      text_drop_events(ctx);
      return ALBERT_E_HIP;
    }
  }
  ctx->time_kind = kind;
  return ALBERT_OK;
}

int albert_text_kernel_time(albert_text_ctx* ctx, int* launches, double* total_ms) {
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

void albert_text_free(albert_text_ctx* ctx) {
  if (!ctx) return;
  text_drop_events(ctx);
  (void)hipFree(ctx->mem);
  delete ctx;
}

}  // extern "C"
