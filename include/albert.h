/*
 * albert.h -- C ABI of the MI355X (gfx950) Kokoro ALBERT phoneme encoder.
 *
 * The encoder is the front end of Kokoro TTS, as described on the page
 * "ALBERT: How Kokoro's Phoneme Encoder Works, and Where CKE Has Reached It"
 * (sections "What ALBERT Changed: Two Kinds of Sharing" and "Inside One Real
 * ALBERT Layer"):
 *   phoneme IDs -> word + position + type tables (width 128), summed and
 *   LayerNormed -> 128->768 projection -> n_iter executions of ONE shared
 *   post-LayerNorm transformer layer (12 heads of 64, bidirectional masked
 *   attention, 768->2048->768 tanh-GELU FFN) -> 768->512 projection.
 * ALBERT's intermediate grouping (several layer weight sets, each reused
 * over a block of executions) is the n_groups option of albert_config.
 *
 * Every call takes plain pointers and sizes.  Unless stated otherwise:
 *   - "dev" pointers are device memory on the current HIP device,
 *   - hip_stream is a hipStream_t (NULL = the null stream); all device work
 *     of a call is enqueued on it, in stream order,
 *   - the return value is an albert_status (0 = ALBERT_OK).
 * The library never allocates device memory per request: the caller owns the
 * inputs, the output and a workspace of albert_workspace_bytes() bytes.
 */
#ifndef ALBERT_H
#define ALBERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  A request that fails validation writes nothing to `out`
 * (the checked, validate-before-write contract of the page "ALBERT: How
 * Kokoro's Phoneme Encoder Works", section "How CKE Represents It"), and the
 * context stays usable for the next request. */
enum albert_status {
  ALBERT_OK = 0,
  ALBERT_E_ARG = 1,       /* null pointer, bad size, bad dtype or config     */
  ALBERT_E_WORKSPACE = 2, /* ws_bytes smaller than albert_workspace_bytes()  */
  ALBERT_E_LENGTH = 3,    /* a length outside [1, T] / bad cu_seqlens        */
  ALBERT_E_ID = 4,        /* an ID at a valid slot outside [0, vocab-1]      */
  ALBERT_E_ALIAS = 5,     /* `out` overlaps an input or the workspace        */
  ALBERT_E_HIP = 6,       /* a HIP runtime call failed                       */
  ALBERT_E_SYNC = 7,      /* cooperating workgroups did not meet: the two
                             halves of a LayerNorm row tile (bf16, FP8) or
                             the text path's multi-workgroup LSTM
                             recurrence; a workgroup waited too long for a
                             partner that was not resident                 */
  ALBERT_E_SCRATCH = 8    /* albert_encode_noalloc: the request needs more
                             workspace than ALBERT_SCRATCH_BYTES           */
};

/* Compute/storage type of tables, weight matrices and activations.
 * Accumulation, biases, LayerNorm, softmax and GELU are always fp32.
 * ALBERT_FP8 is the low-precision variant: every matrix-product input is an
 * OCP FP8 E4M3 code (weights per output row times a power-of-two scale, so
 * the largest magnitude of each row is at most 448; activations rounded to
 * nearest even and saturated at +-448) while the residual stream, Q|K|V and
 * the tables stay bf16 and attention runs on bf16 matrix cores.  Its
 * fidelity is scored as on the page "Kokoro-82M-encoder-hailo10h" ("Eval
 * results"): N(0,1) inputs at the embedding LayerNorm output, cosine of the
 * [128,512] outputs against full precision. */
enum albert_dtype { ALBERT_F32 = 0, ALBERT_BF16 = 1, ALBERT_FP8 = 2 };

/* flags for albert_encode / albert_encode_varlen */
#define ALBERT_ASYNC 1u /* return after enqueueing; read the status later
                           with albert_read_status()                        */
#define ALBERT_UNFUSED 2u /* bf16 and FP8: run Q|K|V and attention as
                             separate kernels (otherwise fused when every
                             sequence has at most 256 tokens), so that the
                             QKV tap holds its checkpoint.  Text path: run the LSTM
                             recurrence as one workgroup per direction and
                             32 sequences instead of four cooperating ones */
#define ALBERT_LN_HANDOFF 4u /* testing aid, bf16 and FP8: the two workgroups that
                             share each LayerNorm row tile do not wait for
                             each other's row statistics, so the fallback in
                             which one hands its rows to the other runs
                             (results equal to the default within bf16
                             rounding) */

typedef struct albert_config {
  int32_t vocab;    /* word-table rows (Kokoro: 178)                       */
  int32_t max_pos;  /* position-table rows, also the longest sequence (512)*/
  int32_t n_types;  /* type-table rows (2); type id is always 0            */
  int32_t emb;      /* embedding width E (must be 128)                     */
  int32_t hidden;   /* hidden width H (must be 768)                        */
  int32_t heads;    /* attention heads (must be 12)                        */
  int32_t head_dim; /* per-head width (must be 64)                         */
  int32_t ffn;      /* FFN width (Kokoro: 2048; multiple of 256)           */
  int32_t n_iter;   /* executions of the shared layer (Kokoro: 12; >= 0)   */
  int32_t n_groups; /* distinct layer weight sets G (Kokoro: 1, i.e. full
                       sharing); 1 <= G <= max(n_iter, 1).  Execution i
                       (from 0) uses set floor(i * G / n_iter): contiguous,
                       near-equal blocks of executions per set ("What ALBERT
                       Changed", part 2: intermediate grouping)             */
  int32_t out_dim;  /* output width (Kokoro: 512; multiple of 256)         */
  float ln_eps;     /* LayerNorm epsilon (Kokoro: 1e-12)                   */
} albert_config;

/* Weight tensors and their canonical order (index: name [shape]) for one
 * layer weight set (n_groups = 1).  Linear weights are [out, in] row-major,
 * y_j = b_j + sum_i x_i W[j][i] (contract A of "Qwen3-TTS and Kokoro: Two
 * Routes from Text to Speech").
 *   0 emb.word [vocab,E]    1 emb.pos [max_pos,E]   2 emb.type [n_types,E]
 *   3 emb.ln.g [E]          4 emb.ln.b [E]
 *   5 proj.w [H,E]          6 proj.b [H]
 *   7 q.w [H,H]  8 q.b [H]  9 k.w [H,H] 10 k.b [H] 11 v.w [H,H] 12 v.b [H]
 *  13 o.w [H,H] 14 o.b [H] 15 attn_ln.g [H] 16 attn_ln.b [H]
 *  17 ffn1.w [F,H] 18 ffn1.b [F] 19 ffn2.w [H,F] 20 ffn2.b [H]
 *  21 ffn_ln.g [H] 22 ffn_ln.b [H]
 *  23 out.w [O,H] 24 out.b [O]                                            */
#define ALBERT_N_TENSORS 25
/* With G = n_groups sets, indices 7..22 repeat once per set: tensor 7+16g+j
 * is tensor 7+j of set g (0 <= j < 16), and out.w, out.b move to 7+16G and
 * 8+16G, for albert_n_tensors(cfg) = 9 + 16G tensors in all. */
#define ALBERT_LAYER_TENSORS 16

typedef struct albert_ctx albert_ctx; /* opaque; owns the device weights */

/* Fill *cfg with the Kokoro configuration. */
int albert_default_config(albert_config* cfg);

/* Number of weight tensors under cfg (9 + 16 * n_groups), or -1 for a bad
 * config. */
int albert_n_tensors(const albert_config* cfg);

/* Canonical name of tensor `index` under cfg, NULL for a bad index or
 * config.  A layer tensor's name is its role ("q.w", ...); its weight set
 * is (index - 7) / 16. */
const char* albert_tensor_name(const albert_config* cfg, int index);

/* Shape of tensor `index` under cfg: writes rows/cols (cols = 1 for
 * vectors).  Returns ALBERT_E_ARG for a bad index or config. */
int albert_tensor_shape(const albert_config* cfg, int index, int64_t* rows, int64_t* cols);

/* Create a context holding ONE copy of the encoder weights on the current
 * device -- one layer weight set serves all n_iter executions of the shared
 * layer (page "ALBERT: How Kokoro's Phoneme Encoder Works", "Cross-layer
 * parameter sharing", and the canonical-name weight binding of "How CKE
 * Represents It"); with n_groups = G each of the G sets serves its block of
 * executions.
 *
 * host_tensors: albert_n_tensors(cfg) host pointers to fp32 arrays in
 *   canonical order and shape.  They are read during the call and may be
 *   freed after.
 * dtype: ALBERT_BF16 stores tables and weight matrices as bfloat16 (round to
 *   nearest even); ALBERT_F32 stores them as given; ALBERT_FP8 stores the
 *   tables as bfloat16 and each weight matrix row j as E4M3 codes of
 *   W[j,:] * 2^k_j (k_j the largest integer with max_i |W[j,i]| * 2^k_j
 *   <= 448, 0 for a zero row) plus the exponent.  Biases and LayerNorm
 *   vectors are fp32 in all three.  The query weights and bias are stored scaled
 *   by 1/sqrt(head_dim) = 1/8, a power of two, so the attention scores need
 *   no further scaling and the stored values are exact.
 * This is the only call that allocates device memory (and it synchronises
 * hip_stream before returning).  On failure *ctx is NULL. */
int albert_load_weights(albert_ctx** ctx, const albert_config* cfg,
                        const float* const* host_tensors, int dtype, void* hip_stream);

/* Bytes of workspace for a request of n_seq sequences and max_rows token
 * rows: padded calls use (B, B*T); packed calls use (n, total).
 * Returns 0 for invalid arguments.  Size is linear in max_rows.
 * The workspace is the caller-owned arena of the page "ALBERT: How Kokoro's
 * Phoneme Encoder Works", section "How CKE Represents It": every
 * intermediate buffer of a request sits at an offset planned here from the
 * request's sizes, and nothing is allocated while encoding. */
size_t albert_workspace_bytes(const albert_ctx* ctx, int n_seq, int64_t max_rows);

/* Padded batch.
 * ids     dev int32 [B, T], row-major; slots t >= lengths[b] are padding
 *         and are never read.
 * lengths dev int32 [B]; each in [1, T].
 * B >= 1, 1 <= T <= max_pos.  B == 0 is an empty request: ALBERT_OK, nothing
 * is read, written or enqueued.
 * out     dev fp32 [B, T, out_dim]; rows t >= lengths[b] are written as 0.
 * ws      dev workspace of ws_bytes >= albert_workspace_bytes(ctx, B, B*T),
 *         256-byte aligned; its contents on entry are ignored.
 * Attention of sequence b reads keys 0..lengths[b]-1 only (the pad mask of
 * "How Kokoro TTS Works and Where CKE Stands", "What ALBERT does here");
 * positions are 0..lengths[b]-1 and the token type is 0.
 * IDs and lengths are validated on the device before anything is written to
 * `out`; on ALBERT_E_LENGTH / ALBERT_E_ID `out` is left byte-for-byte
 * unchanged.  Argument errors (E_ARG, E_WORKSPACE, E_ALIAS) are detected on
 * the host before any work is enqueued.  Without ALBERT_ASYNC the call waits
 * for the stream and returns the device status; with it, the call returns
 * ALBERT_OK after enqueueing and the device status is read with
 * albert_read_status(ws, stream).  Calls that share a workspace must be
 * ordered on one stream; calls with distinct workspaces (and outputs) may
 * run concurrently on different streams, since the context is only read
 * while encoding (kernel timing aside). */
int albert_encode(albert_ctx* ctx, const int32_t* ids, const int32_t* lengths,
                  int B, int T, float* out, void* ws, size_t ws_bytes,
                  void* hip_stream, unsigned flags);

/* Bytes of the static device scratch behind albert_encode_noalloc (64 MiB
 * on every GPU the library runs on, held until the process ends). */
#define ALBERT_SCRATCH_BYTES (64u << 20)

/* albert_encode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is the library's own static device scratch instead of a
 * caller buffer; the call allocates nothing, frees nothing and never waits
 * for the stream (ALBERT_ASYNC is implied; ALBERT_UNFUSED and
 * ALBERT_LN_HANDOFF work as for albert_encode).
 * ids, lengths, B, T, out, hip_stream: as albert_encode (same kernels, same
 * results bit for bit).
 * status     dev int32 [1] (caller-owned output): after the request's
 *            kernels, the device status (ALBERT_OK, ALBERT_E_LENGTH or
 *            ALBERT_E_ID; on an error `out` is unchanged).
 * Host-side errors as albert_encode, plus ALBERT_E_SCRATCH (nothing
 * enqueued) when albert_workspace_bytes(ctx, B, B*T) > ALBERT_SCRATCH_BYTES:
 * about 3,800 token rows B*T in bf16 (4,300 with FP8 operands, 2,300 in
 * fp32), e.g. one utterance of up to 512 tokens or 30 of 128.
 * Every call on one GPU uses that GPU's one scratch, which keeps the last
 * call's contents (each request sets up what it needs): calls that overlap
 * on one GPU race, so order them on one stream. */
int albert_encode_noalloc(albert_ctx* ctx, const int32_t* ids, const int32_t* lengths,
                          int B, int T, float* out, int32_t* status, void* hip_stream,
                          unsigned flags);

/* Packed (varlen) batch of n sequences with no padding.
 * This entry point is the library's own (the pages compile one static
 * length with padding); it serves packed workloads such as 1,024
 * utterances of geometric lengths, and drops pad rows outright where the
 * "Kokoro-82M-LiteRT" card trims pad outputs after the fact.  The
 * arithmetic per sequence is that of albert_encode.
 * ids        dev int32 [total]; sequence s occupies rows cu[s] .. cu[s+1]-1.
 * cu_seqlens dev int32 [n + 1]; cu[0] = 0, cu[n] = total, and every length
 *            cu[s+1]-cu[s] in [1, max_len]; positions restart at 0 per
 *            sequence.
 * max_len    host-side bound on every length, 1 <= max_len <= max_pos.
 * out        dev fp32 [total, out_dim].
 * ws         workspace of albert_workspace_bytes(ctx, n, total) bytes.
 * n == 0 with total == 0 is an empty request (ALBERT_OK, nothing enqueued).
 * Validation, errors and flags as albert_encode. */
int albert_encode_varlen(albert_ctx* ctx, const int32_t* ids, const int32_t* cu_seqlens,
                         int n, int total, int max_len, float* out, void* ws,
                         size_t ws_bytes, void* hip_stream, unsigned flags);

/* Packed batch that starts from the embedding LayerNorm output instead of
 * phoneme IDs: the encoder block without its embedding, as deployed when the
 * embedding runs elsewhere ("Kokoro-82M-encoder-hailo10h", "What this is
 * not"; the low-precision fidelity method of its "Eval results" feeds this
 * point).
 * x          dev fp32 [total, emb], row-major; rows packed as cu_seqlens
 *            says.  Values are used as given (non-finite values propagate).
 * Other arguments, validation (lengths only: there are no IDs), errors,
 * workspace and flags as albert_encode_varlen. */
int albert_encode_features(albert_ctx* ctx, const float* x, const int32_t* cu_seqlens, int n,
                           int total, int max_len, float* out, void* ws, size_t ws_bytes,
                           void* hip_stream, unsigned flags);

/* Wait for hip_stream and return the device status word that the last
 * request enqueued with this workspace left there (ALBERT_E_HIP if the read
 * fails).  This is the integer status of the "checked" kernel contracts
 * (validate before write) of the page "ALBERT: How Kokoro's Phoneme Encoder
 * Works", section "How CKE Represents It", read back for requests enqueued
 * with ALBERT_ASYNC. */
int albert_read_status(const void* ws, void* hip_stream);

/* Debug taps: where a request's intermediate tensors sit in the workspace
 * after it completes (checkpoints at fixed boundaries of the graph, in graph
 * order: the connected X-Ray checkpoints of the page "ALBERT: How Kokoro's
 * Phoneme Encoder Works", section "Evidence and the Open Edges", which
 * compare a running chain at declared boundaries).  Rows are packed tokens (sequence s at rows cu[s]..cu[s+1]-1);
 * elements are the context's dtype (fp32 or bf16) unless noted.  Under
 * ALBERT_FP8, EMB, CTX and G hold E4M3 codes (one byte each), X, QKV and X1
 * are bf16, and taps 10 and 11 are the E4M3 copies of X and X1 that feed
 * the next products (ALBERT_E_ARG for other dtypes).
 *   0 STATUS  int32 [1]          1 CU     int32 [n_seq + 1]
 *   2 ROW_SEQ int32 [rows]       3 ROW_POS int32 [rows]
 *   4 EMB  [rows, E]   embedding sum after LayerNorm
 *   5 X    [rows, H]   input projection (n_iter = 0) or last layer output
 *   6 QKV  [rows, 3H]  last execution's q/8 | k | v, head h at h*64 (written
 *                      only by the separate kernels: ALBERT_UNFUSED, fp32,
 *                      or a sequence over 256 tokens)
 *   7 CTX  [rows, H]   last execution's attention context (token-major)
 *   8 X1   [rows, H]   last execution's post-attention LayerNorm output
 *   9 G    [rows, F]   last execution's GELU output
 *  10 X8   [rows, H]   E4M3 copy of X (ALBERT_FP8 only)
 *  11 X1_8 [rows, H]   E4M3 copy of X1 (ALBERT_FP8 only)
 * Writes the byte offset from ws, the byte size, and the row stride in
 * elements (0 for the int32 taps).  Host-only; enqueues nothing. */
enum albert_tap {
  ALBERT_TAP_STATUS = 0, ALBERT_TAP_CU = 1, ALBERT_TAP_ROW_SEQ = 2,
  ALBERT_TAP_ROW_POS = 3, ALBERT_TAP_EMB = 4, ALBERT_TAP_X = 5,
  ALBERT_TAP_QKV = 6, ALBERT_TAP_CTX = 7, ALBERT_TAP_X1 = 8, ALBERT_TAP_G = 9,
  ALBERT_TAP_X8 = 10, ALBERT_TAP_X1_8 = 11
};
int albert_tap(const albert_ctx* ctx, int n_seq, int64_t max_rows, int tap,
               size_t* offset, size_t* bytes, int64_t* row_stride);

/* Kernel kinds of the launch sequence, for albert_time_kernel(). */
enum albert_kernel_kind {
  ALBERT_K_EMBED = 0,       /* embedding sum + LayerNorm (or features in)   */
  ALBERT_K_PROJ = 1,        /* 128 -> 768 input projection                  */
  ALBERT_K_QKV = 2,         /* fused Q|K|V projection, once per execution   */
  ALBERT_K_ATTN = 3,        /* masked-softmax attention, once per execution */
  ALBERT_K_ATTN_OUT_LN = 4, /* output projection + residual + LayerNorm     */
  ALBERT_K_FFN1_GELU = 5,   /* 768 -> 2048 + GELU                           */
  ALBERT_K_FFN2_LN = 6,     /* 2048 -> 768 + residual + LayerNorm           */
  ALBERT_K_OUT = 7,         /* 768 -> 512 output projection                 */
  ALBERT_K_QKV_ATTN = 8,    /* fused Q|K|V projection + attention (bf16)    */
  ALBERT_K_COUNT = 9
};

/* Measurement hook for benchmarks and profilers.  After this call every
 * launch of kernel `kind` in later requests on `ctx` (up to max_launches of
 * them) is bracketed by two HIP events recorded on the request's stream;
 * kind = -1 switches timing off.  Creates 2*max_launches events (host
 * call, no device allocation per request).  Not thread-safe: one host thread
 * per context while timing. */
int albert_time_kernel(albert_ctx* ctx, int kind, int max_launches);

/* Wait for the recorded events and report how many launches were timed
 * since albert_time_kernel() and their summed duration in milliseconds. */
int albert_kernel_time(albert_ctx* ctx, int* launches, double* total_ms);

/* ---- Length regulation (the step after the encoder) -----------------------
 * Kokoro expands token-level features to audio-aligned frames by integer
 * durations ("How Kokoro TTS Works and Where CKE Stands", section "The time
 * axis is where a circuit becomes difficult"; the [p1,p2,p3], d=[2,1,3] ->
 * [p1,p1,p2,p3,p3,p3] example of "Qwen3-TTS and Kokoro: Two Routes from Text
 * to Speech", section "Path one").  These calls need no context. */

/* Durations from duration logits: dur[t] = max(1, rint(sum_k sigmoid(
 * logits[t,k]) / speed)), fp32 arithmetic, rounding half to even.
 * logits dev fp32 [total, K]; dur dev int32 [total] (written).
 * total >= 1, K >= 1, speed finite and > 0.  Returns after enqueueing. */
int albert_durations(const float* logits, int total, int K, float speed, int32_t* dur,
                     void* hip_stream);

/* Workspace bytes for albert_expand over `total` tokens (0 if total < 1). */
size_t albert_expand_workspace_bytes(int total);

/* Expand packed token features to frames.
 * feat      dev fp32 [total, C], C a multiple of 4.
 * dur       dev int32 [total], every value >= 1.
 * cu_tok    dev int32 [n + 1] token offsets of the n sequences (cu[0] = 0,
 *           cu[n] = total, every sequence non-empty).
 * out       dev fp32 [max_frames, C]: row cu_frames[s] + r holds the feature
 *           row of the token whose frames cover it, tokens in order; rows
 *           past the frame count A = sum dur are not written.
 * cu_frames dev int32 [n + 1] (written): first frame of each sequence, with
 *           cu_frames[n] = A.
 * ws        workspace of albert_expand_workspace_bytes(total) bytes,
 *           256-byte aligned.
 * Durations < 1, bad offsets or A > max_frames give ALBERT_E_LENGTH with
 * `out` and `cu_frames` unchanged.  Flags and status as albert_encode. */
int albert_expand(const float* feat, const int32_t* dur, const int32_t* cu_tok, int n,
                  int total, int C, float* out, int64_t max_frames, int32_t* cu_frames,
                  void* ws, size_t ws_bytes, void* hip_stream, unsigned flags);

/* ---- Kokoro's parallel text encoder ----------------------------------------
 * The second path on the same phoneme IDs ("How Kokoro TTS Works and Where
 * CKE Stands", the component list: embedding -> three weight-normalized
 * convolutions -> bidirectional LSTM, beside the ALBERT; "How I want CKE to
 * stitch it": its own [512, T] features).  Sizes and blocks the pages leave
 * open follow the StyleTTS 2 text encoder Kokoro inherits: 512 channels,
 * convolutions of width 5 zero-padded at each sequence's ends, each followed
 * by a LayerNorm over the channels and a LeakyReLU; an LSTM of 256 units
 * per direction (gates i, f, g, o; zero initial state) whose backward scan
 * starts at each sequence's own last token (the masking the
 * "Kokoro-82M-LiteRT" card calls for).  Storage is bf16 with fp32
 * accumulation, gate arithmetic and cell state; output fp32, token-major
 * [.., 512] (forward half, then backward half). */
typedef struct albert_text_config {
  int32_t vocab;    /* embedding rows (Kokoro: 178)                         */
  int32_t channels; /* width C of the embedding and convolutions (512)      */
  int32_t kernel;   /* convolution width: odd, 1..7 (5)                     */
  int32_t n_conv;   /* convolution blocks: 1..8 (3)                         */
  int32_t hidden;   /* LSTM units per direction (must be 256)              */
  float ln_eps;     /* LayerNorm epsilon (1e-5)                             */
  float slope;      /* LeakyReLU negative slope (0.2)                       */
} albert_text_config;

typedef struct albert_text_ctx albert_text_ctx; /* opaque; owns device weights */

/* Fill *cfg with the configuration above. */
int albert_text_default_config(albert_text_config* cfg);

/* Weight tensors in canonical order:
 *   emb [vocab, C];
 *   per block i: conv<i>.v [C, C*K] (row-major [C_out][C_in][K], the
 *     direction of the weight-normalized kernel), conv<i>.g [C] (its norm:
 *     W = g * v / ||v|| over each output channel's C*K values), conv<i>.b
 *     [C], conv<i>.ln.g [C], conv<i>.ln.b [C];
 *   per direction (fwd, then bwd): lstm.<d>.w_ih [4H, C], lstm.<d>.w_hh
 *     [4H, H], lstm.<d>.b_ih [4H], lstm.<d>.b_hh [4H].
 * albert_text_n_tensors returns 1 + 5*n_conv + 8 (-1 for a bad config). */
int albert_text_n_tensors(const albert_text_config* cfg);
const char* albert_text_tensor_name(const albert_text_config* cfg, int index);
int albert_text_tensor_shape(const albert_text_config* cfg, int index, int64_t* rows,
                             int64_t* cols);

/* One device copy of the text encoder's weights (bf16; vectors fp32).  The
 * weight normalization is applied here, in double precision (a zero
 * direction row is ALBERT_E_ARG); the two LSTM biases are summed.  Host
 * tensors as albert_load_weights; allocates, and synchronises hip_stream. */
int albert_text_load_weights(albert_text_ctx** ctx, const albert_text_config* cfg,
                             const float* const* host_tensors, void* hip_stream);

/* Workspace bytes for n_seq sequences and max_rows token rows (0 for
 * invalid arguments). */
size_t albert_text_workspace_bytes(const albert_text_ctx* ctx, int n_seq, int64_t max_rows);

/* Padded batch: ids dev int32 [B, T], lengths dev int32 [B] in [1, T]
 * (T >= 1, B*T < 2^31); out dev fp32 [B, T, 2*hidden], pad rows written
 * as 0.  Validation, errors, workspace rules and flags as albert_encode. */
int albert_text_encode(albert_text_ctx* ctx, const int32_t* ids, const int32_t* lengths, int B,
                       int T, float* out, void* ws, size_t ws_bytes, void* hip_stream,
                       unsigned flags);

/* Packed batch: ids dev int32 [total], cu_seqlens dev int32 [n + 1], every
 * length in [1, max_len]; out dev fp32 [total, 2*hidden].  As
 * albert_encode_varlen. */
int albert_text_encode_varlen(albert_text_ctx* ctx, const int32_t* ids, const int32_t* cu_seqlens,
                              int n, int total, int max_len, float* out, void* ws,
                              size_t ws_bytes, void* hip_stream, unsigned flags);

/* Checkpoints in the workspace after a request (as albert_tap):
 *   0 STATUS int32 [1]   1 CU int32 [n_seq + 1]
 *   2 EMB  bf16 [rows, C]    embedding rows
 *   3 CONV bf16 [rows, C]    the last convolution block's output
 *   4 XG   fp32 [rows, 8H]   LSTM input projection plus both biases,
 *                            forward gates then backward gates */
enum albert_text_tap_kind {
  ALBERT_TT_STATUS = 0, ALBERT_TT_CU = 1, ALBERT_TT_EMB = 2, ALBERT_TT_CONV = 3, ALBERT_TT_XG = 4
};
int albert_text_tap(const albert_text_ctx* ctx, int n_seq, int64_t max_rows, int tap,
                    size_t* offset, size_t* bytes, int64_t* row_stride);

/* Kernel kinds of the text path, for albert_text_time_kernel() (same
 * contract as albert_time_kernel). */
enum albert_text_kernel_kind {
  ALBERT_TK_EMBED = 0,    /* embedding gather                               */
  ALBERT_TK_TAPS = 1,     /* per-row convolution taps, once per request     */
  ALBERT_TK_CONV = 2,     /* convolution GEMM + LayerNorm + LeakyReLU       */
  ALBERT_TK_LSTM_IN = 3,  /* LSTM input projection, both directions         */
  ALBERT_TK_LSTM = 4,     /* LSTM recurrence, both directions               */
  ALBERT_TK_COUNT = 5
};
int albert_text_time_kernel(albert_text_ctx* ctx, int kind, int max_launches);
int albert_text_kernel_time(albert_text_ctx* ctx, int* launches, double* total_ms);

/* Release the text context's device memory.  NULL is accepted. */
void albert_text_free(albert_text_ctx* ctx);

/* Release the context's device memory.  NULL is accepted. */
void albert_free(albert_ctx* ctx);

/* Static description of a status code. */
const char* albert_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* ALBERT_H */
