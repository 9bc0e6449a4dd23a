"""Plain float64 definition of the Kokoro ALBERT phoneme-encoder forward pass.

TEST INFRASTRUCTURE ONLY: used by the tests, the graft smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Sources (the pages this follows):
  [ALBERT]  "ALBERT: How Kokoro's Phoneme Encoder Works, and Where CKE Has
            Reached It" -- sections "What ALBERT Changed: Two Kinds of
            Sharing", "Inside One Real ALBERT Layer" (steps 1-6 and the
            paragraph after them) and "How CKE Represents It" (the contract
            list: LayerNorm epsilon 1e-12, GELU variant, additive mask, 12
            heads of 64, 128->768 projection).
  [TTS]     "How Kokoro TTS Works and Where CKE Stands" -- sections "What
            ALBERT does here" (softmax(QK^T/sqrt(d) + mask) V), "The time axis
            is where a circuit becomes difficult" (durations, A = sum d) and
            "How I want CKE to stitch it" (the header checks IDs).
  [ROUTES]  "Qwen3-TTS and Kokoro: Two Routes from Text to Speech" -- section
            "Path one" (the [p1,p2,p3], d=[2,1,3] toy) and "Six kernels, six
            mathematical contracts", contract A (a biased projection
            y_j = b_j + sum_i x_i W[j,i], weights stored [out, in]).
  [HAILO]   "Kokoro-82M-encoder-hailo10h" model card -- "What this is": the
            GELU is the tanh approximation and contains a cubic; "Eval
            results": low-precision fidelity is scored with N(0,1) inputs fed
            at the embedding LayerNorm output ([128,128] per sample) and the
            per-sample cosine of the flattened [128,512] outputs.

Everything is evaluated in float64.  For the bf16 path the oracle consumes the
exact weight values the GPU consumes (matrices and tables rounded to bf16 by
``bf16_round``, then widened), so a comparison measures activation rounding
only.  Readings taken where the pages are silent are listed at each function.
"""
from __future__ import annotations

import math

import numpy as np

# Tensors stored in the compute dtype (bf16 on the bf16 path); biases and
# LayerNorm vectors always stay float32.
_MATRIX_NAMES = ("emb.word", "emb.pos", "emb.type", "proj.w", "q.w", "k.w",
                 "v.w", "o.w", "ffn1.w", "ffn2.w", "out.w")


class OracleError(ValueError):
    """A request the encoder must reject; ``code`` names the status."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    bfloat16 keeps the top 16 bits of an IEEE binary32 value (8 exponent bits,
    7 stored mantissa bits).  Rounding adds half an ulp of the kept part minus
    one, plus the kept part's lowest bit (so that exact halves go to the even
    neighbour), then truncates.  Inputs must be finite.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16_round expects finite values")
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    u = (u + 0x7FFF + keep_lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest OCP FP8 E4M3 value, ties to even, saturating.

    E4M3 has 4 exponent bits (bias 7) and 3 stored mantissa bits: normal
    values m * 2^(e-3) with 8 <= m < 16 and -6 <= e <= 8, subnormals
    m * 2^-9 with m < 8, largest finite 448 (the all-ones pattern is NaN,
    so there is no infinity).  Reading for the low-precision variant:
    magnitudes beyond 448 saturate to 448.  Works in float64 on any input.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)                      # a = f * 2^e, 0.5 <= f < 1
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)  # spacing at a's binade
    r = np.minimum(np.round(a / step) * step, E4M3_MAX)  # np.round: half to even
    return np.copysign(r, x)


def fp8_row_exponents(w) -> np.ndarray:
    """Per-output-row power-of-two scale for an [out, in] weight matrix.

    Reading for the low-precision variant: row j is stored as
    e4m3(W[j, :] * 2^k_j) with the largest integer k_j such that
    max_i |W[j, i]| * 2^k_j <= 448 (k_j = 0 for an all-zero row, and at most
    127 so that 2^-k_j is an E8M0 scale), and the product is multiplied back
    by 2^-k_j, which is exact.
    """
    w = np.asarray(w, dtype=np.float64)
    m = np.abs(w).max(axis=1)
    k = np.zeros(m.shape, dtype=np.int64)
    nz = m > 0
    k[nz] = np.floor(np.log2(E4M3_MAX / m[nz])).astype(np.int64)
    # settle log2's rounding at exact powers of two
    k[nz] += (m[nz] * np.ldexp(1.0, k[nz] + 1) <= E4M3_MAX).astype(np.int64)
    k[nz] -= (m[nz] * np.ldexp(1.0, k[nz]) > E4M3_MAX).astype(np.int64)
    # an E8M0 scale 2^-k needs k <= 127 (rows below 448 * 2^-127 keep k = 127)
    return np.minimum(k, 127)


def fp8_quantize_rows(w) -> np.ndarray:
    """The weight values the low-precision variant multiplies with."""
    w = np.asarray(w, dtype=np.float64)
    sc = np.ldexp(1.0, fp8_row_exponents(w))[:, None]
    return e4m3_round(w * sc) / sc


def prepare_weights(w: dict, dtype: str) -> dict:
    """Widen the float32 weight set to float64, as the given path stores it.

    dtype "f32": every tensor exactly as given.
    dtype "bf16": tables and linear weight matrices rounded to bf16 first;
    biases and LayerNorm gains/shifts kept in float32 (the library's storage
    rule, so that both sides see identical parameter values).
    dtype "fp8": tables rounded to bf16, linear weight matrices quantized
    per row to E4M3 (``fp8_quantize_rows``), vectors kept in float32.
    """
    if dtype not in ("f32", "bf16", "fp8"):
        raise ValueError(dtype)
    out = {}
    for name, t in w.items():
        t32 = np.asarray(t, dtype=np.float32)
        head, _, rest = name.partition(".")
        role = rest if head[:1] == "g" and head[1:].isdigit() else name
        if dtype == "fp8" and role in _MATRIX_NAMES and role.endswith(".w"):
            out[name] = fp8_quantize_rows(t32)
        elif dtype in ("bf16", "fp8") and role in _MATRIX_NAMES:
            out[name] = bf16_round(t32)
        else:
            out[name] = t32.astype(np.float64)
    return out


def param_counts(cfg) -> dict:
    """Weight counts of the factorized embedding and of a BERT-style one.

    [ALBERT] "What ALBERT Changed", part 1: the tables live at width E and one
    E x H projection follows the sum; the unfactorized variant keeps all three
    tables at width H.  Weights only (no biases), as the page counts them.
    """
    E, H = cfg.emb, cfg.hidden
    word, pos, typ = cfg.vocab * E, cfg.max_pos * E, cfg.n_types * E
    proj = E * H
    tables = word + pos + typ
    unfact = (cfg.vocab + cfg.max_pos + cfg.n_types) * H
    return {"word": word, "position": pos, "type": typ, "tables": tables,
            "projection": proj, "factorized_total": tables + proj,
            "unfactorized_total": unfact,
            "savings": unfact - (tables + proj)}


def validate(ids, lengths, T: int, cfg) -> None:
    """Reject what the encoder's header check rejects.

    [TTS] "How I want CKE to stitch it": the encoder's header checks IDs
    before the embedding runs.  Reading: each length must lie in [1, T],
    T <= max positions, and every ID at a valid slot (t < length) must index
    the word table.  Slots at t >= length are padding and are never read.
    """
    ids = np.asarray(ids)
    lengths = np.asarray(lengths)
    if T < 1 or T > cfg.max_pos:
        raise OracleError("E_ARG", f"T={T} outside [1, {cfg.max_pos}]")
    for b, L in enumerate(lengths):
        if L < 1 or L > T:
            raise OracleError("E_LENGTH", f"sequence {b} length {L} outside [1, {T}]")
    for b, L in enumerate(lengths):
        row = ids[b, :L]
        if np.any(row < 0) or np.any(row >= cfg.vocab):
            raise OracleError("E_ID", f"sequence {b} has an id outside [0, {cfg.vocab - 1}]")


def layer_norm(x, g, b, eps: float) -> np.ndarray:
    """LayerNorm over the last axis.

    [ALBERT] step 1 and "How CKE Represents It" (epsilon 1e-12).  Reading:
    population variance (divide by the width) and epsilon added to the
    variance inside the square root.
    """
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu_tanh(x) -> np.ndarray:
    """GELU, tanh approximation: x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).

    [HAILO] "What this is": the encoder's GELU is the tanh approximation and
    contains a cubic; the constants are those of Hendrycks and Gimpel's
    approximation.  The cubic is formed as x*x*x.
    """
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x * x * x)))


def softmax(s) -> np.ndarray:
    """Row softmax over the last axis, with the row maximum subtracted first."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def dense(x, w, b) -> np.ndarray:
    """Biased projection y[t, j] = b[j] + sum_i x[t, i] * w[j, i].

    [ROUTES] contract A, with weights stored [out, in]; Kokoro's projections
    are the biased form.
    """
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T + b


def attention(q, k, v, heads: int) -> np.ndarray:
    """Bidirectional multi-head attention over one sequence.

    [ALBERT] step 4: q, k, v of width H split into `heads` heads of H/heads;
    per head softmax(q k^T / sqrt(head_dim)) v over every position on both
    sides; heads concatenated back to width H.  The pad mask is applied by
    the caller passing only the sequence's valid rows (an additive mask of
    -inf on pad keys contributes exactly zero weight).
    """
    L, H = q.shape
    d = H // heads
    out = np.empty((L, H), dtype=np.float64)
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        s = (q[:, sl] @ k[:, sl].T) / math.sqrt(d)
        out[:, sl] = softmax(s) @ v[:, sl]
    return out


def embed_ln(ids_seq, W: dict, cfg) -> np.ndarray:
    """Three-table embedding summed, then LayerNorm over the width E.

    [ALBERT] step 1: the ID indexes the word table, the position (0..L-1)
    indexes the position table, the token type (always 0 here) indexes the
    type table; the three rows are summed and LayerNormed.
    """
    ids_seq = np.asarray(ids_seq)
    L = ids_seq.shape[0]
    e = W["emb.word"][ids_seq] + W["emb.pos"][:L] + W["emb.type"][0]
    return layer_norm(e, W["emb.ln.g"], W["emb.ln.b"], cfg.ln_eps)


def shared_layer(h, W: dict, cfg, taps: dict | None = None) -> np.ndarray:
    """One execution of the shared transformer layer (post-LayerNorm).

    [ALBERT] steps 3-6: Q/K/V projections, bidirectional attention, output
    projection + residual + LayerNorm, then 768->2048, GELU, 2048->768,
    residual + LayerNorm.  When `taps` is a dict, the intermediate tensors
    are stored in it under "q", "k", "v", "ctx", "h1", "g".
    """
    q = dense(h, W["q.w"], W["q.b"])
    k = dense(h, W["k.w"], W["k.b"])
    v = dense(h, W["v.w"], W["v.b"])
    ctx = attention(q, k, v, cfg.heads)
    h1 = layer_norm(h + dense(ctx, W["o.w"], W["o.b"]),
                    W["attn_ln.g"], W["attn_ln.b"], cfg.ln_eps)
    g = gelu_tanh(dense(h1, W["ffn1.w"], W["ffn1.b"]))
    out = layer_norm(h1 + dense(g, W["ffn2.w"], W["ffn2.b"]),
                     W["ffn_ln.g"], W["ffn_ln.b"], cfg.ln_eps)
    if taps is not None:
        taps.update(q=q, k=k, v=v, ctx=ctx, h1=h1, g=g)
    return out


def group_schedule(n_iter: int, n_groups: int) -> list:
    """Which weight set each of the n_iter layer executions uses.

    [ALBERT] "What ALBERT Changed", part 2: besides full sharing, ALBERT can
    keep several distinct weight sets, each one serving a contiguous run of
    the layer executions.
    Reading: the blocks are contiguous and as equal as integers allow,
    execution i (from 0) using set floor(i * G / n_iter); G = 1 is full
    sharing and G = n_iter gives every execution its own set.
    """
    if n_groups < 1 or (n_iter > 0 and n_groups > n_iter):
        raise OracleError("E_ARG", f"{n_groups} weight sets for {n_iter} executions")
    return [i * n_groups // n_iter for i in range(n_iter)]


def layer_set(W: dict, cfg, g: int) -> dict:
    """The layer tensors of weight set g under their plain names."""
    if getattr(cfg, "n_groups", 1) == 1:
        return W
    pre = f"g{g}."
    return {k[len(pre):]: v for k, v in W.items() if k.startswith(pre)}


def encode_sequence(ids_seq, W: dict, cfg, n_iter: int | None = None,
                    taps: dict | None = None) -> np.ndarray:
    """Encode one sequence of valid IDs: returns [L, out_dim].

    [ALBERT] "Inside One Real ALBERT Layer" and "What ALBERT Changed", part 2:
    embedding + LayerNorm, the E->H projection, then `n_iter` executions of
    the shared layer, each on the previous execution's output (all with the
    same weights, or with the weight set ``group_schedule`` assigns), then
    the H->512 projection.
    """
    n_iter = cfg.n_iter if n_iter is None else n_iter
    sched = group_schedule(n_iter, getattr(cfg, "n_groups", 1))
    sets = [layer_set(W, cfg, g) for g in range(getattr(cfg, "n_groups", 1))]
    e = embed_ln(ids_seq, W, cfg)
    h = dense(e, W["proj.w"], W["proj.b"])
    if taps is not None:
        taps["emb"] = e
        taps["x0"] = h
    for it in range(n_iter):
        layer_taps = {} if taps is not None else None
        h = shared_layer(h, sets[sched[it]], cfg, layer_taps)
        if taps is not None:
            taps[f"iter{it}"] = dict(layer_taps, out=h)
    return dense(h, W["out.w"], W["out.b"])


def encode(ids, lengths, W: dict, cfg, n_iter: int | None = None,
           seqs=None) -> np.ndarray:
    """Padded batch: ids [B, T], lengths [B] -> [B, T, out_dim].

    Each sequence is encoded over its own valid tokens only, so pad slots
    never influence real tokens; output rows at t >= length are zero.
    `seqs` restricts the work to the listed sequences (the others stay 0).
    """
    ids = np.asarray(ids)
    lengths = np.asarray(lengths)
    B, T = ids.shape
    validate(ids, lengths, T, cfg)
    out = np.zeros((B, T, cfg.out_dim), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(lengths[b])
        out[b, :L] = encode_sequence(ids[b, :L], W, cfg, n_iter)
    return out


def encode_varlen(ids, cu_seqlens, W: dict, cfg, n_iter: int | None = None,
                  seqs=None) -> np.ndarray:
    """Packed batch: ids [total], cu_seqlens [n + 1] -> [total, out_dim].

    Sequence s occupies rows cu[s] .. cu[s+1]-1; positions restart at 0 for
    every sequence.
    """
    ids = np.asarray(ids)
    cu = np.asarray(cu_seqlens)
    total = ids.shape[0]
    if cu[0] != 0 or cu[-1] != total:
        raise OracleError("E_LENGTH", "cu_seqlens must start at 0 and end at total")
    lengths = np.diff(cu)
    if np.any(lengths < 1) or np.any(lengths > cfg.max_pos):
        raise OracleError("E_LENGTH", "sequence length outside [1, max positions]")
    if np.any(ids < 0) or np.any(ids >= cfg.vocab):
        raise OracleError("E_ID", "id outside the vocabulary")
    out = np.zeros((total, cfg.out_dim), dtype=np.float64)
    for s in (range(len(lengths)) if seqs is None else seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        out[a:b] = encode_sequence(ids[a:b], W, cfg, n_iter)
    return out


def encode_features(x_ln, W: dict, cfg, n_iter: int | None = None) -> np.ndarray:
    """Encode from the embedding LayerNorm output [L, E] of one sequence.

    The split the Hailo deployment uses ([HAILO] "What this is not": the
    embedding and its LayerNorm run elsewhere and the encoder block starts
    at the projection): E->H projection, the layer executions, H->512.
    """
    n_iter = cfg.n_iter if n_iter is None else n_iter
    sched = group_schedule(n_iter, getattr(cfg, "n_groups", 1))
    sets = [layer_set(W, cfg, g) for g in range(getattr(cfg, "n_groups", 1))]
    h = dense(x_ln, W["proj.w"], W["proj.b"])
    for it in range(n_iter):
        h = shared_layer(h, sets[sched[it]], cfg)
    return dense(h, W["out.w"], W["out.b"])


def _bf16_of(x):
    """bf16 storage of a float64 activation (rounded via float32)."""
    return bf16_round(np.asarray(x, dtype=np.float64).astype(np.float32))


# Storage roundings of the low-precision variant (module level so that a
# test can replace them with the identity).
fp8_operand = e4m3_round
fp8_store = _bf16_of


def encode_fp8_features(x_ln, W8: dict, cfg, n_iter: int | None = None,
                        taps: dict | None = None) -> np.ndarray:
    """The low-precision (FP8) variant from the LayerNorm output [L, E].

    Same steps as ``encode_features``; what changes is where values are
    rounded (the variant's definition, a reading of "FP8 GEMM operands"):
    every matrix-product input is an E4M3 value (``fp8_operand``) and every
    stored activation that is not a product input -- the residual stream,
    Q|K|V -- is bf16 (``fp8_store``).  W8 comes from
    prepare_weights(..., "fp8").  Products, biases, softmax, GELU and
    LayerNorm are exact (float64) here.  When `taps` is a dict, the values
    before each rounding are stored in it: "x0" (projection), and for the
    last execution "qkv", "ctx", "h1", "f1" (FFN1 output before GELU), "g"
    (after GELU) and "out" (the execution's output).
    """
    n_iter = cfg.n_iter if n_iter is None else n_iter
    sched = group_schedule(n_iter, getattr(cfg, "n_groups", 1))
    sets = [layer_set(W8, cfg, g) for g in range(getattr(cfg, "n_groups", 1))]
    op, st = fp8_operand, fp8_store
    y = dense(op(x_ln), W8["proj.w"], W8["proj.b"])
    if taps is not None:
        taps["x0"] = y
    h, h8 = st(y), op(y)
    for it in range(n_iter):
        Wl = sets[sched[it]]
        qkv = [dense(h8, Wl[n + ".w"], Wl[n + ".b"]) for n in ("q", "k", "v")]
        q, k, v = (st(t) for t in qkv)
        c = attention(q, k, v, cfg.heads)
        c8 = op(c)
        y = layer_norm(h + dense(c8, Wl["o.w"], Wl["o.b"]), Wl["attn_ln.g"], Wl["attn_ln.b"],
                       cfg.ln_eps)
        h1, h18 = st(y), op(y)
        f1 = dense(h18, Wl["ffn1.w"], Wl["ffn1.b"])
        g8 = op(gelu_tanh(f1))
        y2 = layer_norm(h1 + dense(g8, Wl["ffn2.w"], Wl["ffn2.b"]), Wl["ffn_ln.g"], Wl["ffn_ln.b"],
                        cfg.ln_eps)
        if taps is not None:
            taps.update(qkv=np.concatenate(qkv, axis=1), ctx=c, h1=y, f1=f1, g=gelu_tanh(f1),
                        out=y2)
        h, h8 = st(y2), op(y2)
    return dense(h8, W8["out.w"], W8["out.b"])


def duration_from_logits(logits, speed: float = 1.0) -> np.ndarray:
    """Integer durations from duration logits [T, C].

    [TTS] "The time axis is where a circuit becomes difficult": sigmoid of the
    duration channels, summed, divided by speed, rounded and clamped to at
    least one frame.  Reading: round to nearest, halves to even.
    """
    x = np.asarray(logits, dtype=np.float64)
    s = (1.0 / (1.0 + np.exp(-x))).sum(axis=-1) / speed
    return np.maximum(np.rint(s), 1).astype(np.int64)


def expand_durations(x, d) -> tuple[np.ndarray, int]:
    """Length regulation: repeat row t of x d[t] times; A = sum(d).

    [ROUTES] "Path one" and [TTS] "The time axis": durations are integers
    >= 1 and the aligned stream has A = sum(d) rows in token order.
    """
    x = np.asarray(x)
    d = np.asarray(d)
    if d.ndim != 1 or d.shape[0] != x.shape[0] or np.any(d < 1):
        raise OracleError("E_LENGTH", "durations must be >= 1, one per token")
    A = int(d.sum())
    out = np.empty((A,) + x.shape[1:], dtype=x.dtype)
    r = 0
    for t in range(x.shape[0]):
        for _ in range(int(d[t])):
            out[r] = x[t]
            r += 1
    return out, A
