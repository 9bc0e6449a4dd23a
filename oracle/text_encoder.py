"""Plain float64 definition of Kokoro's parallel text encoder.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the tests
and the benchmark's CPU-baseline leg, never by the product path, and it
shares no code with the HIP library.

Sources:
  [TTS]    "How Kokoro TTS Works and Where CKE Stands" -- the component list
           (a small separate path: embedding, three weight-normalized
           convolutions, a bidirectional LSTM; it runs beside the ALBERT on
           the same phoneme IDs) and "How I want CKE to stitch it" (the text
           path publishes its own [512, T] features).
  [LITERT] "Kokoro-82M-LiteRT" -- the LSTMs are masked: a plain LSTM over a
           padded batch lets pad tokens into the backward pass.
Readings where the pages are silent (the StyleTTS 2 text encoder, which the
pages name as Kokoro's base in [HAILO] and [LITERT]): 512 channels; kernel
5 with zero padding of 2 at each end of every sequence; after each
convolution a LayerNorm over the channels (epsilon 1e-5) and a LeakyReLU of
slope 0.2; an LSTM of 256 units per direction with the i, f, g, o gate
order and both biases; zero initial state; output [L, 512] token-major
(forward half, then backward half).
"""
from __future__ import annotations

import numpy as np

from .albert_oracle import OracleError, bf16_round, layer_norm


def weight_norm(v, g) -> np.ndarray:
    """Weight normalization: W = g * v / ||v|| per output channel.

    [TTS] (component list: the text path's convolutions carry weight
    normalization); the reparameterization of
    Salimans and Kingma (2016), the norm taken over all of an output
    channel's weights (input channels and taps).
    """
    v = np.asarray(v, dtype=np.float64)
    norm = np.sqrt((v * v).reshape(v.shape[0], -1).sum(axis=1))
    return np.asarray(g, np.float64).reshape(-1, *([1] * (v.ndim - 1))) * v / \
        norm.reshape(-1, *([1] * (v.ndim - 1)))


def conv1d_same(x, w, b) -> np.ndarray:
    """out[t, o] = b[o] + sum_j sum_i w[o, i, j] * x[t + j - K//2, i], with x
    taken as zero outside the sequence (x is [L, C_in], w [C_out, C_in, K])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L = x.shape[0]
    K = w.shape[2]
    p = K // 2
    xp = np.zeros((L + 2 * p, x.shape[1]))
    xp[p:p + L] = x
    out = np.zeros((L, w.shape[0])) + b
    for j in range(K):
        out += xp[j:j + L] @ w[:, :, j].T
    return out


def leaky_relu(x, slope: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, x, slope * x)


def sigmoid(x) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def lstm(x, w_ih, w_hh, b_ih, b_hh, reverse: bool = False) -> np.ndarray:
    """One LSTM direction over one sequence x [L, I] -> h [L, H].

    gates = W_ih x_t + b_ih + W_hh h_prev + b_hh, split i, f, g, o;
    c = sigmoid(f) c_prev + sigmoid(i) tanh(g); h = sigmoid(o) tanh(c);
    h and c start at zero.  reverse runs t = L-1 .. 0 over the sequence's
    own tokens only, so padding never enters it ([LITERT]).
    """
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    H = np.asarray(w_hh).shape[1]
    h = np.zeros(H)
    c = np.zeros(H)
    out = np.zeros((L, H))
    xg = x @ np.asarray(w_ih, np.float64).T + b_ih + b_hh
    for t in (range(L - 1, -1, -1) if reverse else range(L)):
        z = xg[t] + np.asarray(w_hh, np.float64) @ h
        i, f, g, o = z[:H], z[H:2 * H], z[2 * H:3 * H], z[3 * H:]
        c = sigmoid(f) * c + sigmoid(i) * np.tanh(g)
        h = sigmoid(o) * np.tanh(c)
        out[t] = h
    return out


def prepare_text_weights(w: dict, cfg, dtype: str) -> dict:
    """Float64 weights as the given path stores them: the convolutions'
    effective weights (weight norm applied in float64, then stored as
    float32 -- or bf16 on the bf16 path, like the embedding and LSTM
    matrices); vectors float32.  dtype "f64" keeps the effective weights
    unrounded (the definition itself)."""
    if dtype not in ("f64", "f32", "bf16"):
        raise ValueError(dtype)
    if dtype == "bf16":
        rnd = lambda a: bf16_round(np.asarray(a, np.float32))
    elif dtype == "f32":
        rnd = lambda a: np.asarray(a, np.float32).astype(np.float64)
    else:
        rnd = lambda a: np.asarray(a, np.float64)
    out = {"emb": rnd(np.asarray(w["emb"], np.float32))}
    for i in range(cfg.n_conv):
        wn = weight_norm(np.asarray(w[f"conv{i}.v"], np.float32), np.asarray(w[f"conv{i}.g"], np.float32))
        out[f"conv{i}.w"] = rnd(wn if dtype == "f64" else wn.astype(np.float32))
        for k in ("b", "ln.g", "ln.b"):
            out[f"conv{i}.{k}"] = np.asarray(w[f"conv{i}.{k}"], np.float32).astype(np.float64)
    for d in ("fwd", "bwd"):
        for k in ("w_ih", "w_hh"):
            out[f"lstm.{d}.{k}"] = rnd(np.asarray(w[f"lstm.{d}.{k}"], np.float32))
        for k in ("b_ih", "b_hh"):
            out[f"lstm.{d}.{k}"] = np.asarray(w[f"lstm.{d}.{k}"], np.float32).astype(np.float64)
    return out


def text_encode_sequence(ids_seq, TW: dict, cfg) -> np.ndarray:
    """One sequence of valid IDs -> [L, 2 * hidden] (512 for Kokoro)."""
    ids_seq = np.asarray(ids_seq)
    x = TW["emb"][ids_seq]
    for i in range(cfg.n_conv):
        x = conv1d_same(x, TW[f"conv{i}.w"], TW[f"conv{i}.b"])
        x = leaky_relu(layer_norm(x, TW[f"conv{i}.ln.g"], TW[f"conv{i}.ln.b"], cfg.ln_eps), cfg.slope)
    args = lambda d: (TW[f"lstm.{d}.w_ih"], TW[f"lstm.{d}.w_hh"], TW[f"lstm.{d}.b_ih"],
                      TW[f"lstm.{d}.b_hh"])
    return np.concatenate([lstm(x, *args("fwd")), lstm(x, *args("bwd"), reverse=True)], axis=1)


def text_encode(ids, lengths, TW: dict, cfg, seqs=None) -> np.ndarray:
    """Padded batch ids [B, T], lengths [B] -> [B, T, 2 * hidden]; rows at
    t >= length are zero and pad IDs are never read."""
    ids = np.asarray(ids)
    lengths = np.asarray(lengths)
    B, T = ids.shape
    for b, L in enumerate(lengths):
        if L < 1 or L > T:
            raise OracleError("E_LENGTH", f"sequence {b} length {L} outside [1, {T}]")
        if np.any(ids[b, :L] < 0) or np.any(ids[b, :L] >= cfg.vocab):
            raise OracleError("E_ID", f"sequence {b} has an id outside the vocabulary")
    out = np.zeros((B, T, 2 * cfg.hidden))
    for b in (range(B) if seqs is None else seqs):
        L = int(lengths[b])
        out[b, :L] = text_encode_sequence(ids[b, :L], TW, cfg)
    return out
