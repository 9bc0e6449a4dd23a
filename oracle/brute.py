"""Pure-Python, loop-by-loop encoder for tiny shapes.

TEST INFRASTRUCTURE ONLY.  A second, independent reading of the same
definition as ``albert_oracle`` (it imports nothing from it), written with
explicit loops over lists so that each sum can be checked by eye.  It also
accepts a list of per-execution layer weight sets, so that a model with N
distinct layers can be compared against the shared-layer schedule.

Sources: "ALBERT: How Kokoro's Phoneme Encoder Works" (sections "What ALBERT
Changed" and "Inside One Real ALBERT Layer"), the Hailo-10H model card for the
tanh GELU, and contract A of "Qwen3-TTS and Kokoro: Two Routes from Text to
Speech" for y_j = b_j + sum_i x_i W[j][i].
"""
from __future__ import annotations

import math

LAYER_KEYS = ("q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "o.w", "o.b",
              "attn_ln.g", "attn_ln.b", "ffn1.w", "ffn1.b", "ffn2.w",
              "ffn2.b", "ffn_ln.g", "ffn_ln.b")


def _lin(x, W, b):
    # x: list of rows; W: rows of out x in; b: list
    out = []
    for row in x:
        y = []
        for j in range(len(W)):
            acc = b[j]
            for i in range(len(row)):
                acc += row[i] * W[j][i]
            y.append(acc)
        out.append(y)
    return out


def _ln(x, g, b, eps):
    out = []
    for row in x:
        n = len(row)
        mu = sum(row) / n
        var = sum((v - mu) * (v - mu) for v in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(row[i] - mu) * inv * g[i] + b[i] for i in range(n)])
    return out


def _gelu(v):
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * v * (1.0 + math.tanh(c * (v + 0.044715 * v * v * v)))


def _attn(q, k, v, heads):
    L = len(q)
    H = len(q[0])
    d = H // heads
    scale = 1.0 / math.sqrt(d)
    out = [[0.0] * H for _ in range(L)]
    for h in range(heads):
        o = h * d
        for t in range(L):
            scores = []
            for u in range(L):
                s = 0.0
                for c in range(d):
                    s += q[t][o + c] * k[u][o + c]
                scores.append(s * scale)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = sum(w)
            for c in range(d):
                acc = 0.0
                for u in range(L):
                    acc += w[u] / z * v[u][o + c]
                out[t][o + c] = acc
    return out


def _layer(x, P, cfg):
    q = _lin(x, P["q.w"], P["q.b"])
    k = _lin(x, P["k.w"], P["k.b"])
    v = _lin(x, P["v.w"], P["v.b"])
    c = _attn(q, k, v, cfg.heads)
    a = _lin(c, P["o.w"], P["o.b"])
    h1 = _ln([[x[t][i] + a[t][i] for i in range(len(x[t]))] for t in range(len(x))],
             P["attn_ln.g"], P["attn_ln.b"], cfg.ln_eps)
    f = [[_gelu(val) for val in row] for row in _lin(h1, P["ffn1.w"], P["ffn1.b"])]
    f2 = _lin(f, P["ffn2.w"], P["ffn2.b"])
    return _ln([[h1[t][i] + f2[t][i] for i in range(len(h1[t]))] for t in range(len(h1))],
               P["ffn_ln.g"], P["ffn_ln.b"], cfg.ln_eps)


def _tolist(W):
    return {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in W.items()}


def encode_brute(ids_seq, W, cfg, layers=None):
    """Encode one sequence; `layers` optionally lists one weight dict per
    execution (a model with distinct layers); by default the shared layer in
    W is used cfg.n_iter times."""
    Wl = _tolist(W)
    ids_seq = [int(i) for i in ids_seq]
    L = len(ids_seq)
    E = len(Wl["emb.word"][0])
    e = [[Wl["emb.word"][ids_seq[t]][i] + Wl["emb.pos"][t][i] + Wl["emb.type"][0][i]
          for i in range(E)] for t in range(L)]
    e = _ln(e, Wl["emb.ln.g"], Wl["emb.ln.b"], cfg.ln_eps)
    x = _lin(e, Wl["proj.w"], Wl["proj.b"])
    if layers is None:
        shared = {k: Wl[k] for k in LAYER_KEYS}
        layers = [shared] * cfg.n_iter
    else:
        layers = [_tolist(P) for P in layers]
    for P in layers:
        x = _layer(x, P, cfg)
    return _lin(x, Wl["out.w"], Wl["out.b"])
