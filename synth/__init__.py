"""Seeded synthetic weights and inputs for the Kokoro ALBERT phoneme encoder.

This module only draws random numbers and lays them out in the shapes the
encoder consumes.  It performs none of the encoder's arithmetic, so both the
float64 oracle and the HIP library can be fed from it without sharing any
computation.

Shapes follow the pinned Kokoro configuration described on the page "ALBERT:
How Kokoro's Phoneme Encoder Works" (section "What ALBERT Changed", the worked
parameter arithmetic, and section "Inside One Real ALBERT Layer"): vocabulary
178, 512 positions, 2 token types, embedding width 128, hidden width 768, 12
heads of 64, FFN width 2048, one shared layer executed 12 times, and an output
projection to 512.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_SEED = 20261203

# Canonical tensor order.  Linear weights are [out, in] row-major.
TENSOR_NAMES = (
    "emb.word", "emb.pos", "emb.type", "emb.ln.g", "emb.ln.b",
    "proj.w", "proj.b",
    "q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "o.w", "o.b",
    "attn_ln.g", "attn_ln.b",
    "ffn1.w", "ffn1.b", "ffn2.w", "ffn2.b",
    "ffn_ln.g", "ffn_ln.b",
    "out.w", "out.b",
)
# The tensors of one transformer layer (indices 7..22 above).
LAYER_NAMES = TENSOR_NAMES[7:23]


@dataclass(frozen=True)
class Config:
    vocab: int = 178
    max_pos: int = 512
    n_types: int = 2
    emb: int = 128
    hidden: int = 768
    heads: int = 12
    head_dim: int = 64
    ffn: int = 2048
    n_iter: int = 12
    out_dim: int = 512
    ln_eps: float = 1e-12
    n_groups: int = 1           # distinct layer weight sets (Kokoro: one)

    def shapes(self) -> dict:
        E, H, F, O = self.emb, self.hidden, self.ffn, self.out_dim
        return {
            "emb.word": (self.vocab, E), "emb.pos": (self.max_pos, E),
            "emb.type": (self.n_types, E), "emb.ln.g": (E,), "emb.ln.b": (E,),
            "proj.w": (H, E), "proj.b": (H,),
            "q.w": (H, H), "q.b": (H,), "k.w": (H, H), "k.b": (H,),
            "v.w": (H, H), "v.b": (H,), "o.w": (H, H), "o.b": (H,),
            "attn_ln.g": (H,), "attn_ln.b": (H,),
            "ffn1.w": (F, H), "ffn1.b": (F,), "ffn2.w": (H, F), "ffn2.b": (H,),
            "ffn_ln.g": (H,), "ffn_ln.b": (H,),
            "out.w": (O, H), "out.b": (O,),
        }


KOKORO = Config()


def tensor_names(cfg: Config = KOKORO) -> tuple:
    """Canonical tensor order for cfg.n_groups layer weight sets.

    One set: TENSOR_NAMES.  G > 1 sets: the seven embedding/projection
    tensors, then the 16 layer tensors of set 0, 1, ..., G-1 named
    "g<set>.<name>", then the output projection.
    """
    if cfg.n_groups == 1:
        return TENSOR_NAMES
    names = list(TENSOR_NAMES[:7])
    for g in range(cfg.n_groups):
        names += [f"g{g}.{n}" for n in LAYER_NAMES]
    return tuple(names + list(TENSOR_NAMES[23:]))


def base_name(name: str) -> str:
    """Strip a "g<set>." prefix: the tensor's role in the layer."""
    head, _, rest = name.partition(".")
    return rest if head[:1] == "g" and head[1:].isdigit() else name

# A tiny configuration for brute-force cross checks.
TINY = Config(vocab=11, max_pos=6, n_types=2, emb=4, hidden=8, heads=2,
              head_dim=4, ffn=16, n_iter=3, out_dim=4)


def make_weights(cfg: Config = KOKORO, seed: int = WEIGHT_SEED) -> dict:
    """Draw every tensor in canonical order (``tensor_names``) from one
    generator.

    Matrices, tables and biases ~ N(0, 0.02); LayerNorm gains 1 + N(0, 0.01)
    and shifts N(0, 0.01).  Drawn in float64, returned as float32.
    """
    rng = np.random.default_rng(seed)
    shapes = cfg.shapes()
    out = {}
    for name in tensor_names(cfg):
        shp = shapes[base_name(name)]
        if name.endswith(".g"):
            a = 1.0 + rng.normal(0.0, 0.01, size=shp)
        elif name.endswith("ln.b"):
            a = rng.normal(0.0, 0.01, size=shp)
        else:
            a = rng.normal(0.0, 0.02, size=shp)
        out[name] = np.ascontiguousarray(a.astype(np.float32))
    return out


@dataclass
class Workload:
    """One batch of encoder input.

    Padded form: ``ids`` is int32 [B, T] and ``lengths`` int32 [B].
    Packed form: ``ids`` is int32 [total] and ``cu_seqlens`` int32 [n + 1].
    """
    name: str
    dtype: str                  # "f32" or "bf16"
    ids: np.ndarray
    lengths: np.ndarray
    T: int
    packed: bool = False
    cu_seqlens: np.ndarray | None = None
    notes: dict = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def rows(self) -> int:
        """Rows the caller's output buffer holds."""
        return self.tokens if self.packed else self.n_seq * self.T


def _pad_boundary(rng, B, T, lengths):
    ids = rng.integers(1, 178, size=(B, T)).astype(np.int32)
    for b in range(B):
        L = int(lengths[b])
        ids[b, 0] = 0
        ids[b, L - 1] = 0
        ids[b, L:] = 0
    return ids


def make_workload(k: int) -> Workload:
    """Configuration k in 1..5 (see module doc for the recipe)."""
    rng = np.random.default_rng(1000 + k)
    if k == 1:
        ids = np.concatenate([[0], rng.integers(1, 178, size=34), [0]]).astype(np.int32)
        return Workload("single utterance B=1 T=36", "f32", ids[None, :],
                        np.array([36], np.int32), 36)
    if k == 2:
        B, T = 64, 128
        lengths = rng.integers(16, 129, size=B).astype(np.int32)
        return Workload("padded batch B=64 T=128", "bf16",
                        _pad_boundary(rng, B, T, lengths), lengths, T)
    if k == 3:
        B, T = 256, 128
        lengths = np.full(B, T, np.int32)
        ids = rng.integers(1, 178, size=(B, T)).astype(np.int32)
        return Workload("full batch B=256 T=128", "bf16", ids, lengths, T)
    if k == 4:
        B, T = 32, 512
        lengths = rng.integers(256, 513, size=B).astype(np.int32)
        return Workload("long sequences B=32 T=512", "bf16",
                        _pad_boundary(rng, B, T, lengths), lengths, T)
    if k == 5:
        n = 1024
        lengths = np.clip(rng.geometric(1.0 / 60.0, size=n), 8, 510).astype(np.int32)
        total = int(lengths.sum())
        ids = rng.integers(1, 178, size=total).astype(np.int32)
        cu = np.zeros(n + 1, np.int32)
        cu[1:] = np.cumsum(lengths)
        return Workload("varlen packed n=1024 mean 60", "bf16", ids, lengths,
                        int(lengths.max()), packed=True, cu_seqlens=cu)
    raise ValueError(f"no workload {k}")


def random_padded(seed: int, B: int, T: int, lo: int = 1, hi: int | None = None,
                  vocab: int = 178, dtype: str = "bf16") -> Workload:
    """Padded batch with lengths uniform in [lo, hi] and random pad-slot ids."""
    rng = np.random.default_rng(seed)
    hi = T if hi is None else hi
    lengths = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    ids = rng.integers(0, vocab, size=(B, T)).astype(np.int32)
    return Workload(f"random padded B={B} T={T}", dtype, ids, lengths, T)


def random_packed(seed: int, lengths, vocab: int = 178, dtype: str = "bf16") -> Workload:
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int32)
    total = int(lengths.sum())
    ids = rng.integers(0, vocab, size=total).astype(np.int32)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return Workload(f"random packed n={len(lengths)}", dtype, ids, lengths,
                    int(lengths.max()), packed=True, cu_seqlens=cu)


# ------------------------------------------------------- text encoder ----
# Kokoro's parallel text path: embedding -> three weight-normalized
# convolutions -> bidirectional LSTM ("How Kokoro TTS Works and Where CKE
# Stands", the component list; [512, T] features per "How I want CKE to
# stitch it").  Sizes the pages leave open follow the StyleTTS 2 text
# encoder that Kokoro inherits: 512 channels, kernel 5, 256 LSTM units per
# direction.

TEXT_WEIGHT_SEED = 20261204


@dataclass(frozen=True)
class TextConfig:
    vocab: int = 178
    channels: int = 512
    kernel: int = 5
    n_conv: int = 3
    hidden: int = 256          # LSTM units per direction
    ln_eps: float = 1e-5
    slope: float = 0.2         # LeakyReLU negative slope

    def tensor_names(self) -> tuple:
        names = ["emb"]
        for i in range(self.n_conv):
            names += [f"conv{i}.v", f"conv{i}.g", f"conv{i}.b", f"conv{i}.ln.g", f"conv{i}.ln.b"]
        for d in ("fwd", "bwd"):
            names += [f"lstm.{d}.w_ih", f"lstm.{d}.w_hh", f"lstm.{d}.b_ih", f"lstm.{d}.b_hh"]
        return tuple(names)

    def shapes(self) -> dict:
        C, K, Hh = self.channels, self.kernel, self.hidden
        s = {"emb": (self.vocab, C)}
        for i in range(self.n_conv):
            s.update({f"conv{i}.v": (C, C, K), f"conv{i}.g": (C,), f"conv{i}.b": (C,),
                      f"conv{i}.ln.g": (C,), f"conv{i}.ln.b": (C,)})
        for d in ("fwd", "bwd"):
            s.update({f"lstm.{d}.w_ih": (4 * Hh, C), f"lstm.{d}.w_hh": (4 * Hh, Hh),
                      f"lstm.{d}.b_ih": (4 * Hh,), f"lstm.{d}.b_hh": (4 * Hh,)})
        return s


TEXT = TextConfig()
TEXT_TINY = TextConfig(vocab=7, channels=6, kernel=3, n_conv=2, hidden=3)


def make_text_weights(cfg: TextConfig = TEXT, seed: int = TEXT_WEIGHT_SEED) -> dict:
    """Draw the text encoder's tensors in canonical order from one generator.

    Embedding N(0, 1); convolution directions v ~ N(0, 0.02) with gains
    g = 1 + N(0, 0.01) (so each output channel's effective weight has norm
    close to 1) and biases N(0, 0.02); LayerNorm gains 1 + N(0, 0.01),
    shifts N(0, 0.01); LSTM matrices N(0, 0.05) and biases N(0, 0.02).
    Drawn in float64, returned as float32.
    """
    rng = np.random.default_rng(seed)
    shapes = cfg.shapes()
    out = {}
    for name in cfg.tensor_names():
        shp = shapes[name]
        if name == "emb":
            a = rng.normal(0.0, 1.0, size=shp)
        elif name.endswith(".g"):
            a = 1.0 + rng.normal(0.0, 0.01, size=shp)
        elif name.endswith("ln.b"):
            a = rng.normal(0.0, 0.01, size=shp)
        elif name.startswith("lstm") and ".w_" in name:
            a = rng.normal(0.0, 0.05, size=shp)
        else:
            a = rng.normal(0.0, 0.02, size=shp)
        out[name] = np.ascontiguousarray(a.astype(np.float32))
    return out
