"""Randomized batch shapes through the C ABI against the oracle.

Each case draws a batch size, a padded length and sequence lengths (some
batches all full length), runs it padded or packed, in bf16, fp32 or with
E4M3 operands, and checks the longest, the shortest and three random
sequences against the float64 oracle at the path's tolerance (pad slots
must be exactly zero).  The shapes cross every
tile boundary the kernels choose between (split-K products up to 256 rows,
64-, 128- and 256-row LayerNorm pairs, fused and separate Q|K|V +
attention, sequences over 256 tokens), so a mistake in one of the rarer
tilings shows up here even where the fixed-shape tests do not reach it.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check, dev, encoder, oracle_weights, row_cosines

pytestmark = pytest.mark.gpu
K = synth.KOKORO
FP8_MAX_ABS, FP8_MIN_COS = 0.2, 0.997  # the full-depth E4M3 bound (test_gpu_fp8)
BATCHES = (1, 2, 3, 7, 31, 64, 97, 200, 257, 600)
LENGTHS = (1, 5, 36, 100, 128, 129, 255, 256, 300, 512)


def _case(seed):
    """dtype, packed, workload and the sequences checked, from one seed."""
    rng = np.random.default_rng(seed)
    dtype = "f32" if seed % 4 == 3 else "fp8" if seed % 8 == 5 else "bf16"
    packed = bool(rng.integers(0, 2))
    B, T = int(rng.choice(BATCHES)), int(rng.choice(LENGTHS))
    B = max(1, min(B, 80_000 // T))
    full = rng.random() < 0.3
    wl = synth.random_padded(seed, B, T, lo=T if full else 1, dtype=dtype)
    L = wl.lengths
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), *map(int, rng.integers(0, B, 3))})
    return dtype, packed, wl, seqs


def _check(got, ids_seq, dtype, W, ref_row, what):
    """The path's tolerance; E4M3 operands against the oracle's emulation
    fed by its own embedding, at the full-depth bound."""
    if dtype != "fp8":
        check(got, ref_row, dtype, what)
        return
    ref = oracle.encode_fp8_features(oracle.embed_ln(ids_seq, W, K), W, K)
    err = float(np.max(np.abs(got - ref)))
    cos = float(np.min(row_cosines(got, ref)))
    print(f"[random] {what} fp8 max_abs={err:.3e} min_cos={cos:.6f}", flush=True)
    assert err <= FP8_MAX_ABS and cos >= FP8_MIN_COS, (what, err, cos)


@pytest.mark.parametrize("seed", range(24))
def test_random_batch(seed):
    import torch
    dtype, packed, wl, seqs = _case(seed)
    B, T = wl.ids.shape
    L = wl.lengths
    enc = encoder(dtype)
    W = oracle_weights(dtype)
    print(f"[random] seed={seed} dtype={dtype} packed={packed} B={B} T={T} rows={int(L.sum())}", flush=True)
    if packed:
        flat = np.concatenate([wl.ids[b, :n] for b, n in enumerate(L)]).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        out = torch.full((int(cu[-1]), K.out_dim), float("nan"), device="cuda")
        ws = enc.new_workspace(B, int(cu[-1]))
        assert enc.encode_varlen_raw(dev(flat), dev(cu), T, out, ws) == 0
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        ref = oracle.encode_varlen(flat, cu, W, K, seqs=seqs) if dtype != "fp8" else None
        for s in seqs:
            _check(got[cu[s]:cu[s + 1]], flat[cu[s]:cu[s + 1]], dtype, W,
                   None if ref is None else ref[cu[s]:cu[s + 1]], f"seed {seed} seq {s}")
    else:
        out = torch.full((B, T, K.out_dim), float("nan"), device="cuda")
        ws = enc.new_workspace(B, B * T)
        assert enc.encode_raw(dev(wl.ids), dev(L), out, ws) == 0
        got = out.cpu().numpy().astype(np.float64)
        ref = oracle.encode(wl.ids, L, W, K, seqs=seqs) if dtype != "fp8" else None
        for s in seqs:
            _check(got[s, :L[s]], wl.ids[s, :L[s]], dtype, W, None if ref is None else ref[s, :L[s]],
                   f"seed {seed} seq {s}")
        pad = np.arange(T)[None, :] >= L[:, None]
        assert np.all(got[pad] == 0.0)
