"""GPU parity of Kokoro's parallel text encoder (embedding, weight-normalized
convolution blocks, masked bidirectional LSTM) against the float64 oracle,
through the C ABI.  bf16 storage with fp32 accumulation and cell state, so
the encoder's bf16 tolerances apply; the embedding gather is bit-exact."""
import functools

import numpy as np
import pytest

import synth
from oracle import text_encoder as te

from _gpu import check, dev

pytestmark = pytest.mark.gpu
TC = synth.TEXT


@functools.lru_cache(maxsize=None)
def _w():
    return synth.make_text_weights()


@functools.lru_cache(maxsize=None)
def _tw():
    return te.prepare_text_weights(_w(), TC, "bf16")


_ENC = {}


def _enc():
    import albert_transformer_amd as A
    if "e" not in _ENC:
        _ENC["e"] = A.TextEncoder(_w())
    return _ENC["e"]


def _run(enc, ids, lengths):
    import torch
    B, T = ids.shape
    out = torch.full((B, T, 512), float("nan"), device="cuda")
    ws = enc.new_workspace(B, B * T)
    assert enc.encode_raw(dev(ids), dev(lengths), out, ws) == 0
    return out.cpu().numpy().astype(np.float64), ws


def _tap(enc, ws, n, rows_cap, name, rows, dtype):
    import torch
    off, nb, stride = enc.tap(n, rows_cap, name)
    t = ws[off:off + nb].cpu().view(dtype)
    return t.view(-1, stride)[:rows].double().numpy()


def test_text_stages():
    """Embedding rows bit-exact; the last convolution block and the LSTM
    input projection against the oracle; then the output."""
    import torch
    enc = _enc()
    TW = _tw()
    wl = synth.random_padded(51, B=3, T=70, lo=1, hi=70)
    wl.lengths[:] = [70, 33, 1]
    out, ws = _run(enc, wl.ids, wl.lengths)
    B, T = wl.ids.shape
    rows = int(wl.lengths.sum())
    emb = _tap(enc, ws, B, B * T, "emb", rows, torch.bfloat16)
    conv = _tap(enc, ws, B, B * T, "conv", rows, torch.bfloat16)
    xg = _tap(enc, ws, B, B * T, "xg", rows, torch.float32)
    r0 = 0
    for b in range(B):
        L = int(wl.lengths[b])
        ids = wl.ids[b, :L]
        sl = slice(r0, r0 + L)
        assert np.array_equal(emb[sl], TW["emb"][ids])
        x = TW["emb"][ids]
        for i in range(TC.n_conv):
            x = te.conv1d_same(x, TW[f"conv{i}.w"], TW[f"conv{i}.b"])
            x = te.leaky_relu(te.layer_norm(x, TW[f"conv{i}.ln.g"], TW[f"conv{i}.ln.b"], TC.ln_eps),
                              TC.slope)
        check(conv[sl], x, "bf16", f"text seq{b} conv")
        ref_xg = np.concatenate(
            [x @ TW[f"lstm.{d}.w_ih"].T + TW[f"lstm.{d}.b_ih"] + TW[f"lstm.{d}.b_hh"]
             for d in ("fwd", "bwd")], axis=1)
        check(xg[sl], ref_xg, "bf16", f"text seq{b} lstm input")
        check(out[b, :L], te.text_encode_sequence(ids, TW, TC), "bf16", f"text seq{b} output")
        assert np.all(out[b, L:] == 0.0)
        r0 += L


def test_text_packed_equals_padded_and_pad_invariance():
    import torch
    enc = _enc()
    wl = synth.random_padded(52, B=5, T=40, lo=1, hi=40)
    out, _ = _run(enc, wl.ids, wl.lengths)
    # other pad IDs and a wider T leave every valid row unchanged
    ids2 = np.concatenate([wl.ids, np.full((5, 9), 3, np.int32)], axis=1)
    for b, L in enumerate(wl.lengths):
        ids2[b, L:] = 177
    out2, _ = _run(enc, ids2, wl.lengths)
    cu = np.concatenate([[0], np.cumsum(wl.lengths)]).astype(np.int32)
    flat = np.concatenate([wl.ids[b, :L] for b, L in enumerate(wl.lengths)]).astype(np.int32)
    outp = torch.full((len(flat), 512), float("nan"), device="cuda")
    ws = enc.new_workspace(5, len(flat))
    assert enc.encode_varlen_raw(dev(flat), dev(cu), 40, outp, ws) == 0
    outp = outp.cpu().numpy()
    for b, L in enumerate(wl.lengths):
        assert np.array_equal(out[b, :L], out2[b, :L])
        assert np.array_equal(out[b, :L], outp[cu[b]:cu[b + 1]])


def test_text_full_size_sampled():
    """The full B=256, T=128 batch (all 8 sequence groups of both
    directions); sampled sequences against the oracle."""
    enc = _enc()
    TW = _tw()
    wl = synth.make_workload(3)
    out, _ = _run(enc, wl.ids, wl.lengths)
    for b in (0, 37, 255):
        check(out[b], te.text_encode_sequence(wl.ids[b], TW, TC), "bf16", f"text full seq{b}")


def test_text_long_ragged_batch():
    """Lengths spanning 1..512 in one batch of 33 sequences (two groups of
    the recurrence, the second holding one sequence)."""
    enc = _enc()
    TW = _tw()
    rng = np.random.default_rng(53)
    lengths = rng.integers(1, 513, 33).astype(np.int32)
    lengths[:3] = [512, 1, 2]
    ids = rng.integers(0, 178, (33, 512)).astype(np.int32)
    out, _ = _run(enc, ids, lengths)
    for b in (0, 1, 2, 20, 32):
        L = int(lengths[b])
        check(out[b, :L], te.text_encode_sequence(ids[b, :L], TW, TC), "bf16", f"text L={L}")


def test_text_rejections_leave_output_untouched():
    import torch
    import albert_transformer_amd as A
    enc = _enc()
    ids = np.ones((2, 8), np.int32)
    canary = torch.full((2, 8, 512), 5.0, device="cuda")
    ws = enc.new_workspace(2, 16)
    out = canary.clone()
    assert enc.encode_raw(dev(ids), dev(np.array([8, 0], np.int32)), out, ws) == A.E_LENGTH
    assert torch.equal(out, canary)
    bad = ids.copy()
    bad[1, 3] = 178
    assert enc.encode_raw(dev(bad), dev(np.array([8, 8], np.int32)), out, ws) == A.E_ID
    assert torch.equal(out, canary)
    bad[1, 3] = 1
    bad[1, 6] = -5    # beyond the length: never read
    assert enc.encode_raw(dev(bad), dev(np.array([8, 5], np.int32)), out, ws) == A.OK
    assert enc.encode_raw(dev(ids), dev(np.array([8, 8], np.int32)), out, ws, ws_bytes=16) == \
        A.E_WORKSPACE


def test_text_recurrence_variants_agree_bitwise():
    """The four-workgroup recurrence (default) and the one-workgroup one
    (ALBERT_UNFUSED) add the same products in the same order: identical
    outputs, on a ragged batch of three groups of 32 sequences."""
    import torch
    import albert_transformer_amd as A
    enc = _enc()
    TW = _tw()
    rng = np.random.default_rng(54)
    lengths = rng.integers(1, 97, 70).astype(np.int32)
    lengths[:2] = [96, 1]
    ids = rng.integers(0, 178, (70, 96)).astype(np.int32)
    outs = []
    for flags in (0, A.UNFUSED):
        out = torch.full((70, 96, 512), float("nan"), device="cuda")
        ws = enc.new_workspace(70, 70 * 96)
        assert enc.encode_raw(dev(ids), dev(lengths), out, ws, flags=flags) == A.OK
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    for b in (0, 1, 69):
        L = int(lengths[b])
        check(outs[0][b, :L].astype(np.float64), te.text_encode_sequence(ids[b, :L], TW, TC),
              "bf16", f"text recurrence L={L}")


def test_text_many_short_sequences():
    """More sequences than one cooperative launch of the recurrence holds
    (several launches, the last one partial); packed rows; sampled
    sequences against the oracle and the whole output against the
    one-workgroup recurrence."""
    import torch
    import albert_transformer_amd as A
    enc = _enc()
    TW = _tw()
    rng = np.random.default_rng(55)
    n = 64 * 32 * 2 + 37
    lengths = rng.integers(1, 7, n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    flat = rng.integers(0, 178, total).astype(np.int32)
    outs = []
    for flags in (0, A.UNFUSED):
        out = torch.full((total, 512), float("nan"), device="cuda")
        ws = enc.new_workspace(n, total)
        assert enc.encode_varlen_raw(dev(flat), dev(cu), 6, out, ws, flags=flags) == A.OK
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    for b in (0, 2047, 2048, 4095, n - 1):
        check(outs[0][cu[b]:cu[b + 1]].astype(np.float64),
              te.text_encode_sequence(flat[cu[b]:cu[b + 1]], TW, TC), "bf16", f"text short seq{b}")
