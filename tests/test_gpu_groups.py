"""GPU parity of ALBERT's intermediate grouping (G layer weight sets, each
reused over a contiguous block of the executions) against the float64
oracle, through the C ABI.  Tolerances as in the other parity tests."""
import functools

import numpy as np
import pytest

import oracle
import synth

from _gpu import check, dev

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _weights(G: int, n_iter: int = 12):
    cfg = synth.Config(n_groups=G, n_iter=n_iter)
    return cfg, synth.make_weights(cfg, seed=777 + G)


def _encoder(G, dtype, n_iter=12):
    import albert_transformer_amd as A
    cfg, w = _weights(G, n_iter)
    return cfg, w, A.Encoder(w, dtype, n_groups=G, n_iter=n_iter)


def _run(enc, wl):
    import torch
    B, T = wl.ids.shape
    out = torch.full((B, T, 512), float("nan"), device="cuda")
    ws = enc.new_workspace(B, B * T)
    assert enc.encode_raw(dev(wl.ids), dev(wl.lengths), out, ws) == 0
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("G,dtype,n_iter", [(3, "bf16", 12), (12, "bf16", 12), (5, "f32", 12),
                                            (2, "bf16", 3)])
def test_grouped_padded_batch(G, dtype, n_iter):
    cfg, w, enc = _encoder(G, dtype, n_iter)
    W = oracle.prepare_weights(w, dtype)
    wl = synth.random_padded(60 + G, B=3, T=72, lo=1, hi=72)
    wl.lengths[:] = [72, 37, 1]
    got = _run(enc, wl)
    ref = oracle.encode(wl.ids, wl.lengths, W, cfg)
    for b in range(3):
        L = int(wl.lengths[b])
        check(got[b, :L], ref[b, :L], dtype, f"G={G} n_iter={n_iter} seq{b}")
        assert np.all(got[b, L:] == 0.0)
    enc.close()


def test_identical_sets_equal_full_sharing_bitwise():
    """G copies of one layer set run the same kernels on the same values as
    the fully shared model, so the outputs are identical bit for bit."""
    import albert_transformer_amd as A
    w1 = synth.make_weights()
    cfg4 = synth.Config(n_groups=4)
    w4 = {n: w1[synth.base_name(n)] for n in synth.tensor_names(cfg4)}
    wl = synth.random_padded(70, B=4, T=64, lo=10, hi=64)
    e1 = A.Encoder(w1, "bf16")
    e4 = A.Encoder(w4, "bf16", n_groups=4)
    assert np.array_equal(_run(e1, wl), _run(e4, wl))
    e1.close()
    e4.close()


def test_grouped_full_size_headline_shape():
    """Twelve distinct sets (a BERT-style stack) at the full B=256, T=128
    batch; sampled sequences checked against the oracle."""
    cfg, w, enc = _encoder(12, "bf16")
    W = oracle.prepare_weights(w, "bf16")
    wl = synth.make_workload(3)
    got = _run(enc, wl)
    for b in (0, 131, 255):
        ref = oracle.encode_sequence(wl.ids[b], W, cfg)
        check(got[b], ref, "bf16", f"G=12 full batch seq{b}")
    enc.close()
