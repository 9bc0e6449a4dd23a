"""Pins of the float64 text-encoder oracle against library routines it does
not call (torch's weight_norm, conv1d, LayerNorm, LeakyReLU and LSTM with
packed sequences) and against invariants of its definition."""
import numpy as np
import pytest
import torch

import synth
from oracle import text_encoder as te

T = synth.TEXT
TT = synth.TEXT_TINY


def _tw(cfg, seed=None, dtype="f64"):
    w = synth.make_text_weights(cfg) if seed is None else synth.make_text_weights(cfg, seed)
    return w, te.prepare_text_weights(w, cfg, dtype)


def test_weight_norm_matches_torch():
    w, _ = _tw(TT, seed=3)
    conv = torch.nn.Conv1d(TT.channels, TT.channels, TT.kernel).double()
    conv = torch.nn.utils.parametrizations.weight_norm(conv, dim=0)
    with torch.no_grad():
        conv.parametrizations.weight.original0.copy_(
            torch.from_numpy(w["conv0.g"].astype(np.float64)).view(-1, 1, 1))
        conv.parametrizations.weight.original1.copy_(torch.from_numpy(w["conv0.v"].astype(np.float64)))
    ref = conv.weight.detach().numpy()
    got = te.weight_norm(w["conv0.v"], w["conv0.g"])
    assert np.max(np.abs(got - ref)) < 1e-14
    # each output channel's effective weight has norm g
    assert np.allclose(np.sqrt((got ** 2).sum(axis=(1, 2))), w["conv0.g"], rtol=1e-12)


def test_conv1d_same_matches_torch():
    rng = np.random.default_rng(1)
    for L, K in ((1, 5), (2, 5), (9, 5), (7, 3)):
        x = rng.normal(0, 1, (L, 6))
        w = rng.normal(0, 1, (4, 6, K))
        b = rng.normal(0, 1, 4)
        ref = torch.nn.functional.conv1d(torch.from_numpy(x.T[None]), torch.from_numpy(w),
                                         torch.from_numpy(b), padding=K // 2)[0].numpy().T
        assert np.max(np.abs(te.conv1d_same(x, w, b) - ref)) < 1e-12


def test_lstm_matches_torch_both_directions():
    rng = np.random.default_rng(2)
    I, H, L = 5, 4, 7
    m = torch.nn.LSTM(I, H, batch_first=True, bidirectional=True).double()
    x = rng.normal(0, 1, (L, I))
    with torch.no_grad():
        ref = m(torch.from_numpy(x[None]))[0][0].numpy()
    p = {k: v.detach().numpy() for k, v in m.named_parameters()}
    fwd = te.lstm(x, p["weight_ih_l0"], p["weight_hh_l0"], p["bias_ih_l0"], p["bias_hh_l0"])
    bwd = te.lstm(x, p["weight_ih_l0_reverse"], p["weight_hh_l0_reverse"], p["bias_ih_l0_reverse"],
                  p["bias_hh_l0_reverse"], reverse=True)
    assert np.max(np.abs(np.concatenate([fwd, bwd], 1) - ref)) < 1e-13


def _torch_text_encoder(w, cfg):
    """The same architecture assembled from torch modules (weight-normed
    Conv1d, LayerNorm over channels, LeakyReLU, packed bidirectional LSTM)."""
    C = cfg.channels
    emb = torch.nn.Embedding(cfg.vocab, C).double()
    convs, lns = [], []
    for i in range(cfg.n_conv):
        c = torch.nn.utils.parametrizations.weight_norm(
            torch.nn.Conv1d(C, C, cfg.kernel, padding=cfg.kernel // 2).double(), dim=0)
        ln = torch.nn.LayerNorm(C, eps=cfg.ln_eps).double()
        with torch.no_grad():
            c.parametrizations.weight.original0.copy_(
                torch.from_numpy(w[f"conv{i}.g"].astype(np.float64)).view(-1, 1, 1))
            c.parametrizations.weight.original1.copy_(torch.from_numpy(w[f"conv{i}.v"].astype(np.float64)))
            c.bias.copy_(torch.from_numpy(w[f"conv{i}.b"].astype(np.float64)))
            ln.weight.copy_(torch.from_numpy(w[f"conv{i}.ln.g"].astype(np.float64)))
            ln.bias.copy_(torch.from_numpy(w[f"conv{i}.ln.b"].astype(np.float64)))
        convs.append(c)
        lns.append(ln)
    lstm = torch.nn.LSTM(C, cfg.hidden, batch_first=True, bidirectional=True).double()
    with torch.no_grad():
        emb.weight.copy_(torch.from_numpy(w["emb"].astype(np.float64)))
        for d, suf in (("fwd", ""), ("bwd", "_reverse")):
            for k, hk in (("w_ih", "weight_ih_l0"), ("w_hh", "weight_hh_l0"),
                          ("b_ih", "bias_ih_l0"), ("b_hh", "bias_hh_l0")):
                getattr(lstm, hk + suf).copy_(torch.from_numpy(w[f"lstm.{d}.{k}"].astype(np.float64)))

    def run(ids, lengths):
        ids = torch.from_numpy(ids.astype(np.int64))
        lengths = torch.from_numpy(np.asarray(lengths))
        mask = (torch.arange(ids.shape[1])[None, :] < lengths[:, None]).double()[:, None, :]
        x = emb(ids).transpose(1, 2) * mask             # [B, C, T], pads zero
        for c, ln in zip(convs, lns):
            x = c(x)
            x = torch.nn.functional.leaky_relu(ln(x.transpose(1, 2)), cfg.slope).transpose(1, 2)
            x = x * mask                                  # pads stay zero for the next taps
        packed = torch.nn.utils.rnn.pack_padded_sequence(x.transpose(1, 2), lengths,
                                                         batch_first=True, enforce_sorted=False)
        out, _ = lstm(packed)
        out, _ = torch.nn.utils.rnn.pad_packed_sequence(out, batch_first=True,
                                                        total_length=ids.shape[1])
        return out.detach().numpy()
    return run


@pytest.mark.parametrize("cfg", [TT, T], ids=["tiny", "kokoro"])
def test_text_encoder_matches_torch_assembly(cfg):
    w, TW = _tw(cfg)
    rng = np.random.default_rng(4)
    B, Tn = 3, 12
    ids = rng.integers(0, cfg.vocab, (B, Tn))
    lengths = np.array([12, 5, 1])
    ids[1, 5:] = cfg.vocab - 1     # pad IDs are never read
    with torch.no_grad():
        ref = _torch_text_encoder(w, cfg)(ids, lengths)
    got = te.text_encode(ids, lengths, TW, cfg)
    assert np.max(np.abs(got - ref)) < 1e-11
    assert np.all(got[1, 5:] == 0) and np.all(got[2, 1:] == 0)


def test_reversal_swaps_the_directions():
    """Reversing a sequence and swapping the forward and backward LSTM
    weights reverses the output and swaps its halves (the backward scan
    starts at the sequence's own last token)."""
    w, TW = _tw(TT, seed=9)
    ids = np.array([1, 4, 2, 6, 0, 3])
    sw = dict(TW)
    for k in ("w_ih", "w_hh", "b_ih", "b_hh"):
        sw[f"lstm.fwd.{k}"], sw[f"lstm.bwd.{k}"] = TW[f"lstm.bwd.{k}"], TW[f"lstm.fwd.{k}"]
    # the convolutions must be mirrored too: reverse each kernel's taps
    for i in range(TT.n_conv):
        sw[f"conv{i}.w"] = TW[f"conv{i}.w"][:, :, ::-1]
    a = te.text_encode_sequence(ids, TW, TT)
    b = te.text_encode_sequence(ids[::-1], sw, TT)
    H = TT.hidden
    assert np.max(np.abs(a[::-1, :H] - b[:, H:])) < 1e-13
    assert np.max(np.abs(a[::-1, H:] - b[:, :H])) < 1e-13


def test_text_pad_invariance():
    w, TW = _tw(TT, seed=11)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, TT.vocab, (2, 9))
    a = te.text_encode(ids, [6, 9], TW, TT)
    ids2 = np.concatenate([ids, rng.integers(0, TT.vocab, (2, 4))], axis=1)
    ids2[0, 6:] = 0
    b = te.text_encode(ids2, [6, 9], TW, TT)
    assert np.array_equal(a, b[:, :9])
    assert np.array_equal(te.text_encode_sequence(ids[0, :6], TW, TT), a[0, :6])
