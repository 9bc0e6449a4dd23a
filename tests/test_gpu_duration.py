"""GPU parity of length regulation (durations and frame expansion) against
the oracle.  Expansion copies values, so it is compared bit for bit."""
import json
import os

import numpy as np
import pytest

import oracle

from _gpu import dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle_expand(feat, dur, cu):
    parts, cu_f = [], [0]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        rows, A = oracle.expand_durations(feat[a:b], dur[a:b])
        parts.append(rows)
        cu_f.append(cu_f[-1] + A)
    return np.concatenate(parts), np.array(cu_f, np.int32)


def test_toy_from_page():
    import albert_transformer_amd as A
    g = json.load(open(os.path.join(GOLDEN, "duration_toy.json")))
    # p1, p2, p3 as three distinct feature rows
    feat = np.stack([np.full(8, k + 1.0, np.float32) for k in range(3)])
    out, cuf = A.expand(dev(feat), dev(np.array(g["durations"], np.int32)),
                        dev(np.array([0, 3], np.int32)), max_frames=16)
    got = out.cpu().numpy()
    names = {1.0: "p1", 2.0: "p2", 3.0: "p3"}
    assert [names[float(r[0])] for r in got] == g["aligned"]
    assert cuf.cpu().numpy().tolist() == [0, g["frames"]]


@pytest.mark.parametrize("seed,n,C", [(1, 1, 4), (2, 7, 512), (3, 300, 512), (4, 40, 132)])
def test_random_packed_expansion_bitexact(seed, n, C):
    import torch
    import albert_transformer_amd as A
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 200, n)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    feat = rng.normal(0, 1, (total, C)).astype(np.float32)
    dur = rng.integers(1, 9, total).astype(np.int32)
    ref, ref_cu = _oracle_expand(feat, dur, cu)
    max_frames = len(ref) + 5
    out = torch.full((max_frames, C), -3.0, device="cuda")
    cuf = torch.full((n + 1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(A.expand_workspace_bytes(total), dtype=torch.uint8, device="cuda")
    assert A.expand_raw(dev(feat), dev(dur), dev(cu), max_frames, out, cuf, ws) == 0
    got = out.cpu().numpy()
    assert np.array_equal(cuf.cpu().numpy(), ref_cu)
    assert np.array_equal(got[: len(ref)], ref)
    assert np.all(got[len(ref):] == -3.0)  # rows past A untouched


def test_expansion_rejections_leave_outputs_untouched():
    import torch
    import albert_transformer_amd as A
    feat = np.ones((10, 8), np.float32)
    cu = np.array([0, 4, 10], np.int32)
    ws = torch.empty(A.expand_workspace_bytes(10), dtype=torch.uint8, device="cuda")
    canary = torch.full((40, 8), 9.0, device="cuda")
    cu_canary = torch.full((3,), 77, dtype=torch.int32, device="cuda")

    def call(d, c, max_frames=40):
        out, cuf = canary.clone(), cu_canary.clone()
        rc = A.expand_raw(dev(feat), dev(np.asarray(d, np.int32)), dev(np.asarray(c, np.int32)),
                          max_frames, out, cuf, ws)
        assert torch.equal(out, canary) and torch.equal(cuf, cu_canary)
        return rc

    assert call([1] * 9 + [0], cu) == A.E_LENGTH          # a zero duration
    assert call([1] * 9 + [-2], cu) == A.E_LENGTH         # a negative duration
    assert call([5] * 10, cu) == A.E_LENGTH               # 50 frames > 40
    assert call([1] * 10, [0, 4, 9]) == A.E_LENGTH        # cu[n] != total
    assert call([1] * 10, [0, 0, 10]) == A.E_LENGTH       # empty sequence


def test_expansion_exact_fit():
    import albert_transformer_amd as A
    feat = np.arange(40, dtype=np.float32).reshape(10, 4)
    out, cuf = A.expand(dev(feat), dev(np.full(10, 4, np.int32)), dev(np.array([0, 4, 10], np.int32)),
                        max_frames=40)
    assert cuf.cpu().numpy().tolist() == [0, 16, 40]
    assert np.array_equal(out.cpu().numpy(), np.repeat(feat, 4, axis=0))


def test_durations_rule():
    import albert_transformer_amd as A
    rng = np.random.default_rng(9)
    for total, K, speed in ((1, 1, 1.0), (1000, 50, 1.0), (777, 7, 0.8), (300, 64, 1.7)):
        logits = rng.normal(0, 3, (total, K)).astype(np.float32)
        got = A.durations(dev(logits), speed).cpu().numpy()
        ref = oracle.duration_from_logits(logits.astype(np.float64), speed)
        s = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).sum(-1) / speed
        near_tie = np.abs(s - np.floor(s) - 0.5) < 1e-3
        assert np.all(got >= 1)
        assert np.array_equal(got[~near_tie], ref[~near_tie])
        # at a near-tie either neighbour is a correct rounding
        ok = (got[near_tie] == np.maximum(np.floor(s[near_tie]), 1)) | \
             (got[near_tie] == np.maximum(np.ceil(s[near_tie]), 1))
        assert np.all(ok)


def test_expansion_full_size():
    """The encoder's packed output shape (the long packed workload, 63k
    tokens x 512) expanded by seeded durations; every row checked."""
    import albert_transformer_amd as A
    import synth
    wl = synth.make_workload(5)
    rng = np.random.default_rng(55)
    feat = rng.normal(0, 0.5, (wl.tokens, 512)).astype(np.float32)
    d = rng.integers(1, 9, wl.tokens).astype(np.int32)
    ref, ref_cu = _oracle_expand(feat, d, wl.cu_seqlens)
    out, cuf = A.expand(dev(feat), dev(d), dev(wl.cu_seqlens), max_frames=len(ref))
    assert np.array_equal(cuf.cpu().numpy(), ref_cu)
    assert np.array_equal(out.cpu().numpy(), ref)
