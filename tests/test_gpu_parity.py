"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Tolerances: bf16 path max |error| <= 3e-2 and per-token cosine >= 0.999;
fp32 debug path max |error| <= 1e-4; integer bookkeeping bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check, dev, encoder, oracle_weights, read_tap

pytestmark = pytest.mark.gpu
K = synth.KOKORO


def _expected_rows(lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    row_seq = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    row_pos = np.concatenate([np.arange(L) for L in lengths]).astype(np.int32)
    return cu, row_seq, row_pos


def _run_padded(enc, wl, flags=0):
    import torch
    ids, lens = dev(wl.ids), dev(wl.lengths)
    B, T = wl.ids.shape
    ws = enc.new_workspace(B, B * T)
    out = torch.full((B, T, K.out_dim), float("nan"), device="cuda")
    rc = enc.encode_raw(ids, lens, out, ws, flags=flags)
    assert rc == 0, rc
    return out.cpu().numpy().astype(np.float64), ws


@pytest.mark.parametrize("dtype,fused", [("f32", False), ("bf16", False), ("bf16", True)])
def test_stage_checkpoints_one_execution(dtype, fused):
    """Checkpoints in graph order with one execution of the layer: integer
    bookkeeping, embedding LN, Q|K|V (unfused sequence only), attention
    context, both LayerNorms, GELU, output."""
    import albert_transformer_amd as A
    enc = encoder(dtype, n_iter=1)
    W = oracle_weights(dtype)
    wl = synth.random_padded(31, B=3, T=70, lo=1, hi=70)
    wl.lengths[:] = [70, 33, 1]
    out, ws = _run_padded(enc, wl, flags=0 if fused else A.UNFUSED)
    B, T = wl.ids.shape
    rows = int(wl.lengths.sum())
    cu, row_seq, row_pos = _expected_rows(wl.lengths)
    assert np.array_equal(read_tap(enc, ws, B, B * T, "cu", 0)[:B + 1], cu)
    assert np.array_equal(read_tap(enc, ws, B, B * T, "row_seq", 0)[:rows], row_seq)
    assert np.array_equal(read_tap(enc, ws, B, B * T, "row_pos", 0)[:rows], row_pos)
    assert read_tap(enc, ws, B, B * T, "status", 0)[0] == 0
    taps = {n: read_tap(enc, ws, B, B * T, n, rows) for n in ("emb", "qkv", "ctx", "x1", "g", "x")}
    for b in range(B):
        L = int(wl.lengths[b])
        sl = slice(int(cu[b]), int(cu[b + 1]))
        t = {}
        ref = oracle.encode_sequence(wl.ids[b, :L], W, K, n_iter=1, taps=t)
        it = t["iter0"]
        check(taps["emb"][sl], t["emb"], dtype, f"seq{b} emb")
        if not fused:
            qkv = np.concatenate([it["q"] / 8.0, it["k"], it["v"]], axis=1)
            check(taps["qkv"][sl], qkv, dtype, f"seq{b} qkv")
        check(taps["ctx"][sl], it["ctx"], dtype, f"seq{b} ctx")
        check(taps["x1"][sl], it["h1"], dtype, f"seq{b} x1")
        check(taps["g"][sl], it["g"], dtype, f"seq{b} gelu")
        check(taps["x"][sl], it["out"], dtype, f"seq{b} layer out")
        check(out[b, :L], ref, dtype, f"seq{b} out")
        assert np.all(out[b, L:] == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_executions_is_projection_chain(dtype):
    enc = encoder(dtype, n_iter=0)
    W = oracle_weights(dtype)
    wl = synth.random_padded(32, B=2, T=40, lo=1, hi=40)
    out, _ = _run_padded(enc, wl)
    for b in range(2):
        L = int(wl.lengths[b])
        check(out[b, :L], oracle.encode_sequence(wl.ids[b, :L], W, K, n_iter=0), dtype,
              f"n_iter=0 seq{b}")


def test_single_utterance_t36_fp32():
    wl = synth.make_workload(1)
    enc = encoder("f32")
    out, _ = _run_padded(enc, wl)
    ref = oracle.encode(wl.ids, wl.lengths, oracle_weights("f32"), K)
    check(out, ref, "f32", "single utterance B=1 T=36")


def test_fp32_ragged_batch():
    enc = encoder("f32")
    wl = synth.random_padded(33, B=4, T=150, lo=1, hi=150)
    wl.lengths[:] = [150, 37, 129, 1]
    out, _ = _run_padded(enc, wl)
    ref = oracle.encode(wl.ids, wl.lengths, oracle_weights("f32"), K)
    check(out, ref, "f32", "fp32 ragged")


def test_bf16_ragged_tails_packed():
    """Lengths around the 32-key block, the 128-query tile and the 256-row
    GEMM tile boundaries, the longest sequence, and a single token."""
    import torch
    lengths = [1, 31, 32, 33, 127, 128, 129, 257, 512]
    wl = synth.random_packed(34, lengths)
    enc = encoder("bf16")
    out = torch.full((wl.tokens, K.out_dim), float("nan"), device="cuda")
    ws = enc.new_workspace(len(lengths), wl.tokens)
    rc = enc.encode_varlen_raw(dev(wl.ids), dev(wl.cu_seqlens), 512, out, ws)
    assert rc == 0
    ref = oracle.encode_varlen(wl.ids, wl.cu_seqlens, oracle_weights("bf16"), K)
    check(out.cpu().numpy(), ref, "bf16", "packed ragged tails")


def _sample(lengths, k, rng):
    order = np.argsort(lengths)
    pick = {int(order[0]), int(order[-1])}
    while len(pick) < min(k, len(lengths)):
        pick.add(int(rng.integers(0, len(lengths))))
    return sorted(pick)


@pytest.mark.parametrize("k,nsample", [(2, 64), (3, 32), (4, 32), (5, 64)])
def test_full_size_configs_sampled(k, nsample):
    """The bench's launch at full size; the oracle checks sampled sequences
    (the longest, the shortest and random others: every sequence of the
    B=64 and B=32 workloads, 32 of the 256 full-length ones, 64 of the 1,024
    packed ones)."""
    import torch
    wl = synth.make_workload(k)
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    rng = np.random.default_rng(500 + k)
    seqs = _sample(wl.lengths, nsample, rng)
    if wl.packed:
        out = torch.full((wl.tokens, K.out_dim), float("nan"), device="cuda")
        ws = enc.new_workspace(wl.n_seq, wl.tokens)
        rc = enc.encode_varlen_raw(dev(wl.ids), dev(wl.cu_seqlens), wl.T, out, ws)
        assert rc == 0
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        ref = oracle.encode_varlen(wl.ids, wl.cu_seqlens, W, K, seqs=seqs)
        cu = wl.cu_seqlens
        for s in seqs:
            check(got[cu[s]:cu[s + 1]], ref[cu[s]:cu[s + 1]], "bf16", f"{wl.name} seq{s}")
    else:
        got, _ = _run_padded(enc, wl)
        assert np.all(np.isfinite(got))
        ref = oracle.encode(wl.ids, wl.lengths, W, K, seqs=seqs)
        for s in seqs:
            L = int(wl.lengths[s])
            check(got[s, :L], ref[s, :L], "bf16", f"{wl.name} seq{s}")
        pad = np.arange(wl.T)[None, :] >= wl.lengths[:, None]
        assert np.all(got[pad] == 0.0)


def test_packed_equals_padded_bitwise():
    """Every row is computed independently of the others apart from its own
    sequence's keys, so the same sequences give identical bits whether they
    arrive padded or packed."""
    import torch
    enc = encoder("bf16")
    wl = synth.random_padded(35, B=6, T=200, lo=1, hi=200)
    out_pad, _ = _run_padded(enc, wl)
    packed = np.concatenate([wl.ids[b, :L] for b, L in enumerate(wl.lengths)]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(wl.lengths)]).astype(np.int32)
    out = torch.empty((int(cu[-1]), K.out_dim), device="cuda")
    ws = enc.new_workspace(6, int(cu[-1]))
    assert enc.encode_varlen_raw(dev(packed), dev(cu), 200, out, ws) == 0
    got = out.cpu().numpy()
    for b, L in enumerate(wl.lengths):
        assert np.array_equal(got[cu[b]:cu[b + 1]], out_pad[b, :L].astype(np.float32))


def test_pad_slots_and_more_padding_do_not_change_real_tokens():
    """Pad-slot contents never matter (bit for bit).  More padding (a larger
    T) is bit-for-bit invisible to the separate Q|K|V and attention kernels
    as long as the request stays on the same side of the split-K boundary
    (at most 256 token rows B*T: products split over K; more: one pass),
    which changes the products' summation order: across it the outputs agree
    to the bf16 tolerance.  The fused kernel groups 256 // T sequences per
    tile, so a larger T can regroup them and reorder the softmax's rounding:
    there the outputs agree to the bf16 tolerance as well."""
    import albert_transformer_amd as A
    enc = encoder("bf16")
    for B, T, T_more, T_split in ((3, 64, 164, 80), (5, 64, 164, None)):
        wl = synth.random_padded(36, B=B, T=T, lo=5, hi=60)
        wl2 = synth.Workload(wl.name, wl.dtype, wl.ids.copy(), wl.lengths, wl.T)
        for b, L in enumerate(wl.lengths):
            wl2.ids[b, L:] = 999  # pad slots are never read, even out of range
        more = []
        for T2 in (T_more, T_split):
            if T2 is None:
                continue
            ids3 = np.concatenate([wl.ids, np.zeros((B, T2 - T), np.int32)], axis=1)
            more.append(synth.Workload(wl.name, wl.dtype, ids3, wl.lengths, T2))
        for flags in (0, A.UNFUSED):
            a, _ = _run_padded(enc, wl, flags)
            b_, _ = _run_padded(enc, wl2, flags)
            for b, L in enumerate(wl.lengths):
                assert np.array_equal(a[b, :L], b_[b, :L])
            for wl3 in more:
                c, _ = _run_padded(enc, wl3, flags)
                same_side = (B * T <= 256) == (B * wl3.T <= 256)
                for b, L in enumerate(wl.lengths):
                    if flags and same_side:
                        assert np.array_equal(a[b, :L], c[b, :L]), (B, wl3.T, b)
                    else:
                        check(c[b, :L], a[b, :L], "bf16", f"T={wl3.T} vs T={T} seq{b}")


def test_determinism_and_no_carry_over():
    """Bitwise-identical repeats, and a different request in between leaves
    no state behind (second request with a different length)."""
    enc = encoder("bf16")
    wa = synth.random_padded(37, B=5, T=90)
    wb = synth.random_padded(38, B=9, T=300)
    a1, _ = _run_padded(enc, wa)
    _run_padded(enc, wb)
    a2, _ = _run_padded(enc, wa)
    assert np.array_equal(a1, a2)


def test_repeated_ids():
    enc = encoder("bf16")
    ids = np.full((2, 50), 7, np.int32)
    lengths = np.array([50, 20], np.int32)
    wl = synth.Workload("repeated ids", "bf16", ids, lengths, 50)
    out, _ = _run_padded(enc, wl)
    ref = oracle.encode(ids, lengths, oracle_weights("bf16"), K)
    check(out[0, :50], ref[0, :50], "bf16", "repeated ids 50")
    check(out[1, :20], ref[1, :20], "bf16", "repeated ids 20")


def test_rejections_leave_output_untouched():
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    B, T = 3, 32
    ids = np.ones((B, T), np.int32)
    lengths = np.array([32, 10, 5], np.int32)
    ws = enc.new_workspace(B, B * T)
    canary = torch.full((B, T, K.out_dim), 12345.0, device="cuda")

    def call(i, l, **kw):
        out = canary.clone()
        rc = enc.encode_raw(dev(i), dev(l), out, ws, **kw)
        assert torch.equal(out, canary), "output changed on a rejected request"
        return rc

    bad_id = ids.copy()
    bad_id[1, 9] = 178
    assert call(bad_id, lengths) == A.E_ID
    bad_id[1, 9] = -1
    assert call(bad_id, lengths) == A.E_ID
    assert call(ids, np.array([32, 0, 5], np.int32)) == A.E_LENGTH
    assert call(ids, np.array([33, 1, 5], np.int32)) == A.E_LENGTH
    need = enc.workspace_bytes(B, B * T)
    assert call(ids, lengths, ws_bytes=need - 1) == A.E_WORKSPACE
    # an id beyond the length is a pad slot: accepted
    ok_ids = ids.copy()
    ok_ids[2, 7] = 5000
    out = canary.clone()
    assert enc.encode_raw(dev(ok_ids), dev(lengths), out, ws) == 0
    # aliasing: output inside the workspace
    wsv = ws[: B * T * K.out_dim * 4].view(torch.float32)
    assert lib_encode_alias(enc, ids, lengths, wsv, ws) == A.E_ALIAS
    # T beyond the position table
    big = np.ones((1, 513), np.int32)
    out2 = torch.empty((1, 513, K.out_dim), device="cuda")
    ws2 = enc.new_workspace(1, 513)
    assert enc.encode_raw(dev(big), dev(np.array([513], np.int32)), out2, ws2) == A.E_ARG
    # the context is still usable
    assert enc.encode_raw(dev(ids), dev(lengths), out, ws) == 0


def lib_encode_alias(enc, ids, lengths, out_view, ws):
    return enc.encode_raw(dev(ids), dev(lengths), out_view, ws)


def test_packed_rejections():
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    ids = np.ones(40, np.int32)
    ws = enc.new_workspace(3, 40)
    canary = torch.full((40, K.out_dim), -7.0, device="cuda")
    for cu, max_len, code in (([0, 10, 10, 40], 40, A.E_LENGTH),   # empty sequence
                              ([0, 10, 25, 39], 40, A.E_LENGTH),   # cu[n] != total
                              ([1, 10, 25, 40], 40, A.E_LENGTH),   # cu[0] != 0
                              ([0, 10, 25, 40], 12, A.E_LENGTH)):  # longer than max_len
        out = canary.clone()
        rc = enc.encode_varlen_raw(dev(ids), dev(np.array(cu, np.int32)), max_len, out, ws)
        assert rc == code, (cu, rc)
        assert torch.equal(out, canary)
    bad = ids.copy()
    bad[39] = 178
    out = canary.clone()
    assert enc.encode_varlen_raw(dev(bad), dev(np.array([0, 10, 25, 40], np.int32)), 40,
                                 out, ws) == A.E_ID
    assert torch.equal(out, canary)


def test_async_flag_and_empty_batch():
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    wl = synth.random_padded(39, B=2, T=16)
    ws = enc.new_workspace(2, 32)
    out = torch.empty((2, 16, K.out_dim), device="cuda")
    assert enc.encode_raw(dev(wl.ids), dev(wl.lengths), out, ws, flags=A.ASYNC) == 0
    assert A.read_status(ws) == 0
    bad = wl.ids.copy()
    bad[0, 0] = 400
    assert enc.encode_raw(dev(bad), dev(wl.lengths), out, ws, flags=A.ASYNC) == 0
    assert A.read_status(ws) == A.E_ID
    empty = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    assert enc.encode_raw(empty, torch.empty(0, dtype=torch.int32, device="cuda"), out, ws) == 0


def test_fused_equals_unfused_on_aligned_groups():
    """Full-length sequences of 128 tokens: the fused Q|K|V + attention kernel
    and the separate kernels do the same arithmetic in the same order (the
    same K slices, 32-key blocks from each sequence's start), so the outputs
    are identical bit for bit."""
    import albert_transformer_amd as A
    enc = encoder("bf16")
    wl = synth.random_padded(61, B=12, T=128, lo=128, hi=128)
    a, _ = _run_padded(enc, wl)
    b, _ = _run_padded(enc, wl, flags=A.UNFUSED)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,lo,hi,seed", [(36, 1, 36, 62), (100, 1, 100, 63), (200, 1, 200, 64),
                                          (256, 200, 256, 65), (129, 129, 129, 66)])
def test_fused_groups_vs_oracle(T, lo, hi, seed):
    """Groups of S = 256 // T whole sequences per workgroup (7, 2, 1, 1, 1),
    ragged lengths so sequences start anywhere in a group's tile; sampled
    sequences against the oracle."""
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    wl = synth.random_padded(seed, B=23, T=T, lo=lo, hi=hi)
    wl.lengths[0] = hi
    wl.lengths[1] = lo
    out, _ = _run_padded(enc, wl)
    for b in (0, 1, 7, 22):
        L = int(wl.lengths[b])
        check(out[b, :L], oracle.encode_sequence(wl.ids[b, :L], W, K), "bf16", f"fused T={T} seq{b}")


@pytest.mark.parametrize("max_len,n", [(1, 300), (60, 40)])
def test_fused_packed_short_sequences(max_len, n):
    """Packed batches of short sequences: S = 256 (one-token sequences) and
    S = 4 per group."""
    import torch
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    rng = np.random.default_rng(67 + max_len)
    lengths = rng.integers(1, max_len + 1, n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ids = rng.integers(0, 178, int(cu[-1])).astype(np.int32)
    out = torch.full((int(cu[-1]), 512), float("nan"), device="cuda")
    ws = enc.new_workspace(n, int(cu[-1]))
    assert enc.encode_varlen_raw(dev(ids), dev(cu), max_len, out, ws) == 0
    got = out.cpu().numpy().astype(np.float64)
    for s in (0, 1, n // 2, n - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        check(got[a:b], oracle.encode_sequence(ids[a:b], W, K), "bf16", f"fused packed L<={max_len} seq{s}")


def test_attention_grids_agree_bitwise():
    """The unfused attention runs on packed 128-row query blocks when the
    mean length is under 128 and on per-sequence query tiles otherwise.
    A lane sees its own sequence's keys in the same 32-key blocks either
    way, so the same sequences give the same bits: packed (mean < 128, a
    block may hold several whole sequences and parts of two more) against
    padded to T=256 (256 rows per sequence: per-sequence tiles).  Sampled
    sequences also against the oracle."""
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    rng = np.random.default_rng(68)
    lengths = rng.integers(1, 200, 45).astype(np.int32)
    lengths[:6] = [1, 256, 2, 129, 128, 255]
    n = len(lengths)
    assert lengths.sum() < n * 128
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ids = rng.integers(0, 178, int(cu[-1])).astype(np.int32)
    out = torch.full((int(cu[-1]), 512), float("nan"), device="cuda")
    ws = enc.new_workspace(n, int(cu[-1]))
    assert enc.encode_varlen_raw(dev(ids), dev(cu), 256, out, ws, flags=A.UNFUSED) == 0
    got = out.cpu().numpy()
    padded = np.zeros((n, 256), np.int32)
    for s in range(n):
        padded[s, :lengths[s]] = ids[cu[s]:cu[s + 1]]
    wl = synth.Workload("grids", "bf16", padded, lengths, 256)
    out_pad, _ = _run_padded(enc, wl, flags=A.UNFUSED)
    for s in range(n):
        assert np.array_equal(got[cu[s]:cu[s + 1]], out_pad[s, :lengths[s]].astype(np.float32)), s
    for s in (0, 1, 3, n - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        check(got[a:b].astype(np.float64), oracle.encode_sequence(ids[a:b], W, K), "bf16",
              f"packed attention blocks seq{s}")


@pytest.mark.parametrize("B,T,seed", [(6, 200, 71), (256, 128, 72)])
def test_layernorm_pair_handoff(B, T, seed):
    """bf16 LayerNorm products split each 768-wide row tile between two
    workgroups that swap row statistics.  ALBERT_LN_HANDOFF stops them from
    waiting for each other, so in every row tile one half hands its rows
    over (its fp32 values before normalisation) and the other normalises
    both: the fallback for a partner that is late or not resident.  Outputs
    equal the default run bit for bit (the same values, statistics and
    arithmetic, whichever block normalises them) and, on sampled sequences,
    match the oracle.  B=6 runs 128-row tiles, B=256 x T=128 256-row
    tiles."""
    import albert_transformer_amd as A
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    wl = synth.random_padded(seed, B=B, T=T, lo=1, hi=T)
    wl.lengths[0] = T
    a, _ = _run_padded(enc, wl)
    for rep in range(2):  # which half hands over varies from run to run
        b, _ = _run_padded(enc, wl, flags=A.LN_HANDOFF)
        for s in range(B):
            L = int(wl.lengths[s])
            check(b[s, :L], a[s, :L], "bf16", f"handoff vs default seq{s} run{rep}")
        assert np.array_equal(a, b), f"handoff run {rep}: bits differ from the default run"
        pad = np.arange(T)[None, :] >= wl.lengths[:, None]
        assert np.all(b[pad] == 0.0)
    for s in (0, B - 1):
        L = int(wl.lengths[s])
        check(b[s, :L], oracle.encode_sequence(wl.ids[s, :L], W, K), "bf16", f"handoff seq{s}")


@pytest.mark.parametrize("n,lo,hi,seed", [(200, 1, 256, 73), (8192, 1, 3, 77), (8193, 1, 3, 78),
                                          (9000, 1, 3, 74)])
def test_fused_group_packing(n, lo, hi, seed):
    """The fused kernel's groups: consecutive sequences packed greedily on
    the device while their rows fit 256 (n = 200, lengths 1..256, so a
    group may hold one long sequence or many short ones; n = 8,192, the
    most the device grouping takes), or, beyond 8,192 sequences, S = 256 /
    longest per group chosen on the host (n = 8,193 and 9,000 of 1..3
    tokens).  Sampled sequences against the oracle, and every
    sequence against the separate kernels' run."""
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, n).astype(np.int32)
    lengths[0] = hi
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ids = rng.integers(0, 178, int(cu[-1])).astype(np.int32)
    outs = []
    for flags in (0, A.UNFUSED):
        out = torch.full((int(cu[-1]), 512), float("nan"), device="cuda")
        ws = enc.new_workspace(n, int(cu[-1]))
        assert enc.encode_varlen_raw(dev(ids), dev(cu), hi, out, ws, flags=flags) == 0
        outs.append(out.cpu().numpy().astype(np.float64))
    check(outs[0], outs[1], "bf16", f"fused vs separate n={n}")
    for s in (0, 1, n // 2, n - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        check(outs[0][a:b], oracle.encode_sequence(ids[a:b], W, K), "bf16", f"grouped seq{s}")


def test_concurrent_calls_on_two_streams_match_single_calls():
    """Every per-request state lives in the caller's workspace, so two calls
    with their own workspaces may run at the same time on two streams: each
    output equals, bit for bit, the one its batch gives alone.  (With the
    other call's blocks on the chip a paired LayerNorm block may find its
    partner late and hand its rows over; the partner then normalises the
    same fp32 values with the same statistics, so the bits do not change.)"""
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    batches = [synth.random_padded(81, B=48, T=128, lo=1, hi=128),
               synth.random_padded(82, B=40, T=96, lo=1, hi=96)]
    alone = []
    for wl in batches:
        B, T = wl.ids.shape
        out = torch.full((B, T, 512), float("nan"), device="cuda")
        ws = enc.new_workspace(B, B * T)
        assert enc.encode_raw(dev(wl.ids), dev(wl.lengths), out, ws) == 0
        alone.append(out.cpu().numpy())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, wss, args = [], [], []
    for wl in batches:
        B, T = wl.ids.shape
        outs.append(torch.full((B, T, 512), float("nan"), device="cuda"))
        wss.append(enc.new_workspace(B, B * T))
        args.append((dev(wl.ids), dev(wl.lengths)))
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            assert enc.encode_raw(args[i][0], args[i][1], outs[i], wss[i], stream=streams[i],
                                  flags=A.ASYNC) == 0
        torch.cuda.synchronize()
        for i in range(2):
            assert A.read_status(wss[i]) == A.OK
            T = batches[i].ids.shape[1]
            valid = np.arange(T)[None, :] < batches[i].lengths[:, None]
            got = outs[i].cpu().numpy()
            check(got[valid], alone[i][valid], "bf16", f"concurrent batch {i} repeat {rep}")
            assert np.array_equal(got, alone[i]), f"concurrent batch {i} repeat {rep}: bits differ"
            assert np.all(got[~valid] == 0), "pad slots"


@pytest.mark.parametrize("flags_name", ["fused", "unfused", "handoff"])
def test_poisoned_workspace_ragged_tail(flags_name):
    """The workspace's contents on entry are ignored.  Filled with 0xFF bytes
    (NaN in bf16 and fp32) before a packed call whose last group ends inside
    a 32-row block, the rows past the last token stay stale: products read
    them (the buffer range check does not cover a DMA's row offset), the
    fused attention must not let them reach a valid context (0 times NaN is
    not 0).  Outputs must be finite and match the oracle."""
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    W = oracle_weights("bf16")
    flags = {"fused": 0, "unfused": A.UNFUSED, "handoff": A.LN_HANDOFF}[flags_name]
    rng = np.random.default_rng(91)
    lengths = np.array([100, 90, 37, 5], np.int32)   # 232 rows: one group, ends mid-block
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ids = rng.integers(0, 178, int(cu[-1])).astype(np.int32)
    n, total = len(lengths), int(cu[-1])
    ws = enc.new_workspace(n, total)
    ws.fill_(0xFF)
    for call in range(2):   # the second call reuses the workspace the first wrote
        out = torch.full((total, 512), float("nan"), device="cuda")
        print(f"[poison] {flags_name} call {call}", flush=True)
        assert enc.encode_varlen_raw(dev(ids), dev(cu), 128, out, ws, flags=flags) == 0
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        for s in range(n):
            a, b = int(cu[s]), int(cu[s + 1])
            check(got[a:b], oracle.encode_sequence(ids[a:b], W, K), "bf16",
                  f"poisoned workspace {flags_name} seq{s}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiny_batches_split_k(dtype):
    """Requests of at most 256 token rows run their products split over K
    (partial sums, then a reduce kernel with the epilogue).  The split depends
    on the product only, so padded and packed give the same bits there too,
    and the outputs match the oracle (one utterance of 36 tokens, and three
    short sequences padded to 80)."""
    import torch
    enc = encoder(dtype)
    W = oracle_weights(dtype)
    for seed, B, T in ((140, 1, 36), (141, 3, 80)):
        wl = synth.random_padded(seed, B=B, T=T, lo=1, hi=T)
        wl.lengths[0] = T
        out_pad, _ = _run_padded(enc, wl)
        packed = np.concatenate([wl.ids[b, :L] for b, L in enumerate(wl.lengths)]).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(wl.lengths)]).astype(np.int32)
        out = torch.empty((int(cu[-1]), K.out_dim), device="cuda")
        ws = enc.new_workspace(B, int(cu[-1]))
        assert enc.encode_varlen_raw(dev(packed), dev(cu), T, out, ws) == 0
        got = out.cpu().numpy()
        for b, L in enumerate(wl.lengths):
            assert np.array_equal(got[cu[b]:cu[b + 1]], out_pad[b, :L].astype(np.float32)), (seed, b)
            check(out_pad[b, :L], oracle.encode_sequence(wl.ids[b, :L], W, K), dtype,
                  f"split-K B={B} T={T} seq{b}")
