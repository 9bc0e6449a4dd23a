"""albert_encode_noalloc: the padded entry point on the library's static
device scratch, for callers that cannot allocate.  Checked through the C ABI
against albert_encode with a caller workspace (the same kernels: the same
bits), on two calls in a row, the second smaller, and against the oracle on
sampled sequences; oversized requests and bad IDs are rejected with `out`
unchanged."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check, dev, encoder, oracle_weights

pytestmark = pytest.mark.gpu
K = synth.KOKORO


def _with_workspace(enc, wl):
    import torch
    B, T = wl.ids.shape
    ws = enc.new_workspace(B, B * T)
    out = torch.full((B, T, K.out_dim), float("nan"), device="cuda")
    assert enc.encode_raw(dev(wl.ids), dev(wl.lengths), out, ws) == 0
    return out.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    import torch
    import albert_transformer_amd as A
    enc = encoder(dtype)
    W = oracle_weights(dtype)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    shapes = [(101, 24, 128), (102, 3, 40)] if dtype == "bf16" else [(103, 16, 100), (104, 1, 36)]
    for call, (seed, B, T) in enumerate(shapes):   # the second call is smaller
        wl = synth.random_padded(seed, B=B, T=T, lo=1, hi=T)
        wl.lengths[0] = T
        assert enc.workspace_bytes(B, B * T) <= A.SCRATCH_BYTES
        ref = _with_workspace(enc, wl)
        out = torch.full((B, T, K.out_dim), float("nan"), device="cuda")
        status.fill_(-1)
        print(f"[noalloc] {dtype} call {call} B={B} T={T}", flush=True)
        assert enc.encode_noalloc_raw(dev(wl.ids), dev(wl.lengths), out, status) == A.OK
        torch.cuda.synchronize()
        assert int(status.item()) == A.OK
        got = out.cpu().numpy()
        valid = np.arange(T)[None, :] < wl.lengths[:, None]
        check(got[valid], ref[valid], dtype, f"noalloc vs workspace call {call}")
        assert np.array_equal(got, ref), f"call {call}: bits differ from albert_encode"
        for b in (0, B - 1):
            L = int(wl.lengths[b])
            check(got[b, :L], oracle.encode_sequence(wl.ids[b, :L], W, K), dtype,
                  f"noalloc call {call} seq{b}")


def test_noalloc_rejections_leave_out_unchanged():
    import torch
    import albert_transformer_amd as A
    enc = encoder("bf16")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    # larger than the scratch: refused on the host, nothing enqueued
    B, T = 64, 128
    assert enc.workspace_bytes(B, B * T) > A.SCRATCH_BYTES
    ids = dev(np.ones((B, T), np.int32))
    lens = dev(np.full(B, T, np.int32))
    canary = torch.full((B, T, K.out_dim), 5.0, device="cuda")
    out = canary.clone()
    assert enc.encode_noalloc_raw(ids, lens, out, status) == A.E_SCRATCH
    torch.cuda.synchronize()
    assert torch.equal(out, canary) and int(status.item()) == -1
    # an ID outside the vocabulary: the device status says so, out unchanged
    wl = synth.random_padded(105, B=4, T=50, lo=1, hi=50)
    bad = wl.ids.copy()
    bad[2, 0] = 178
    out = torch.full((4, 50, K.out_dim), 5.0, device="cuda")
    assert enc.encode_noalloc_raw(dev(bad), dev(wl.lengths), out, status) == A.OK
    torch.cuda.synchronize()
    assert int(status.item()) == A.E_ID
    assert torch.all(out == 5.0)
    # the scratch still serves the next request
    ref = _with_workspace(enc, wl)
    out = torch.full((4, 50, K.out_dim), float("nan"), device="cuda")
    assert enc.encode_noalloc_raw(dev(wl.ids), dev(wl.lengths), out, status) == A.OK
    torch.cuda.synchronize()
    assert int(status.item()) == A.OK
    assert np.array_equal(out.cpu().numpy(), ref)
