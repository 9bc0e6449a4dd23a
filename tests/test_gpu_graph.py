"""The encoder's launch sequence captured in a HIP graph and replayed.

Every kernel of a request reads its sizes and pointers from its arguments
and the workspace, and the sequence has no memset nodes (the workspace
clears are kernels), so one captured request can be replayed: each replay,
with other eager requests and synchronisations between replays, must give
the eager result bit for bit.  Small batches are bound by launch overhead,
which replaying a graph removes."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check, dev, encoder, oracle_weights

pytestmark = pytest.mark.gpu
K = synth.KOKORO


@pytest.mark.parametrize("dtype,B,T,noalloc", [("f32", 1, 36, False), ("bf16", 1, 36, False),
                                               ("bf16", 16, 128, False), ("bf16", 16, 128, True)])
def test_graph_replays_equal_eager(dtype, B, T, noalloc):
    import torch
    import albert_transformer_amd as A
    enc = encoder(dtype)
    W = oracle_weights(dtype)
    wl = synth.random_padded(120 + B, B=B, T=T, lo=1, hi=T)
    wl.lengths[0] = T
    ids, lens = dev(wl.ids), dev(wl.lengths)
    out = torch.full((B, T, K.out_dim), float("nan"), device="cuda")
    ws = enc.new_workspace(B, B * T)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        if noalloc:
            return enc.encode_noalloc_raw(ids, lens, out, status)
        return enc.encode_raw(ids, lens, out, ws, flags=A.ASYNC)

    assert step() == A.OK
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    for b in (0, B - 1):
        L = int(wl.lengths[b])
        check(eager[b, :L], oracle.encode_sequence(wl.ids[b, :L], W, K), dtype, f"eager seq{b}")

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            assert step() == A.OK
    torch.cuda.synchronize()
    other = synth.random_padded(130 + B, B=3, T=50, lo=1, hi=50)
    for rep in range(3):
        out.fill_(float("nan"))
        print(f"[graph] {dtype} B={B} T={T} noalloc={noalloc} replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, eager), f"replay {rep}: differs from the eager run"
        if noalloc:
            assert int(status.item()) == A.OK
        else:
            assert A.read_status(ws) == A.OK
        # eager work between replays (another request, on its own workspace)
        enc.encode(dev(other.ids), dev(other.lengths))
        torch.cuda.synchronize()
    del graph
