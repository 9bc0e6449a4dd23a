"""The bench's FLOP accounting (host arithmetic, no GPU).

The encoder's algorithmic work per sequence of L tokens, counted here
independently from the architecture ("Inside One Real ALBERT Layer": the
128 -> 768 projection, twelve executions of one layer with Q/K/V, 12 heads of
64, output projection, FFN 768 -> 2048 -> 768, then the 768 -> 512 output),
must equal the bench's seq_flops, and the per-kernel figures the roofline
divides by must add up to it over one step's launches, with the fused or the
separate Q|K|V and attention kernels.
"""
import numpy as np
import pytest

import bench

H, E, F, O, HEADS, DH, ITERS = 768, 128, 2048, 512, 12, 64, 12


def arch_flops(L: int) -> float:
    per_token = 2 * E * H + 2 * H * O  # input and output projections
    per_token += ITERS * (2 * H * 3 * H + 2 * H * H + 2 * H * F + 2 * F * H)
    per_seq_attention = ITERS * HEADS * (2 * L * L * DH + 2 * L * L * DH)  # q k^T and p v
    return float(per_token * L + per_seq_attention)


@pytest.mark.parametrize("L", [1, 36, 128, 257, 512])
def test_seq_flops_matches_the_architecture(L):
    assert bench.seq_flops(np.array([L])) == arch_flops(L)


@pytest.mark.parametrize("fused", [True, False])
def test_kernel_flops_add_up_to_one_step(fused):
    rng = np.random.default_rng(5)
    lengths = rng.integers(1, 513, 40)
    per_step = {"embed": 1, "proj": 1, "attn_out_ln": ITERS, "ffn1_gelu": ITERS,
                "ffn2_ln": ITERS, "out": 1}
    per_step.update({"qkv_attn": ITERS} if fused else {"qkv": ITERS, "attn": ITERS})
    total = sum(bench.kernel_flops(k, lengths) * n for k, n in per_step.items())
    assert total == pytest.approx(bench.seq_flops(lengths), rel=1e-12)
    assert bench.seq_flops(lengths) == pytest.approx(sum(arch_flops(int(L)) for L in lengths), rel=1e-12)
