"""Shared helpers for the GPU parity tests (imported only by GPU tests)."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

BF16_MAX_ABS = 3e-2     # bf16 path vs the float64 oracle, max |error|
BF16_MIN_COS = 0.999    # bf16 path vs the oracle, per-token cosine
F32_MAX_ABS = 1e-4      # fp32 debug path vs the oracle, max |error|


@functools.lru_cache(maxsize=None)
def weights32():
    return synth.make_weights()


@functools.lru_cache(maxsize=None)
def oracle_weights(dtype: str):
    return oracle.prepare_weights(weights32(), dtype)


_ENC = {}


def encoder(dtype: str, **cfg):
    import albert_transformer_amd as A
    key = (dtype, tuple(sorted(cfg.items())))
    if key not in _ENC:
        _ENC[key] = A.Encoder(weights32(), dtype, **cfg)
    return _ENC[key]


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def read_tap(enc, ws, n_seq, max_rows, name, rows):
    """Copy a workspace checkpoint to host as float64 [rows, stride] (or int)."""
    import torch
    off, nb, stride = enc.tap(n_seq, max_rows, name)
    raw = ws[off:off + nb]
    if stride == 0:
        return raw.view(torch.int32).cpu().numpy()
    t = raw.view(torch.bfloat16 if enc.dtype == "bf16" else torch.float32)
    return t.view(-1, stride)[:rows].float().cpu().numpy().astype(np.float64)


def row_cosines(got, ref):
    num = (got * ref).sum(-1)
    den = np.linalg.norm(got, axis=-1) * np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def check(got, ref, dtype: str, what: str = ""):
    """Assert the tolerance of the path; return (max_abs, min_cos)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    cos = float(np.min(row_cosines(got.reshape(-1, got.shape[-1]),
                                   ref.reshape(-1, ref.shape[-1])))) if got.size else 1.0
    print(f"[parity] {what} dtype={dtype} max_abs={err:.3e} min_cos={cos:.6f}", flush=True)
    if dtype == "bf16":
        assert err <= BF16_MAX_ABS, f"{what}: max abs {err}"
        assert cos >= BF16_MIN_COS, f"{what}: min cosine {cos}"
    else:
        assert err <= F32_MAX_ABS, f"{what}: max abs {err}"
    return err, cos
