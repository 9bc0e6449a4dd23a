"""ctypes binding of libalbert.so (the C ABI in include/albert.h).

Argument marshalling only: every step of the encoder runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  The
binding refuses to work without the compiled library -- there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libalbert.so")

OK, E_ARG, E_WORKSPACE, E_LENGTH, E_ID, E_ALIAS, E_HIP, E_SYNC, E_SCRATCH = range(9)
STATUS_NAMES = {OK: "OK", E_ARG: "E_ARG", E_WORKSPACE: "E_WORKSPACE",
                E_LENGTH: "E_LENGTH", E_ID: "E_ID", E_ALIAS: "E_ALIAS", E_HIP: "E_HIP",
                E_SYNC: "E_SYNC", E_SCRATCH: "E_SCRATCH"}
SCRATCH_BYTES = 64 << 20   # ALBERT_SCRATCH_BYTES
F32, BF16, FP8 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8}
ASYNC = 1
UNFUSED = 2
LN_HANDOFF = 4
N_TENSORS = 25
TAPS = {"status": 0, "cu": 1, "row_seq": 2, "row_pos": 3, "emb": 4, "x": 5,
        "qkv": 6, "ctx": 7, "x1": 8, "g": 9, "x8": 10, "x1_8": 11}

EXPORTS = ("albert_default_config", "albert_n_tensors", "albert_tensor_name",
           "albert_tensor_shape", "albert_load_weights", "albert_workspace_bytes", "albert_encode",
           "albert_encode_noalloc",
           "albert_encode_varlen", "albert_encode_features", "albert_read_status", "albert_tap", "albert_free",
           "albert_status_str", "albert_time_kernel", "albert_kernel_time",
           "albert_durations", "albert_expand_workspace_bytes", "albert_expand",
           "albert_text_default_config", "albert_text_n_tensors", "albert_text_tensor_name",
           "albert_text_tensor_shape", "albert_text_load_weights", "albert_text_workspace_bytes",
           "albert_text_encode", "albert_text_encode_varlen", "albert_text_tap",
           "albert_text_time_kernel", "albert_text_kernel_time", "albert_text_free")
TEXT_TAPS = {"status": 0, "cu": 1, "emb": 2, "conv": 3, "xg": 4}
TEXT_KERNEL_KINDS = ("embed", "taps", "conv", "lstm_in", "lstm")
KERNEL_KINDS = ("embed", "proj", "qkv", "attn", "attn_out_ln", "ffn1_gelu", "ffn2_ln", "out",
                "qkv_attn")


class Config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("n_types", ctypes.c_int32), ("emb", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_iter", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("out_dim", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class TextConfig(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("n_conv", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("slope", ctypes.c_float)]


_LIB = None


def lib():
    """Load libalbert.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m albert_transformer_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.albert_default_config.argtypes = [ctypes.POINTER(Config)]
    L.albert_default_config.restype = i32
    L.albert_n_tensors.argtypes = [ctypes.POINTER(Config)]
    L.albert_n_tensors.restype = i32
    L.albert_tensor_name.argtypes = [ctypes.POINTER(Config), i32]
    L.albert_tensor_name.restype = ctypes.c_char_p
    L.albert_tensor_shape.argtypes = [ctypes.POINTER(Config), i32,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.albert_tensor_shape.restype = i32
    L.albert_load_weights.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(Config),
                                      ctypes.POINTER(vp), i32, vp]
    L.albert_load_weights.restype = i32
    L.albert_workspace_bytes.argtypes = [vp, i32, i64]
    L.albert_workspace_bytes.restype = sz
    L.albert_encode.argtypes = [vp, vp, vp, i32, i32, vp, vp, sz, vp, ctypes.c_uint]
    L.albert_encode.restype = i32
    L.albert_encode_noalloc.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, ctypes.c_uint]
    L.albert_encode_noalloc.restype = i32
    L.albert_encode_varlen.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp,
                                       ctypes.c_uint]
    L.albert_encode_varlen.restype = i32
    L.albert_encode_features.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp,
                                         ctypes.c_uint]
    L.albert_encode_features.restype = i32
    L.albert_read_status.argtypes = [vp, vp]
    L.albert_read_status.restype = i32
    L.albert_tap.argtypes = [vp, i32, i64, i32, ctypes.POINTER(sz), ctypes.POINTER(sz),
                             ctypes.POINTER(i64)]
    L.albert_tap.restype = i32
    L.albert_free.argtypes = [vp]
    L.albert_free.restype = None
    L.albert_status_str.argtypes = [i32]
    L.albert_status_str.restype = ctypes.c_char_p
    L.albert_time_kernel.argtypes = [vp, i32, i32]
    L.albert_time_kernel.restype = i32
    L.albert_kernel_time.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
    L.albert_kernel_time.restype = i32
    L.albert_durations.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp]
    L.albert_durations.restype = i32
    L.albert_expand_workspace_bytes.argtypes = [i32]
    L.albert_expand_workspace_bytes.restype = sz
    L.albert_expand.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, vp, vp, sz, vp, ctypes.c_uint]
    L.albert_expand.restype = i32
    tc = ctypes.POINTER(TextConfig)
    L.albert_text_default_config.argtypes = [tc]
    L.albert_text_default_config.restype = i32
    L.albert_text_n_tensors.argtypes = [tc]
    L.albert_text_n_tensors.restype = i32
    L.albert_text_tensor_name.argtypes = [tc, i32]
    L.albert_text_tensor_name.restype = ctypes.c_char_p
    L.albert_text_tensor_shape.argtypes = [tc, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.albert_text_tensor_shape.restype = i32
    L.albert_text_load_weights.argtypes = [ctypes.POINTER(vp), tc, ctypes.POINTER(vp), vp]
    L.albert_text_load_weights.restype = i32
    L.albert_text_workspace_bytes.argtypes = [vp, i32, i64]
    L.albert_text_workspace_bytes.restype = sz
    L.albert_text_encode.argtypes = [vp, vp, vp, i32, i32, vp, vp, sz, vp, ctypes.c_uint]
    L.albert_text_encode.restype = i32
    L.albert_text_encode_varlen.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp,
                                            ctypes.c_uint]
    L.albert_text_encode_varlen.restype = i32
    L.albert_text_tap.argtypes = [vp, i32, i64, i32, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                  ctypes.POINTER(i64)]
    L.albert_text_tap.restype = i32
    L.albert_text_time_kernel.argtypes = [vp, i32, i32]
    L.albert_text_time_kernel.restype = i32
    L.albert_text_kernel_time.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
    L.albert_text_kernel_time.restype = i32
    L.albert_text_free.argtypes = [vp]
    L.albert_text_free.restype = None
    _LIB = L
    return L


def default_config(**overrides) -> Config:
    c = Config()
    lib().albert_default_config(ctypes.byref(c))
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


def status_str(code: int) -> str:
    return lib().albert_status_str(code).decode()


class AlbertError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(code, code)} ({status_str(code)})")
        self.code = code


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _need(t, name: str, dtype=None, numel: int | None = None):
    """Refuse a tensor the library would misread: wrong element type, not on
    the GPU, not contiguous, or fewer elements than the call will touch.
    (The library sees only a pointer, so an int64 ID tensor would be read as
    pairs of int32 values that are all in range.)"""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs {numel}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(int(s.cuda_stream))


class Encoder:
    """One device-resident copy of the encoder weights (an albert_ctx).

    weights: dict of canonical name -> float32 numpy array (see
    ``synth.tensor_names``: with n_groups = G > 1 the layer tensors of set g
    are named "g<g>.<name>"); dtype "bf16", "fp8" (E4M3 matrix-product
    operands) or "f32"; config overrides as keyword arguments (e.g.
    n_iter=1, n_groups=3).
    """

    def __init__(self, weights: dict, dtype: str = "bf16", stream=None, **cfg):
        import torch  # noqa: F401  (HIP runtime shared with torch)
        L = lib()
        self.cfg = default_config(**cfg)
        self.dtype = dtype
        cf = ctypes.byref(self.cfg)
        nt = L.albert_n_tensors(cf)
        if nt < 0:
            raise AlbertError(E_ARG, "albert_n_tensors")
        names = []
        for i in range(nt):
            n = L.albert_tensor_name(cf, i).decode()
            if self.cfg.n_groups > 1 and 7 <= i < 7 + 16 * self.cfg.n_groups:
                n = f"g{(i - 7) // 16}.{n}"
            names.append(n)
        self._host = []
        for i, n in enumerate(names):
            a = np.ascontiguousarray(np.asarray(weights[n], dtype=np.float32))
            r, c = ctypes.c_int64(), ctypes.c_int64()
            rc = L.albert_tensor_shape(cf, i, ctypes.byref(r), ctypes.byref(c))
            if rc != OK:
                raise AlbertError(rc, "albert_tensor_shape")
            if a.size != r.value * c.value:
                raise ValueError(f"{n}: expected {r.value}x{c.value}, got {a.shape}")
            self._host.append(a)
        ptrs = (ctypes.c_void_p * nt)(*[a.ctypes.data for a in self._host])
        h = ctypes.c_void_p()
        rc = L.albert_load_weights(ctypes.byref(h), cf, ptrs, DTYPES[dtype], _stream(stream))
        self._host = None
        if rc != OK:
            raise AlbertError(rc, "albert_load_weights")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().albert_free(self.handle)
            self.handle = None

    __del__ = close

    # -------------------------------------------------------------- sizes --
    def workspace_bytes(self, n_seq: int, max_rows: int) -> int:
        return int(lib().albert_workspace_bytes(self.handle, n_seq, max_rows))

    def tap(self, n_seq: int, max_rows: int, name: str):
        off, nb, st = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
        rc = lib().albert_tap(self.handle, n_seq, max_rows, TAPS[name], ctypes.byref(off),
                              ctypes.byref(nb), ctypes.byref(st))
        if rc != OK:
            raise AlbertError(rc, "albert_tap")
        return off.value, nb.value, st.value

    def time_kernel(self, kind: str | None, max_launches: int = 1024) -> None:
        """Bracket later launches of one kernel kind with HIP events."""
        k = -1 if kind is None else KERNEL_KINDS.index(kind)
        rc = lib().albert_time_kernel(self.handle, k, max_launches)
        if rc != OK:
            raise AlbertError(rc, "albert_time_kernel")

    def kernel_time(self) -> tuple[int, float]:
        """(launches timed, summed milliseconds) since time_kernel()."""
        n, ms = ctypes.c_int(), ctypes.c_double()
        rc = lib().albert_kernel_time(self.handle, ctypes.byref(n), ctypes.byref(ms))
        if rc != OK:
            raise AlbertError(rc, "albert_kernel_time")
        return n.value, ms.value

    def new_workspace(self, n_seq: int, max_rows: int):
        import torch
        return torch.empty(self.workspace_bytes(n_seq, max_rows), dtype=torch.uint8,
                           device="cuda")

    # ------------------------------------------------------------- encode --
    def encode_raw(self, ids, lengths, out, ws, stream=None, flags=0, ws_bytes=None) -> int:
        """Padded call on caller tensors; returns the status code."""
        import torch
        if ids.dim() != 2:
            raise ValueError(f"ids: expected [B, T], got {tuple(ids.shape)}")
        B, T = ids.shape
        _need(ids, "ids", torch.int32)
        _need(lengths, "lengths", torch.int32, B)
        _need(out, "out", torch.float32, B * T * self.cfg.out_dim)
        _need(ws, "ws")
        nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
        return lib().albert_encode(self.handle, _ptr(ids), _ptr(lengths), B, T, _ptr(out),
                                   _ptr(ws), nb, _stream(stream), flags)

    def encode_noalloc_raw(self, ids, lengths, out, status, stream=None, flags=0) -> int:
        """Padded call on the library's static scratch (no workspace); the
        device status lands in status (int32 [1]).  Returns the host status."""
        import torch
        if ids.dim() != 2:
            raise ValueError(f"ids: expected [B, T], got {tuple(ids.shape)}")
        B, T = ids.shape
        _need(ids, "ids", torch.int32)
        _need(lengths, "lengths", torch.int32, B)
        _need(out, "out", torch.float32, B * T * self.cfg.out_dim)
        _need(status, "status", torch.int32, 1)
        return lib().albert_encode_noalloc(self.handle, _ptr(ids), _ptr(lengths), B, T,
                                           _ptr(out), _ptr(status), _stream(stream), flags)

    def encode_varlen_raw(self, ids, cu, max_len, out, ws, stream=None, flags=0,
                          ws_bytes=None, n=None, total=None) -> int:
        import torch
        n = cu.numel() - 1 if n is None else n
        total = ids.numel() if total is None else total
        _need(ids, "ids", torch.int32, total)
        _need(cu, "cu_seqlens", torch.int32, n + 1)
        _need(out, "out", torch.float32, total * self.cfg.out_dim)
        _need(ws, "ws")
        nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
        return lib().albert_encode_varlen(self.handle, _ptr(ids), _ptr(cu), n, total, max_len,
                                          _ptr(out), _ptr(ws), nb, _stream(stream), flags)

    def encode_features_raw(self, x, cu, max_len, out, ws, stream=None, flags=0,
                            ws_bytes=None, n=None, total=None) -> int:
        """Packed call from embedding LayerNorm output x fp32 [total, 128]."""
        import torch
        n = cu.numel() - 1 if n is None else n
        total = x.shape[0] if total is None else total
        _need(x, "x", torch.float32, total * self.cfg.emb)
        _need(cu, "cu_seqlens", torch.int32, n + 1)
        _need(out, "out", torch.float32, total * self.cfg.out_dim)
        _need(ws, "ws")
        nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
        return lib().albert_encode_features(self.handle, _ptr(x), _ptr(cu), n, total, max_len,
                                            _ptr(out), _ptr(ws), nb, _stream(stream), flags)

    def encode_features(self, x, cu, max_len, out=None, ws=None, stream=None):
        """x fp32 [total, 128], cu int32 [n+1] (CUDA tensors) -> fp32 [total, 512]."""
        import torch
        total = x.shape[0]
        if out is None:
            out = torch.empty(total, self.cfg.out_dim, dtype=torch.float32, device="cuda")
        if ws is None:
            ws = self.new_workspace(cu.numel() - 1, total)
        rc = self.encode_features_raw(x, cu, max_len, out, ws, stream)
        if rc != OK:
            raise AlbertError(rc, "albert_encode_features")
        return out

    def encode(self, ids, lengths, out=None, ws=None, stream=None):
        """ids int32 [B, T], lengths int32 [B] (CUDA tensors) -> fp32 [B, T, 512]."""
        import torch
        B, T = ids.shape
        if out is None:
            out = torch.empty(B, T, self.cfg.out_dim, dtype=torch.float32, device="cuda")
        if ws is None:
            ws = self.new_workspace(B, B * T)
        rc = self.encode_raw(ids, lengths, out, ws, stream)
        if rc != OK:
            raise AlbertError(rc, "albert_encode")
        return out

    def encode_varlen(self, ids, cu, max_len, out=None, ws=None, stream=None):
        """ids int32 [total], cu int32 [n+1] (CUDA tensors) -> fp32 [total, 512]."""
        import torch
        total = ids.numel()
        if out is None:
            out = torch.empty(total, self.cfg.out_dim, dtype=torch.float32, device="cuda")
        if ws is None:
            ws = self.new_workspace(cu.numel() - 1, total)
        rc = self.encode_varlen_raw(ids, cu, max_len, out, ws, stream)
        if rc != OK:
            raise AlbertError(rc, "albert_encode_varlen")
        return out


def durations(logits, speed: float = 1.0, dur=None, stream=None):
    """Durations from duration logits [total, K] (CUDA fp32) -> int32 [total]."""
    import torch
    total, K = logits.shape
    _need(logits, "logits", torch.float32)
    if dur is None:
        dur = torch.empty(total, dtype=torch.int32, device="cuda")
    _need(dur, "dur", torch.int32, total)
    rc = lib().albert_durations(_ptr(logits), total, K, float(speed), _ptr(dur), _stream(stream))
    if rc != OK:
        raise AlbertError(rc, "albert_durations")
    return dur


def expand_workspace_bytes(total: int) -> int:
    return int(lib().albert_expand_workspace_bytes(total))


def expand_raw(feat, dur, cu_tok, max_frames, out, cu_frames, ws, stream=None, flags=0,
               ws_bytes=None) -> int:
    """Length regulation on caller tensors; returns the status code."""
    import torch
    total, C = feat.shape
    _need(feat, "feat", torch.float32)
    _need(dur, "dur", torch.int32, total)
    _need(cu_tok, "cu_tok", torch.int32)
    _need(out, "out", torch.float32, int(max_frames) * C)
    _need(cu_frames, "cu_frames", torch.int32, cu_tok.numel())
    _need(ws, "ws")
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    return lib().albert_expand(_ptr(feat), _ptr(dur), _ptr(cu_tok), cu_tok.numel() - 1, total, C,
                               _ptr(out), int(max_frames), _ptr(cu_frames), _ptr(ws), nb,
                               _stream(stream), flags)


def expand(feat, dur, cu_tok, max_frames, stream=None):
    """feat fp32 [total, C], dur int32 [total], cu_tok int32 [n+1] (CUDA)
    -> (frames fp32 [A, C], cu_frames int32 [n+1])."""
    import torch
    total, C = feat.shape
    out = torch.empty((int(max_frames), C), dtype=torch.float32, device="cuda")
    cuf = torch.empty(cu_tok.numel(), dtype=torch.int32, device="cuda")
    ws = torch.empty(expand_workspace_bytes(total), dtype=torch.uint8, device="cuda")
    rc = expand_raw(feat, dur, cu_tok, max_frames, out, cuf, ws, stream)
    if rc != OK:
        raise AlbertError(rc, "albert_expand")
    return out[: int(cuf[-1].item())], cuf


def read_status(ws, stream=None) -> int:
    return int(lib().albert_read_status(_ptr(ws), _stream(stream)))


def text_default_config(**overrides) -> TextConfig:
    c = TextConfig()
    lib().albert_text_default_config(ctypes.byref(c))
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


class TextEncoder:
    """Device copy of the parallel text encoder's weights (an albert_text_ctx).

    weights: dict of canonical name -> float32 array (``synth.TextConfig``
    names; conv<i>.v may be [C, C, K]); config overrides as keywords.
    """

    def __init__(self, weights: dict, stream=None, **cfg):
        import torch  # noqa: F401  (HIP runtime shared with torch)
        L = lib()
        self.cfg = text_default_config(**cfg)
        cf = ctypes.byref(self.cfg)
        nt = L.albert_text_n_tensors(cf)
        if nt < 0:
            raise AlbertError(E_ARG, "albert_text_n_tensors")
        host = []
        for i in range(nt):
            n = L.albert_text_tensor_name(cf, i).decode()
            a = np.ascontiguousarray(np.asarray(weights[n], dtype=np.float32))
            r, c = ctypes.c_int64(), ctypes.c_int64()
            rc = L.albert_text_tensor_shape(cf, i, ctypes.byref(r), ctypes.byref(c))
            if rc != OK:
                raise AlbertError(rc, "albert_text_tensor_shape")
            if a.size != r.value * c.value:
                raise ValueError(f"{n}: expected {r.value}x{c.value} values, got {a.shape}")
            host.append(a)
        ptrs = (ctypes.c_void_p * nt)(*[a.ctypes.data for a in host])
        h = ctypes.c_void_p()
        rc = L.albert_text_load_weights(ctypes.byref(h), cf, ptrs, _stream(stream))
        if rc != OK:
            raise AlbertError(rc, "albert_text_load_weights")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().albert_text_free(self.handle)
            self.handle = None

    __del__ = close

    @property
    def out_dim(self) -> int:
        return 2 * self.cfg.hidden

    def workspace_bytes(self, n_seq: int, max_rows: int) -> int:
        return int(lib().albert_text_workspace_bytes(self.handle, n_seq, max_rows))

    def new_workspace(self, n_seq: int, max_rows: int):
        import torch
        return torch.empty(self.workspace_bytes(n_seq, max_rows), dtype=torch.uint8,
                           device="cuda")

    def tap(self, n_seq: int, max_rows: int, name: str):
        off, nb, st = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
        rc = lib().albert_text_tap(self.handle, n_seq, max_rows, TEXT_TAPS[name],
                                   ctypes.byref(off), ctypes.byref(nb), ctypes.byref(st))
        if rc != OK:
            raise AlbertError(rc, "albert_text_tap")
        return off.value, nb.value, st.value

    def time_kernel(self, kind: str | None, max_launches: int = 1024) -> None:
        k = -1 if kind is None else TEXT_KERNEL_KINDS.index(kind)
        rc = lib().albert_text_time_kernel(self.handle, k, max_launches)
        if rc != OK:
            raise AlbertError(rc, "albert_text_time_kernel")

    def kernel_time(self) -> tuple[int, float]:
        n, ms = ctypes.c_int(), ctypes.c_double()
        rc = lib().albert_text_kernel_time(self.handle, ctypes.byref(n), ctypes.byref(ms))
        if rc != OK:
            raise AlbertError(rc, "albert_text_kernel_time")
        return n.value, ms.value

    def encode_raw(self, ids, lengths, out, ws, stream=None, flags=0, ws_bytes=None) -> int:
        import torch
        if ids.dim() != 2:
            raise ValueError(f"ids: expected [B, T], got {tuple(ids.shape)}")
        B, T = ids.shape
        _need(ids, "ids", torch.int32)
        _need(lengths, "lengths", torch.int32, B)
        _need(out, "out", torch.float32, B * T * self.out_dim)
        _need(ws, "ws")
        nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
        return lib().albert_text_encode(self.handle, _ptr(ids), _ptr(lengths), B, T, _ptr(out),
                                        _ptr(ws), nb, _stream(stream), flags)

    def encode_varlen_raw(self, ids, cu, max_len, out, ws, stream=None, flags=0,
                          ws_bytes=None) -> int:
        import torch
        _need(ids, "ids", torch.int32)
        _need(cu, "cu_seqlens", torch.int32)
        _need(out, "out", torch.float32, ids.numel() * self.out_dim)
        _need(ws, "ws")
        nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
        return lib().albert_text_encode_varlen(self.handle, _ptr(ids), _ptr(cu), cu.numel() - 1,
                                               ids.numel(), max_len, _ptr(out), _ptr(ws), nb,
                                               _stream(stream), flags)

    def encode(self, ids, lengths, out=None, ws=None, stream=None):
        """ids int32 [B, T], lengths int32 [B] (CUDA) -> fp32 [B, T, 512]."""
        import torch
        B, T = ids.shape
        if out is None:
            out = torch.empty(B, T, self.out_dim, dtype=torch.float32, device="cuda")
        if ws is None:
            ws = self.new_workspace(B, B * T)
        rc = self.encode_raw(ids, lengths, out, ws, stream)
        if rc != OK:
            raise AlbertError(rc, "albert_text_encode")
        return out
