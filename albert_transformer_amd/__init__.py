"""MI355X-native Kokoro ALBERT phoneme encoder.

The compute path is the C-ABI library ``libalbert.so`` (HIP kernels for
gfx950, declared in include/albert.h); this package only binds it.
"""
from ._lib import (  # noqa: F401
    ASYNC, UNFUSED, LN_HANDOFF, BF16, F32, FP8, DTYPES, OK, E_ARG, E_WORKSPACE, E_LENGTH, E_ID, E_ALIAS, E_HIP,
    E_SYNC, E_SCRATCH, SCRATCH_BYTES,
    STATUS_NAMES, TAPS, EXPORTS, KERNEL_KINDS, AlbertError, Config, Encoder, default_config, lib,
    read_status, status_str, durations, expand, expand_raw, expand_workspace_bytes,
    TextConfig, TextEncoder, text_default_config, TEXT_TAPS, TEXT_KERNEL_KINDS,
)
