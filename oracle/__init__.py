"""Float64 CPU oracle for the Kokoro ALBERT phoneme encoder.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package; only the tests, the graft smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library: the only common module is ``synth``, which draws seeded random inputs
and does none of the encoder's arithmetic.
"""
from .albert_oracle import (  # noqa: F401
    bf16_round, prepare_weights, validate, layer_norm, gelu_tanh, softmax,
    dense, attention, shared_layer, embed_ln, encode_sequence, encode,
    encode_varlen, expand_durations, duration_from_logits, param_counts,
    group_schedule, layer_set, encode_features, encode_fp8_features, e4m3_round,
    fp8_row_exponents, fp8_quantize_rows, E4M3_MAX,
    OracleError,
)
