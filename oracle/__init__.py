"""CPU fp64 oracle for exact attention. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never does, and this package never
imports the GPU library.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    bf16_bits_to_f64,
    f16_bits_to_f64,
    causal_visible,
    exact_scale,
    head_backward,
    head_forward,
    head_probs,
    key_mass,
    kv_head,
    online_softmax_stats,
    rows_forward,
)
from .fp8 import (  # noqa: F401
    block_exponent,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    fp8_attention_forward,
    mx_fp8_attention_forward,
    quantize_e4m3_blocks,
    quantize_e4m3_rows32,
)
