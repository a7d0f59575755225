"""CPU oracle for KV-cache importance scoring and eviction.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The library never calls
it, and it shares no code with the GPU kernels.

Everything here is fp64 numpy, written as the plain definitions from the pages
(see ``oracle.reference``). Parity is pinned by the tests in
``tests/test_oracle_*.py`` (closed forms, library routines, brute force).
"""
from .reference import (  # noqa: F401
    REPEAT,
    CAUSAL,
    bf16_bits_to_f64,
    visible_logits,
    kv_head_of,
    outside_window,
    lse,
    attention,
    attention_weights,
    max_scores,
    future_mass,
    decode_attention,
    value_norms,
    select,
    compact,
    stream_states,
)
