"""CPU float64 oracle for attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
GPU library never calls it, and nothing here imports the GPU library.

See ``ref.py`` for the definitions and ``brute.py`` for the pure-Python
brute force used to pin them.
"""
from .ref import (  # noqa: F401
    rope_inv_freq,
    rope_rotate,
    repeat_kv,
    softmax,
    attention_probs,
    prefill,
    prefill_rows,
    kv_append,
    prefill_chunk,
    decode_gqa,
    decode_mla,
    mla_absorb_query,
    mla_unabsorbed,
    partial_attention,
    merge_pair,
    merge,
    combine_splits,
)
