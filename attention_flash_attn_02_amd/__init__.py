"""MI355X (gfx950) attention forward: HIP kernels behind a C ABI (include/attn.h).

Python entry points (same names as the C calls, without the ``attn_`` prefix):
prefill_gqa_rope, rope_rotate, decode_gqa, decode_gqa_noalloc, decode_mla,
combine_splits, kv_append, prefill_chunk, prefill_chunk_step, and the workspace size queries;
prefill_gqa_rope_unfused composes rope_rotate with the attention call.
libattn.so is loaded on first use; every call raises ImportError if it has
not been built (there is no other code path).
"""
from ._lib import AttnError, lib  # noqa: F401
from .ops import (  # noqa: F401
    combine_splits,
    decode_gqa,
    decode_gqa_noalloc,
    decode_gqa_workspace_bytes,
    decode_mla,
    decode_mla_workspace_bytes,
    kv_append,
    prefill_chunk,
    prefill_chunk_step,
    prefill_chunk_workspace_bytes,
    prefill_gqa_rope,
    prefill_gqa_rope_unfused,
    prefill_gqa_rope_workspace_bytes,
    prefill_num_configs,
    rope_rotate,
)
