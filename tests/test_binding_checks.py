"""The Python binding checks every tensor it is handed before any library
call (no GPU needed): shapes and dtypes of inputs, caches, lengths, outputs
and workspaces, then that every tensor is a GPU tensor.  A narrower cache, a
short output or a small workspace would otherwise be read or written past
its allocation by the kernels, which size their accesses from q's shape."""
import pytest
import torch

import attention_flash_attn_02_amd as attn

bf = torch.bfloat16


def _t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_decode_gqa_checks():
    q, kc, vc = _t(2, 16, 128), _t(2, 4, 64, 128), _t(2, 4, 64, 128)
    L = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="v_cache"):
        attn.decode_gqa(q, kc, _t(2, 4, 32, 128), L, 0.1)             # shorter V cache
    with pytest.raises(ValueError, match="k_cache"):
        attn.decode_gqa(q, _t(2, 4, 64, 64), vc, L, 0.1)              # head dim mismatch
    with pytest.raises(TypeError, match="k_cache"):
        attn.decode_gqa(q, kc.to(torch.float16), vc, L, 0.1)          # dtype mismatch
    with pytest.raises(TypeError, match="kv_len"):
        attn.decode_gqa(q, kc, vc, L.to(torch.int64), 0.1)
    with pytest.raises(ValueError, match="kv_len"):
        attn.decode_gqa(q, kc, vc, torch.zeros(3, dtype=torch.int32), 0.1)
    with pytest.raises(ValueError, match="out"):
        attn.decode_gqa(q, kc, vc, L, 0.1, out=_t(2, 16, 64))          # short output
    with pytest.raises(TypeError, match="out"):
        attn.decode_gqa(q, kc, vc, L, 0.1, out=_t(2, 16, 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace"):  # 3 workgroups per KV head at split 32: partials
        attn.decode_gqa(q, _t(2, 4, 300, 128), _t(2, 4, 300, 128), L, 0.1, split=32,
                        workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.decode_gqa(q, kc, vc, L, 0.1)                             # all well formed, but on the CPU


def test_decode_mla_checks():
    q, c = _t(2, 16, 512), _t(2, 64, 512)
    L = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="kv_cache"):
        attn.decode_mla(q, _t(2, 64, 448), L, 0.07)                   # latent + rope width mismatch
    with pytest.raises(TypeError, match="kv_cache"):
        attn.decode_mla(q, c.to(torch.float16), L, 0.07)
    with pytest.raises(ValueError, match="out"):
        attn.decode_mla(q, c, L, 0.07, out=_t(2, 16, 512))              # output is the 448-d latent
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.decode_mla(q, c, L, 0.07)


def test_prefill_checks():
    q, k, v = _t(1, 8, 100, 128), _t(1, 2, 100, 128), _t(1, 2, 100, 128)
    with pytest.raises(ValueError, match="v"):
        attn.prefill_gqa_rope(q, k, _t(1, 2, 99, 128), 0.1)
    with pytest.raises(TypeError, match="k"):
        attn.prefill_gqa_rope(q, k.to(torch.float16), v, 0.1)
    with pytest.raises(ValueError, match="out"):
        attn.prefill_gqa_rope(q, k, v, 0.1, out=_t(1, 8, 50, 128))
    with pytest.raises(TypeError, match="out"):
        attn.prefill_gqa_rope(q, k, v, 0.1, out=_t(1, 8, 100, 128, dtype=torch.float16), out_dtype=bf)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.prefill_gqa_rope(q, k, v, 0.1)


def test_prefill_chunk_and_append_checks():
    q, kc, vc = _t(1, 8, 32, 128), _t(1, 2, 256, 128), _t(1, 2, 256, 128)
    L = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="v_cache"):
        attn.prefill_chunk(q, kc, _t(1, 2, 128, 128), L, 0.1)
    with pytest.raises(ValueError, match="out"):
        attn.prefill_chunk(q, kc, vc, L, 0.1, out=_t(1, 8, 16, 128))
    kn, vn = _t(1, 2, 32, 128), _t(1, 2, 32, 128)
    with pytest.raises(ValueError, match="v_new"):
        attn.kv_append(kn, _t(1, 2, 16, 128), kc, vc, L)
    with pytest.raises(ValueError, match="q"):
        attn.kv_append(kn, vn, kc, vc, L, q=_t(1, 8, 32, 64))
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.kv_append(kn, vn, kc, vc, L)


def test_combine_and_rope_checks():
    o, lse = torch.zeros(4, 3, 128), torch.zeros(4, 2)
    with pytest.raises(ValueError, match="lse_part"):
        attn.combine_splits(o, lse)
    with pytest.raises(ValueError, match="out"):
        attn.combine_splits(o, torch.zeros(4, 3), out=torch.zeros(4, 64))
    x = _t(1, 2, 16, 128)
    with pytest.raises(ValueError, match="out"):
        attn.rope_rotate(x, 10000.0, out=_t(1, 2, 8, 128))
