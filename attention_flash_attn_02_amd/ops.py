"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Every function takes device tensors, checks that they are contiguous CUDA
(HIP) tensors of the expected dtype and shape, and passes raw pointers and
torch's current stream to the library.  All arithmetic runs in the
library's kernels.  Output tensors (and decode workspaces) may be passed in;
otherwise they are allocated with torch.
"""
from __future__ import annotations

import torch

from . import _lib

_DT = {torch.float32: _lib.ATTN_F32, torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16,
       torch.float8_e5m2: _lib.ATTN_FP8_E5M2}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def prefill_num_configs() -> int:
    return int(_lib.lib().attn_prefill_num_configs())


def prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, dtype, rope_theta) -> int:
    return int(_lib.lib().attn_prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, _DT[dtype], float(rope_theta)))


def prefill_gqa_rope(q, k, v, softmax_scale: float, causal: bool = True, rope_theta: float = 0.0,
                     out_dtype=None, out=None, return_lse: bool = False, q_descale: float = 1.0,
                     k_descale: float = 1.0, v_descale: float = 1.0, stream=None, config=None,
                     k_rope: str = "once", workspace=None, k_rotated: bool = False):
    """q [B,Hq,S,D], k/v [B,Hkv,S,D] -> o [B,Hq,S,D] (and lse [B,Hq,S]).

    ``k_rope`` picks where RoPE is applied to K: "once" (attn_prefill_gqa_rope_ws:
    every key rotated once into ``workspace``, allocated if not given, then the
    attention kernel) or "per_tile" (attn_prefill_gqa_rope: K tiles rotated
    inside the attention kernel as they are staged).  ``config`` selects a
    tile configuration (attn_prefill_gqa_rope_with_config); None = global.
    ``k_rotated`` (with a configuration and a workspace): the workspace already
    holds this K rotated by an earlier call, so only the attention kernel runs."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, S, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if k_rope not in ("once", "per_tile"):
        raise ValueError("k_rope must be 'once' or 'per_tile'")
    if k_rotated and (config is None or workspace is None or k_rope != "once"):
        raise ValueError("k_rotated needs a configuration and the workspace holding the rotated K")
    if out_dtype is None:
        out_dtype = torch.float16 if q.dtype == torch.float8_e5m2 else q.dtype
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if return_lse else None
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse") if lse is not None else None,
            B, Hq, Hkv, S, D, _dtype_code(q), _dtype_code(out), float(softmax_scale), int(bool(causal)),
            float(rope_theta), float(q_descale), float(k_descale), float(v_descale)]
    ws_ptr, ws_bytes = None, 0
    if k_rope == "once":
        need = int(_lib.lib().attn_prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, _dtype_code(q), float(rope_theta)))
        if need > 0:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    if config is None:
        if k_rope == "once":
            code = _lib.lib().attn_prefill_gqa_rope_ws(*args, ws_ptr, ws_bytes, _stream(stream))
        else:
            code = _lib.lib().attn_prefill_gqa_rope(*args, _stream(stream))
    else:
        cfg = int(config) | (_lib.ATTN_CONFIG_K_ROTATED if k_rotated else 0)
        code = _lib.lib().attn_prefill_gqa_rope_with_config(*args, cfg, ws_ptr, ws_bytes, _stream(stream))
    _lib.check(code)
    return (out, lse) if return_lse else out


def rope_rotate(x, rope_theta: float, out=None, stream=None):
    """attn_rope_rotate: rotate x [B,H,S,D] by position (rotate-half RoPE,
    positions 0..S-1).  ``out`` may be ``x`` itself (in place)."""
    B, H, S, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _lib.check(_lib.lib().attn_rope_rotate(_dev(x, "x"), _dev(out, "out"), B, H, S, D, _dtype_code(x),
                                           float(rope_theta), _stream(stream)))
    return out


def prefill_gqa_rope_unfused(q, k, v, softmax_scale: float, causal: bool = True, rope_theta: float = 0.0,
                             out_dtype=None, out=None, return_lse: bool = False, q_rot=None, k_rot=None,
                             stream=None, config=None):
    """The unfused form of prefill_gqa_rope: attn_rope_rotate on Q and on K
    (into ``q_rot`` / ``k_rot``, allocated if not given), then the attention
    kernel without RoPE.  Three launches instead of one."""
    if rope_theta > 0:
        q = rope_rotate(q, rope_theta, out=q_rot, stream=stream)
        k = rope_rotate(k, rope_theta, out=k_rot, stream=stream)
    return prefill_gqa_rope(q, k, v, softmax_scale, causal=causal, rope_theta=0.0, out_dtype=out_dtype, out=out,
                            return_lse=return_lse, stream=stream, config=config)


def kv_append(k_new, v_new, k_cache, v_cache, kv_len, rope_theta: float = 0.0, q=None, advance: bool = True,
              stream=None):
    """attn_kv_append: write k_new, v_new [B,Hkv,T,D] into the caches
    [B,Hkv,cap,D] at slots kv_len[b].., K (and ``q`` [B,Hq,T,D], in place)
    rotated to those positions when rope_theta > 0; kv_len (int32 [B]) then
    advances by T unless ``advance`` is False."""
    B, Hkv, T, D = k_new.shape
    cap = k_cache.shape[2]
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,):
        raise ValueError("kv_len must be int32 [B]")
    for name, t in (("v_new", v_new),):
        if t.shape != k_new.shape or t.dtype != k_new.dtype:
            raise ValueError(f"{name} must match k_new")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.shape != (B, Hkv, cap, D) or t.dtype != k_new.dtype:
            raise ValueError(f"{name} must be [B,Hkv,cap,D] of k_new's dtype")
    Hq = 0
    if q is not None:
        if q.dim() != 4 or q.shape[0] != B or q.shape[2:] != (T, D) or q.dtype != k_new.dtype:
            raise ValueError("q must be [B,Hq,T,D] of k_new's dtype")
        Hq = q.shape[1]
    _lib.check(_lib.lib().attn_kv_append(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(q, "q") if q is not None else None,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"), B, Hkv, Hq, T, D, cap,
        _dtype_code(k_new), float(rope_theta), 1 if advance else 0, _stream(stream)))
    return k_cache, v_cache


def prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split=0) -> int:
    return int(_lib.lib().attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split))


def prefill_chunk(q, k_cache, v_cache, kv_len, softmax_scale: float, out_dtype=None, out=None,
                  return_lse: bool = False, split: int = 0, workspace=None, stream=None):
    """attn_prefill_chunk: q [B,Hq,T,D] (rotated) against the cache prefix;
    kv_len (int32 [B]) counts the chunk's own tokens -> o [B,Hq,T,D].  The
    key ranges of ``split`` keys (0: default) use ``workspace`` (allocated if
    not given and needed)."""
    B, Hq, T, D = q.shape
    _, Hkv, cap, _ = k_cache.shape
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,):
        raise ValueError("kv_len must be int32 [B]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    need = prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_lib.lib().attn_prefill_chunk(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"),
        _dev(out, "out"), _dev(lse, "lse") if lse is not None else None, ws_ptr, ws_bytes, B, Hq, Hkv, T, D,
        cap, int(split), _dtype_code(q), _dtype_code(out), float(softmax_scale), _stream(stream)))
    return (out, lse) if return_lse else out


def decode_gqa_workspace_bytes(B, Hq, cap, D, split=0) -> int:
    return int(_lib.lib().attn_decode_gqa_workspace_bytes(B, Hq, cap, D, split))


def decode_gqa(q, k_cache, v_cache, kv_len, softmax_scale: float, split: int = 0, out=None,
               workspace=None, stream=None):
    """attn_decode_gqa: q [B,Hq,D], caches [B,Hkv,cap,D], kv_len int32 [B] -> o [B,Hq,D]."""
    B, Hq, D = q.shape
    _, Hkv, cap, _ = k_cache.shape
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,):
        raise ValueError("kv_len must be int32 [B]")
    if out is None:
        out = torch.empty_like(q)
    need = decode_gqa_workspace_bytes(B, Hq, cap, D, split)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = _lib.lib().attn_decode_gqa(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"),
        _dev(out, "out"), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        B, Hq, Hkv, D, cap, int(split), _dtype_code(q), float(softmax_scale), _stream(stream))
    _lib.check(code)
    return out


def decode_mla_workspace_bytes(B, H, cap, d_latent, split=0) -> int:
    return int(_lib.lib().attn_decode_mla_workspace_bytes(B, H, cap, d_latent, split))


def decode_mla(q, kv_cache, kv_len, softmax_scale: float, d_latent: int = 448, split: int = 0,
               out=None, workspace=None, stream=None):
    """attn_decode_mla: q [B,H,dl+dr], cache [B,cap,dl+dr], kv_len int32 [B] -> o [B,H,dl]."""
    B, H, dq = q.shape
    cap = kv_cache.shape[1]
    d_rope = dq - d_latent
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,):
        raise ValueError("kv_len must be int32 [B]")
    if out is None:
        out = torch.empty((B, H, d_latent), dtype=q.dtype, device=q.device)
    need = decode_mla_workspace_bytes(B, H, cap, d_latent, split)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = _lib.lib().attn_decode_mla(
        _dev(q, "q"), _dev(kv_cache, "kv_cache"), _dev(kv_len, "kv_len"), _dev(out, "out"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), B, H, d_latent,
        d_rope, cap, int(split), _dtype_code(q), float(softmax_scale), _stream(stream))
    _lib.check(code)
    return out


def combine_splits(o_part, lse_part, out_dtype=torch.float32, out=None, stream=None):
    """attn_combine_splits: o_part [R,nsplit,D] f32, lse_part [R,nsplit] f32 -> o [R,D]."""
    R, ns, D = o_part.shape
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32 or lse_part.shape != (R, ns):
        raise ValueError("o_part [R,nsplit,D] and lse_part [R,nsplit] must be float32")
    if out is None:
        out = torch.empty((R, D), dtype=out_dtype, device=o_part.device)
    code = _lib.lib().attn_combine_splits(_dev(o_part, "o_part"), _dev(lse_part, "lse_part"),
                                          _dev(out, "out"), R, ns, D, _dtype_code(out), _stream(stream))
    _lib.check(code)
    return out
