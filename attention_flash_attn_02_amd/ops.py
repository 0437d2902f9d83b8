"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Every function checks each tensor it is given (inputs, caches, lengths,
outputs and workspaces) for shape, dtype, contiguity and device before any
library call: the kernels size their loads and stores from the shapes
passed, so a narrower cache or a short output would otherwise be read or
written past its allocation.  Shapes and dtypes are checked first (so a
wrong argument is reported as such even before the device is looked at),
then that every tensor is a contiguous GPU tensor on q's device.  Raw
pointers and torch's current stream go to the library; all arithmetic runs
in its kernels.  Output tensors (and workspaces) may be passed in, otherwise
they are allocated with torch.
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


def _shape(t, name: str, shape, dtype=None) -> None:
    """t must be a tensor of exactly `shape` (and `dtype`, if given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ndim(t, name: str, n: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got {t.dim()}")


def _same_device(ref: torch.Tensor, ref_name: str = "q", **named) -> None:
    """ref and every given tensor are contiguous GPU tensors on ref's device."""
    _dev(ref, ref_name)
    for name, t in named.items():
        if t is None:
            continue
        _dev(t, name)
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _check_workspace(ws, need: int) -> None:
    """A workspace the caller passes must hold `need` bytes."""
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")


def _workspace(ws, need: int, device) -> torch.Tensor:
    """The caller's workspace (checked to hold `need` bytes) or a new one."""
    _check_workspace(ws, need)
    return ws if ws is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=device)


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
    _ndim(q, "q", 4)
    _ndim(k, "k", 4)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, S, D), q.dtype)
    _shape(v, "v", (B, Hkv, S, D), q.dtype)
    if k_rope not in ("once", "per_tile"):
        raise ValueError("k_rope must be 'once' or 'per_tile'")
    if k_rotated and (config is None or workspace is None or k_rope != "once"):
        raise ValueError("k_rotated needs a configuration and the workspace holding the rotated K")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else (torch.float16 if q.dtype == torch.float8_e5m2 else q.dtype)
    if out is not None:
        _shape(out, "out", (B, Hq, S, D), out_dtype)
    _same_device(q, k=k, v=v, out=out, workspace=workspace)
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
            workspace = _workspace(workspace, need, q.device)
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
    _ndim(x, "x", 4)
    B, H, S, D = x.shape
    if out is not None:
        _shape(out, "out", tuple(x.shape), x.dtype)
    _same_device(x, "x", out=out)
    if out is None:
        out = torch.empty_like(x)
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
    _ndim(k_new, "k_new", 4)
    _ndim(k_cache, "k_cache", 4)
    B, Hkv, T, D = k_new.shape
    cap = k_cache.shape[2]
    _shape(kv_len, "kv_len", (B,), torch.int32)
    _shape(v_new, "v_new", (B, Hkv, T, D), k_new.dtype)
    _shape(k_cache, "k_cache", (B, Hkv, cap, D), k_new.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, cap, D), k_new.dtype)
    Hq = 0
    if q is not None:
        _ndim(q, "q", 4)
        _shape(q, "q", (B, q.shape[1], T, D), k_new.dtype)
        Hq = q.shape[1]
    _same_device(k_new, "k_new", v_new=v_new, k_cache=k_cache, v_cache=v_cache, kv_len=kv_len, q_rotated=q)
    _lib.check(_lib.lib().attn_kv_append(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(q, "q") if q is not None else None,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"), B, Hkv, Hq, T, D, cap,
        _dtype_code(k_new), float(rope_theta), 1 if advance else 0, _stream(stream)))
    return k_cache, v_cache


def prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split=0) -> int:
    return int(_lib.lib().attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split))


def prefill_chunk(q, k_cache, v_cache, kv_len, softmax_scale: float, out_dtype=None, out=None,
                  return_lse: bool = False, split: int = 0, workspace=None, rope_theta: float = 0.0,
                  stream=None):
    """attn_prefill_chunk: q [B,Hq,T,D] against the cache prefix; kv_len
    (int32 [B]) counts the chunk's own tokens -> o [B,Hq,T,D].  With
    ``rope_theta`` > 0 the kernel rotates q to the chunk's positions (the
    cached K rows already rotated); otherwise q is used as given.  The key
    ranges of ``split`` keys (0: default) use ``workspace`` (allocated if not
    given and needed)."""
    _ndim(q, "q", 4)
    _ndim(k_cache, "k_cache", 4)
    B, Hq, T, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, "k_cache", (B, Hkv, cap, D), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, cap, D), q.dtype)
    _shape(kv_len, "kv_len", (B,), torch.int32)
    if out is not None:
        _shape(out, "out", (B, Hq, T, D), out_dtype or out.dtype)
    need = prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split)
    _check_workspace(workspace, need)
    _same_device(q, k_cache=k_cache, v_cache=v_cache, kv_len=kv_len, out=out, workspace=workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    if need > 0:
        workspace = _workspace(workspace, need, q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_lib.lib().attn_prefill_chunk(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"),
        _dev(out, "out"), _dev(lse, "lse") if lse is not None else None, ws_ptr, ws_bytes, B, Hq, Hkv, T, D,
        cap, int(split), _dtype_code(q), _dtype_code(out), float(softmax_scale), float(rope_theta),
        _stream(stream)))
    return (out, lse) if return_lse else out


def prefill_chunk_step(q, k_new, v_new, k_cache, v_cache, kv_len, softmax_scale: float, out_dtype=None,
                       out=None, return_lse: bool = False, split: int = 0, workspace=None,
                       rope_theta: float = 0.0, stream=None):
    """attn_prefill_chunk_step: one chunked-prefill step into a static append
    cache.  q [B,Hq,T,D] (not rotated), k_new/v_new [B,Hkv,T,D] are appended
    at slots kv_len[b].. (K rotated there when rope_theta > 0), q attends to
    the cache prefix including the chunk, and kv_len (int32 [B], EXCLUDING
    the chunk on entry) advances by T -> o [B,Hq,T,D]."""
    _ndim(q, "q", 4)
    _ndim(k_new, "k_new", 4)
    _ndim(k_cache, "k_cache", 4)
    B, Hq, T, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _shape(k_new, "k_new", (B, Hkv, T, D), q.dtype)
    _shape(v_new, "v_new", (B, Hkv, T, D), q.dtype)
    _shape(k_cache, "k_cache", (B, Hkv, cap, D), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, cap, D), q.dtype)
    _shape(kv_len, "kv_len", (B,), torch.int32)
    if out is not None:
        _shape(out, "out", (B, Hq, T, D), out_dtype or out.dtype)
    need = prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split)
    _check_workspace(workspace, need)
    _same_device(q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, kv_len=kv_len, out=out,
                 workspace=workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    if need > 0:
        workspace = _workspace(workspace, need, q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_lib.lib().attn_prefill_chunk_step(
        _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None, ws_ptr, ws_bytes, B, Hq, Hkv, T, D, cap, int(split),
        _dtype_code(q), _dtype_code(out), float(softmax_scale), float(rope_theta), _stream(stream)))
    return (out, lse) if return_lse else out


def decode_gqa_workspace_bytes(B, Hq, cap, D, split=0) -> int:
    return int(_lib.lib().attn_decode_gqa_workspace_bytes(B, Hq, cap, D, split))


def decode_gqa(q, k_cache, v_cache, kv_len, softmax_scale: float, split: int = 0, out=None,
               workspace=None, stream=None):
    """attn_decode_gqa: q [B,Hq,D], caches [B,Hkv,cap,D], kv_len int32 [B] -> o [B,Hq,D]."""
    _ndim(q, "q", 3)
    _ndim(k_cache, "k_cache", 4)
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, "k_cache", (B, Hkv, cap, D), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, cap, D), q.dtype)
    _shape(kv_len, "kv_len", (B,), torch.int32)
    if out is not None:
        _shape(out, "out", (B, Hq, D), q.dtype)
    need = decode_gqa_workspace_bytes(B, Hq, cap, D, split)
    _check_workspace(workspace, need)
    _same_device(q, k_cache=k_cache, v_cache=v_cache, kv_len=kv_len, out=out, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    workspace = _workspace(workspace, need, q.device)
    code = _lib.lib().attn_decode_gqa(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"),
        _dev(out, "out"), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        B, Hq, Hkv, D, cap, int(split), _dtype_code(q), float(softmax_scale), _stream(stream))
    _lib.check(code)
    return out


def decode_gqa_noalloc(q, k_cache, v_cache, kv_len, softmax_scale: float, split: int = 0, out=None, stream=None):
    """attn_decode_gqa_noalloc: decode_gqa with the split partials in the
    library's static device scratch (no workspace, no device allocation when
    ``out`` is given).  Calls that overlap on one GPU race on that scratch."""
    _ndim(q, "q", 3)
    _ndim(k_cache, "k_cache", 4)
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, "k_cache", (B, Hkv, cap, D), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, cap, D), q.dtype)
    _shape(kv_len, "kv_len", (B,), torch.int32)
    if out is not None:
        _shape(out, "out", (B, Hq, D), q.dtype)
    _same_device(q, k_cache=k_cache, v_cache=v_cache, kv_len=kv_len, out=out)
    if out is None:
        out = torch.empty_like(q)
    code = _lib.lib().attn_decode_gqa_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(kv_len, "kv_len"),
        _dev(out, "out"), B, Hq, Hkv, D, cap, int(split), _dtype_code(q), float(softmax_scale), _stream(stream))
    _lib.check(code)
    return out


def decode_mla_workspace_bytes(B, H, cap, d_latent, split=0) -> int:
    return int(_lib.lib().attn_decode_mla_workspace_bytes(B, H, cap, d_latent, split))


def decode_mla(q, kv_cache, kv_len, softmax_scale: float, d_latent: int = 448, split: int = 0,
               out=None, workspace=None, stream=None):
    """attn_decode_mla: q [B,H,dl+dr], cache [B,cap,dl+dr], kv_len int32 [B] -> o [B,H,dl]."""
    _ndim(q, "q", 3)
    _ndim(kv_cache, "kv_cache", 3)
    B, H, dq = q.shape
    cap = kv_cache.shape[1]
    d_rope = dq - d_latent
    _shape(kv_cache, "kv_cache", (B, cap, dq), q.dtype)
    _shape(kv_len, "kv_len", (B,), torch.int32)
    if out is not None:
        _shape(out, "out", (B, H, d_latent), q.dtype)
    need = decode_mla_workspace_bytes(B, H, cap, d_latent, split)
    _check_workspace(workspace, need)
    _same_device(q, kv_cache=kv_cache, kv_len=kv_len, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((B, H, d_latent), dtype=q.dtype, device=q.device)
    workspace = _workspace(workspace, need, q.device)
    code = _lib.lib().attn_decode_mla(
        _dev(q, "q"), _dev(kv_cache, "kv_cache"), _dev(kv_len, "kv_len"), _dev(out, "out"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), B, H, d_latent,
        d_rope, cap, int(split), _dtype_code(q), float(softmax_scale), _stream(stream))
    _lib.check(code)
    return out


def combine_splits(o_part, lse_part, out_dtype=torch.float32, out=None, stream=None):
    """attn_combine_splits: o_part [R,nsplit,D] f32, lse_part [R,nsplit] f32 -> o [R,D]."""
    _ndim(o_part, "o_part", 3)
    R, ns, D = o_part.shape
    _shape(o_part, "o_part", (R, ns, D), torch.float32)
    _shape(lse_part, "lse_part", (R, ns), torch.float32)
    if out is not None:
        _shape(out, "out", (R, D), out.dtype)
    _same_device(o_part, "o_part", lse_part=lse_part, out=out)
    if out is None:
        out = torch.empty((R, D), dtype=out_dtype, device=o_part.device)
    code = _lib.lib().attn_combine_splits(_dev(o_part, "o_part"), _dev(lse_part, "lse_part"),
                                          _dev(out, "out"), R, ns, D, _dtype_code(out), _stream(stream))
    _lib.check(code)
    return out
