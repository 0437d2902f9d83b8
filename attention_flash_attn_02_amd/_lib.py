"""ctypes loader for libattn.so (the C ABI declared in include/attn.h).

The library is loaded from this package directory.  There is no fallback:
if the shared library is missing or lacks a symbol, importing the binding
raises, so nothing can silently run on another code path.
"""
from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libattn.so")

# status codes and dtype enum (values fixed by include/attn.h)
ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE",
                4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_UNSUPPORTED",
                7: "ATTN_ERR_LAUNCH"}
ATTN_F32, ATTN_F16, ATTN_BF16, ATTN_FP8_E5M2 = 0, 1, 2, 3
ATTN_CONFIG_K_ROTATED = 0x100  # or-ed into a prefill configuration id: the workspace holds the rotated K

_c_int, _c_float, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/attn.h
SIGNATURES = {
    "attn_status_str": (ctypes.c_char_p, [_c_int]),
    "attn_prefill_gqa_rope": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_int, _c_float, _c_int, _c_float, _c_float, _c_float,
                                       _c_float, _vp]),
    "attn_prefill_gqa_rope_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float]),
    "attn_prefill_gqa_rope_ws": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_float, _c_int, _c_float, _c_float, _c_float,
                                          _c_float, _vp, _sz, _vp]),
    "attn_prefill_num_configs": (_c_int, []),
    "attn_prefill_gqa_rope_with_config": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                                   _c_int, _c_int, _c_int, _c_float, _c_int, _c_float,
                                                   _c_float, _c_float, _c_float, _c_int, _vp, _sz, _vp]),
    "attn_decode_gqa_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_decode_gqa": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_float, _vp]),
    "attn_decode_gqa_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _c_float, _vp]),
    "attn_decode_mla_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_decode_mla": (_c_int, [_vp, _vp, _vp, _vp, _vp, _sz, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_float, _vp]),
    "attn_combine_splits": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "attn_rope_rotate": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp]),
    "attn_kv_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _c_float, _c_int, _vp]),
    "attn_prefill_chunk_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_prefill_chunk": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_float, _vp]),
    "attn_prefill_chunk_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                         _c_float, _vp]),
}


class AttnError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m attention_flash_attn_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is absent
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(code: int) -> None:
    if code != ATTN_OK:
        raise AttnError(code, lib().attn_status_str(code).decode())
