"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/attn.h, and rejects bad arguments on the host before
anything is launched."""
import ctypes
import os
import re

import pytest

from attention_flash_attn_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# Fake but 256-byte aligned device addresses: every call below must fail its
# host-side checks before any use of them.
P = 0x100000
P2 = 0x200000
ODD = 0x100002


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"attn_prefill_gqa_rope", "attn_decode_gqa", "attn_decode_mla", "attn_combine_splits",
            "attn_status_str", "attn_decode_gqa_workspace_bytes",
            "attn_decode_mla_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings(lib):
    for code in range(8):
        s = lib.attn_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.attn_status_str(99).decode() == "unknown status"


def _prefill(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P2, lse=None, B=1, Hq=4, Hkv=2, S=16, D=64, in_dt=_lib.ATTN_BF16,
             out_dt=_lib.ATTN_BF16, scale=0.125, causal=1, theta=0.0, qd=1.0, kd=1.0, vd=1.0)
    a.update(kw)
    return lib.attn_prefill_gqa_rope(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                     a["S"], a["D"], a["in_dt"], a["out_dt"], a["scale"], a["causal"],
                                     a["theta"], a["qd"], a["kd"], a["vd"], None)


def test_prefill_rejects(lib):
    assert _prefill(lib, q=None) == 1
    assert _prefill(lib, o=None) == 1
    assert _prefill(lib, S=0) == 2
    assert _prefill(lib, B=-1) == 2
    assert _prefill(lib, Hq=6, Hkv=4) == 2
    assert _prefill(lib, in_dt=7) == 3
    assert _prefill(lib, out_dt=_lib.ATTN_FP8_E5M2) == 3
    assert _prefill(lib, D=96) == 6
    assert _prefill(lib, in_dt=_lib.ATTN_FP8_E5M2, out_dt=_lib.ATTN_F16, theta=10000.0) == 6
    assert _prefill(lib, q=ODD) == 4
    assert _prefill(lib, lse=P + 2) == 4
    assert _prefill(lib, scale=float("nan")) == 2


def _prefill_ws(lib, ws=P, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P2, lse=None, B=1, Hq=4, Hkv=2, S=16, D=64, in_dt=_lib.ATTN_BF16,
             out_dt=_lib.ATTN_BF16, scale=0.125, causal=1, theta=10000.0, qd=1.0, kd=1.0, vd=1.0)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.attn_prefill_gqa_rope_workspace_bytes(a["B"], a["Hkv"], a["S"], a["D"], a["in_dt"],
                                                             a["theta"])
    return lib.attn_prefill_gqa_rope_ws(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                        a["S"], a["D"], a["in_dt"], a["out_dt"], a["scale"], a["causal"],
                                        a["theta"], a["qd"], a["kd"], a["vd"], ws, ws_bytes, None)


def test_prefill_k_rotated_flag_needs_workspace(lib):
    # ATTN_CONFIG_K_ROTATED says the workspace holds the rotated K: without one it is rejected on the host
    code = lib.attn_prefill_gqa_rope_with_config(P, P, P, P2, None, 1, 4, 2, 16, 64, _lib.ATTN_BF16, _lib.ATTN_BF16,
                                                 0.125, 1, 10000.0, 1.0, 1.0, 1.0, _lib.ATTN_CONFIG_K_ROTATED,
                                                 None, 0, None)
    assert code == 5
    code = lib.attn_prefill_gqa_rope_with_config(P, P, P, P2, None, 1, 4, 2, 16, 64, _lib.ATTN_BF16, _lib.ATTN_BF16,
                                                 0.125, 1, 10000.0, 1.0, 1.0, 1.0, _lib.ATTN_CONFIG_K_ROTATED | 9,
                                                 P, 1 << 20, None)
    assert code == 6  # configuration 9 does not exist


def test_prefill_config_ids(lib):
    # ids 0..8 are the sweep configurations (7 the global one); anything else is rejected on the host
    assert lib.attn_prefill_num_configs() == 9
    for bad in (-1, 9, 1000):
        code = lib.attn_prefill_gqa_rope_with_config(P, P, P, P2, None, 1, 4, 2, 16, 64, _lib.ATTN_BF16,
                                                     _lib.ATTN_BF16, 0.125, 1, 0.0, 1.0, 1.0, 1.0, bad, None, 0, None)
        assert code == 6


def test_prefill_ws_workspace_size(lib):
    f = lib.attn_prefill_gqa_rope_workspace_bytes
    # rotated K: B * Hkv * S * D 16-bit elements
    assert f(1, 8, 2048, 128, _lib.ATTN_BF16, 10000.0) == 1 * 8 * 2048 * 128 * 2
    assert f(3, 2, 17, 64, _lib.ATTN_F16, 500.0) == 3 * 2 * 17 * 64 * 2
    assert f(1, 8, 2048, 128, _lib.ATTN_BF16, 0.0) == 0  # no RoPE: no pre-pass
    assert f(1, 8, 2048, 128, _lib.ATTN_F32, 10000.0) == 0  # fp32 kernel rotates K itself
    assert f(1, 8, 2048, 128, _lib.ATTN_FP8_E5M2, 10000.0) == 0
    assert f(0, 8, 2048, 128, _lib.ATTN_BF16, 10000.0) == 0


def test_prefill_ws_rejects(lib):
    assert _prefill_ws(lib, ws=None) == 5
    assert _prefill_ws(lib, ws_bytes=16 * 64 * 2 * 2 - 1) == 5
    assert _prefill_ws(lib, ws=P + 8) == 4
    assert _prefill_ws(lib, q=None) == 1
    assert _prefill_ws(lib, Hq=6, Hkv=4) == 2
    assert _prefill_ws(lib, D=96) == 6
    assert _prefill_ws(lib, S=70000) == 6  # exact angle reduction needs positions < 2^16
    assert _prefill_ws(lib, in_dt=_lib.ATTN_FP8_E5M2, out_dt=_lib.ATTN_F16) == 6


def _gqa(lib, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, L=P, o=P2, ws=P, B=2, Hq=16, Hkv=4, D=128, cap=3000, split=128,
             dt=_lib.ATTN_BF16, scale=0.1)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_gqa_workspace_bytes(a["B"], a["Hq"], a["cap"], a["D"], a["split"])
    return lib.attn_decode_gqa(a["q"], a["k"], a["v"], a["L"], a["o"], a["ws"], ws_bytes, a["B"], a["Hq"],
                               a["Hkv"], a["D"], a["cap"], a["split"], a["dt"], a["scale"], None)


def test_decode_gqa_rejects(lib):
    assert _gqa(lib, L=None) == 1
    assert _gqa(lib, cap=0) == 2
    assert _gqa(lib, Hq=16, Hkv=3) == 2
    assert _gqa(lib, D=64) == 6
    assert _gqa(lib, Hq=64, Hkv=2) == 6            # 32 query heads per KV head
    assert _gqa(lib, dt=_lib.ATTN_F32) == 6
    assert _gqa(lib, dt=11) == 3
    assert _gqa(lib, split=100) == 2
    assert _gqa(lib, split=2048) == 2
    assert _gqa(lib, ws=None) == 5                 # 6 workgroups per KV head: partials need a workspace
    assert _gqa(lib, ws_bytes=1024) == 5
    assert _gqa(lib, ws=P + 16) == 4
    assert _gqa(lib, o=ODD) == 4
    # the score scale must be positive and finite (as for the prefill)
    for bad in (0.0, -0.1, float("nan"), float("inf"), float("-inf")):
        assert _gqa(lib, scale=bad) == 2


def test_decode_gqa_workspace_size(lib):
    # a KV head gets ceil(cap / (4 waves * split)) workgroups; with more than
    # one, their partial outputs [B*Hq, n_wg, D] f32 then lse [B*Hq, n_wg] f32
    # go to the workspace (256-byte aligned pieces); with one, none is needed
    B, Hq, cap, D, split = 128, 16, 2056, 128, 128
    ns = -(-cap // (4 * split))
    assert ns == 5
    o_bytes = B * Hq * ns * D * 4
    lse_bytes = B * Hq * ns * 4
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    assert lib.attn_decode_gqa_workspace_bytes(B, Hq, cap, D, split) == up(o_bytes) + up(lse_bytes)
    assert lib.attn_decode_gqa_workspace_bytes(B, Hq, cap, D, 0) == lib.attn_decode_gqa_workspace_bytes(B, Hq, cap, D, 128)
    # 1024 slots per wave cover caps up to 4096 with one workgroup: no workspace
    assert lib.attn_decode_gqa_workspace_bytes(B, Hq, cap, D, 1024) == 0
    assert lib.attn_decode_gqa_workspace_bytes(B, Hq, 4096, D, 1024) == 0
    assert lib.attn_decode_gqa_workspace_bytes(B, Hq, 4097, D, 1024) > 0
    assert lib.attn_decode_gqa_workspace_bytes(0, Hq, cap, D, split) == 0


def test_decode_gqa_no_workspace_when_one_workgroup(lib):
    # cap 3000 at split 1024: one workgroup per KV head, the workspace is not
    # used, so NULL passes the host checks; a bad pointer elsewhere still
    # fails them before anything is launched
    assert _gqa(lib, split=1024, ws=None, ws_bytes=0, o=ODD) == 4


def _mla(lib, ws_bytes=None, **kw):
    a = dict(q=P, c=P, L=P, o=P2, ws=P, B=2, H=16, dl=448, dr=64, cap=300, split=128,
             dt=_lib.ATTN_BF16, scale=0.07)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_mla_workspace_bytes(a["B"], a["H"], a["cap"], a["dl"], a["split"])
    return lib.attn_decode_mla(a["q"], a["c"], a["L"], a["o"], a["ws"], ws_bytes, a["B"], a["H"], a["dl"],
                               a["dr"], a["cap"], a["split"], a["dt"], a["scale"], None)


def test_decode_mla_rejects(lib):
    assert _mla(lib, q=None) == 1
    assert _mla(lib, B=0) == 2
    assert _mla(lib, dl=512, dr=0) == 6
    assert _mla(lib, H=32) == 6
    assert _mla(lib, dt=_lib.ATTN_FP8_E5M2) == 6
    assert _mla(lib, split=48) == 2
    assert _mla(lib, ws_bytes=16) == 5
    assert _mla(lib, c=ODD) == 4
    for bad in (0.0, -0.07, float("nan"), float("inf")):
        assert _mla(lib, scale=bad) == 2
    # the split index is the second grid dimension: at most 65535 splits
    assert _mla(lib, B=1, cap=32 * 65536, split=32) == 2


def test_combine_rejects(lib):
    f = lib.attn_combine_splits
    assert f(None, P, P2, 4, 3, 128, _lib.ATTN_F32, None) == 1
    assert f(P, P, P2, 0, 3, 128, _lib.ATTN_F32, None) == 2
    assert f(P, P, P2, 4, 3, 2048, _lib.ATTN_F32, None) == 2
    assert f(P, P, P2, 4, 3, 128, _lib.ATTN_FP8_E5M2, None) == 3
    assert f(P + 1, P, P2, 4, 3, 128, _lib.ATTN_F32, None) == 4


def test_rope_rejects(lib):
    def rope(x=P, y=P, B=1, H=2, S=16, D=128, dt=_lib.ATTN_BF16, theta=10000.0):
        return lib.attn_rope_rotate(x, y, B, H, S, D, dt, theta, None)
    assert rope(x=None) == 1
    assert rope(S=0) == 2 and rope(D=63) == 2
    assert rope(theta=0.0) == 2 and rope(theta=float("nan")) == 2 and rope(theta=float("inf")) == 2
    assert rope(dt=_lib.ATTN_FP8_E5M2) == 6 and rope(dt=9) == 3
    assert rope(D=258) == 6 and rope(D=24) == 6       # half rows not whole 16-byte chunks (16-bit)
    assert rope(S=65537) == 6
    assert rope(x=P + 8) == 4


def test_kv_append_rejects(lib):
    def app(kn=P, vn=P, q=None, kc=P2, vc=P2, L=P, B=2, Hkv=2, Hq=8, T=1, D=128, cap=64,
            dt=_lib.ATTN_BF16, theta=10000.0, adv=1):
        return lib.attn_kv_append(kn, vn, q, kc, vc, L, B, Hkv, Hq, T, D, cap, dt, theta, adv, None)
    assert app(kn=None) == 1 and app(L=None) == 1
    assert app(T=0) == 2 and app(cap=0) == 2 and app(D=63) == 2
    assert app(q=P, Hq=0) == 2
    assert app(theta=float("nan")) == 2 and app(theta=float("inf")) == 2
    assert app(dt=_lib.ATTN_FP8_E5M2) == 6 and app(dt=9) == 3
    assert app(D=258) == 6 and app(cap=70000) == 6
    assert app(kc=P + 8) == 4 and app(L=P + 2) == 4 and app(q=P + 8) == 4


def test_prefill_chunk_rejects(lib):
    def chunk(q=P, kc=P, vc=P, L=P, o=P2, lse=None, ws=P, wsb=None, B=2, Hq=16, Hkv=4, T=32, D=128, cap=2056,
              split=0, dt=_lib.ATTN_BF16, odt=_lib.ATTN_BF16, scale=0.088, theta=0.0):
        if wsb is None:
            wsb = lib.attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split)
        return lib.attn_prefill_chunk(q, kc, vc, L, o, lse, ws, wsb, B, Hq, Hkv, T, D, cap, split, dt, odt, scale,
                                      theta, None)
    assert chunk(L=None) == 1 and chunk(o=None) == 1
    assert chunk(T=0) == 2 and chunk(T=3000) == 2 and chunk(Hq=6, Hkv=4) == 2 and chunk(split=100) == 2
    assert chunk(scale=0.0) == 2 and chunk(scale=float("nan")) == 2
    assert chunk(theta=float("nan")) == 2 and chunk(theta=float("inf")) == 2
    assert chunk(theta=10000.0, cap=70000, T=32) == 6  # RoPE positions past 2^16
    assert chunk(dt=_lib.ATTN_F32) == 6 and chunk(dt=_lib.ATTN_FP8_E5M2) == 6 and chunk(D=96) == 6
    assert chunk(odt=_lib.ATTN_FP8_E5M2) == 3 and chunk(dt=8) == 3
    assert chunk(q=ODD) == 4 and chunk(L=P + 2) == 4 and chunk(lse=P + 2) == 4
    assert chunk(ws=None) == 5 and chunk(wsb=256) == 5 and chunk(ws=P + 16) == 4


def test_prefill_chunk_step_rejects(lib):
    """The fused chunk step fails every host check of the two calls it fuses,
    before anything is launched (so a rejected call writes nothing)."""
    def step(q=P, kn=P, vn=P, kc=P, vc=P, L=P, o=P2, lse=None, ws=P, wsb=None, B=2, Hq=16, Hkv=4, T=32, D=128,
             cap=2056, split=0, dt=_lib.ATTN_BF16, odt=_lib.ATTN_BF16, scale=0.088, theta=0.0):
        if wsb is None:
            wsb = lib.attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, split)
        return lib.attn_prefill_chunk_step(q, kn, vn, kc, vc, L, o, lse, ws, wsb, B, Hq, Hkv, T, D, cap, split, dt,
                                           odt, scale, theta, None)
    assert step(kn=None) == 1 and step(vn=None) == 1 and step(L=None) == 1 and step(o=None) == 1
    assert step(T=0) == 2 and step(T=3000) == 2 and step(Hq=6, Hkv=4) == 2 and step(split=100) == 2
    assert step(scale=0.0) == 2 and step(scale=float("inf")) == 2 and step(theta=float("nan")) == 2
    assert step(theta=10000.0, cap=70000, T=32) == 6
    assert step(dt=_lib.ATTN_F32) == 6 and step(D=96) == 6 and step(odt=_lib.ATTN_FP8_E5M2) == 3
    assert step(kn=ODD) == 4 and step(vn=P + 8) == 4 and step(L=P + 2) == 4 and step(lse=P + 2) == 4
    assert step(ws=None) == 5 and step(wsb=256) == 5 and step(ws=P + 16) == 4


def test_prefill_chunk_workspace_size(lib):
    # partials [B*Hq*T, nsplit, D] f32 then lse [B*Hq*T, nsplit] f32, 256-byte aligned pieces
    B, Hq, Hkv, T, D, cap = 2, 16, 4, 32, 128, 2056
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    ns = -(-cap // 256)
    assert lib.attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, 256) == \
        up(B * Hq * T * ns * D * 4) + up(B * Hq * T * ns * 4)
    assert lib.attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, 4096) == 0  # one range: none needed
    assert lib.attn_prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, cap, 0) > 0


def test_binding_rejects_cpu_tensors():
    import torch

    import attention_flash_attn_02_amd as attn
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.prefill_gqa_rope(q, q, q, 0.125)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "libattn.so"))


def test_noalloc_documented_limit(lib):
    """The allocation-free GQA decode's static array is 8 MiB: at the default
    split and capacity 2056 its parts fit B * Hq = 3251 query rows and not
    one more (the figure the header states)."""
    need = lambda rows: lib.attn_decode_gqa_workspace_bytes(1, rows, 2056, 128, 0)  # noqa: E731
    assert need(3251) <= 8 << 20 < need(3252)
