"""The allocation-free GQA decode entry point (attn_decode_gqa_noalloc),
called through the C ABI: its output equals attn_decode_gqa's (the same
kernels, with the split partials in the library's static device scratch
instead of a caller workspace) and the oracle's, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents);
sizes beyond the 8 MiB scratch are rejected before anything is launched."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import decode_gqa_inputs, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_flash_attn_02_amd as a
    return a._lib.lib()


def _call(lib, fn, q, kc, vc, L, o, split, ws=None):
    B, Hq, D = q.shape
    Hkv, cap = kc.shape[1], kc.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in (q, kc, vc, L, o)]
    if ws is None:
        return fn(*ptrs, B, Hq, Hkv, D, cap, split, 2, 1 / math.sqrt(D), stream)  # 2 = ATTN_BF16
    return fn(*ptrs, ws.data_ptr(), ws.numel(), B, Hq, Hkv, D, cap, split, 2, 1 / math.sqrt(D), stream)


@pytest.mark.parametrize("split", [0, 64, 1024])
def test_noalloc_equals_workspace_form(lib, split):
    for B, lengths in ((64, None), (8, [2048, 1, 0, 7, 33, 2000, 129, 1024])):  # second call smaller
        q, kc, vc, L = decode_gqa_inputs(B, 16, 4, 128, 2056, 2048, "bf16", seed=B + split, nan_tail=True,
                                         lengths=lengths)
        q, kc, vc, L = [t.cuda() for t in (q, kc, vc, L)]
        need = lib.attn_decode_gqa_workspace_bytes(B, 16, 2056, 128, split)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        o_ws = torch.empty_like(q)
        o_na = torch.empty_like(q)
        assert _call(lib, lib.attn_decode_gqa, q, kc, vc, L, o_ws, split, ws) == 0
        assert _call(lib, lib.attn_decode_gqa_noalloc, q, kc, vc, L, o_na, split) == 0
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws)
        want = oracle.decode_gqa(to_f64(q.cpu()), to_f64(kc.cpu()), to_f64(vc.cpu()), L.cpu().numpy(),
                                 1 / math.sqrt(128))
        got = to_f64(o_na.cpu())
        assert np.all(np.isfinite(got))
        assert float(np.max(np.abs(got - want))) <= 2e-2


def test_noalloc_rejects_beyond_scratch(lib):
    # 4096 sequences x 16 heads x 5 parts x (128 + 1) floats > 8 MiB: rejected on the host
    P = 1 << 20
    code = lib.attn_decode_gqa_noalloc(P, P, P, P, P, 4096, 16, 4, 128, 2056, 0, 2, 0.088, None)
    assert code == 5  # ATTN_ERR_WORKSPACE
