"""Seeded synthetic inputs for the attention forward workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It draws random tensors and names shapes; it holds none of
the attention arithmetic.  Every tensor is drawn as float32 N(0, 1) on the
CPU generator and then cast to the storage dtype of the workload, so the GPU
and the oracle see exactly the same bytes (the oracle upcasts them to float64,
which is lossless for float32, float16, bfloat16 and float8 e5m2).

Workloads (the five configurations the method is evaluated on):

* ``tiny_f32``   causal GQA prefill, fp32, B=1, Hq=4, Hkv=2, S=128, D=64,
  scale 1/sqrt(64), no RoPE.
* ``gqa_rope``   causal GQA prefill with fused RoPE, bf16 in / bf16 out,
  B=1, Hq=32, Hkv=8, S=2048, D=128, theta=10000, rotate-half on all dims.
* ``decode_gqa`` GQA decode, bf16, Hq=16, Hkv=4, D=128, context 2048 in a
  static cache of capacity 2056, split 128, batch 1/8/32/64/128.
* ``mha_fwd``    MHA forward Z=4, H=32, D=64 non-causal and D=128 causal,
  N_CTX 1024..16384, fp16 or fp8 e5m2 inputs, fp16 output.
* ``decode_mla`` absorbed-MLA decode, bf16, H=16, latent 448 + rope 64,
  context 2048 (capacity 2056), scale 1/sqrt(192), batch 1/32/128.
"""
from __future__ import annotations

import math

import numpy as np
import torch

SEED = 123

# Per-tensor seed offsets: each named tensor of a workload draws from its own
# stream so that changing one shape does not shift the others.
_OFFSETS = {"q": 0, "k": 1, "v": 2, "kv": 3, "q_nope": 4, "q_rope": 5,
            "w_uk": 6, "w_uv": 7, "c": 8, "part_o": 9, "part_lse": 10, "rope_x": 11}

CONFIGS = {
    "tiny_f32": dict(B=1, Hq=4, Hkv=2, S=128, D=64, dtype="f32", out="f32",
                     causal=True, rope_theta=0.0, scale=1.0 / math.sqrt(64)),
    "gqa_rope": dict(B=1, Hq=32, Hkv=8, S=2048, D=128, dtype="bf16", out="bf16",
                     causal=True, rope_theta=10000.0, scale=1.0 / math.sqrt(128)),
    "decode_gqa": dict(Hq=16, Hkv=4, D=128, cap=2056, L=2048, split=128, dtype="bf16",
                       scale=1.0 / math.sqrt(128), batches=(1, 8, 32, 64, 128)),
    "mha_fwd_d64": dict(Z=4, H=32, D=64, causal=False, out="f16",
                        n_ctx=(1024, 2048, 4096, 8192, 16384), dtypes=("f16", "fp8_e5m2")),
    "mha_fwd_d128": dict(Z=4, H=32, D=128, causal=True, out="f16",
                         n_ctx=(1024, 2048, 4096, 8192, 16384), dtypes=("f16", "fp8_e5m2")),
    "decode_mla": dict(H=16, d_latent=448, d_rope=64, cap=2056, L=2048, dtype="bf16",
                       scale=1.0 / math.sqrt(192), batches=(1, 32, 128),
                       d_nope=128, d_v=128),
}

TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e5m2": torch.float8_e5m2,
}


def _gen(seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + _OFFSETS[name])
    return g


def randn(shape, dtype: str, seed: int, name: str) -> torch.Tensor:
    """N(0,1) float32 draw cast to ``dtype`` (a key of TORCH_DTYPES)."""
    x = torch.randn(*shape, generator=_gen(seed, name), dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype])


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU or GPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def prefill_inputs(B, Hq, Hkv, S, D, dtype, seed=SEED):
    """q [B,Hq,S,D], k and v [B,Hkv,S,D] in ``dtype``, D innermost."""
    q = randn((B, Hq, S, D), dtype, seed, "q")
    k = randn((B, Hkv, S, D), dtype, seed, "k")
    v = randn((B, Hkv, S, D), dtype, seed, "v")
    return q, k, v


def decode_gqa_inputs(B, Hq, Hkv, D, cap, L, dtype="bf16", seed=SEED, nan_tail=False,
                      lengths=None):
    """q [B,Hq,D], k_cache and v_cache [B,Hkv,cap,D], kv_len int32 [B].

    ``lengths`` overrides the per-sequence valid length (default L for all).
    With ``nan_tail`` every slot at or past a sequence's length holds NaN, so
    a kernel that reads an unused slot produces NaN in its output.
    """
    q = randn((B, Hq, D), dtype, seed, "q")
    kc = randn((B, Hkv, cap, D), dtype, seed, "k")
    vc = randn((B, Hkv, cap, D), dtype, seed, "v")
    if lengths is None:
        lengths = [L] * B
    kv_len = torch.tensor(lengths, dtype=torch.int32)
    if nan_tail:
        for b, n in enumerate(lengths):
            kc[b, :, n:, :] = float("nan")
            vc[b, :, n:, :] = float("nan")
    return q, kc, vc, kv_len


def decode_mla_inputs(B, H, d_latent, d_rope, cap, L, dtype="bf16", seed=SEED, nan_tail=False,
                      lengths=None):
    """Absorbed query [B,H,dl+dr] and latent cache [B,cap,dl+dr] (latent first, then rope)."""
    dq = d_latent + d_rope
    q = randn((B, H, dq), dtype, seed, "q")
    c = randn((B, cap, dq), dtype, seed, "kv")
    if lengths is None:
        lengths = [L] * B
    kv_len = torch.tensor(lengths, dtype=torch.int32)
    if nan_tail:
        for b, n in enumerate(lengths):
            c[b, n:, :] = float("nan")
    return q, c, kv_len


def mla_projection_inputs(B, H, d_latent, d_rope, d_nope, d_v, seed=SEED):
    """Unabsorbed-MLA inputs: q_nope [B,H,d_nope], q_rope [B,H,d_rope] (float64),
    W_UK and W_UV [H, d_latent, d_nope|d_v] drawn N(0,1)/sqrt(d_latent) (float64)."""
    q_nope = randn((B, H, d_nope), "f32", seed, "q_nope").double()
    q_rope = randn((B, H, d_rope), "f32", seed, "q_rope").double()
    w_uk = randn((H, d_latent, d_nope), "f32", seed, "w_uk").double() / math.sqrt(d_latent)
    w_uv = randn((H, d_latent, d_v), "f32", seed, "w_uv").double() / math.sqrt(d_latent)
    return q_nope.numpy(), q_rope.numpy(), w_uk.numpy(), w_uv.numpy()


def split_partials(R, nsplit, D, seed=SEED, empty_every=0):
    """Random split-softmax partials for exercising a combine step on its own:
    o_part [R,nsplit,D] float32 and lse_part [R,nsplit] float32 (natural log).
    With ``empty_every`` = k > 0, every k-th split holds an empty part (lse=-inf, o=0)."""
    o = randn((R, nsplit, D), "f32", seed, "part_o")
    lse = randn((R, nsplit), "f32", seed, "part_lse") * 3.0
    if empty_every > 0:
        idx = torch.arange(nsplit) % empty_every == empty_every - 1
        lse[:, idx] = float("-inf")
        o[:, idx, :] = 0.0
    return o, lse
