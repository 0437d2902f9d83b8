"""Plain float64 CPU oracle for scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke entry point and the
benchmark's CPU-baseline leg, never by the GPU library, and it imports nothing
from the GPU library.

Sources (the pages are cited by title and section):

* "Lesson: shape adaptive attention negative 20260722" (row "Conditions"):
  causal GQA prefill and decode with RoPE fused into attention.
* "Fixed-budget decode audit", sections "Which implementation was tested" and
  "Setup and interpretation": split-context GQA decode against a static
  append cache, and MLA with a 448-d latent plus a 64-d RoPE part per token
  using matrix absorption.
* "Fixed-budget decode audit", section "A: group-entry queries and one joint
  history scan": the merge of two softmax parts,
  alpha = sigmoid(score_b - lse_a), out = (1 - alpha) out_a + alpha out_b.
* Persistent-attention digest (hada.io), section on benchmarks: Z=4, H=32
  forward in fp16 and fp8 (float8e5).

None of the pages prints the attention formula itself, so what the oracle
computes is the textbook definition: for each query row,
O = softmax(scale * q K^T) V with the softmax taken over keys.  Readings of
points the pages leave open (each also listed in the design notes):

* GQA: query head h reads KV head floor(h / G) with G = Hq / Hkv.
* Causal: key j is visible to query i iff j <= i (equal query and key lengths).
* RoPE: rotate-half pairing (i, i + D/2), inverse frequency theta^(-2i/D),
  angle = position * inverse frequency, positions 0..S-1, applied to Q and K
  (after KV-head repetition) and never to V.
* MLA: the absorbed query is [W_UK[h] q_nope ; q_rope] (latent first, rope
  last) and the value is the 448-d latent part of the cache row.
* An empty key set yields a zero output and lse = -inf.

Everything is float64 with library primitives (matmul, exp) as single steps.
Loops over (batch, head) and over chunks of query rows only bound memory; each
row's softmax is always taken over its complete key set.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# RoPE (reading: rotate-half, theta^(-2i/D), positions from 0)
# ----------------------------------------------------------------------------
def rope_inv_freq(D: int, theta: float) -> np.ndarray:
    """Inverse frequencies theta^(-2i/D) for the D/2 rotated pairs."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / D)


def rope_rotate(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotate x [..., S, D] by position: the pair (x[i], x[i+D/2]) turns by
    angle positions[s] * theta^(-2i/D)."""
    D = x.shape[-1]
    half = D // 2
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * rope_inv_freq(D, theta)[None, :]          # [S, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# Building blocks
# ----------------------------------------------------------------------------
def repeat_kv(k: np.ndarray, G: int) -> np.ndarray:
    """Explicit KV-head repetition: [B, Hkv, ...] -> [B, Hkv*G, ...] where head
    h holds KV head h // G."""
    return np.repeat(k, G, axis=1)


def softmax(t: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax along ``axis``, shifted by the row maximum before exp."""
    m = np.max(t, axis=axis, keepdims=True)
    e = np.exp(t - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def _causal_mask(rows: np.ndarray, n_keys: int) -> np.ndarray:
    """True where key j is NOT visible to query row i (j > i)."""
    return np.arange(n_keys)[None, :] > np.asarray(rows)[:, None]


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                    rows=None) -> np.ndarray:
    """Probabilities softmax(scale q k^T) for one head: q [R, D] (query rows
    ``rows``, default 0..R-1), k [S, D] -> [R, S]."""
    t = scale * (q @ k.T)
    if causal:
        if rows is None:
            rows = np.arange(q.shape[0])
        t = np.where(_causal_mask(rows, k.shape[0]), -np.inf, t)
    return softmax(t, axis=-1)


def _logsumexp_rows(t: np.ndarray) -> np.ndarray:
    m = np.max(t, axis=-1)
    return m + np.log(np.sum(np.exp(t - m[:, None]), axis=-1))


# ----------------------------------------------------------------------------
# Prefill: causal (or not) GQA attention with optional RoPE
# ----------------------------------------------------------------------------
def prefill(q, k, v, scale: float, causal: bool, rope_theta: float = 0.0,
            return_lse: bool = False, row_chunk: int = 1024):
    """q [B,Hq,S,D], k and v [B,Hkv,S,D] (float64) -> O [B,Hq,S,D]
    (and LSE [B,Hq,S] in natural-log units when ``return_lse``).

    KV heads are repeated explicitly (repeat_kv) before RoPE and the scores."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    k_rep = repeat_kv(k, G)
    v_rep = repeat_kv(v, G)
    if rope_theta > 0:
        pos = np.arange(S)
        q = rope_rotate(q, pos, rope_theta)
        k_rep = rope_rotate(k_rep, pos, rope_theta)
    out = np.empty((B, Hq, S, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, Hq, S), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, S, row_chunk):
                rows = np.arange(r0, min(S, r0 + row_chunk))
                t = scale * (q[b, h, rows] @ k_rep[b, h].T)
                if causal:
                    t = np.where(_causal_mask(rows, S), -np.inf, t)
                p = softmax(t, axis=-1)
                out[b, h, rows] = p @ v_rep[b, h]
                if return_lse:
                    lse[b, h, rows] = _logsumexp_rows(t)
    return (out, lse) if return_lse else out


def prefill_rows(q, k, v, scale: float, causal: bool, rope_theta: float,
                 b: int, h: int, rows):
    """Selected query rows of one head of ``prefill`` (for sampled checks at
    sizes where the full output is too costly).  q [B,Hq,S,D] and k, v
    [B,Hkv,S,D] may be any float arrays; only head h of batch b and its KV
    head are converted.  Returns O [len(rows), D] and LSE [len(rows)]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    S = q.shape[2]
    rows = np.asarray(rows)
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, h // G], dtype=np.float64)
    vh = np.asarray(v[b, h // G], dtype=np.float64)
    if rope_theta > 0:
        qh = rope_rotate(qh[rows], rows, rope_theta)
        kh = rope_rotate(kh, np.arange(S), rope_theta)
    else:
        qh = qh[rows]
    t = scale * (qh @ kh.T)
    if causal:
        t = np.where(_causal_mask(rows, S), -np.inf, t)
    return softmax(t, axis=-1) @ vh, _logsumexp_rows(t)


# ----------------------------------------------------------------------------
# Decode neighbours: appending tokens to the static cache, and a chunk of
# queries against the cache prefix ("Fixed-budget decode audit", "Setup and
# interpretation": a static append cache; prompts prefilled in chunks of 32)
# ----------------------------------------------------------------------------
def kv_append(k_cache, v_cache, kv_len, k_new, v_new, rope_theta: float, q_new=None):
    """Append T tokens per sequence: k_new, v_new [B,Hkv,T,D] go to slots
    kv_len[b] .. kv_len[b]+T-1 of the caches [B,Hkv,cap,D].  The slot index is
    the token's position: K is rotated by it when rope_theta > 0, V is copied.
    q_new [B,Hq,T,D], if given, is rotated at the same positions.  Returns
    float64 copies (k_cache, v_cache, kv_len + T, q); slots outside the
    appended range keep their contents."""
    k2 = np.array(k_cache, dtype=np.float64)
    v2 = np.array(v_cache, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, _, T, _ = k_new.shape
    q2 = None if q_new is None else np.array(q_new, dtype=np.float64)
    for b in range(B):
        L = int(kv_len[b])
        pos = L + np.arange(T)
        kb = rope_rotate(k_new[b], pos, rope_theta) if rope_theta > 0 else k_new[b]
        k2[b, :, L:L + T] = kb
        v2[b, :, L:L + T] = v_new[b]
        if q2 is not None and rope_theta > 0:
            q2[b] = rope_rotate(q2[b], pos, rope_theta)
    return k2, v2, np.asarray(kv_len, dtype=np.int64) + T, q2


def prefill_chunk(q, k_cache, v_cache, kv_len, scale: float, return_lse: bool = False):
    """A chunk of T queries per sequence against the cache prefix: q
    [B,Hq,T,D] (already rotated), caches [B,Hkv,cap,D], kv_len [B] counting
    the chunk's own tokens.  Row t sits at position p = kv_len[b] - T + t and
    attends to slots 0..p (causal, aligned at the end of the prefix).  A row
    with p < 0 sees no key: zero output, lse -inf."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, T, v_cache.shape[-1]), dtype=np.float64)
    lse = np.full((B, Hq, T), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(kv_len[b])
        pos = L - T + np.arange(T)
        live = pos >= 0
        if L == 0 or not live.any():
            continue
        kb = repeat_kv(np.asarray(k_cache[b:b + 1, :, :L], dtype=np.float64), G)[0]
        vb = repeat_kv(np.asarray(v_cache[b:b + 1, :, :L], dtype=np.float64), G)[0]
        for h in range(Hq):
            t = scale * (q[b, h][live] @ kb[h].T)
            t = np.where(_causal_mask(pos[live], L), -np.inf, t)
            out[b, h, live] = softmax(t, axis=-1) @ vb[h]
            lse[b, h, live] = _logsumexp_rows(t)
    return (out, lse) if return_lse else out


# ----------------------------------------------------------------------------
# Decode against a static cache
# ----------------------------------------------------------------------------
def decode_gqa(q, k_cache, v_cache, kv_len, scale: float):
    """One new query token per sequence: q [B,Hq,D], caches [B,Hkv,cap,D],
    kv_len [B] -> O [B,Hq,D].  Query head h attends to the first kv_len[b]
    slots of KV head h // G; later slots are never read.  No mask applies:
    the query's own key is already in the cache."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, v_cache.shape[-1]), dtype=np.float64)
    for b in range(B):
        n = int(kv_len[b])
        if n == 0:
            continue
        kb = repeat_kv(np.asarray(k_cache[b:b + 1, :, :n], dtype=np.float64), G)[0]
        vb = repeat_kv(np.asarray(v_cache[b:b + 1, :, :n], dtype=np.float64), G)[0]
        for h in range(Hq):
            p = softmax(scale * (kb[h] @ q[b, h]))
            out[b, h] = p @ vb[h]
    return out


def decode_mla(q, cache, kv_len, scale: float, d_latent: int):
    """Absorbed MLA decode: q [B,H,dl+dr], cache [B,cap,dl+dr] (latent then
    rope) -> O [B,H,dl].  Scores use all dl+dr dims; values are the latent
    part of the same cache rows."""
    q = np.asarray(q, dtype=np.float64)
    B, H, _ = q.shape
    out = np.zeros((B, H, d_latent), dtype=np.float64)
    for b in range(B):
        n = int(kv_len[b])
        if n == 0:
            continue
        c = np.asarray(cache[b, :n], dtype=np.float64)
        t = scale * (q[b] @ c.T)                      # [H, n]
        out[b] = softmax(t, axis=-1) @ c[:, :d_latent]
    return out


def mla_absorb_query(q_nope, q_rope, w_uk):
    """Absorbed query [W_UK[h] q_nope[b,h] ; q_rope[b,h]]: q_nope [B,H,dn],
    q_rope [B,H,dr], w_uk [H,dl,dn] -> [B,H,dl+dr]."""
    q_lat = np.einsum("hld,bhd->bhl", w_uk, q_nope)
    return np.concatenate([q_lat, q_rope], axis=-1)


def mla_unabsorbed(q_nope, q_rope, c_lat, c_rope, w_uk, w_uv, kv_len, scale: float):
    """MLA with the latent explicitly up-projected per head:
    K_h = [C_lat W_UK[h] ; C_rope], V_h = C_lat W_UV[h],
    o_h = softmax(scale [q_nope ; q_rope] K_h^T) V_h.
    q_nope [B,H,dn], q_rope [B,H,dr], c_lat [B,cap,dl], c_rope [B,cap,dr],
    w_uk [H,dl,dn], w_uv [H,dl,dv] -> [B,H,dv]."""
    B, H, _ = q_nope.shape
    dv = w_uv.shape[-1]
    out = np.zeros((B, H, dv), dtype=np.float64)
    for b in range(B):
        n = int(kv_len[b])
        if n == 0:
            continue
        for h in range(H):
            k_h = np.concatenate([c_lat[b, :n] @ w_uk[h], c_rope[b, :n]], axis=-1)
            v_h = c_lat[b, :n] @ w_uv[h]
            qh = np.concatenate([q_nope[b, h], q_rope[b, h]])
            out[b, h] = softmax(scale * (k_h @ qh)) @ v_h
    return out


# ----------------------------------------------------------------------------
# Softmax over a part of the keys, and the merge of parts
# ----------------------------------------------------------------------------
def partial_attention(q, k, v, scale: float):
    """Attention of q [D] over the keys k [n,D] / values v [n,Dv] alone:
    returns (normalised output [Dv], lse).  An empty part gives (0, -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1]), -np.inf
    t = scale * (k @ q)
    m = np.max(t)
    e = np.exp(t - m)
    return (e @ v) / np.sum(e), m + np.log(np.sum(e))


def merge_pair(o_a, lse_a, o_b, lse_b):
    """Merge two softmax parts (o normalised within its part, lse its
    log-sum-exp): alpha = sigmoid(lse_b - lse_a),
    o = (1 - alpha) o_a + alpha o_b, lse = log(exp(lse_a) + exp(lse_b))."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    if lse_a == -np.inf and lse_b == -np.inf:
        return np.zeros_like(o_a), -np.inf
    with np.errstate(over="ignore"):
        alpha = 1.0 / (1.0 + np.exp(lse_a - lse_b))
    return (1.0 - alpha) * o_a + alpha * o_b, np.logaddexp(lse_a, lse_b)


def merge(parts):
    """Fold ``merge_pair`` over a list of (o, lse) parts, left to right."""
    o, lse = parts[0]
    for o_b, lse_b in parts[1:]:
        o, lse = merge_pair(o, lse, o_b, lse_b)
    return o, lse


def combine_splits(o_part, lse_part):
    """Merge split partials: o_part [R,nsplit,D] (each normalised within its
    split), lse_part [R,nsplit] (natural log, -inf for an empty split)
    -> O [R,D] by folding ``merge_pair`` over the splits."""
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    R, ns, D = o_part.shape
    out = np.zeros((R, D), dtype=np.float64)
    for r in range(R):
        out[r] = merge([(o_part[r, s], lse_part[r, s]) for s in range(ns)])[0]
    return out
