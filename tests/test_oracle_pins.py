"""Pins for the float64 CPU oracle (no GPU).

Each check ties the oracle to something other than itself: a pure-Python
brute force, a library routine (torch's CPU scaled_dot_product_attention in
float64), closed forms, invariants of softmax attention and RoPE, and the
merge rule printed in the fixed-budget decode audit.  The mutation tests at
the end plant plausible mistakes in the oracle and check that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
from oracle import ref
from workloads import (decode_gqa_inputs, decode_mla_inputs, mla_projection_inputs,
                       prefill_inputs, split_partials, to_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_MATH = {k: getattr(math, k) for k in ("exp", "log", "cos", "sin", "sqrt")}


def _ev(s):
    return float(eval(s, {"__builtins__": {}}, _MATH))  # closed-form fixture strings


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# Pins written as functions of the oracle module, so that the mutation tests
# can run the same checks against a deliberately broken copy.
# ---------------------------------------------------------------------------
def pin_brute_force(mod, causal, rope_theta, B=2, Hq=4, Hkv=2, S=6, D=8, seed=0):
    q, k, v = _rand((B, Hq, S, D), seed), _rand((B, Hkv, S, D), seed + 1), _rand((B, Hkv, S, D), seed + 2)
    scale = 0.37
    got = mod.prefill(q, k, v, scale, causal, rope_theta)
    want = np.array(brute.prefill(q.tolist(), k.tolist(), v.tolist(), scale, causal, rope_theta))
    return np.max(np.abs(got - want))


def pin_sdpa(mod, causal, B=2, Hq=8, Hkv=2, S=33, D=16, seed=3):
    q, k, v = _rand((B, Hq, S, D), seed), _rand((B, Hkv, S, D), seed + 1), _rand((B, Hkv, S, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    got = mod.prefill(q, k, v, scale, causal)
    want = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          is_causal=causal, scale=scale, enable_gqa=True).numpy()
    return np.max(np.abs(got - want))


def pin_rope_complex(mod, D=16, theta=10000.0, seed=5):
    """RoPE as complex multiplication: z_i = x_i + j x_{i+D/2} turns by
    e^{j p w_i}, with w_0 = 1 and a constant ratio w_{i+1}/w_i = theta^(-2/D)."""
    x = _rand((7, D), seed)
    pos = np.arange(7) * 13
    got = mod.rope_rotate(x, pos, theta)
    half = D // 2
    w = np.empty(half)
    w[0] = 1.0
    for i in range(1, half):
        w[i] = w[i - 1] * theta ** (-2.0 / D)
    z = (x[:, :half] + 1j * x[:, half:]) * np.exp(1j * pos[:, None] * w[None, :])
    want = np.concatenate([z.real, z.imag], axis=-1)
    return np.max(np.abs(got - want))


def pin_merge_identity(mod, seed=7):
    rng = np.random.default_rng(seed)
    n, D = 40, 12
    q, k, v = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, 5))
    scale = 0.5
    o_full, lse_full = mod.partial_attention(q, k, v, scale)
    cuts = [0, 0, 7, 7, 19, 33, 40]          # includes empty parts
    parts = [mod.partial_attention(q, k[a:b], v[a:b], scale) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = mod.merge(parts)
    return max(np.max(np.abs(o - o_full)), abs(lse - lse_full))


# ---------------------------------------------------------------------------
# The pins proper
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rope_theta", [0.0, 10000.0, 50.0])
def test_brute_force_tiny(causal, rope_theta):
    assert pin_brute_force(ref, causal, rope_theta) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    assert pin_sdpa(ref, causal) <= 1e-12


def test_matches_torch_sdpa_mha_fp32_config_shape():
    # the tiny fp32 workload's shape, values exactly as the GPU would see them
    q, k, v = prefill_inputs(1, 4, 2, 128, 64, "f32")
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    got = oracle.prefill(qd, kd, vd, 1 / 8, True)
    want = F.scaled_dot_product_attention(torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(vd),
                                          is_causal=True, scale=1 / 8, enable_gqa=True).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((20, 16)), rng.standard_normal((20, 16))
    for causal in (False, True):
        p = oracle.attention_probs(q, k, 0.25, causal)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12
        assert np.all(p >= 0)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)
    t = rng.standard_normal((5, 9))
    assert np.max(np.abs(oracle.softmax(t) - oracle.softmax(t + 1e3))) <= 1e-12
    # decode and MLA rows also sum to one: a constant value row passes through unchanged
    qd, kc, vc, L = decode_gqa_inputs(2, 4, 2, 8, 12, 9, "f32")
    vc_const = np.ones_like(to_f64(vc))
    o = oracle.decode_gqa(to_f64(qd), to_f64(kc), vc_const, L.numpy(), 0.3)
    assert np.max(np.abs(o - 1.0)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_attention_probs_match_brute_force(causal):
    """attention_probs against the pure-Python brute force: attending to
    one-hot value rows (value j = e_j) returns the probability row itself, so
    brute.attend over the visible keys gives row i of the probabilities
    (zeros past the causal bound).  A doubled or dropped scale fails this."""
    rng = np.random.default_rng(11)
    S, D, scale = 9, 6, 0.37
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    p = oracle.attention_probs(q, k, scale, causal)
    for i in range(S):
        n = i + 1 if causal else S
        eye = [[1.0 if c == j else 0.0 for c in range(n)] for j in range(n)]
        want = brute.attend(list(q[i]), [list(r) for r in k[:n]], eye, scale) + [0.0] * (S - n)
        assert np.max(np.abs(p[i] - np.asarray(want))) <= 1e-12
    # sampled rows: the same probabilities by row index
    rows = [0, 4, 8]
    assert np.max(np.abs(oracle.attention_probs(q[rows], k, scale, causal, rows=rows) - p[rows])) <= 1e-15
    # a planted doubled scale is caught
    bad = oracle.attention_probs(q, k, 2 * scale, causal)
    assert np.max(np.abs(bad - p)) > 1e-3


def test_causal_invariance():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, S, D = 1, 4, 2, 24, 8
    q, k, v = rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    for rope in (0.0, 10000.0):
        base = oracle.prefill(q, k, v, 0.3, True, rope)
        for t in (0, 5, 17):
            k2, v2 = k.copy(), v.copy()
            k2[:, :, t + 1:] += 100 * rng.standard_normal(k2[:, :, t + 1:].shape)
            v2[:, :, t + 1:] -= 50.0
            pert = oracle.prefill(q, k2, v2, 0.3, True, rope)
            assert np.max(np.abs(pert[:, :, :t + 1] - base[:, :, :t + 1])) <= 1e-15
        # row 0 attends only to key 0, so it equals V[0] of its KV head exactly
        assert np.array_equal(base[0, :, 0], np.repeat(v[0, :, 0], Hq // Hkv, axis=0))


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, S, D = 2, 6, 3, 10, 4
    q, k, v = rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    got = oracle.prefill(q, k, v, 0.5, True, 10000.0)
    # brute force indexes KV head h // G; MHA input built by hand head by head
    k_mha = np.stack([k[:, h // 2] for h in range(Hq)], axis=1)
    v_mha = np.stack([v[:, h // 2] for h in range(Hq)], axis=1)
    mha = np.array(brute.prefill(q.tolist(), k_mha.tolist(), v_mha.tolist(), 0.5, True, 10000.0))
    assert np.max(np.abs(got - mha)) <= 1e-12


@pytest.mark.parametrize("rope_theta", [0.0, 10000.0])
def test_decode_equals_prefill_row(rope_theta):
    B, Hq, Hkv, S, D = 2, 8, 2, 200, 16
    q, k, v = prefill_inputs(B, Hq, Hkv, S, D, "f32", seed=11)
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    full = oracle.prefill(qd, kd, vd, 0.25, True, rope_theta)
    cap = S + 8
    for t in (0, 1, 127, S - 1):
        # cache holds rows 0..t (already rotated when RoPE is on), then garbage
        kc = np.full((B, Hkv, cap, D), np.nan)
        vc = np.full((B, Hkv, cap, D), np.nan)
        krot = oracle.rope_rotate(kd, np.arange(S), rope_theta) if rope_theta > 0 else kd
        kc[:, :, :t + 1] = krot[:, :, :t + 1]
        vc[:, :, :t + 1] = vd[:, :, :t + 1]
        qt = qd[:, :, t]
        if rope_theta > 0:
            qt = oracle.rope_rotate(qt[:, :, None, :], [t], rope_theta)[:, :, 0]
        dec = oracle.decode_gqa(qt, kc, vc, np.array([t + 1] * B), 0.25)
        assert np.max(np.abs(dec - full[:, :, t])) <= 1e-12


def test_decode_brute_force_ragged_lengths():
    q, kc, vc, L = decode_gqa_inputs(3, 4, 2, 8, 20, 0, "f32", lengths=[1, 13, 0], nan_tail=True)
    got = oracle.decode_gqa(to_f64(q), to_f64(kc), to_f64(vc), L.numpy(), 0.4)
    want = np.array(brute.decode(to_f64(q).tolist(), to_f64(kc).tolist(), to_f64(vc).tolist(), [1, 13, 0], 0.4))
    assert np.max(np.abs(got - want)) <= 1e-12
    assert np.all(got[2] == 0.0)


def test_mla_absorbed_equals_unabsorbed():
    B, H, dl, dr, dn, dv, cap, L = 2, 16, 448, 64, 128, 128, 40, 33
    q_nope, q_rope, w_uk, w_uv = mla_projection_inputs(B, H, dl, dr, dn, dv)
    _, c, kv_len = decode_mla_inputs(B, H, dl, dr, cap, L, "f32")
    cd = to_f64(c)
    scale = 1 / math.sqrt(dn + dr)
    ref_o = oracle.mla_unabsorbed(q_nope, q_rope, cd[..., :dl], cd[..., dl:], w_uk, w_uv, kv_len.numpy(), scale)
    q_abs = oracle.mla_absorb_query(q_nope, q_rope, w_uk)
    lat = oracle.decode_mla(q_abs, cd, kv_len.numpy(), scale, dl)
    o_abs = np.einsum("bhl,hlv->bhv", lat, w_uv)
    rel = np.max(np.abs(o_abs - ref_o)) / np.max(np.abs(ref_o))
    assert rel <= 1e-10


def test_mla_matches_brute_force_decode():
    # MLA decode is single-KV-head decode whose values are the latent part
    B, H, dl, dr, cap = 2, 3, 6, 2, 9
    q, c, L = decode_mla_inputs(B, H, dl, dr, cap, 0, "f32", lengths=[5, 9])
    qd, cd = to_f64(q), to_f64(c)
    got = oracle.decode_mla(qd, cd, L.numpy(), 0.7, dl)
    kc = cd[:, None]
    vc = cd[:, None, :, :dl]
    want = np.array(brute.decode(qd.tolist(), kc.tolist(), vc.tolist(), [5, 9], 0.7))
    assert np.max(np.abs(got - want)) <= 1e-12


def test_rope_invariants():
    rng = np.random.default_rng(9)
    D, theta = 128, 10000.0
    x = rng.standard_normal((5, D))
    # R_0 is the identity, exactly
    assert np.array_equal(oracle.rope_rotate(x, np.zeros(5), theta), x)
    # rotation preserves norms
    r = oracle.rope_rotate(x, np.arange(5) * 411, theta)
    assert np.max(np.abs(np.linalg.norm(r, axis=1) - np.linalg.norm(x, axis=1))) <= 1e-12
    # scores depend only on the relative position
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n, c in ((3, 10, 100), (0, 2047, 5), (700, 12, 1000)):
        a = oracle.rope_rotate(q[None], [m], theta)[0] @ oracle.rope_rotate(k[None], [n], theta)[0]
        b = oracle.rope_rotate(q[None], [m + c], theta)[0] @ oracle.rope_rotate(k[None], [n + c], theta)[0]
        assert abs(a - b) <= 1e-10
    assert pin_rope_complex(ref) <= 1e-12


def test_rope_golden_d4():
    g = _golden("rope_d4.json")
    x = np.array([[_ev(s) for s in g["x"]]])
    got = oracle.rope_rotate(x, [_ev(g["position"])], _ev(g["theta"]))[0]
    want = np.array([_ev(s) for s in g["expected"]])
    assert np.max(np.abs(got - want)) <= 1e-15


def test_attention_golden_closed_form():
    g = _golden("attention_closed_form.json")
    arr = lambda a: np.array([[_ev(s) for s in row] for row in a])[None, None]  # noqa: E731
    got = oracle.prefill(arr(g["q"]), arr(g["k"]), arr(g["v"]), _ev(g["scale"]), g["causal"])[0, 0]
    want = np.array([[_ev(s) for s in row] for row in g["expected"]])
    assert np.max(np.abs(got - want)) <= 1e-15


def test_closed_forms():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, D = 1, 2, 1, 30, 8
    v = rng.standard_normal((B, Hkv, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    # q = 0: uniform weights, so O_i = mean of V_0..V_i (causal) or of all V
    q0 = np.zeros((B, Hq, S, D))
    o = oracle.prefill(q0, k, v, 0.3, True)
    cum = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    assert np.max(np.abs(o[0, 0] - cum)) <= 1e-12
    o = oracle.prefill(q0, k, v, 0.3, False)
    assert np.max(np.abs(o[0, 1] - v[0, 0].mean(0))) <= 1e-12
    # identical keys: uniform weights whatever q is
    kid = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o = oracle.prefill(rng.standard_normal((B, Hq, S, D)), kid, v, 0.3, True)
    assert np.max(np.abs(o[0, 0] - cum)) <= 1e-12
    # S = 1: the output is V
    o = oracle.prefill(rng.standard_normal((B, Hq, 1, D)), k[:, :, :1], v[:, :, :1], 0.3, True, 10000.0)
    assert np.array_equal(o[0, 0], v[0, 0, :1]) and np.array_equal(o[0, 1], v[0, 0, :1])


def test_lse_output():
    rng = np.random.default_rng(13)
    q, k, v = rng.standard_normal((1, 2, 9, 4)), rng.standard_normal((1, 1, 9, 4)), rng.standard_normal((1, 1, 9, 4))
    _, lse = oracle.prefill(q, k, v, 0.5, True, 0.0, return_lse=True)
    for h in range(2):
        for i in range(9):
            s = [0.5 * math.fsum(q[0, h, i] * k[0, 0, j]) for j in range(i + 1)]
            assert abs(lse[0, h, i] - math.log(math.fsum(math.exp(x) for x in s))) <= 1e-12


def test_prefill_rows_matches_prefill():
    q, k, v = prefill_inputs(1, 4, 1, 300, 32, "f32", seed=21)
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    full, lse = oracle.prefill(qd, kd, vd, 0.2, True, 10000.0, return_lse=True, row_chunk=64)
    rows = [0, 1, 63, 64, 200, 299]
    o, l = oracle.prefill_rows(q.numpy(), k.numpy(), v.numpy(), 0.2, True, 10000.0, 0, 3, rows)
    assert np.max(np.abs(o - full[0, 3, rows])) <= 1e-12
    assert np.max(np.abs(l - lse[0, 3, rows])) <= 1e-12


def test_merge_identity():
    assert pin_merge_identity(ref) <= 1e-12


def test_merge_golden_worked_example():
    g = _golden("merge_worked_example.json")
    hs = np.array([_ev(s) for s in g["history_scores"]])
    hv = np.array([[_ev(s)] for s in g["history_values"]])
    # scores are <q,k> with q = [1] and k = score, scale 1
    o_h, lse_h = oracle.partial_attention(np.array([1.0]), hs[:, None], hv, 1.0)
    assert abs(o_h[0] - _ev(g["expected_history_output"])) <= 1e-15
    assert abs(lse_h - _ev(g["expected_history_lse"])) <= 1e-15
    cs = _ev(g["current_score"])
    o, lse = oracle.merge_pair(o_h, lse_h, np.array([_ev(g["current_value"])]), cs)
    assert abs(o[0] - _ev(g["expected_output"])) <= 1e-14
    assert abs(lse - _ev(g["expected_lse"])) <= 1e-14
    alpha = 1.0 / (1.0 + math.exp(lse_h - cs))
    assert abs(alpha - _ev(g["expected_alpha"])) <= 1e-15


def test_combine_splits_equals_full_softmax():
    # split a decode row's keys at multiples of 32 (a ragged last split and
    # empty splits past the length), then combine
    q, kc, vc, L = decode_gqa_inputs(1, 2, 1, 16, 200, 0, "f32", lengths=[150])
    qd, kd, vd = to_f64(q), to_f64(kc), to_f64(vc)
    full = oracle.decode_gqa(qd, kd, vd, L.numpy(), 0.25)
    split = 32
    ns = (200 + split - 1) // split
    o_part = np.zeros((2, ns, 16))
    lse_part = np.zeros((2, ns))
    for h in range(2):
        for s in range(ns):
            a, b = s * split, min((s + 1) * split, 150)
            o_part[h, s], lse_part[h, s] = oracle.partial_attention(qd[0, h], kd[0, 0, a:max(a, b)], vd[0, 0, a:max(a, b)], 0.25)
    assert np.isinf(lse_part[0, -1])
    got = oracle.combine_splits(o_part, lse_part)
    assert np.max(np.abs(got - full[0])) <= 1e-12


def test_combine_splits_handles_all_empty_rows():
    o, lse = split_partials(3, 4, 8, empty_every=1)
    got = oracle.combine_splits(o.numpy(), lse.numpy())
    assert np.all(got == 0.0)


# ---------------------------------------------------------------------------
# Decode neighbours: cache append and chunked prefill
# ---------------------------------------------------------------------------
def pin_chunked_prefill(mod, S=70, T=32, theta=10000.0, prefix=(0, 9), seed=11):
    """Prefill a prompt chunk by chunk through kv_append + prefill_chunk (each
    sequence may already hold a prefix in its cache) and compare every row
    with the one-shot prefill of the whole sequence.  Returns the max error."""
    B, Hq, Hkv, D = 2, 4, 2, 8
    scale = 0.4
    tot = S + max(prefix)
    q, k, v = _rand((B, Hq, tot, D), seed), _rand((B, Hkv, tot, D), seed + 1), _rand((B, Hkv, tot, D), seed + 2)
    cap = tot + 5
    kc = np.full((B, Hkv, cap, D), np.nan)
    vc = np.full((B, Hkv, cap, D), np.nan)
    L = np.zeros(B, dtype=np.int64)
    err = 0.0
    # the prefix of sequence b goes in first (one append of its own length per sequence)
    for b in range(B):
        if prefix[b]:
            kb, vb, _, _ = mod.kv_append(kc[b:b + 1], vc[b:b + 1], L[b:b + 1], k[b:b + 1, :, :prefix[b]],
                                         v[b:b + 1, :, :prefix[b]], theta)
            kc[b:b + 1], vc[b:b + 1] = kb, vb
            L[b] = prefix[b]
    outs = [[] for _ in range(B)]
    for c0 in range(0, S, T):
        c1 = min(S, c0 + T)
        sl = [slice(prefix[b] + c0, prefix[b] + c1) for b in range(B)]
        kn = np.stack([k[b, :, sl[b]] for b in range(B)])
        vn = np.stack([v[b, :, sl[b]] for b in range(B)])
        qn = np.stack([q[b, :, sl[b]] for b in range(B)])
        kc, vc, L, qr = mod.kv_append(kc, vc, L, kn, vn, theta, qn)
        o = mod.prefill_chunk(qr, kc, vc, L, scale)
        for b in range(B):
            outs[b].append(o[b])
    for b in range(B):
        n = prefix[b] + S
        want = mod.prefill(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale, True, theta)[0]
        got = np.concatenate(outs[b], axis=1)
        e = float(np.max(np.abs(got - want[:, prefix[b]:])))
        err = np.inf if np.isnan(e) else max(err, e)
    return err


@pytest.mark.parametrize("theta,T", [(10000.0, 32), (0.0, 32), (10000.0, 1), (500.0, 17)])
def test_chunked_prefill_equals_one_shot_prefill(theta, T):
    """Chunks of 32 (and 1, and 17) over prefixes of 0 and 9 tokens reproduce
    the one-shot causal RoPE prefill row for row."""
    assert pin_chunked_prefill(ref, T=T, theta=theta) <= 1e-12


def test_decode_equals_chunk_of_one():
    B, Hq, Hkv, D, cap = 3, 8, 2, 16, 40
    k = _rand((B, Hkv, cap, D), 21)
    v = _rand((B, Hkv, cap, D), 22)
    q = _rand((B, Hq, D), 23)
    L = np.array([1, 17, 40])
    want = ref.decode_gqa(q, k, v, L, 0.3)
    got = ref.prefill_chunk(q[:, :, None], k, v, L, 0.3)[:, :, 0]
    assert np.max(np.abs(got - want)) <= 1e-12


def test_kv_append_slots_values_and_positions():
    """Only slots L..L+T-1 change; V is copied bit for bit; with theta = 0 so is
    K; with RoPE, appending one token at a time gives the same cache as one
    append of all of them (the slot index is the position)."""
    B, Hkv, Hq, T, D, cap = 2, 2, 4, 5, 8, 16
    kc = np.full((B, Hkv, cap, D), np.nan)
    vc = np.full((B, Hkv, cap, D), np.nan)
    L = np.array([0, 7])
    kn, vn, qn = _rand((B, Hkv, T, D), 31), _rand((B, Hkv, T, D), 32), _rand((B, Hq, T, D), 33)
    k0, v0, L0, q0 = ref.kv_append(kc, vc, L, kn, vn, 0.0, qn)
    assert np.array_equal(L0, L + T)
    for b in range(B):
        assert np.array_equal(k0[b, :, L[b]:L[b] + T], kn[b]) and np.array_equal(v0[b, :, L[b]:L[b] + T], vn[b])
        outside = np.ones(cap, dtype=bool)
        outside[L[b]:L[b] + T] = False
        assert np.all(np.isnan(k0[b][:, outside])) and np.all(np.isnan(v0[b][:, outside]))
    assert np.array_equal(q0, qn)
    k1, v1, _, q1 = ref.kv_append(kc, vc, L, kn, vn, 10000.0, qn)
    ks, vs, Ls = kc, vc, L
    qs = []
    for t in range(T):
        ks, vs, Ls, qt = ref.kv_append(ks, vs, Ls, kn[:, :, t:t + 1], vn[:, :, t:t + 1], 10000.0, qn[:, :, t:t + 1])
        qs.append(qt)
    assert np.allclose(k1, ks, atol=1e-14, equal_nan=True) and np.array_equal(v1, vs, equal_nan=True)
    assert np.allclose(q1, np.concatenate(qs, axis=2), atol=1e-14)
    # norms are preserved (a rotation) and position 0 is the identity
    for b in range(B):
        np.testing.assert_allclose(np.linalg.norm(k1[b, :, L[b]:L[b] + T], axis=-1), np.linalg.norm(kn[b], axis=-1),
                                   rtol=1e-13)
    assert np.allclose(k1[0, :, 0], kn[0, :, 0], atol=1e-15)


def test_prefill_chunk_rows_without_keys():
    """kv_len below the chunk length: rows at negative positions see no key."""
    k, v, q = _rand((1, 1, 8, 4), 41), _rand((1, 1, 8, 4), 42), _rand((1, 1, 5, 4), 43)
    o, lse = ref.prefill_chunk(q, k, v, np.array([3]), 0.5, return_lse=True)
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.allclose(o[0, 0, 2], v[0, 0, 0])  # position 0 sees only key 0


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin.
# ---------------------------------------------------------------------------
def _mutant_tile_kv(k, G):          # GQA head h -> KV head h % Hkv instead of h // G
    return np.tile(k, (1, G) + (1,) * (k.ndim - 2))


def _mutant_rope_interleaved(x, positions, theta):   # pairs (2i, 2i+1) instead of (i, i+D/2)
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * ref.rope_inv_freq(D, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


_rope_rotate_orig = ref.rope_rotate


def _mutant_rope_sign(x, positions, theta):          # rotation by the opposite angle
    return _rope_rotate_orig(x, -np.asarray(positions, dtype=np.float64), theta)


def _mutant_mask_off_by_one(rows, n_keys):           # hides the diagonal too
    return np.arange(n_keys)[None, :] >= np.asarray(rows)[:, None]


def _mutant_merge_flip(o_a, lse_a, o_b, lse_b):      # alpha = sigmoid(lse_a - lse_b)
    alpha = 1.0 / (1.0 + np.exp(lse_b - lse_a))
    return (1 - alpha) * np.asarray(o_a) + alpha * np.asarray(o_b), np.logaddexp(lse_a, lse_b)


def _mutant_inv_freq(D, theta):                      # exponent i/D instead of 2i/D
    return np.power(float(theta), -np.arange(D // 2) / D)


_kv_append_orig = ref.kv_append
_prefill_chunk_orig = ref.prefill_chunk


def _mutant_append_position(k_cache, v_cache, kv_len, k_new, v_new, rope_theta, q_new=None):
    # K rotated one position too far (slot index + 1)
    k_new = _rope_rotate_orig(np.asarray(k_new, dtype=np.float64), np.ones(k_new.shape[2]), rope_theta)
    return _kv_append_orig(k_cache, v_cache, kv_len, k_new, v_new, rope_theta, q_new)


def _mutant_chunk_offset(q, k_cache, v_cache, kv_len, scale, return_lse=False):
    # chunk rows placed one position early (and the last prefix slot dropped)
    return _prefill_chunk_orig(q, k_cache, v_cache, np.asarray(kv_len) - 1, scale, return_lse)


@pytest.mark.parametrize("name,attr,fn,pin", [
    ("gqa-tile", "repeat_kv", _mutant_tile_kv, lambda m: pin_sdpa(m, True)),
    ("rope-interleaved", "rope_rotate", _mutant_rope_interleaved, lambda m: pin_rope_complex(m)),
    ("rope-sign", "rope_rotate", _mutant_rope_sign, lambda m: pin_rope_complex(m)),
    ("rope-freq", "rope_inv_freq", _mutant_inv_freq, lambda m: pin_rope_complex(m)),
    ("rope-freq-prefill", "rope_inv_freq", _mutant_inv_freq, lambda m: pin_brute_force(m, True, 10000.0)),
    ("mask-off-by-one", "_causal_mask", _mutant_mask_off_by_one, lambda m: pin_sdpa(m, True)),
    ("merge-flip", "merge_pair", _mutant_merge_flip, lambda m: pin_merge_identity(m)),
    ("append-position", "kv_append", _mutant_append_position, lambda m: pin_chunked_prefill(m)),
    ("chunk-offset", "prefill_chunk", _mutant_chunk_offset, lambda m: pin_chunked_prefill(m)),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn, pin):
    monkeypatch.setattr(ref, attr, fn)
    with np.errstate(all="ignore"):
        err = pin(ref)
    assert not (err <= 1e-6), f"planted mistake {name} went unnoticed (err={err})"
