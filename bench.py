"""Benchmark of the attention forward hot path on one MI355X.

A step is one causal GQA prefill with fused RoPE at the full workload
(B=1, Hq=32, Hkv=8, S=2048, D=128, bf16 in and out, theta 10000): the K
rotation into the workspace, then the attention kernel, which rotates its Q
rows in registers.  ``value`` is its throughput in useful TFLOP/s
(4 * B * Hq * D * S(S+1)/2 flops per step, masked work excluded), with inputs
resident in HBM.  The same JSON line carries the roofline of that kernel, the
CPU float64 oracle timed on a bounded sample of the same workload, and the
other paths (GQA and MLA decode in eager and hipGraph modes, MHA forward in
fp16 / fp8, the tiny fp32 prefill) as secondary figures.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick [--prefill-config N]]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s (% MFMA peak); decode µs/step and HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(B, H, S, D, causal):
    return 4.0 * B * H * D * (S * (S + 1) / 2 if causal else S * S)


def gqa_decode_bytes(B, Hq=16, Hkv=4, D=128, L=2048, elem=2):
    return B * (L * Hkv * D * 2 * elem + 2 * Hq * D * elem)


def mla_decode_bytes(B, H=16, dq=512, dl=448, L=2048, elem=2):
    return B * (L * dq * elem + H * dq * elem + H * dl * elem)


GLOBAL_CONFIG = 7  # the library's global 16-bit prefill configuration (what the calls without one use)

SPIN_S = 0.06  # untimed work before each measurement: the clock takes ~45 ms of load to settle


def spin(fn, seconds=SPIN_S):
    """Run fn() back to back for about `seconds` of wall time (untimed), so that
    the measurement that follows sees the clock it settles at under load."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break


def time_loop(fn, iters, warmup):
    """Average ms per call of fn() over `iters` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    spin(fn)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def time_graph(fn, steps_per_graph, replays, warmup=2):
    """ms per step with `steps_per_graph` calls captured in one hipGraph."""
    import torch
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for _ in range(steps_per_graph):
            fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    spin(g.replay)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (replays * steps_per_graph)


LLC_BYTES = 256 << 20         # MI355X last-level (Infinity) cache


def cache_sets(step_bytes):
    """Number of input copies that makes a rotation stream from HBM."""
    return max(2, -(-2 * LLC_BYTES // step_bytes) + 1)


def decode_case(kind, B, split, scale, graph_steps=20, modes=("warm", "cold"), iters=50):
    """Time one decode shape (split kernel + combine) in eager and hipGraph mode."""
    import torch
    import attention_flash_attn_02_amd as attn
    from workloads import decode_gqa_inputs, decode_mla_inputs
    dev = torch.device("cuda:0")
    if kind == "gqa":
        q, kc, vc, L = [t.to(dev) for t in decode_gqa_inputs(B, 16, 4, 128, 2056, 2048, "bf16")]
        by = gqa_decode_bytes(B)
        caches = [(kc, vc)]
        ws = torch.empty(attn.decode_gqa_workspace_bytes(B, 16, 2056, 128, split), dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        mk = lambda c: (lambda: attn.decode_gqa(q, c[0], c[1], L, scale, split=split, out=o, workspace=ws))  # noqa: E731
    else:
        q, cm, L = [t.to(dev) for t in decode_mla_inputs(B, 16, 448, 64, 2056, 2048, "bf16")]
        by = mla_decode_bytes(B)
        caches = [(cm,)]
        ws = torch.empty(attn.decode_mla_workspace_bytes(B, 16, 2056, 448, split), dtype=torch.uint8, device=dev)
        o = torch.empty((B, 16, 448), dtype=torch.bfloat16, device=dev)
        mk = lambda c: (lambda: attn.decode_mla(q, c[0], L, scale, split=split, out=o, workspace=ws))  # noqa: E731
    res = {"bytes": by}
    for mode in modes:
        if mode == "cold":
            n = cache_sets(by)
            while len(caches) < n:
                caches.append(tuple(t.clone() for t in caches[0]))
            fns = [mk(c) for c in caches]
        else:
            fns = [mk(caches[0])]
        k = [0]

        def step():
            fns[k[0] % len(fns)]()
            k[0] += 1
        me = time_loop(step, max(iters, len(fns)), 5)
        mg = time_graph(step, max(graph_steps, len(fns)) if mode == "cold" else graph_steps, 5)
        res[mode] = {"eager_us": round(me * 1e3, 2), "graph_us": round(mg * 1e3, 2),
                     "graph_GBs": round(by / (mg * 1e-3) / 1e9, 1),
                     "graph_frac": round(by / (mg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "eager_GBs": round(by / (me * 1e-3) / 1e9, 1), "sets": len(fns)}
    del caches, ws, o, q
    torch.cuda.empty_cache()
    return res


def rope_factorial(graph_steps=20, iters=50):
    """RoPE fused into the attention kernel (K rotated per staged tile, or
    once per key by a pre-pass into a workspace; Q in registers either way)
    vs RoPE as separate kernels (attn_rope_rotate on Q and K, then attention
    without RoPE), in eager and hipGraph mode, warm (one input set) and cold
    (inputs rotated over enough copies to exceed twice the last-level cache),
    on the causal GQA RoPE prefill workload."""
    import torch
    import attention_flash_attn_02_amd as attn
    from workloads import prefill_inputs
    dev = torch.device("cuda:0")
    B, Hq, Hkv, S, D = 1, 32, 8, 2048, 128
    scale = 1 / math.sqrt(D)
    q, k, v = [t.to(dev) for t in prefill_inputs(B, Hq, Hkv, S, D, "bf16")]
    flops = prefill_flops(B, Hq, S, D, True)
    set_bytes = 2 * (q.numel() + k.numel() + v.numel() + q.numel())  # q, k, v in, o out
    out = {}
    for mode in ("warm", "cold"):
        n = 1 if mode == "warm" else cache_sets(set_bytes)
        sets = [(q, k, v)] + [(q.clone(), k.clone(), v.clone()) for _ in range(n - 1)]
        outs = [torch.empty_like(q) for _ in range(n)]
        qr = [torch.empty_like(q) for _ in range(n)]
        kr = [torch.empty_like(k) for _ in range(n)]
        wsb = attn.prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, torch.bfloat16, 10000.0)
        ws = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(n)]
        for variant in ("fused_k_per_tile", "fused_k_once", "unfused"):
            if variant == "fused_k_per_tile":
                fns = [lambda i=i: attn.prefill_gqa_rope(*sets[i], scale, causal=True, rope_theta=10000.0, out=outs[i],
                                                         k_rope="per_tile")
                       for i in range(n)]
            elif variant == "fused_k_once":
                fns = [lambda i=i: attn.prefill_gqa_rope(*sets[i], scale, causal=True, rope_theta=10000.0, out=outs[i],
                                                         workspace=ws[i])
                       for i in range(n)]
            else:
                fns = [lambda i=i: attn.prefill_gqa_rope_unfused(*sets[i], scale, causal=True, rope_theta=10000.0,
                                                                 out=outs[i], q_rot=qr[i], k_rot=kr[i])
                       for i in range(n)]
            c = [0]

            def step():
                fns[c[0] % n]()
                c[0] += 1
            me = time_loop(step, max(iters, n), 5)
            mg = time_graph(step, max(graph_steps, n), 5)
            out[f"{variant}_{mode}"] = {"eager_us": round(me * 1e3, 2), "graph_us": round(mg * 1e3, 2),
                                        "eager_tflops": round(flops / (me * 1e-3) / 1e12, 1),
                                        "graph_tflops": round(flops / (mg * 1e-3) / 1e12, 1), "sets": n}
        del sets, outs, qr, kr, ws
        torch.cuda.empty_cache()
    return out


def decode_neighbours(iters=50):
    """The steps on either side of decode attention: (1) a decode step of the
    GQA decode workload (B=128) with the new token appended first
    (attn_kv_append with RoPE, then attn_decode_gqa), and the append alone;
    (2) the causal GQA RoPE prefill prompt (S=2048) prefilled in chunks of 32
    (attn_prefill_chunk_step per chunk; also as attn_kv_append then
    attn_prefill_chunk) against the one-shot fused prefill.  hipGraph
    replay, warm."""
    import torch
    import attention_flash_attn_02_amd as attn
    from workloads import decode_gqa_inputs, prefill_inputs, randn
    dev = torch.device("cuda:0")
    out = {}
    B, Hq, Hkv, D, cap = 128, 16, 4, 128, 2056
    scale = 1 / math.sqrt(D)
    q, kc, vc, L = [t.to(dev) for t in decode_gqa_inputs(B, Hq, Hkv, D, cap, 2048, "bf16")]
    L_app = L - 1  # the new token goes to slot 2047, decode then attends 2048 keys
    kn = randn((B, Hkv, 1, D), "bf16", 5, "k").to(dev)
    vn = randn((B, Hkv, 1, D), "bf16", 5, "v").to(dev)
    qn = q.view(B, Hq, 1, D)
    o = torch.empty_like(q)
    ws = torch.empty(attn.decode_gqa_workspace_bytes(B, Hq, cap, D), dtype=torch.uint8, device=dev)
    app = lambda: attn.kv_append(kn, vn, kc, vc, L_app, rope_theta=10000.0, q=qn, advance=False)  # noqa: E731

    def step():
        app()
        attn.decode_gqa(q, kc, vc, L, scale, out=o, workspace=ws)
    ma = time_graph(app, 20, 5)
    ms = time_graph(step, 20, 5)
    by = gqa_decode_bytes(B)
    out["decode_step_B128"] = {"append_us": round(ma * 1e3, 2), "append_plus_decode_us": round(ms * 1e3, 2),
                               "decode_bytes": by, "step_GBs": round(by / (ms * 1e-3) / 1e9, 1)}
    del q, kc, vc, L, o, ws
    B, Hq, Hkv, S, D, T = 1, 32, 8, 2048, 128, 32
    scale = 1 / math.sqrt(D)
    q, k, v = [t.to(dev) for t in prefill_inputs(B, Hq, Hkv, S, D, "bf16")]
    chunks = [(q[:, :, c:c + T].contiguous(), k[:, :, c:c + T].contiguous(), v[:, :, c:c + T].contiguous())
              for c in range(0, S, T)]
    kc = torch.empty((B, Hkv, S, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    Lc = torch.zeros(B, dtype=torch.int32, device=dev)
    oc = [torch.empty_like(c[0]) for c in chunks]
    wsc = torch.empty(max(1, attn.prefill_chunk_workspace_bytes(B, Hq, Hkv, T, D, S)), dtype=torch.uint8,
                      device=dev)

    # per chunk, one call: append K (rotated) and V, the chunk's attention with
    # its queries rotated in the kernel, and the advance of kv_len in its last
    # launch (attn_prefill_chunk_step)
    def chunked():
        Lc.zero_()
        for (qc, kk, vv), oo in zip(chunks, oc):
            attn.prefill_chunk_step(qc, kk, vv, kc, vc, Lc, scale, out=oo, workspace=wsc, rope_theta=10000.0)

    # the same as two calls: append with its own advance, then the attention
    def chunked_two_calls():
        Lc.zero_()
        for (qc, kk, vv), oo in zip(chunks, oc):
            attn.kv_append(kk, vv, kc, vc, Lc, rope_theta=10000.0)
            attn.prefill_chunk(qc, kc, vc, Lc, scale, out=oo, workspace=wsc, rope_theta=10000.0)
    fo = torch.empty_like(q)
    fws = torch.empty(attn.prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, torch.bfloat16, 10000.0),
                      dtype=torch.uint8, device=dev)
    mc = time_graph(chunked, 1, 5)
    m2 = time_graph(chunked_two_calls, 1, 5)
    mf = time_graph(lambda: attn.prefill_gqa_rope(q, k, v, scale, causal=True, rope_theta=10000.0, out=fo,
                                                  workspace=fws), 20, 5)
    flops = prefill_flops(B, Hq, S, D, True)
    out["chunked_prefill_S2048_T32"] = {"chunked_us": round(mc * 1e3, 2), "two_calls_per_chunk_us": round(m2 * 1e3, 2),
                                        "one_shot_fused_us": round(mf * 1e3, 2),
                                        "chunked_tflops": round(flops / (mc * 1e-3) / 1e12, 1),
                                        "chunks": len(chunks)}
    torch.cuda.empty_cache()
    return out


SWEEP_ROUNDS = 3


def sweep(scale):
    """Every tile configuration per shape; gap of the global configuration to the best one.

    Prefill: attn_prefill_gqa_rope_with_config ids (the global one is
    GLOBAL_CONFIG, the software-pipelined kernel, for 16-bit and fp8 inputs;
    fp8 inputs also have configuration 0, the 4-wave kernel with P in e4m3,
    and 1, P in f16), timed in
    SWEEP_ROUNDS interleaved rounds (seeded random order), median per
    configuration.  Decode: the split size (global = the library default),
    hipGraph mode, cold caches."""
    import torch
    import attention_flash_attn_02_amd as attn
    from workloads import prefill_inputs
    dev = torch.device("cuda:0")
    out = {}
    nconf = attn.prefill_num_configs()
    all16 = list(range(nconf))
    shapes = [("C2_gqa_rope_bf16_S2048", (1, 32, 8, 2048, 128, "bf16", True, 10000.0, torch.bfloat16), all16, GLOBAL_CONFIG),
              ("mha_D64_noncausal_N4096_f16", (4, 32, 32, 4096, 64, "f16", False, 0.0, torch.float16), all16, GLOBAL_CONFIG),
              ("mha_D128_causal_N4096_f16", (4, 32, 32, 4096, 128, "f16", True, 0.0, torch.float16), all16, GLOBAL_CONFIG),
              ("mha_D128_causal_N16384_f16", (4, 32, 32, 16384, 128, "f16", True, 0.0, torch.float16), all16,
               GLOBAL_CONFIG),
              ("mha_D64_noncausal_N1024_f16", (4, 32, 32, 1024, 64, "f16", False, 0.0, torch.float16), all16,
               GLOBAL_CONFIG),
              ("mha_D128_causal_N2048_f16", (4, 32, 32, 2048, 128, "f16", True, 0.0, torch.float16), all16, GLOBAL_CONFIG),
              ("mha_D64_noncausal_N8192_f16", (4, 32, 32, 8192, 64, "f16", False, 0.0, torch.float16), all16,
               GLOBAL_CONFIG),
              ("mha_D64_noncausal_N4096_fp8", (4, 32, 32, 4096, 64, "fp8_e5m2", False, 0.0, torch.float16), [0, 1, 7],
               GLOBAL_CONFIG),
              ("mha_D128_causal_N4096_fp8", (4, 32, 32, 4096, 128, "fp8_e5m2", True, 0.0, torch.float16), [0, 1, 7],
               GLOBAL_CONFIG)]
    for name, (B, Hq, Hkv, S, D, dt, causal, theta, odt), confs, glob in shapes:
        q, k, v = [t.to(dev) for t in prefill_inputs(B, Hq, Hkv, S, D, dt, seed=S)]
        o = torch.empty(q.shape, dtype=odt, device=dev)
        ws = torch.empty(max(1, attn.prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, q.dtype, theta)),
                         dtype=torch.uint8, device=dev)
        it = 20 if S <= 4096 else 4
        # configurations interleaved over rounds in a seeded random order, median per configuration
        rng = random.Random(S * 7 + D)
        samples = {c: [] for c in confs}
        for rnd in range(SWEEP_ROUNDS):
            order = list(confs)
            rng.shuffle(order)
            for c in order:
                ms = time_loop(lambda: attn.prefill_gqa_rope(q, k, v, 1 / math.sqrt(D), causal=causal,
                                                            rope_theta=theta, out=o, config=c, workspace=ws),
                               it, 2)
                samples[c].append(ms)
        times = {str(c): round(sorted(v)[len(v) // 2] * 1e3, 2) for c, v in samples.items()}
        best = min(times.values())
        g = str(glob)
        out["prefill_" + name] = {"us": times, "global": g, "best": min(times, key=times.get),
                                  "gap_pct": round(100 * (times[g] / best - 1), 2)}
        del q, k, v, o, ws
    for kind, Bs, sc in (("gqa", (1, 8, 32, 64, 128), scale), ("mla", (1, 8, 32, 64, 128), 1 / math.sqrt(192))):
        for Bd in Bs:
            times = {}
            for sp in (0, 64, 128, 256, 512, 1024):
                r = decode_case(kind, Bd, sp, sc, modes=("cold",), iters=20)
                times["default" if sp == 0 else str(sp)] = r["cold"]["graph_us"]
            best = min(times.values())
            out[f"decode_{kind}_B{Bd}"] = {"graph_us": times, "global": "default",
                                           "best": min(times, key=times.get),
                                           "gap_pct": round(100 * (times["default"] / best - 1), 2)}
    gaps = [v["gap_pct"] for v in out.values()]
    out["summary"] = {"max_gap_pct": max(gaps), "mean_gap_pct": round(sum(gaps) / len(gaps), 2)}
    return out


def prefill_traffic():
    """HBM bytes per launch of the prefill step from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "prefill_gqa_rope_bf16_S2048.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, val = line[2:].split(": ", 1)
            fields[key.strip()] = val.strip().strip("`")
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


PREFILL_SOURCES = ("attention_flash_attn_02_amd/csrc/prefill.hip", "attention_flash_attn_02_amd/csrc/prefill_sp.hip",
                   "attention_flash_attn_02_amd/csrc/prefill_common.hpp", "attention_flash_attn_02_amd/csrc/common.hpp",
                   "attention_flash_attn_02_amd/csrc/rope_common.hpp")


def cpu_baseline(budget_s=15.0):
    """Time the float64 oracle on KV groups of the full prefill workload until
    about `budget_s` seconds of CPU work (or the whole workload) is done."""
    import numpy as np
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        if pools:
            p = pools[0]
            blas = f"{p.get('internal_api', '?')} {p.get('version', '?')} ({p.get('threading_layer', '?')} threads, " \
                   f"{p.get('architecture', '?')})"
    except Exception:  # pragma: no cover
        threads = 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    import oracle
    from workloads import prefill_inputs, to_f64
    q, k, v = prefill_inputs(1, 32, 8, 2048, 128, "bf16")
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    scale = 1 / math.sqrt(128)
    t0 = time.perf_counter()
    groups = 0
    for g in range(8):
        oracle.prefill(qd[:, 4 * g:4 * g + 4], kd[:, g:g + 1], vd[:, g:g + 1], scale, True, 10000.0)
        groups += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = prefill_flops(1, 4 * groups, 2048, 128, True)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "host_cpus": len(os.sched_getaffinity(0)), "blas": blas,
            "numpy": np.__version__,
            "sample": f"{groups} of 8 KV groups ({4 * groups} of 32 query heads) of the causal GQA "
                      f"RoPE prefill B=1 S=2048 D=128, float64 numpy, {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps before the timed ones (the clock settles after ~800 steps)")
    ap.add_argument("--quick", action="store_true", help="prefill step only (for profiling runs)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only GQA and MLA decode at batch 128 with the default splits, `steps` calls "
                         "each (for profiling runs); prints one JSON line of its own")
    ap.add_argument("--neighbours-only", action="store_true",
                    help="only the append + decode step and the chunked prefill prompt (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the tile-config sweep")
    ap.add_argument("--prefill-config", type=int, default=None,
                    help="profiling runs only (with --quick): run the prefill step in this sweep "
                         "configuration instead of the global one")
    ap.add_argument("--mha-only", default=None, metavar="DTYPE,D,N",
                    help="profiling runs: time only the Z=4, H=32 MHA forward of this dtype (f16 or "
                         "fp8_e5m2), head dim (64: non-causal, 128: causal) and length, `steps` calls "
                         "after `warmup`; prints one JSON line of its own")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.prefill_config is not None and not (args.quick or args.mha_only):
        log("--prefill-config is for profiling runs and needs --quick or --mha-only")
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(the prefill shards by KV-head group and decode by batch with no exchange).")
        sys.exit(2)

    import torch
    import attention_flash_attn_02_amd as attn
    from workloads import prefill_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.lib()

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.mha_only:
        dt, D_, N = args.mha_only.split(",")
        D_, N = int(D_), int(N)
        causal = D_ == 128
        qm, km, vm = [t.to(dev) for t in prefill_inputs(4, 32, 32, N, D_, dt, seed=N)]
        om = torch.empty(qm.shape, dtype=torch.float16, device=dev)
        cfg = args.prefill_config
        ms_m = time_loop(lambda: attn.prefill_gqa_rope(qm, km, vm, 1 / math.sqrt(D_), causal=causal, out=om,
                                                      config=cfg), args.steps, args.warmup)
        tf = prefill_flops(4, 32, N, D_, causal) / (ms_m * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if dt.startswith("fp8") else PEAK_BF16_TFLOPS
        print(json.dumps({"mha_only": {"dtype": dt, "D": D_, "N": N, "causal": causal, "config": cfg,
                                       "us": round(ms_m * 1e3, 2), "tflops": round(tf, 1),
                                       "frac": round(tf / peak, 4)}}), flush=True)
        return

    if args.decode_only:
        out = {}
        for kind, sc in (("gqa", 1 / math.sqrt(128)), ("mla", 1 / math.sqrt(192))):
            r = decode_case(kind, 128, 0, sc, graph_steps=args.steps, modes=("cold",), iters=args.steps)
            out[f"decode_{kind}_B128"] = r
            log(f"decode {kind} B=128:", json.dumps(r))
        print(json.dumps({"decode_only": out}), flush=True)
        return
    if args.neighbours_only:
        out = decode_neighbours()
        log("decode neighbours:", json.dumps(out))
        print(json.dumps({"neighbours_only": out}), flush=True)
        return

    # ---- the step: causal GQA prefill with fused RoPE, full workload ----
    # (attn_prefill_gqa_rope_ws: K rotated once into the workspace, then the
    # attention kernel, which rotates its Q rows in registers)
    B, Hq, Hkv, S, D = 1, 32, 8, 2048, 128
    q, k, v = [t.to(dev) for t in prefill_inputs(B, Hq, Hkv, S, D, "bf16")]
    out = torch.empty_like(q)
    scale = 1 / math.sqrt(D)
    ws = torch.empty(attn.prefill_gqa_rope_workspace_bytes(B, Hkv, S, D, torch.bfloat16, 10000.0),
                     dtype=torch.uint8, device=dev)

    cfg = args.prefill_config  # None: the global configuration (attn_prefill_gqa_rope_ws)

    def step():
        attn.prefill_gqa_rope(q, k, v, scale, causal=True, rope_theta=10000.0, out=out, workspace=ws, config=cfg)

    for _ in range(args.warmup):
        step()
    # untimed steps until the clock has settled under load (it takes ~45 ms of
    # back-to-back work), the same settling every other measurement here gets
    spin(step)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = prefill_flops(B, Hq, S, D, True)
    tflops = flops / (ms * 1e-3) / 1e12
    # the step's attention kernel alone: the same launch (global configuration)
    # with the workspace already holding the rotated K, so the rotation kernel
    # is skipped; HIP events on the same stream (torch's current stream, which
    # the binding passes to the library)
    ms_kern = time_loop(lambda: attn.prefill_gqa_rope(q, k, v, scale, causal=True, rope_theta=10000.0, out=out,
                                                      workspace=ws, config=GLOBAL_CONFIG if cfg is None else cfg,
                                                      k_rotated=True),
                        max(args.steps, 50), args.warmup)
    # the K rotation's share of the step: step time minus the attention kernel
    # alone (the rotation kernel plus the one launch gap it adds; inside the
    # step K arrives cold, after the attention kernel has used the caches)
    ms_rot = ms - ms_kern
    # the same rotation launch on its own (attn_rope_rotate of K into the
    # workspace), 20 launches per captured graph so that the host's per-call
    # overhead is not what is timed; back to back, K stays cache-resident and
    # the time includes one dispatch gap per launch
    ws_k = ws.view(torch.bfloat16).view(k.shape)
    ms_rot_alone = time_graph(lambda: attn.rope_rotate(k, 10000.0, out=ws_k), 20, max(args.steps // 10, 10))
    kern_tflops = flops / (ms_kern * 1e-3) / 1e12
    log(f"prefill gqa+rope bf16 S=2048: {ms * 1e3:.1f} us/step; K rotation {ms_rot * 1e3:.1f} us of it "
        f"({ms_rot_alone * 1e3:.1f} us alone in a graph), "
        f"attention kernel alone {ms_kern * 1e3:.1f} us; {tflops:.1f} TFLOP/s per step, "
        f"{kern_tflops:.1f} TFLOP/s attention kernel")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal GQA prefill with fused RoPE", "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "seq_len": S, "head_dim": D, "rope_theta": 10000.0,
                   "in_dtype": "bf16", "out_dtype": "bf16", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": prefill_traffic(),
                     "kernel": "prefill_sp_kernel<bf16,128,causal,RoPE on Q (K rotated once),4 waves>"
                               if cfg is None else f"prefill configuration {cfg}",
                     "kernel_us": round(ms_kern * 1e3, 2), "k_rotation_us": round(ms_rot * 1e3, 2),
                     "k_rotation_alone_graph_us": round(ms_rot_alone * 1e3, 2),
                     "algorithmic_per_launch": flops},
    }

    if not args.quick:
        sec = {}
        # graph replay of the prefill step
        ms_g = time_graph(step, 10, 10)
        sec["prefill_gqa_rope_graph"] = {"us_per_step": round(ms_g * 1e3, 2),
                                         "tflops": round(flops / (ms_g * 1e-3) / 1e12, 1)}
        # tiny fp32 prefill
        qt, kt, vt = [t.to(dev) for t in prefill_inputs(1, 4, 2, 128, 64, "f32")]
        ms_t = time_loop(lambda: attn.prefill_gqa_rope(qt, kt, vt, 1 / 8, causal=True), 100, 10)
        sec["prefill_tiny_f32"] = {"us_per_step": round(ms_t * 1e3, 2)}
        # MHA forward Z=4, H=32, fp16 and fp8 e5m2 (fp16 out)
        mha = {}
        for D_, causal in ((64, False), (128, True)):
            for N in (1024, 2048, 4096, 8192, 16384):
                for dt in ("f16", "fp8_e5m2"):
                    qm, km, vm = [t.to(dev) for t in prefill_inputs(4, 32, 32, N, D_, dt, seed=N)]
                    om = torch.empty(qm.shape, dtype=torch.float16, device=dev)
                    it = 20 if N <= 4096 else 5
                    ms_m = time_loop(lambda: attn.prefill_gqa_rope(qm, km, vm, 1 / math.sqrt(D_), causal=causal,
                                                                  out=om), it, 3)
                    f = prefill_flops(4, 32, N, D_, causal)
                    tf = f / (ms_m * 1e-3) / 1e12
                    peak = PEAK_FP8_TFLOPS if dt == "fp8_e5m2" else PEAK_BF16_TFLOPS
                    mha[f"D{D_}_{'causal' if causal else 'noncausal'}_N{N}_{dt}"] = {
                        "us": round(ms_m * 1e3, 1), "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
                    del qm, km, vm, om
        sec["mha_fwd_Z4_H32"] = mha
        log("mha:", json.dumps(mha))
        # decode: split + combine per step, warm (one cache set) and cold (the
        # step rotates over enough cache copies that the working set exceeds
        # twice the 256 MB last-level cache, so every step streams from HBM)
        gqa = {}
        for Bd in (1, 8, 32, 64, 128):
            gqa[f"B{Bd}"] = decode_case("gqa", Bd, 0, scale)
            log(f"decode gqa B={Bd}:", json.dumps(gqa[f"B{Bd}"]))
        sec["decode_gqa"] = gqa
        mla = {}
        for Bd in (1, 8, 32, 64, 128):
            mla[f"B{Bd}"] = decode_case("mla", Bd, 0, 1 / math.sqrt(192))
            log(f"decode mla B={Bd}:", json.dumps(mla[f"B{Bd}"]))
        sec["decode_mla"] = mla
        sec["rope_fusion_factorial"] = rope_factorial()
        log("rope fusion:", json.dumps(sec["rope_fusion_factorial"]))
        sec["decode_neighbours"] = decode_neighbours()
        log("decode neighbours:", json.dumps(sec["decode_neighbours"]))
        if not args.no_sweep:
            sec["sweep"] = sweep(scale)
            log("sweep:", json.dumps(sec["sweep"]))
        result["secondary"] = sec

    if not args.no_cpu and not args.quick:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
