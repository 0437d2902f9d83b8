"""Host-side checks of bench.py (no GPU): the algorithmic work per step that
the roofline figures divide by, and the one-GPU guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_flops_counts_useful_work_only():
    # causal: 4 B H D S(S+1)/2 (query i sees keys 0..i); non-causal: 4 B H D S^2
    assert bench.prefill_flops(1, 32, 2048, 128, True) == 34376515584.0
    assert bench.prefill_flops(4, 32, 1024, 64, False) == 4 * 4 * 32 * 64 * 1024 * 1024
    assert bench.prefill_flops(1, 4, 1, 64, True) == 4 * 4 * 64  # one query, one key
    # brute count of the visible (query, key) pairs on a small causal case
    S = 37
    pairs = sum(1 for i in range(S) for j in range(S) if j <= i)
    assert bench.prefill_flops(2, 3, S, 16, True) == 4 * 2 * 3 * 16 * pairs


def test_decode_bytes_are_the_compulsory_reads_and_writes():
    # GQA: K and V of 2048 slots x 4 KV heads x 128 dims, plus q in and o out (16 heads), bf16
    assert bench.gqa_decode_bytes(1) == 2048 * 4 * 128 * 2 * 2 + 2 * 16 * 128 * 2 == 4202496
    assert bench.gqa_decode_bytes(128) == 537919488
    # MLA: 2048 rows of 512 dims, plus q (16 x 512) in and o (16 x 448) out, bf16
    assert bench.mla_decode_bytes(1) == 2048 * 512 * 2 + 16 * 512 * 2 + 16 * 448 * 2 == 2127872
    assert bench.mla_decode_bytes(128) == 272367616


def test_prefill_traffic_is_an_int_or_none():
    t = bench.prefill_traffic()
    assert t is None or (isinstance(t, int) and t > 40 * 2 ** 20)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_config_override_needs_quick():
    # a sweep configuration may only replace the global one in profiling runs
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--prefill-config", "1"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "--quick" in r.stderr
    assert r.stdout == ""
