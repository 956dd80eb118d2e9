"""bench.py on the CPU: its algorithmic byte and flop counts agree with brute-force counts over
the visibility rule, the named workloads keep their recipe, the committed traffic record still
matches the decode sources, and a multi-GPU request is refused before any device is touched."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_decode_bytes(spec, lens):
    e = 2 if spec.dtype == "bf16" else 4
    kv = 1 if spec.k_eq_v else 2
    total = 0
    for L in lens:
        t = L - 1  # the decode query's position
        keys = [j for j in range(L) if spec.window == 0 or t - j < spec.window]
        pages = {j // wl.BLOCK_SIZE for j in keys}
        total += len(keys) * spec.num_kv_heads * spec.head_dim * e * kv
        total += len(pages) * 4 * spec.num_kv_heads
    return total + 2 * len(lens) * spec.num_q_heads * spec.head_dim * e


def brute_prefill_flops(spec, lens, news):
    pairs = 0
    for L, n in zip(lens, news):
        for i in range(n):
            t = L - n + i
            pairs += sum(1 for j in range(L) if j <= t and (spec.window == 0 or t - j < spec.window))
    return pairs * spec.num_q_heads * 4 * spec.head_dim


@pytest.mark.parametrize("W,keqv", [(0, False), (40, False), (16, True), (1, False)])
def test_decode_bytes_match_a_brute_force_count(W, keqv):
    spec = wl.LayerSpec("bf16", 8, 4, 256, window=W, k_eq_v=keqv)
    g = np.random.default_rng(W + 3)
    lens = [int(x) for x in g.integers(1, 200, size=9)] + [1, 16, 17, 32]
    assert bench.decode_bytes(spec, lens) == brute_decode_bytes(spec, lens)


@pytest.mark.parametrize("W", [0, 1, 24])
def test_prefill_flops_match_a_brute_force_count(W):
    spec = wl.LayerSpec("bf16", 4, 2, 128, window=W)
    lens, news = [50, 33, 70, 5], [20, 33, 1, 5]
    assert bench.prefill_flops(spec, lens, news) == brute_prefill_flops(spec, lens, news)


def test_named_workloads_keep_their_size():
    """The headline decode step reads 272 487 536 algorithmic bytes and the chunked-prefill stack
    does 5 222 948 667 392 flops (the figures quoted with the committed measurements)."""
    specs, pb = wl.workload("softcap_decode_bf16")
    assert bench.decode_bytes(specs[0], pb.context_lens) == 272487536
    specs, pb = wl.workload("chunked_prefill_bf16")
    assert sum(bench.prefill_flops(s, pb.context_lens, pb.n_new) for s in specs) == 5222948667392


def test_traffic_record_matches_the_decode_sources():
    """The counter record that roofline.traffic reads was taken on the current decode sources
    (bench.py reports null otherwise)."""
    assert bench.recorded_traffic() is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
