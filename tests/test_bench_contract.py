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
    """Algorithmic bytes per decode call and flops of the chunked-prefill stack (the figures
    quoted with the committed measurements)."""
    for name, nbytes in (("softcap_decode_bf16", 272487536), ("sliding_decode_bf16", 1076101120),
                         (bench.HEADLINE, 2128252080)):
        specs, pb = wl.workload(name)
        assert bench.decode_bytes(specs[0], pb.context_lens) == nbytes, name
    specs, pb = wl.workload("chunked_prefill_bf16")
    assert pb.n_new.sum() == 8192 and len(set(pb.n_new.tolist())) == 4  # varlen chunks
    assert sum(bench.prefill_flops(s, pb.context_lens, pb.n_new) for s in specs) == 5087395250176


@pytest.mark.parametrize("workload", [bench.HEADLINE, "sliding_decode_bf16",
                                      "softcap_decode_bf16", bench.HEADLINE + "_exact"])
def test_traffic_records_match_the_decode_sources(workload):
    """The counter records that the roofline blocks' traffic reads were taken on the current
    decode sources (bench.py reports null otherwise)."""
    assert bench.decode_traffic(workload) is not None


def test_prefill_counter_record_matches_the_prefill_sources():
    rec = bench.counter_record("prefill_tiled_kernel.chunked_prefill_bf16.pmc.md",
                               bench.PREFILL_SOURCES)
    assert rec is not None and 1.0 <= rec["mfma_flop_ratio"] < 1.5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
