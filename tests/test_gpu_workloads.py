"""The five named workloads at full size, in the launch configuration the benchmark times.

Small workloads are compared with the oracle on every output; the large ones on sampled
sequences / query rows that the oracle computes one by one (the sample is stated per test),
plus properties that hold at any size (tail-only reads of sliding decode).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from harness import (PagedCase, assert_attn_close, compact_pages, dtype_code,
                     exact_kv_reference_caches, oracle_write, ulp_distance)

pytestmark = pytest.mark.gpu


def _fill_past(case, lens, news, seed, chunk=4096):
    """Write positions 0 .. lens[b]-news[b]-1 through the library, in chunks."""
    past = np.asarray(lens) - np.asarray(news)
    start = np.zeros_like(past)
    k_ = 0
    while (start < past).any():
        n = np.minimum(past - start, chunk)
        case.write(start + n, n, seed + k_, with_q=False, device_gen=True)
        start = start + n
        k_ += 1


def test_tiny_sliding_fp32_prefill_then_16_decodes():
    """1 sequence, 256-token prefill then 16 single-token decode steps, W 128, fp32: every
    output against the oracle (1e-4), and the GPU pipeline against the oracle's own pipeline
    (its own cache and q̂)."""
    specs, pb = wl.workload("tiny_sliding_fp32")
    spec = specs[0]
    case = PagedCase(spec, pb, 1)
    kc_o, vc_o = case.host_caches()
    q, k, v, qd, cu, cl = case.write([256], [256], 1)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    assert_attn_close(out, case.oracle_attention(qd, cu, cl), "fp32", what="prefill")
    # the oracle's pipeline from the raw inputs
    qh = case.oracle_write(kc_o, vc_o, q, k, v, cu, cl)
    e2e = oracle.attention(oracle.FP32, 4, 2, 256, 128, 1.0, 0.0, 0, qh, cu, kc_o, vc_o,
                           pb.block_table, cl)
    assert np.abs(out.cpu().numpy() - e2e).max() <= 1e-4
    for step in range(16):
        L = 257 + step
        q, k, v, qd, cu1, cl1 = case.write([L], [1], 100 + step)
        dec = case.decode(qd, cl1)
        torch.cuda.synchronize()
        assert_attn_close(dec, case.oracle_attention(qd, cu1, cl1), "fp32", what=f"decode {L}")
        qh = case.oracle_write(kc_o, vc_o, q, k, v, cu1, cl1)
        e2e = oracle.attention(oracle.FP32, 4, 2, 256, 128, 1.0, 0.0, 0, qh, cu1, kc_o, vc_o,
                               pb.block_table, cl1)
        assert np.abs(dec.cpu().numpy() - e2e).max() <= 1e-4


@pytest.mark.parametrize("q_scale", [1.0, 20.0])
def test_softcap_decode_bf16_full(q_scale):
    """32 sequences, L ~ U[512, 4096]: all outputs vs the oracle; q x 20 makes the cap bind."""
    specs, pb = wl.workload("softcap_decode_bf16")
    spec = specs[0]
    case = PagedCase(spec, pb, 2)
    lens = pb.context_lens
    _fill_past(case, lens, np.ones_like(lens), 200)
    q, k, v, qd, cu, cl = case.write(lens, np.ones_like(lens), 2, q_scale=q_scale)
    out = case.decode(qd, cl)
    torch.cuda.synchronize()
    mx, mean = assert_attn_close(out, case.oracle_attention(qd, cu, cl), "bf16",
                                 what=f"softcap decode q*{q_scale}")
    print(f"softcap_decode q*{q_scale}: max {mx:.3e} mean {mean:.3e}")


def test_sliding_decode_bf16_full():
    """64 x 8192, W 1024: every sequence vs the oracle; then every page before the window is
    NaN-poisoned and the output must not change by a single bit (tail-only reads)."""
    specs, pb = wl.workload("sliding_decode_bf16")
    spec = specs[0]
    case = PagedCase(spec, pb, 3)
    lens = pb.context_lens
    _fill_past(case, lens, np.ones_like(lens), 300)
    q, k, v, qd, cu, cl = case.write(lens, np.ones_like(lens), 3)
    out = case.decode(qd, cl)
    torch.cuda.synchronize()
    seqs = list(range(pb.batch))
    kc, vc, nbt = compact_pages(case, seqs, lens)
    sub_q = wl.to_numpy_bits(qd[seqs])
    ref = oracle.attn_decode(dtype_code(spec), 32, 16, 256, 1024, 1.0, 0.0, 0, sub_q, kc, vc, nbt,
                             lens[seqs])
    mx, mean = assert_attn_close(out[seqs], ref, "bf16", what="sliding decode")
    print(f"sliding_decode (all 64 seqs): max {mx:.3e} mean {mean:.3e}")
    before = torch.from_numpy(pb.block_table[:, :448].reshape(-1).astype(np.int64)).cuda()
    case.kc.index_fill_(0, before, float("nan"))
    case.vc.index_fill_(0, before, float("nan"))
    out2 = case.decode(qd, cl)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_kv_shared_decode_bf16_full():
    """16 x ~32k, head size 512, K=V: every sequence vs the oracle."""
    specs, pb = wl.workload("kv_shared_decode_bf16")
    spec = specs[0]
    case = PagedCase(spec, pb, 4)
    lens = pb.context_lens
    _fill_past(case, lens, np.ones_like(lens), 400, chunk=8192)
    q, k, v, qd, cu, cl = case.write(lens, np.ones_like(lens), 4)
    out = case.decode(qd, cl)
    torch.cuda.synchronize()
    kc, _ = case.host_caches()
    ref = oracle.attn_decode(dtype_code(spec), 32, 4, 512, 0, 1.0, 0.0, 1, wl.to_numpy_bits(qd),
                             kc, None, pb.block_table, lens)
    mx, mean = assert_attn_close(out, ref, "bf16", what="K=V decode")
    print(f"kv_shared_decode (all 16 seqs): max {mx:.3e} mean {mean:.3e}")


def _sample_rows(cu, W, past, n_random, seed, edge=64):
    """Rows of a chunked prefill checked against the oracle, per sequence: the first and last
    `edge` rows; on a sliding layer every row whose window start lo = past + i - W + 1 sits on a
    page edge (lo % 16 in {0, 15}) or next to the chunk start (|lo - past| <= 1, which includes
    i = W - 1, where the window starts exactly at the chunk), and every row whose own position
    is on a page edge; then `n_random` rows drawn at random."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        pick = set(range(min(edge, n))) | set(range(max(0, n - edge), n))
        if W:
            i = np.arange(n)
            lo = past[b] + i - W + 1
            t = past[b] + i
            sel = ((lo >= 0) & ((lo % 16 == 0) | (lo % 16 == 15) | (np.abs(lo - past[b]) <= 1))) \
                | (t % 16 == 0) | (t % 16 == 15)
            pick |= set(i[sel].tolist())
        pick |= set(rng.choice(n, size=min(n_random, n), replace=False).tolist())
        rows.extend(int(cu[b] + i) for i in sorted(pick))
    return np.array(rows, np.int32)


@pytest.mark.parametrize("layer", ["sliding", "global", "global_keqv"])
def test_chunked_prefill_bf16_full(layer):
    """The varlen chunks (about 2048 new tokens after about 6144 cached, 8192 new in all) of
    one sliding layer (W 1024, D 256, 16 kv heads) or of the global layer (D 512, 4 kv heads;
    also with K=V).  Rows checked per sequence: the first and last 64, 256 at random, and on
    the sliding layer every row whose window start or own position meets a page edge, or whose
    window starts next to the chunk start."""
    specs, pb = wl.workload("chunked_prefill_bf16")
    spec = specs[0] if layer == "sliding" else specs[5]
    if layer == "global_keqv":
        spec = wl.LayerSpec("bf16", 32, 4, 512, window=0, k_eq_v=True, rope_theta=1e6)
    case = PagedCase(spec, pb, 5)
    lens, news = pb.context_lens, pb.n_new
    _fill_past(case, lens, news, 500)
    q, k, v, qd, cu, cl = case.write(lens, news, 5)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    rows = _sample_rows(cu, spec.window, lens - news, 256, 5)
    ref = case.oracle_attention(qd, cu, cl, rows=rows)
    mx, mean = assert_attn_close(out, ref, "bf16", rows=rows, what=f"prefill {layer}")
    print(f"chunked_prefill {layer} ({len(rows)} rows): max {mx:.3e} mean {mean:.3e}")


def test_chunked_prefill_jittered_lengths():
    """Varlen chunks (n, past) = (1, 0), (777, 6144), (2048, 5000), (1500, 1023) on the sliding
    layer and on the global layer, sampled rows vs the oracle (first/last 64 rows and 64 random
    per sequence, plus the sliding layer's page-edge and chunk-start rows)."""
    specs, _ = wl.workload("chunked_prefill_bf16")
    news = np.array([1, 777, 2048, 1500], np.int32)
    past = np.array([0, 6144, 5000, 1023], np.int32)
    lens = past + news
    pb = wl.paged_batch(lens, news, seed=55)
    for spec in (specs[0], specs[5]):
        case = PagedCase(spec, pb, 55)
        _fill_past(case, lens, news, 555)
        q, k, v, qd, cu, cl = case.write(lens, news, 56)
        out = case.prefill(qd, cu, cl)
        torch.cuda.synchronize()
        rows = _sample_rows(cu, spec.window, past, 64, 56)
        ref = case.oracle_attention(qd, cu, cl, rows=rows)
        assert_attn_close(out, ref, "bf16", rows=rows, what=f"jittered W{spec.window}")


def test_chunk_write_matches_oracle_on_sampled_tokens():
    """The 8192-token chunk write of the sliding layer: the pages of 2 sampled sequences vs
    the oracle's write of the same tokens (<= 1 ulp)."""
    specs, pb = wl.workload("chunked_prefill_bf16")
    spec = specs[0]
    lens, news = pb.context_lens, pb.n_new
    case = PagedCase(spec, pb, 9)
    q, k, v, qd, cu, cl = case.write(lens, news, 9)
    torch.cuda.synchronize()
    kc1, vc1 = case.host_caches()
    kc0 = np.full_like(kc1, 0x7FC0)
    vc0 = np.full_like(vc1, 0x7FC0)
    seqs = [0, 3]
    sel_tok = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in seqs])
    sub_cu = np.concatenate([[0], np.cumsum(news[seqs])]).astype(np.int32)
    qh = oracle_write(spec, case.w_cpu, pb.block_table[seqs], kc0, vc0, q[sel_tok], k[sel_tok],
                      v[sel_tok], sub_cu, lens[seqs])
    pages = np.concatenate([pb.block_table[b, (lens[b] - news[b]) // 16:(lens[b] + 15) // 16]
                            for b in seqs])
    assert ulp_distance(kc1[pages], kc0[pages]).max() <= 1
    assert ulp_distance(vc1[pages], vc0[pages]).max() <= 1
    assert ulp_distance(wl.to_numpy_bits(qd)[sel_tok], qh).max() <= 1



def test_kv_shared_decode_bf16_exact_form_full():
    """The K=V decode workload (16 x ~32k, head size 512) in the exact K=V form the bench times
    (unrotated keys, 64 rotated pairs, a v norm weight): 8 of the 16 sequences (the shortest,
    the longest and six more; the fp64 reference caches of all 16 would take about 30 GB of
    host memory) vs the oracle over the stored bytes (K = RoPE(C), V = C * w_v / w_k)."""
    specs, pb = wl.workload("kv_shared_decode_bf16")
    spec = dataclasses.replace(specs[0], k_eq_v=2, rope_angles=64)
    case = PagedCase(spec, pb, 4)
    lens = pb.context_lens
    _fill_past(case, lens, np.ones_like(lens), 400, chunk=8192)
    q, k, v, qd, cu, cl = case.write(lens, np.ones_like(lens), 4)
    out = case.decode(qd, cl)
    torch.cuda.synchronize()
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 3, 7, 9, 12, 15})
    kc, _, nbt = compact_pages(case, seqs, lens)
    K, V = exact_kv_reference_caches(spec, kc, nbt, lens[seqs], case.w_cpu[1], case.w_cpu[2])
    q32 = np.ascontiguousarray(qd[seqs].float().cpu().numpy())
    ref = oracle.attn_decode(oracle.FP32, 32, 4, 512, 0, 1.0, 0.0, 0, q32, K, V, nbt,
                             lens[seqs])
    mx, mean = assert_attn_close(out[seqs], ref, "bf16", what="exact K=V decode")
    print(f"kv_shared_decode exact ({len(seqs)} of 16 seqs): max {mx:.3e} mean {mean:.3e}")


def test_chunked_prefill_global_layer_exact_form_full():
    """The chunked-prefill global layer (the varlen chunks, D 512, 32/4 heads) in the exact
    K=V form the bench times: the first and last 64 rows and 256 random rows per sequence vs
    the oracle over the stored bytes."""
    specs, pb = wl.workload("chunked_prefill_bf16")
    spec = dataclasses.replace(specs[5], k_eq_v=2, rope_angles=64)
    case = PagedCase(spec, pb, 5)
    lens, news = pb.context_lens, pb.n_new
    _fill_past(case, lens, news, 500)
    q, k, v, qd, cu, cl = case.write(lens, news, 5)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    rows = _sample_rows(cu, 0, lens - news, 256, 5)
    kc, _ = case.host_caches()
    K, V = exact_kv_reference_caches(spec, kc, pb.block_table, lens, case.w_cpu[1],
                                     case.w_cpu[2])
    q32 = np.ascontiguousarray(qd.float().cpu().numpy())
    ref = oracle.attention(oracle.FP32, 32, 4, 512, 0, 1.0, 0.0, 0, q32, cu, K, V,
                           pb.block_table, cl, rows=rows)
    mx, mean = assert_attn_close(out, ref, "bf16", rows=rows, what="prefill global exact")
    print(f"chunked_prefill global exact ({len(rows)} rows): max {mx:.3e} mean {mean:.3e}")
