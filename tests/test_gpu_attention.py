"""GPU parity of ga_attn_decode / ga_attn_prefill against the oracle, on small ragged inputs
that span several page pairs and ragged tails, plus exact mask probes."""
import numpy as np
import pytest
import torch

import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import (PagedCase, assert_attn_close, assert_within_rounding_bound, i32,
                     softmax_weights, weight_rounding_sigma)
from layout import logical_k, unit_elems

pytestmark = pytest.mark.gpu


def _decode_case(spec, lens, seed, q_scale=1.0):
    pb = wl.paged_batch(lens, np.ones(len(lens), np.int32), seed=seed)
    case = PagedCase(spec, pb, seed)
    past = [L - 1 for L in lens]
    if max(past) > 0:
        case.write(past, past, seed + 100, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, [1] * len(lens), seed, q_scale=q_scale)
    out = case.decode(qd, cl)
    torch.cuda.synchronize()
    ref = case.oracle_attention(qd, cu, cl)
    return out, ref


DECODE_CASES = [
    # dtype, Hq, Hkv, D, W, cap, k_eq_v, lens
    ("bf16", 8, 4, 256, 0, 50.0, False, [1, 2, 17, 31, 32, 33, 200, 513]),
    ("bf16", 32, 16, 256, 64, 0.0, False, [1, 63, 64, 65, 100, 300]),
    ("bf16", 32, 4, 512, 0, 0.0, True, [1, 16, 47, 700]),
    ("bf16", 16, 1, 512, 100, 30.0, True, [5, 99, 100, 101, 450]),
    ("bf16", 4, 4, 128, 17, 0.0, False, [1, 16, 17, 18, 333]),
    ("bf16", 16, 1, 256, 0, 0.0, False, [129, 1000]),
    ("fp32", 4, 2, 256, 128, 0.0, False, [1, 128, 129, 272]),
    ("fp32", 8, 2, 512, 0, 20.0, True, [3, 150]),
    # fp32 past 64 pages of keys: the kernel's window of block ids moves
    ("fp32", 4, 2, 256, 0, 0.0, False, [1100, 2500]),
    ("fp32", 4, 1, 128, 1500, 10.0, True, [1700, 3000, 1023]),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,W,cap,keqv,lens", DECODE_CASES)
def test_decode_matches_oracle(dtype, Hq, Hkv, D, W, cap, keqv, lens):
    spec = wl.LayerSpec(dtype, Hq, Hkv, D, window=W, softcap=cap, k_eq_v=keqv,
                        scale=1.0 if cap == 0 else 1.0 / 16, rope_theta=1e4 if D < 512 else 1e6)
    out, ref = _decode_case(spec, lens, seed=21)
    assert_attn_close(out, ref, dtype, what=f"decode {dtype} D{D} G{Hq // Hkv} W{W} cap{cap}")


@pytest.mark.parametrize("B", [64, 65, 130])
@pytest.mark.parametrize("D,Hq,Hkv,W", [(256, 8, 4, 0), (512, 16, 2, 48)])
def test_decode_batch_sizes_around_one_wave(B, D, Hq, Hkv, W):
    """The decode set-up keeps the lengths of up to 64 sequences in the lanes of one wave and
    loops over groups of 64 above that: batches at and past that boundary, ragged lengths."""
    spec = wl.LayerSpec("bf16", Hq, Hkv, D, window=W, rope_theta=1e4 if D < 512 else 1e6)
    g = np.random.default_rng(100 + B)
    lens = [int(x) for x in g.integers(1, 120, size=B)]
    out, ref = _decode_case(spec, lens, seed=23 + B)
    assert_attn_close(out, ref, "bf16", what=f"decode B{B} D{D} W{W}")


@pytest.mark.parametrize("B,Hq,Hkv,D,W,keqv,maxlen", [
    (64, 32, 16, 256, 0, False, 3000),
    (64, 32, 4, 512, 0, True, 2000),
    (128, 16, 16, 128, 100, False, 400),
])
def test_decode_many_outputs(B, Hq, Hkv, D, W, keqv, maxlen):
    """Batches of 2048 or more (sequence, query head) outputs whose ragged lengths give both
    segments held whole by one worker (the worker writes the output and the merge skips
    them) and segments split over two to ten workers, side by side in one call."""
    spec = wl.LayerSpec("bf16", Hq, Hkv, D, window=W, k_eq_v=keqv,
                        rope_theta=1e4 if D < 512 else 1e6)
    g = np.random.default_rng(200 + D)
    lens = [int(x) for x in g.integers(1, maxlen, size=B)]
    out, ref = _decode_case(spec, lens, seed=24 + D)
    assert_attn_close(out, ref, "bf16", what=f"decode B{B} Hq{Hq} D{D}")


def test_decode_softcap_binds():
    """q scaled by 20 so that the cap of 50 dominates the scores."""
    spec = wl.LayerSpec("bf16", 8, 4, 256, softcap=50.0, scale=1 / 16, norm_q=False,
                        norm_k=False, norm_v=False)
    out, ref = _decode_case(spec, [700, 1500, 33], seed=22, q_scale=20.0)
    assert_attn_close(out, ref, "bf16", what="decode cap binds")


PREFILL_CASES = [
    # dtype, Hq, Hkv, D, W, cap, k_eq_v, (lens, news)
    ("bf16", 8, 4, 256, 0, 0.0, False, ([70, 33, 200], [70, 33, 64])),
    ("bf16", 32, 16, 256, 40, 0.0, False, ([300, 129], [77, 129])),
    ("bf16", 32, 4, 512, 0, 0.0, False, ([260, 90], [100, 90])),
    ("bf16", 32, 4, 512, 0, 0.0, True, ([260, 90], [100, 1])),
    ("bf16", 8, 1, 512, 33, 25.0, True, ([140], [140])),
    ("bf16", 4, 2, 128, 16, 10.0, False, ([1, 16, 17, 48], [1, 16, 17, 20])),
    # a sequence with no new tokens in the middle of the batch: it contributes no rows
    ("bf16", 8, 4, 256, 24, 0.0, False, ([50, 30, 64], [20, 0, 64])),
    ("fp32", 4, 2, 256, 128, 0.0, False, ([256], [256])),
    ("fp32", 8, 2, 512, 0, 0.0, True, ([90, 31], [30, 31])),
    # fp32 past 64 pages of keys (the window of block ids moves), global and sliding
    ("fp32", 4, 2, 256, 0, 0.0, False, ([2200, 1500], [24, 40])),
    ("fp32", 4, 2, 128, 1100, 0.0, False, ([2300], [37])),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,W,cap,keqv,ln", PREFILL_CASES)
def test_prefill_matches_oracle(dtype, Hq, Hkv, D, W, cap, keqv, ln):
    lens, news = ln
    spec = wl.LayerSpec(dtype, Hq, Hkv, D, window=W, softcap=cap, k_eq_v=keqv,
                        rope_theta=1e4 if D < 512 else 1e6)
    pb = wl.paged_batch(lens, news, seed=31)
    case = PagedCase(spec, pb, 31)
    past = [L - n for L, n in zip(lens, news)]
    if max(past) > 0:
        case.write(past, past, 131, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, news, 31)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    ref = case.oracle_attention(qd, cu, cl)
    assert_attn_close(out, ref, dtype, what=f"prefill {dtype} D{D} W{W}")


@pytest.mark.parametrize("past,n,W,keqv", [(5, 37, 4, False), (0, 40, 16, False),
                                           (20, 33, 1, True), (31, 20, 0, False),
                                           (48, 17, 17, True)])
def test_one_hot_probes_are_bit_exact(past, n, W, keqv):
    """Plant one key that beats every other score by ~200 (2^-288 underflows to 0 in fp32):
    a query that sees it returns its value bit-exactly; one that does not never returns it.
    Probes sit at window edges, page edges and the causal edge."""
    D, L = 256, past + n
    spec = wl.LayerSpec("bf16", 2, 1, D, window=W, rope_theta=0.0, k_eq_v=keqv,
                        norm_q=False, norm_k=False, norm_v=False)
    pb = wl.paged_batch([L], [n], seed=41)
    dev = torch.device("cuda")
    probes = {0, 15, 16, 17, past, L - W, L - W - 1, L - 1, past + W, past + W - 1}
    for jstar in sorted(j for j in probes if 0 <= j < L):
        case = PagedCase(spec, pb, 41)
        k = torch.zeros(L, 1, D)
        k[jstar, 0, 0] = 200.0
        v = torch.zeros(L, 1, D) if not keqv else None
        if v is not None:
            v[:, 0, 1] = torch.arange(L, dtype=torch.float32) / 64.0
            v[jstar, 0, 1] = -3.0
        else:
            k[:, 0, 1] = torch.arange(L, dtype=torch.float32) / 64.0
            k[jstar, 0, 1] = -3.0
        q = torch.zeros(n, 2, D)
        q[:, :, 0] = 1.0
        cu = np.array([0, L], np.int32)
        bt = case.bt
        kb = k.to(torch.bfloat16).to(dev)
        vb = None if v is None else v.to(torch.bfloat16).to(dev)
        ga.kv_cache_write(case.p, None, kb, vb, None, None, None, i32(cu, dev),
                          i32([L], dev), bt, case.kc, case.vc)
        qd = q.to(torch.bfloat16).to(dev)
        cuq = np.array([0, n], np.int32)
        out = case.prefill(qd, cuq, np.array([L], np.int32)).float().cpu()
        for i in range(n):
            t = past + i
            vis = jstar <= t and (W == 0 or t - jstar < W)
            got = out[i, :, 1]
            if vis:
                assert (got == -3.0).all(), (jstar, i)
            else:
                assert (got != -3.0).all(), (jstar, i)
        # decode at the last position agrees bit-for-bit with the last prefill row
        dec = case.decode(qd[-1:].contiguous(), np.array([L], np.int32)).float().cpu()
        vis = jstar <= L - 1 and (W == 0 or L - 1 - jstar < W)
        assert ((dec[0, :, 1] == -3.0).all()) == vis


def test_sliding_decode_ignores_pages_before_the_window():
    """NaN-poison every page that lies entirely before the window: output unchanged."""
    spec = wl.LayerSpec("bf16", 8, 4, 256, window=100, rope_theta=1e4)
    lens = [1000, 640, 101]
    pb = wl.paged_batch(lens, [1, 1, 1], seed=51)
    case = PagedCase(spec, pb, 51)
    case.write([L - 1 for L in lens], [L - 1 for L in lens], 151, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, [1, 1, 1], 51)
    out1 = case.decode(qd, cl).clone()
    for b, L in enumerate(lens):
        first_page = (L - 100) // 16
        for pg in range(first_page):
            case.kc[int(pb.block_table[b, pg])] = float("nan")
            case.vc[int(pb.block_table[b, pg])] = float("nan")
    out2 = case.decode(qd, cl)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_decode_equals_last_prefill_row_and_gqa_equals_repeated_heads():
    """Decode at L equals the last prefill row over the same cache, within a bound derived from
    the two kernels' roundings (weights to bf16 before P.V, outputs to bf16); prefill GQA equals
    prefill over the kv heads repeated G times bit for bit: a row's arithmetic (its scores, its
    weights, the order of its tiles) does not depend on which other rows share its workgroup,
    and tiles that only the other rows need add exact zeros."""
    spec = wl.LayerSpec("bf16", 8, 2, 256, window=50, rope_theta=1e4)
    lens = [130, 77]
    pb = wl.paged_batch(lens, lens, seed=61)
    case = PagedCase(spec, pb, 61)
    q, k, v, qd, cu, cl = case.write(lens, lens, 61)
    pre = case.prefill(qd, cu, cl)
    last = torch.from_numpy(cu[1:] - 1).long().cuda()
    dec = case.decode(qd[last].contiguous(), cl)
    torch.cuda.synchronize()
    # the rounding bound, from the stored bytes: both kernels' row sums add the same
    # bf16-rounded weights that multiply V
    kc, vc = case.host_caches()
    K = logical_k(kc, pb.block_table, lens, unit_elems("bf16"))
    f32 = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    K, V = f32(K), f32(vc)
    qn = f32(wl.to_numpy_bits(qd[last]))
    sigma = np.zeros((len(lens), 8, 256))
    for b, L in enumerate(lens):
        pos = np.arange(max(0, L - spec.window), L)
        blk, r = pb.block_table[b, pos // 16], pos % 16
        for h in range(8):
            g = h // 4
            Kb, Vb = K[blk, g, r, :], V[blk, g, :, r]
            w = softmax_weights(qn[b, h], Kb, spec.scale, spec.softcap)
            out = w @ Vb
            sigma[b, h] = 2.0 * weight_rounding_sigma(w, Vb, out)
    assert_within_rounding_bound(dec, pre[last], sigma)
    # GQA: the same layer with each kv head repeated 4x (MHA) gives the same bits
    spec2 = wl.LayerSpec("bf16", 8, 8, 256, window=50, rope_theta=1e4)
    case2 = PagedCase(spec2, pb, 61)
    case2.kc.copy_(case.kc.repeat_interleave(4, dim=1))
    case2.vc.copy_(case.vc.repeat_interleave(4, dim=1))
    pre2 = case2.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    assert torch.equal(pre2, pre)


def test_k_eq_v_equals_separate_caches_holding_the_same_tensor():
    """Prefill with k_eq_v = 1 equals prefill with a V cache holding the same tensor, bit for
    bit: the value operand reaches the matrix cores in the same key order either way (from the
    K tile by transposing reads, or from the V^T page), so every product and sum is the same."""
    spec = wl.LayerSpec("bf16", 16, 2, 512, window=0, k_eq_v=True, rope_theta=1e6)
    lens = [300, 45]
    pb = wl.paged_batch(lens, lens, seed=71)
    case = PagedCase(spec, pb, 71)
    q, k, v, qd, cu, cl = case.write(lens, lens, 71)
    a = case.prefill(qd, cu, cl)
    spec2 = wl.LayerSpec("bf16", 16, 2, 512, window=0, k_eq_v=False, rope_theta=1e6)
    case2 = PagedCase(spec2, pb, 71)
    case2.kc.copy_(case.kc)
    # the same tensor in the V page layout: K's logical rows (tests/layout.py), transposed
    case2.vc.copy_(logical_k(case.kc, pb.block_table, lens, unit_elems("bf16")).transpose(2, 3))
    b = case2.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_workspace_reused_across_calls_of_other_shapes():
    """One workspace, sized once for the largest call, serves consecutive calls of other batch
    sizes and length mixes: nothing a call leaves in it may leak into the next one."""
    spec = wl.LayerSpec("bf16", 8, 2, 256, window=0, rope_theta=1e4)
    p = None
    ws = None
    for k, lens in enumerate([[900, 17, 3000, 1], [2500, 640], [5, 4096, 333, 1200, 77]]):
        pb = wl.paged_batch(lens, [1] * len(lens), seed=60 + k)
        case = PagedCase(spec, pb, 60 + k)
        case.write([L - 1 for L in lens], [L - 1 for L in lens], 160 + k, with_q=False)
        q, kk, v, qd, cu, cl = case.write(lens, [1] * len(lens), 60 + k)
        if ws is None:
            p = case.p
            ws = ga.decode_workspace(p, 8, 4096)
        out = ga.attn_decode(case.p, qd, case.kc, case.vc, case.bt, i32(cl, "cuda"), max(lens),
                             workspace=ws)
        torch.cuda.synchronize()
        ref = case.oracle_attention(qd, cu, cl)
        assert_attn_close(out, ref, "bf16", what=f"workspace reuse call {k}")


def test_decode_sequence_without_keys_gives_zero_output():
    """A sequence whose context is empty (length 0) has no keys: its output rows are zero,
    and the other sequences of the batch are unaffected."""
    spec = wl.LayerSpec("bf16", 8, 4, 256, window=0, rope_theta=1e4)
    lens = [300, 1, 45]
    pb = wl.paged_batch(lens, [1] * 3, seed=64)
    case = PagedCase(spec, pb, 64)
    case.write([299, 0, 44], [299, 0, 44], 164, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, [1] * 3, 64)
    cl0 = cl.copy()
    cl0[1] = 0
    out = ga.attn_decode(case.p, qd, case.kc, case.vc, case.bt, i32(cl0, "cuda"), 300)
    torch.cuda.synchronize()
    assert (out[1].float() == 0).all()
    ref = case.oracle_attention(qd, cu, cl)
    keep = [0, 2]
    assert_attn_close(out[keep], ref[keep], "bf16", what="decode with an empty sequence")


def _stored_values(case, lens, G):
    """The stored value of every position of every sequence, per query head, as the cache
    holds it: [sum(lens)] rows of [Hq][D] (host bits or fp32), gathered through the table (the
    V^T page is [d][row]; with K=V the stored keys, through the K layout)."""
    kc, vc = case.host_caches()
    unit = unit_elems(case.spec.dtype)
    if vc is None:
        kc = logical_k(kc, case.pb.block_table, lens, unit)  # [nb, Hkv, 16, D] as [row][d]
    rows = []
    for b, L in enumerate(lens):
        for t in range(L):
            blk = case.pb.block_table[b, t // wl.BLOCK_SIZE]
            r = t % wl.BLOCK_SIZE
            per_kv = vc[blk, :, :, r] if vc is not None else kc[blk, :, r, :]
            rows.append(np.repeat(per_kv, G, axis=0))
    return np.stack(rows)


@pytest.mark.parametrize("dtype,keqv,cap", [("bf16", False, 0.0), ("bf16", True, 30.0),
                                            ("fp32", False, 0.0), ("fp32", True, 0.0)])
def test_window_of_one_returns_the_own_value_bit_exactly(dtype, keqv, cap):
    """W = 1: every query sees only its own key, whose weight is exactly 1, so each output row
    is the stored value of its own position, bit for bit (prefill rows and decode)."""
    D, Hq, Hkv = 256, 8, 4
    spec = wl.LayerSpec(dtype, Hq, Hkv, D, window=1, softcap=cap, k_eq_v=keqv, rope_theta=1e4,
                        scale=1.0 if cap == 0 else 1.0 / 16)
    lens, news = [40, 17, 70], [40, 9, 33]
    pb = wl.paged_batch(lens, news, seed=61)
    case = PagedCase(spec, pb, 61)
    past = [L - n for L, n in zip(lens, news)]
    case.write(past, past, 62, with_q=False)
    _, _, _, qd, cu, cl = case.write(lens, news, 63)
    out = wl.to_numpy_bits(case.prefill(qd, cu, cl))
    dec = wl.to_numpy_bits(case.decode(qd[torch.from_numpy(cu[1:] - 1).long().to(qd.device)].contiguous(), cl))
    torch.cuda.synchronize()
    vals = _stored_values(case, lens, Hq // Hkv)
    starts = np.concatenate([[0], np.cumsum(lens)])
    want_pre = np.concatenate([vals[starts[b] + past[b]:starts[b + 1]] for b in range(len(lens))])
    want_dec = np.stack([vals[starts[b + 1] - 1] for b in range(len(lens))])
    bits = (lambda x: x.view(np.uint32)) if dtype == "fp32" else (lambda x: x)
    assert np.array_equal(bits(out), bits(want_pre))
    assert np.array_equal(bits(dec), bits(want_dec))


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 8, 4), (512, 16, 2)])
def test_window_beyond_every_length_equals_global(D, Hq, Hkv):
    """W larger than every context sees exactly what a global layer sees: identical bits."""
    outs = []
    for W in (0, 1 << 20):
        spec = wl.LayerSpec("bf16", Hq, Hkv, D, window=W, rope_theta=1e4)
        lens, news = [300, 45, 129], [64, 45, 1]
        pb = wl.paged_batch(lens, news, seed=71)
        case = PagedCase(spec, pb, 71)
        past = [L - n for L, n in zip(lens, news)]
        case.write(past, past, 72, with_q=False)
        _, _, _, qd, cu, cl = case.write(lens, news, 73)
        pre = case.prefill(qd, cu, cl)
        dec = case.decode(qd[torch.from_numpy(cu[1:] - 1).long().to(qd.device)].contiguous(), cl)
        torch.cuda.synchronize()
        outs.append((wl.to_numpy_bits(pre), wl.to_numpy_bits(dec)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("D,W", [(256, 0), (512, 37)])
def test_prefill_largest_group(D, W):
    """16 query heads per kv head, the largest group the bf16 kernels take."""
    spec = wl.LayerSpec("bf16", 16, 1, D, window=W, rope_theta=1e4 if D < 512 else 1e6)
    lens, news = [150, 40], [70, 40]
    pb = wl.paged_batch(lens, news, seed=81)
    case = PagedCase(spec, pb, 81)
    past = [L - n for L, n in zip(lens, news)]
    case.write(past, past, 82, with_q=False)
    _, _, _, qd, cu, cl = case.write(lens, news, 83)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    ref = case.oracle_attention(qd, cu, cl)
    assert_attn_close(out, ref, "bf16", what=f"prefill G16 D{D} W{W}")
