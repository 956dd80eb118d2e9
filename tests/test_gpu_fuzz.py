"""Seeded shape fuzz: decode and chunked prefill against the oracle over random layer shapes.

Each case draws the head size D from {128, 256, 512}, the group G = Hq / Hkv from
{1, 2, 4, 8, 16}, a window from {0, 1, 15, 16, 17, 31, 32, 33, 64, 100} or a random one, the soft
cap, the K=V form and the dtype, then a ragged batch whose lengths sit on both sides of page
(16) and key-tile (32) edges, with chunks of new tokens after a cached past.  The write, the
prefill of the chunks and the decode of the last token of every sequence are compared with
the oracle (the attention stage over the stored bytes, at the parity bars).  Every case is
printed before it runs, and the first failing case stops the test.

A second set draws the exact K=V form (k_eq_v = 2: unrotated keys stored once, rotated in the
attention kernels) with random counts of rotated pairs (1 .. 64, partial units included), a
linear RoPE factor or none, windows, soft cap and ragged chunks; its chunked prefill and decode
are compared with the oracle over what the stored keys mean (K = RoPE(C), V = C w_v / w_k).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, assert_attn_close, i32
from test_gpu_exact_kv import ExactCase

pytestmark = pytest.mark.gpu

EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 95, 96, 97, 127, 128, 129]
WINDOWS = [0, 1, 15, 16, 17, 31, 32, 33, 64, 100]


def draw_case(rng):
    dtype = "fp32" if rng.random() < 0.15 else "bf16"
    D = int(rng.choice([128, 256, 512]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2])) if G >= 8 else int(rng.choice([1, 2, 4]))
    W = int(rng.choice(WINDOWS)) if rng.random() < 0.8 else int(rng.integers(2, 300))
    cap = float(rng.choice([0.0, 0.0, 30.0]))
    keqv = bool(rng.random() < 0.3)
    B = int(rng.integers(1, 6))
    lens, news = [], []
    for _ in range(B):
        L = int(rng.choice(EDGES)) + 32 * int(rng.integers(0, 12)) if rng.random() < 0.7 \
            else int(rng.integers(1, 700))
        n = int(rng.choice([1, L, int(rng.integers(1, L + 1))]))
        lens.append(L)
        news.append(n)
    return dict(dtype=dtype, D=D, Hq=G * Hkv, Hkv=Hkv, W=W, cap=cap, keqv=keqv, lens=lens,
                news=news)


def run_case(c, seed):
    spec = wl.LayerSpec(c["dtype"], c["Hq"], c["Hkv"], c["D"], window=c["W"], softcap=c["cap"],
                        k_eq_v=c["keqv"], scale=1.0 / 16 if c["cap"] else 1.0,
                        rope_theta=1e4 if c["D"] < 512 else 1e6)
    pb = wl.paged_batch(c["lens"], c["news"], seed=seed)
    case = PagedCase(spec, pb, seed)
    past = [L - n for L, n in zip(c["lens"], c["news"])]
    if max(past) > 0:
        case.write(past, past, seed + 7, with_q=False)
    q, k, v, qd, cu, cl = case.write(c["lens"], c["news"], seed)
    out = case.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    assert_attn_close(out, case.oracle_attention(qd, cu, cl), c["dtype"], what="prefill")
    last = torch.from_numpy(cu[1:] - 1).long().to(qd.device)
    dec = case.decode(qd[last].contiguous(), cl)
    torch.cuda.synchronize()
    ref = case.oracle_attention(qd, cu, cl, rows=(cu[1:] - 1).astype(np.int32))
    assert_attn_close(dec, ref[cu[1:] - 1], c["dtype"], what="decode")


@pytest.mark.parametrize("block", range(4))
def test_seeded_shape_fuzz(block):
    """10 cases per block (seeds 9000 + 10 block ..), 40 in all."""
    rng = np.random.default_rng(9000 + block)
    for i in range(10):
        c = draw_case(rng)
        seed = 9000 + 10 * block + i
        print(f"fuzz case {seed}: {c}", flush=True)
        try:
            run_case(c, seed)
        except AssertionError as e:
            raise AssertionError(f"fuzz case {seed} {c}: {e}") from None


ANGLES = [1, 7, 8, 9, 20, 31, 32, 33, 63, 64]


def draw_exact_case(rng):
    c = draw_case(rng)
    c.pop("keqv")
    c["angles"] = min(int(rng.choice(ANGLES)), c["D"] // 2)
    c["f"] = float(rng.choice([0.0, 0.0, 4.0, 8.0]))
    return c


def run_exact_case(c, seed):
    theta = 1e4 if c["D"] < 512 else 1e6
    e = ExactCase(c["dtype"], c["Hq"], c["Hkv"], c["D"], c["W"], theta, c["angles"], c["f"],
                  c["lens"], seed, softcap=c["cap"])
    cl = np.asarray(c["lens"], np.int32)
    news = np.asarray(c["news"], np.int32)
    past = cl - news
    if past.max() > 0:
        e.write(past, past, seed + 7, with_q=False)
    qd, _, cu = e.write(cl, news, seed)
    p = e.params(1.0)
    out = ga.attn_prefill(p, qd, i32(cu, e.dev), e.kc, None, e.bt, i32(cl, e.dev), int(news.max()))
    last = cu[1:] - 1
    dec = ga.attn_decode(p, qd[torch.from_numpy(last).long().to(e.dev)].contiguous(), e.kc, None,
                         e.bt, i32(cl, e.dev), int(cl.max()))
    torch.cuda.synchronize()
    ref = e.oracle_stored(qd, cu, cl, 1.0)
    assert_attn_close(out, ref, c["dtype"], what="exact K=V prefill")
    assert_attn_close(dec, ref[last], c["dtype"], what="exact K=V decode")


@pytest.mark.parametrize("block", range(2))
def test_seeded_exact_kv_fuzz(block):
    """10 exact K=V cases per block (seeds 9500 + 10 block ..), 20 in all."""
    rng = np.random.default_rng(9500 + block)
    for i in range(10):
        c = draw_exact_case(rng)
        seed = 9500 + 10 * block + i
        print(f"exact fuzz case {seed}: {c}", flush=True)
        try:
            run_exact_case(c, seed)
        except AssertionError as e:
            raise AssertionError(f"exact fuzz case {seed} {c}: {e}") from None
