"""GPU parity of sliding-window page recycling: block-table rows used as rings of pages
(logical page p in column p mod max_blocks), written chunk by chunk as a serving loop would.

Each case runs the same chunks through a plain table and through a ring table: the attention
outputs must be identical bit for bit (the window's pages hold the same bytes, and nothing
else is read), and they are compared with the oracle's ring path as well."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, assert_attn_close, dtype_code, i32, oracle_write, ulp_distance

pytestmark = pytest.mark.gpu


def _pair(spec, lens, ring, seed):
    """A plain-table case and a ring-table case of the same layer."""
    plain = PagedCase(spec, wl.paged_batch(lens, lens, seed=seed), seed)
    rspec = wl.LayerSpec(**{**spec.__dict__, "page_ring": True})
    ringc = PagedCase(rspec, wl.ring_batch(lens, lens, ring, seed=seed), seed)
    return plain, ringc


def _chunks(lens, done, chunk):
    n = np.minimum(np.asarray(lens) - done, chunk).astype(np.int32)
    return n, (done + n).astype(np.int32)


@pytest.mark.parametrize("D,Hq,Hkv,W", [(256, 32, 16, 1024), (128, 4, 4, 100)])
def test_ring_decode_over_long_sequences(D, Hq, Hkv, W):
    """Sequences far longer than the ring (36k positions through 65 pages for W = 1024): the
    decode output equals the plain table's bit for bit and the oracle's within tolerance."""
    spec = wl.LayerSpec("bf16", Hq, Hkv, D, window=W, scale=1.0, rope_theta=1e4)
    lens = [36000, 1500, W + 1, 17, 1040] if W == 1024 else [3000, 101, 5, 260]
    ring = (W - 1) // 16 + 2
    plain, ringc = _pair(spec, lens, ring, seed=50)
    done = np.zeros(len(lens), np.int64)
    step = 0
    while (done < lens).any():
        n, cl = _chunks(lens, done, ring * 16)  # a chunk never wraps onto itself
        for c in (plain, ringc):
            c.write(cl, n, 500 + step, with_q=False)
        done += n
        step += 1
    cl = np.asarray(lens, np.int32)
    cu = np.arange(len(lens) + 1, dtype=np.int32)
    q, _, _ = wl.raw_qkv(spec, len(lens), 77)
    outs = []
    for c in (plain, ringc):
        qd = q.to(c.dev)
        ga.kv_cache_write(c.p, qd, None, None, c.w[0], None, None, i32(cu, c.dev), i32(cl, c.dev),
                          None, None, None)
        outs.append((qd, c.decode(qd, cl)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1]), "ring and plain tables disagree"
    kc, vc = ringc.host_caches()
    ref = oracle.attn_decode(oracle.BF16, Hq, Hkv, D, W, 1.0, 0.0, 0,
                             wl.to_numpy_bits(outs[1][0]), kc, vc, ringc.pb.block_table, cl,
                             page_ring=True)
    assert_attn_close(outs[1][1], ref, "bf16", what="ring decode")


@pytest.mark.parametrize("dtype,D,Hq,Hkv,W,chunk", [
    ("bf16", 256, 8, 2, 512, 256),
    ("bf16", 128, 4, 4, 100, 48),
    ("fp32", 128, 4, 2, 40, 24),
])
def test_ring_chunked_prefill(dtype, D, Hq, Hkv, W, chunk):
    """Chunked prefill through the smallest ring the library accepts,
    floor((chunk + W - 2) / 16) + 3 pages: every chunk's output equals the plain table's bit
    for bit, and the last chunk matches the oracle's ring path."""
    spec = wl.LayerSpec(dtype, Hq, Hkv, D, window=W, scale=1.0, rope_theta=1e4,
                        softcap=30.0 if D == 128 else 0.0)
    lens = [1500, 700, W + 13] if dtype == "bf16" else [400, 90]
    ring = (chunk + W - 2) // 16 + 3
    plain, ringc = _pair(spec, lens, ring, seed=51)
    done = np.zeros(len(lens), np.int64)
    step = 0
    while (done < lens).any():
        n, cl = _chunks(lens, done, chunk)
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        outs = []
        for c in (plain, ringc):
            _, _, _, qd, _, _ = c.write(cl, n, 600 + step)
            outs.append((qd, c.prefill(qd, cu, cl, max_q_len=chunk)))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][1], outs[1][1]), f"chunk {step}: ring and plain disagree"
        done += n
        step += 1
    kc, vc = ringc.host_caches()
    ref = ringc.oracle_attention(outs[1][0], cu, cl, caches=(kc, vc))
    assert_attn_close(outs[1][1], ref, dtype, what="ring prefill, last chunk")


def test_ring_write_matches_the_oracle_ring_write():
    """The write through a ring: every stored element within 1 ulp of the oracle's ring write,
    positions that wrapped included, and q as well."""
    spec = wl.LayerSpec("bf16", 8, 2, 256, window=64, rope_theta=1e4, page_ring=True)
    lens = [300, 77, 5]
    ring = (40 + 64 - 2) // 16 + 3
    case = PagedCase(spec, wl.ring_batch(lens, lens, ring, seed=52), 52)
    done = np.zeros(len(lens), np.int64)
    step = 0
    while (done < lens).any():
        n, cl = _chunks(lens, done, 40)
        kc0, vc0 = case.host_caches()
        q, k, v, qd, cu, cl = case.write(cl, n, 700 + step)
        torch.cuda.synchronize()
        kc1, vc1 = case.host_caches()
        qh = case.oracle_write(kc0, vc0, q, k, v, cu, cl)
        assert ulp_distance(kc1, kc0).max() <= 1, step
        assert ulp_distance(vc1, vc0).max() <= 1, step
        assert ulp_distance(wl.to_numpy_bits(qd), qh).max() <= 1, step
        done += n
        step += 1


def _draw_ring_case(rng):
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([128, 256, 512]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    W = int(rng.choice([1, 15, 16, 17, 31, 32, 33, 64, 100])) if rng.random() < 0.7 \
        else int(rng.integers(2, 400))
    B = int(rng.integers(1, 5))
    lens = [int(rng.integers(1, 1600)) for _ in range(B)]
    chunk = max(int(rng.integers(1, 2 * W + 48)), -(-max(lens) // 12))  # at most 12 chunks
    return dict(dtype=dtype, D=D, Hq=G * Hkv, Hkv=Hkv, W=W, cap=float(rng.choice([0.0, 30.0])),
                keqv=bool(rng.random() < 0.3), lens=lens, chunk=chunk)


@pytest.mark.parametrize("block", range(2))
def test_seeded_ring_fuzz(block):
    """Seeded ring-table cases (seeds 9700 + 6 block ..): random shapes, windows, chunk sizes
    and lengths, each through the smallest ring the library accepts for its chunk.  Every
    chunk's prefill and the final decode equal the plain table's bit for bit; the last chunk
    matches the oracle's ring path.  Every case is printed before it runs."""
    rng = np.random.default_rng(9700 + block)
    for i in range(6):
        c = _draw_ring_case(rng)
        seed = 9700 + 6 * block + i
        print(f"ring fuzz case {seed}: {c}", flush=True)
        spec = wl.LayerSpec(c["dtype"], c["Hq"], c["Hkv"], c["D"], window=c["W"], scale=1.0,
                            softcap=c["cap"], k_eq_v=c["keqv"],
                            rope_theta=1e4 if c["D"] < 512 else 1e6)
        lens, chunk = c["lens"], c["chunk"]
        ring = (chunk + c["W"] - 2) // 16 + 3
        plain, ringc = _pair(spec, lens, ring, seed=seed)
        done = np.zeros(len(lens), np.int64)
        step = 0
        while (done < lens).any():
            n, cl = _chunks(lens, done, chunk)
            cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
            outs = []
            for case in (plain, ringc):
                _, _, _, qd, _, _ = case.write(cl, n, seed * 100 + step)
                outs.append((qd, case.prefill(qd, cu, cl, max_q_len=chunk)))
            torch.cuda.synchronize()
            assert torch.equal(outs[0][1], outs[1][1]), \
                f"ring fuzz case {seed} chunk {step}: ring and plain disagree"
            done += n
            step += 1
        kc, vc = ringc.host_caches()
        ref = ringc.oracle_attention(outs[1][0], cu, cl, caches=(kc, vc))
        assert_attn_close(outs[1][1], ref, c["dtype"], what=f"ring fuzz case {seed}, last chunk")
        qdec = wl.raw_qkv(spec, len(lens), seed + 1)[0].to(ringc.dev)  # one query per sequence
        dec = [case.decode(qdec, cl) for case in (plain, ringc)]
        torch.cuda.synchronize()
        assert torch.equal(dec[0], dec[1]), f"ring fuzz case {seed}: decode disagrees"
