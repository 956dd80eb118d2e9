"""GPU parity of ga_kv_cache_write against the oracle's write (element by element)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, assert_attn_close, oracle_write, ulp_distance
from layout import logical_k, unit_elems

pytestmark = pytest.mark.gpu


def _run(spec, lens, news, seed, with_q=True):
    pb = wl.paged_batch(lens, news, seed=seed)
    case = PagedCase(spec, pb, seed)
    # past tokens first (GPU), then the call under test
    past = [L - n for L, n in zip(lens, news)]
    if max(past) > 0:
        case.write(past, past, seed + 100, with_q=False)
    kc0, vc0 = case.host_caches()
    q, k, v, qd, cu, cl = case.write(lens, news, seed, with_q=with_q)
    torch.cuda.synchronize()
    kc1, vc1 = case.host_caches()
    qh = case.oracle_write(kc0, vc0, q if with_q else None, k, v, cu, cl)
    dk = ulp_distance(kc1, kc0)
    dv = None if vc1 is None else ulp_distance(vc1, vc0)
    dq = None if not with_q else ulp_distance(wl.to_numpy_bits(qd), qh)
    return dk, dv, dq


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("k_eq_v", [False, True])
def test_plain_scatter_bit_exact(dtype, D, k_eq_v):
    """Norms off and no rotation: the cache must hold the input bits, nothing else changes."""
    spec = wl.LayerSpec(dtype, 4, 2, D, rope_theta=0.0, k_eq_v=k_eq_v, norm_q=False,
                        norm_k=False, norm_v=False)
    dk, dv, dq = _run(spec, [37, 16, 1, 50], [5, 16, 1, 50], seed=11)
    assert dk.max() == 0 and dq.max() == 0
    if dv is not None:
        assert dv.max() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,theta", [(256, 1e4), (512, 1e6), (128, 1e4)])
@pytest.mark.parametrize("k_eq_v", [False, True])
def test_norm_rope_within_one_ulp(dtype, D, theta, k_eq_v):
    """Norm + rotation in double, rounded once: at most 1 ulp from the oracle, and almost
    always equal (both round a value that agrees to ~1e-15)."""
    spec = wl.LayerSpec(dtype, 8, 2, D, rope_theta=theta, k_eq_v=k_eq_v)
    dk, dv, dq = _run(spec, [300, 17, 65], [300, 1, 20], seed=12)
    for d in (dk, dv, dq):
        if d is None:
            continue
        assert d.max() <= 1
        assert (d > 0).mean() < 1e-3


def test_rope_at_long_positions():
    """Positions up to ~36k with theta 1e6 (the global-layer case): still within 1 ulp."""
    spec = wl.LayerSpec("bf16", 8, 1, 512, rope_theta=1e6, k_eq_v=True)
    lens = [36044, 29491]
    news = [3, 2]
    pb = wl.paged_batch(lens, news, seed=13)
    case = PagedCase(spec, pb, 13)
    kc0, vc0 = case.host_caches()
    q, k, v, qd, cu, cl = case.write(lens, news, 13)
    torch.cuda.synchronize()
    kc1, _ = case.host_caches()
    qh = case.oracle_write(kc0, vc0, q, k, v, cu, cl)
    assert ulp_distance(kc1, kc0).max() <= 1
    assert ulp_distance(wl.to_numpy_bits(qd), qh).max() <= 1


@pytest.mark.parametrize("lens,news", [
    ([40, 9], [7, 9]),  # a decode-sized call (one workgroup per token)
    # chunks: 16-token tiles that straddle sequences and page boundaries (the value pass)
    ([40, 70, 33, 5], [37, 50, 20, 5]),
])
def test_only_owned_slots_change(lens, news):
    """Pages and rows outside the written slots keep their NaN fill (no stray stores)."""
    spec = wl.LayerSpec("bf16", 4, 2, 256)
    pb = wl.paged_batch(lens, news, seed=14)
    case = PagedCase(spec, pb, 14)
    case.write(lens, news, 14)
    torch.cuda.synchronize()
    kc, vc = case.host_caches()
    kc = logical_k(kc, pb.block_table, lens, unit_elems("bf16"))  # rows of used pages in order
    written_k = np.zeros(kc.shape[:3], bool)
    for b, (L, n) in enumerate(zip(lens, news)):
        for t in range(L - n, L):
            written_k[pb.block_table[b, t // 16], :, t % 16] = True
    is_nan_k = (kc & 0x7FFF) > 0x7F80
    assert (~is_nan_k.all(-1) == written_k).all()
    is_nan_v = (vc & 0x7FFF) > 0x7F80
    assert (~is_nan_v.all(-2) == written_k).all()


@pytest.mark.parametrize("dtype,D,theta,angles,scale", [
    ("bf16", 512, 1e6, 64, 8.0),     # global layer: a quarter of the pairs rotated, factor 8
    ("fp32", 256, 1e4, 32, 0.0),
    ("bf16", 256, 1e4, 0, 4.0),
    ("fp32", 512, 1e6, 1, 8.0),
])
def test_proportional_and_scaled_rope_within_one_ulp(dtype, D, theta, angles, scale):
    """Partial rotation (pairs >= angles pass through) and the linear position factor: the
    same one-rounding bound as the full rotation."""
    spec = wl.LayerSpec(dtype, 8, 2, D, rope_theta=theta, k_eq_v=(D == 512),
                        rope_angles=angles, rope_scale=scale)
    dk, dv, dq = _run(spec, [300, 17, 4165], [300, 1, 20], seed=15)
    for d in (dk, dv, dq):
        if d is None:
            continue
        assert d.max() <= 1
        assert (d > 0).mean() < 1e-3


@pytest.mark.parametrize("dtype,D,k_eq_v", [("bf16", 256, False), ("bf16", 512, True),
                                            ("fp32", 128, False)])
def test_q_only_write_for_a_shared_cache_layer(dtype, D, k_eq_v):
    """k = v = None (a layer that reads another layer's cache): the caches keep every bit, the
    block table and caches are not needed, and q comes out as the full write makes it."""
    spec = wl.LayerSpec(dtype, 8, 2, D, rope_theta=1e4, k_eq_v=k_eq_v, rope_angles=D // 8)
    lens, news = [70, 33, 1], [9, 33, 1]
    pb = wl.paged_batch(lens, news, seed=16)
    case = PagedCase(spec, pb, 16)
    case.write(lens, news, 16)                     # fills the caches and makes a reference q
    torch.cuda.synchronize()
    kc0, vc0 = case.host_caches()
    cu = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q, k, v = wl.raw_qkv(spec, int(cu[-1]), 17)
    qd = q.to(case.dev)
    dev = case.dev
    ga.kv_cache_write(case.p, qd, None, None, case.w[0], None, None,
                      torch.from_numpy(cu).to(dev),
                      torch.from_numpy(np.asarray(lens, np.int32)).to(dev), None, None, None)
    torch.cuda.synchronize()
    kc1, vc1 = case.host_caches()
    assert (kc1 == kc0).all() if dtype == "bf16" else (kc1.view(np.uint32) ==
                                                       kc0.view(np.uint32)).all()
    if vc0 is not None:
        assert (vc1.view(np.uint8) == vc0.view(np.uint8)).all()
    # the full write of the same q on a scratch copy of the caches gives the same bits
    qf = q.to(dev)
    kcs, vcs = case.kc.clone(), None if case.vc is None else case.vc.clone()
    ga.kv_cache_write(case.p, qf, k.to(dev), None if v is None else v.to(dev), *case.w,
                      torch.from_numpy(cu).to(dev),
                      torch.from_numpy(np.asarray(lens, np.int32)).to(dev), case.bt, kcs, vcs)
    torch.cuda.synchronize()
    assert ulp_distance(wl.to_numpy_bits(qd), wl.to_numpy_bits(qf)).max() == 0
    # and within one ulp of the oracle's q-only write
    qh = oracle_write(spec, case.w_cpu, pb.block_table, kc0.copy(),
                      None if vc0 is None else vc0.copy(), q, None, None, cu,
                      np.asarray(lens, np.int32))
    assert ulp_distance(wl.to_numpy_bits(qd), qh).max() <= 1


def test_shared_cache_layer_attends_over_the_owner_cache():
    """A cache-owning layer writes its keys; a second layer with its own q norm shares that
    cache (q-only write) and runs prefill attention over it: matches the oracle's attention
    of the oracle's q-only write over the same pages."""
    spec = wl.LayerSpec("bf16", 8, 2, 256, rope_theta=1e4, window=64, softcap=50.0,
                        scale=1.0 / 16)
    lens, news = [150, 40], [30, 40]
    pb = wl.paged_batch(lens, news, seed=18)
    owner = PagedCase(spec, pb, 18)
    owner.write_all(lens, 18)
    torch.cuda.synchronize()
    shared_spec = wl.LayerSpec("bf16", 8, 2, 256, rope_theta=1e4, window=64, softcap=50.0,
                               scale=1.0 / 16)
    w_shared = wl.norm_weights(shared_spec, 19)
    cu = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    cl = np.asarray(lens, np.int32)
    q, _, _ = wl.raw_qkv(shared_spec, int(cu[-1]), 20)
    dev = owner.dev
    qd = q.to(dev)
    ga.kv_cache_write(owner.p, qd, None, None, w_shared[0].to(dev), None, None,
                      torch.from_numpy(cu).to(dev), torch.from_numpy(cl).to(dev), None, None,
                      None)
    out = owner.prefill(qd, cu, cl)
    torch.cuda.synchronize()
    kc, vc = owner.host_caches()
    qh = oracle_write(shared_spec, w_shared, pb.block_table, kc.copy(), vc.copy(), q, None, None,
                      cu, cl)
    s = spec
    ref = oracle.attention(oracle.BF16, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window,
                           float(np.float32(s.scale)), float(np.float32(s.softcap)), 0, qh, cu,
                           kc, vc, pb.block_table, cl)
    assert_attn_close(out, ref, "bf16", what="shared-cache layer")


def test_kv_sharing_topology_sliding_and_global_sources():
    """[MNN] §4.1 sharing pattern in small: one sliding source layer and one global source
    layer own caches; shared layers (sliding, sliding, global, sliding) each normalise and
    rotate their own q with the q-only write and decode over their source's cache."""
    lens = [333, 1, 90, 17]
    sliding = wl.LayerSpec("bf16", 8, 4, 256, window=64, scale=1.0, rope_theta=1e4)
    glob = wl.LayerSpec("bf16", 8, 2, 512, window=0, scale=1.0, k_eq_v=True, rope_theta=1e6,
                        rope_angles=64, rope_scale=8.0)
    sources = {}
    for name, spec, seed in (("s", sliding, 21), ("g", glob, 22)):
        pb = wl.paged_batch(lens, lens, seed=seed)
        case = PagedCase(spec, pb, seed)
        case.write_all(lens, seed)
        sources[name] = (spec, pb, case)
    torch.cuda.synchronize()
    cu = np.arange(len(lens) + 1, dtype=np.int32)
    cl = np.asarray(lens, np.int32)
    for i, which in enumerate("ssgs"):
        spec, pb, case = sources[which]
        w = wl.norm_weights(spec, 30 + i)
        q, _, _ = wl.raw_qkv(spec, len(lens), 40 + i)
        qd = q.to(case.dev)
        ga.kv_cache_write(case.p, qd, None, None, w[0].to(case.dev), None, None,
                          torch.from_numpy(cu).to(case.dev), torch.from_numpy(cl).to(case.dev),
                          None, None, None)
        out = case.decode(qd, cl)
        torch.cuda.synchronize()
        kc, vc = case.host_caches()
        qh = oracle_write(spec, w, pb.block_table, kc.copy(), None if vc is None else vc.copy(),
                          q, None, None, cu, cl)
        assert ulp_distance(wl.to_numpy_bits(qd), qh).max() <= 1
        ref = oracle.attn_decode(oracle.BF16, spec.num_q_heads, spec.num_kv_heads,
                                 spec.head_dim, spec.window, float(np.float32(spec.scale)),
                                 float(np.float32(spec.softcap)), int(spec.k_eq_v),
                                 wl.to_numpy_bits(qd), kc, vc, pb.block_table, cl)
        assert_attn_close(out, ref, "bf16", what=f"shared layer {i} ({which})")


def _draw_write_case(rng):
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([128, 256, 512]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    theta = 0.0 if rng.random() < 0.1 else float(rng.choice([1e4, 1e6]))
    angles = int(rng.choice([0, 1, 8, 20, D // 4, D // 2]))
    scale_f = float(rng.choice([0.0, 0.0, 4.0, 8.0]))
    norms = [bool(rng.random() < 0.8) for _ in range(3)]
    keqv = bool(rng.random() < 0.3)
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 3000, size=B)]
    if rng.random() < 0.5:  # a decode step: one new token per sequence
        news = [1] * B
    else:                   # chunks, one of them possibly the whole sequence
        news = [int(rng.integers(1, min(L, 600) + 1)) for L in lens]
    return dict(dtype=dtype, D=D, Hq=G * Hkv, Hkv=Hkv, theta=theta, angles=angles, f=scale_f,
                norms=norms, keqv=keqv, lens=lens, news=news)


@pytest.mark.parametrize("block", range(2))
def test_seeded_write_fuzz(block):
    """Seeded write cases (seeds 9800 + 8 block ..): random head sizes, group sizes, dtypes,
    RoPE bases, rotated-pair counts, linear factors, norms on or off, K=V, and ragged batches
    written as a decode step or as chunks after a cached past.  Every stored key and value
    and the returned q within 1 ulp of the oracle's write (bit-exact where nothing is
    normalised or rotated).  Every case is printed before it runs."""
    rng = np.random.default_rng(9800 + block)
    for i in range(8):
        c = _draw_write_case(rng)
        seed = 9800 + 8 * block + i
        print(f"write fuzz case {seed}: {c}", flush=True)
        spec = wl.LayerSpec(c["dtype"], c["Hq"], c["Hkv"], c["D"], rope_theta=c["theta"],
                            rope_angles=c["angles"], rope_scale=c["f"], k_eq_v=c["keqv"],
                            norm_q=c["norms"][0], norm_k=c["norms"][1], norm_v=c["norms"][2])
        dk, dv, dq = _run(spec, c["lens"], c["news"], seed=seed)
        for name, d in (("k", dk), ("v", dv), ("q", dq)):
            if d is not None:
                assert d.max() <= 1, f"write fuzz case {seed}: {name} differs by {d.max()} ulp"
