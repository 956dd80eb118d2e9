"""GPU parity of ga_kv_cache_write against the oracle's write (element by element)."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import PagedCase, ulp_distance
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


def test_only_owned_slots_change():
    """Pages and rows outside the written slots keep their NaN fill (no stray stores)."""
    spec = wl.LayerSpec("bf16", 4, 2, 256)
    lens, news = [40, 9], [7, 9]
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
