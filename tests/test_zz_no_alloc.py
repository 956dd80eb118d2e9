"""The allocation-free decode entry point (ga_attn_decode_noalloc) against ga_attn_decode.

Both run the same kernels on the same launch plan; only where the scratch lives differs (the
library's own device array instead of a caller workspace), so their outputs must agree bit for
bit.  Calls follow each other on one device and share the array, so a later, smaller call
must not see anything an earlier one left there.  Run this file on its own and after the rest
of the suite: it must pass both ways.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, assert_attn_close, i32

pytestmark = pytest.mark.gpu


def _prepared(spec, lens, seed):
    pb = wl.paged_batch(lens, np.ones(len(lens), np.int32), seed=seed)
    case = PagedCase(spec, pb, seed)
    past = [L - 1 for L in lens]
    if max(past) > 0:
        case.write(past, past, seed + 100, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, [1] * len(lens), seed)
    return case, qd, cu, cl


def _both(case, qd, cl):
    """(ga_attn_decode with its own workspace, ga_attn_decode_noalloc) on the same inputs."""
    cl_d = i32(cl, case.dev)
    mcl = int(np.max(cl))
    ref = ga.attn_decode(case.p, qd, case.kc, case.vc, case.bt, cl_d, mcl)
    out = torch.full_like(ref, float("nan"))
    ga.attn_decode_noalloc(case.p, qd, case.kc, case.vc, case.bt, cl_d, mcl, out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("big,small", [
    # (dtype, Hq, Hkv, D, W, cap, k_eq_v, lens) of the larger call, then of the smaller one
    (("bf16", 8, 4, 256, 0, 50.0, False, [3000, 512, 4096, 1777, 900, 2500, 64, 3333]),
     ("bf16", 8, 4, 256, 0, 50.0, False, [70, 33, 1])),
    (("bf16", 32, 4, 512, 0, 0.0, True, [9000, 4100, 7000]),
     ("bf16", 32, 4, 512, 0, 0.0, True, [300, 17])),
    (("bf16", 32, 16, 256, 1024, 0.0, False, [4096] * 12),
     ("bf16", 8, 2, 128, 40, 0.0, False, [100, 45])),
])
def test_noalloc_decode_equals_workspace_decode(big, small):
    """Two calls in a row, the second smaller: each equals ga_attn_decode bit for bit, and
    the smaller one also matches the oracle."""
    results = []
    for i, (dt, Hq, Hkv, D, W, cap, keqv, lens) in enumerate((big, small)):
        spec = wl.LayerSpec(dt, Hq, Hkv, D, window=W, softcap=cap, k_eq_v=keqv,
                            scale=1.0 if cap == 0 else 1.0 / 16,
                            rope_theta=1e4 if D < 512 else 1e6)
        case, qd, cu, cl = _prepared(spec, lens, seed=300 + i)
        ws = ga.decode_workspace_bytes(case.p, len(lens), int(max(lens)))
        assert ws <= ga.DECODE_NOALLOC_SCRATCH_BYTES
        ref, out = _both(case, qd, cl)
        assert torch.equal(ref, out), f"call {i}: noalloc output differs from the workspace call"
        results.append((case, qd, cu, cl, out))
    case, qd, cu, cl, out = results[1]
    assert_attn_close(out, case.oracle_attention(qd, cu, cl), "bf16", what="noalloc small")


def test_noalloc_decode_fp32_needs_no_scratch():
    """The fp32 path uses no scratch: the entry point still serves it, equal to ga_attn_decode."""
    spec = wl.LayerSpec("fp32", 4, 2, 256, window=128, rope_theta=1e4)
    case, qd, cu, cl = _prepared(spec, [272, 129, 1], seed=310)
    ref, out = _both(case, qd, cl)
    assert torch.equal(ref, out)


def test_noalloc_decode_refuses_oversize_before_touching_the_device():
    """A shape whose workspace exceeds the array is refused with GA_ERR_WORKSPACE and leaves
    `out` untouched."""
    spec = wl.LayerSpec("bf16", 32, 2, 512, window=0, rope_theta=1e6)
    p = ga.layer_params("bf16", 32, 2, 512, rope_theta=1e6)
    lens = [60000] * 64
    assert ga.decode_workspace_bytes(p, 64, 60000) > ga.DECODE_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    kc, vc = wl.empty_caches(spec, 4, dev)
    bt = torch.zeros(64, 3750, dtype=torch.int32, device=dev)
    cl = i32(lens, dev)
    q = torch.zeros(64, 32, 512, dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 7.0)
    with pytest.raises(ga.GAError) as ei:
        ga.attn_decode_noalloc(p, q, kc, vc, bt, cl, 60000, out)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
