"""The library's calls captured into a HIP graph and replayed: every replay must reproduce the
eager result bit for bit (the kernels are deterministic and allocate nothing), also with
unrelated eager work and synchronisations between the replays."""
import pytest
import torch

import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, i32

pytestmark = pytest.mark.gpu


def test_decode_and_write_graph_replays_match_eager():
    spec = wl.LayerSpec("bf16", 8, 4, 256, softcap=50.0, scale=1 / 16, rope_theta=1e4)
    lens = [700, 33, 1500, 2]
    pb = wl.paged_batch(lens, [1] * 4, seed=81)
    case = PagedCase(spec, pb, 81)
    case.write([L - 1 for L in lens], [L - 1 for L in lens], 181, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, [1] * 4, 81)
    kd, vd = k.cuda(), v.cuda()
    cu_d, cl_d = i32(cu, "cuda"), i32(cl, "cuda")
    out = torch.empty_like(qd)
    ws = ga.decode_workspace(case.p, 4, max(lens))

    def step():  # rewrite the newest token's k/v (no q: q is updated in place), then decode
        ga.kv_cache_write(case.p, None, kd, vd, *case.w, cu_d, cl_d, case.bt, case.kc, case.vc)
        ga.attn_decode(case.p, qd, case.kc, case.vc, case.bt, cl_d, max(lens), out=out,
                       workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        # unrelated eager work between replays (another decode into another buffer)
        other = case.decode(qd, cl)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        assert torch.equal(other, eager)


def test_prefill_graph_replays_match_eager():
    spec = wl.LayerSpec("bf16", 16, 2, 512, window=0, rope_theta=1e6)
    lens, news = [300, 90], [100, 90]
    pb = wl.paged_batch(lens, news, seed=82)
    case = PagedCase(spec, pb, 82)
    case.write([200, 0], [200, 0], 182, with_q=False)
    q, k, v, qd, cu, cl = case.write(lens, news, 82)
    cu_d, cl_d = i32(cu, "cuda"), i32(cl, "cuda")
    out = torch.empty_like(qd)

    def run():
        ga.attn_prefill(case.p, qd, cu_d, case.kc, case.vc, case.bt, cl_d, max(news), out=out)

    run()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
