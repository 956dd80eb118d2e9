"""Benchmark of the paged-KV Gemma attention hot path on one MI355X.

A step is one pass of the path over one batch: ga_kv_cache_write of the batch's new tokens
(norm + RoPE + scatter), then the attention call over the paged cache.  The headline line
measures the bf16 soft-capped decode workload (32 sequences, lengths U[512, 4096], 8 query /
4 kv heads, head size 256, cap 50, scale 1/16); the same JSON line also carries the chunked
prefill workload (4 x 2048 new tokens after 6144 cached, 5 sliding + 1 global layer) and the
two other decode workloads, each with its own roofline fraction.

value = algorithmic KV bytes read by decode attention per step / wall time per step (GB/s),
with the timed steps replayed as one HIP graph of exactly that many consecutive steps (a
serving loop replays one graph per iteration over all its layers).  Inputs are
resident in HBM; the caches are rotated over several copies so that the 256 MB last-level
cache cannot hold a step's working set.  The roofline figure times the attention call alone:
back-to-back calls between two HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_write_amd as ga  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
BS = wl.BLOCK_SIZE


# Sources of the decode kernels: the HBM traffic recorded under profiles/ applies only while
# their hash is unchanged.
DECODE_SOURCES = ("decode.hip", "attn_common.hpp", "device_common.hpp", "launch.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stream_kernel.softcap_decode_bf16.pmc.md")


def decode_sources_sha256():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_write_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per attn_decode call of the headline workload from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the copy-kernel calibration), or None
    when there is none or the decode sources changed since it was taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    blob = text[text.index("```json") + 7:]
    rec = json.loads(blob[:blob.index("```")])
    if rec.get("sources_sha256") != decode_sources_sha256():
        return None
    return float(rec["hbm_bytes_per_call"])


def copy_probe(mib):
    """A plain device copy of known size (for calibrating the byte counters)."""
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def params(spec):
    return ga.layer_params(spec.dtype, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                           window=spec.window, scale=spec.scale, softcap=spec.softcap,
                           k_eq_v=spec.k_eq_v, rope_theta=spec.rope_theta, rms_eps=spec.rms_eps,
                           rope_angles=spec.rope_angles, rope_scale=spec.rope_scale,
                           page_ring=spec.page_ring)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


# ----------------------------------------------------------------------------- work models ---

def decode_bytes(spec, lens):
    """Algorithmic bytes of one decode attention call: the visible keys' K (and V) rows, the
    query, the output and the block-table entries read."""
    e = 2 if spec.dtype == "bf16" else 4
    kv_mult = 1 if spec.k_eq_v else 2
    total = 0
    for L in lens:
        keys = min(int(L), spec.window) if spec.window > 0 else int(L)
        lo = int(L) - keys
        pages = (int(L) - 1) // BS - lo // BS + 1
        total += keys * spec.num_kv_heads * spec.head_dim * e * kv_mult
        total += pages * 4 * spec.num_kv_heads
    total += 2 * len(lens) * spec.num_q_heads * spec.head_dim * e
    return total


def prefill_flops(spec, lens, news):
    """4*D flop per visible (query, key, query head) triple (QK^T and PV)."""
    total = 0
    for L, n in zip(lens, news):
        past = int(L) - int(n)
        t = past + np.arange(int(n), dtype=np.int64)
        if spec.window > 0:
            vis = np.minimum(t + 1, spec.window)
        else:
            vis = t + 1
        total += int(vis.sum())
    return total * spec.num_q_heads * 4 * spec.head_dim


# ----------------------------------------------------------------------------- set-up ---------

class DecodeBench:
    """Caches for one decode workload, the past written by the library, `copies` copies.
    exact=True (a K=V workload): the exact K=V form instead, unrotated keys stored once with 64
    rotated pairs (Gemma-4's proportional RoPE at head size 512) and a v_norm weight."""

    def __init__(self, name, copies, dev, seed=0, exact=False):
        specs, pb = wl.workload(name)
        self.name, self.spec, self.pb, self.dev = name, specs[0], pb, dev
        s = self.spec
        if exact:
            ws = wl.norm_weights(dataclasses.replace(s, k_eq_v=False), seed)
            self.w = [ws[0].to(dev), ws[1].to(dev), None]
            self.spec = s = dataclasses.replace(s, k_eq_v=2, rope_angles=64)
            self.kvw = (self.w[1], ws[2].to(dev))
            self.p = ga.layer_params(s.dtype, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                     window=s.window, scale=s.scale, softcap=s.softcap, k_eq_v=2,
                                     rope_theta=s.rope_theta, rms_eps=s.rms_eps,
                                     rope_angles=s.rope_angles, kv_norm_w=self.kvw)
        else:
            self.p = params(s)
            self.w = [None if x is None else x.to(dev) for x in wl.norm_weights(s, seed)]
        lens = pb.context_lens
        past = lens - 1
        self.bt = i32(pb.block_table, dev)
        self.cl = i32(lens, dev)
        self.cu1 = i32(np.arange(pb.batch + 1), dev)
        kc, vc = wl.empty_caches(s, pb.num_blocks, dev)
        # the past, written by the library in chunks (not timed)
        self._write_past(kc, vc, past, seed)
        self.kcs, self.vcs = [kc], [vc]
        for _ in range(copies - 1):
            self.kcs.append(kc.clone())
            self.vcs.append(None if vc is None else vc.clone())
        q, k, v = wl.raw_qkv(s, pb.batch, seed + 1, device=dev)
        self.q, self.k, self.v = q, k, v
        self.out = torch.empty(pb.batch, s.num_q_heads, s.head_dim, dtype=s.torch_dtype,
                               device=dev)
        self.max_len = int(lens.max())
        self.ws = ga.decode_workspace(self.p, pb.batch, self.max_len, dev)
        self.bytes = decode_bytes(s, lens)
        ga.check_metadata_host(self.p, torch.from_numpy(np.arange(pb.batch + 1, dtype=np.int32)),
                               torch.from_numpy(lens), torch.from_numpy(pb.block_table),
                               pb.num_blocks)

    def _write_past(self, kc, vc, past, seed):
        s, dev = self.spec, self.dev
        B = len(past)
        chunk = 4096
        start = np.zeros(B, np.int64)
        while (start < past).any():
            n = np.minimum(past - start, chunk).astype(np.int32)
            cl = (start + n).astype(np.int32)
            cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
            T = int(cu[-1])
            _, k, v = wl.raw_qkv(s, T, seed + 1000 + int(start.max()), device=dev)
            ga.kv_cache_write(self.p, None, k, v, *self.w, i32(cu, dev), i32(cl, dev), self.bt,
                              kc, vc)
            start = start + n
        torch.cuda.synchronize()

    def write(self, i):
        c = i % len(self.kcs)
        ga.kv_cache_write(self.p, self.q, self.k, self.v, *self.w, self.cu1, self.cl, self.bt,
                          self.kcs[c], self.vcs[c])

    def attend(self, i):
        c = i % len(self.kcs)
        ga.attn_decode(self.p, self.q, self.kcs[c], self.vcs[c], self.bt, self.cl, self.max_len,
                       out=self.out, workspace=self.ws)


class PrefillBench:
    """The 6-layer chunked-prefill stack: per layer a write of the 4 x 2048 chunk + prefill."""

    def __init__(self, dev, seed=0):
        specs, pb = wl.workload("chunked_prefill_bf16")
        self.specs, self.pb, self.dev = specs, pb, dev
        self.layers = []
        lens, news = pb.context_lens, pb.n_new
        past = lens - news
        self.bt = i32(pb.block_table, dev)
        self.cu = i32(pb.cu_seqlens, dev)
        self.cl = i32(lens, dev)
        cu_past = np.concatenate([[0], np.cumsum(past)]).astype(np.int32)
        for li, s in enumerate(specs):
            p = params(s)
            w = [None if x is None else x.to(dev) for x in wl.norm_weights(s, 50 + li)]
            kc, vc = wl.empty_caches(s, pb.num_blocks, dev)
            _, kp, vp = wl.raw_qkv(s, int(cu_past[-1]), 500 + li, device=dev)
            ga.kv_cache_write(p, None, kp, vp, *w, i32(cu_past, dev), i32(past, dev), self.bt,
                              kc, vc)
            q, k, v = wl.raw_qkv(s, pb.total_new, 600 + li, device=dev)
            out = torch.empty_like(q)
            self.layers.append(dict(p=p, w=w, kc=kc, vc=vc, q=q, k=k, v=v, out=out, spec=s))
            del kp, vp
        torch.cuda.synchronize()
        self.flops = sum(prefill_flops(s, lens, news) for s in specs)
        self.max_q = int(news.max())

    def write(self, li):
        L = self.layers[li]
        ga.kv_cache_write(L["p"], L["q"], L["k"], L["v"], *L["w"], self.cu, self.cl, self.bt,
                          L["kc"], L["vc"])

    def attend(self, li):
        L = self.layers[li]
        ga.attn_prefill(L["p"], L["q"], self.cu, L["kc"], L["vc"], self.bt, self.cl, self.max_q,
                        out=L["out"])


def prefill_global_kv_forms(pf: "PrefillBench", reps: int):
    """The chunked-prefill workload's global layer (D 512, 32/4 heads) in its two K=V forms:
    k_eq_v = 1 (the stored rotated keys serve as values) and exact K=V (unrotated keys stored
    once, 64 rotated pairs, values scaled by w_v / w_k).  Returns {form: attention ms}."""
    dev, pb = pf.dev, pf.pb
    base = pf.specs[-1]
    lens, news = pb.context_lens, pb.n_new
    past = lens - news
    cu_past = i32(np.concatenate([[0], np.cumsum(past)]), dev)
    res = {}
    for form in ("k_eq_v", "exact_k_eq_v"):
        exact = form == "exact_k_eq_v"
        s = dataclasses.replace(base, k_eq_v=2 if exact else True,
                                rope_angles=64 if exact else 0)
        ws = [x.to(dev) for x in wl.norm_weights(dataclasses.replace(s, k_eq_v=False), 70)]
        p = ga.layer_params(s.dtype, s.num_q_heads, s.num_kv_heads, s.head_dim, window=s.window,
                            scale=s.scale, softcap=s.softcap, k_eq_v=s.k_eq_v,
                            rope_theta=s.rope_theta, rms_eps=s.rms_eps,
                            rope_angles=s.rope_angles,
                            kv_norm_w=(ws[1], ws[2]) if exact else None)
        kc, _ = wl.empty_caches(s, pb.num_blocks, dev)
        _, kp, _ = wl.raw_qkv(s, int(past.sum()), 71, device=dev)
        ga.kv_cache_write(p, None, kp, None, None, ws[1], None, cu_past, i32(past, dev), pf.bt,
                          kc, None)
        q, k, _ = wl.raw_qkv(s, pb.total_new, 72, device=dev)
        ga.kv_cache_write(p, q, k, None, ws[0], ws[1], None, pf.cu, pf.cl, pf.bt, kc, None)
        out = torch.empty_like(q)
        res[form] = time_calls(lambda i: ga.attn_prefill(p, q, pf.cu, kc, None, pf.bt, pf.cl,
                                                         pf.max_q, out=out), 1, reps, 1)
        del kc, kp, q, k, out
        torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- timing ---------

def capture_chain(step_fn, n):
    """One HIP graph holding n consecutive steps step_fn(0) .. step_fn(n - 1).  A serving loop
    replays one graph per decode iteration over all its layers, so a graph launch is paid once
    per many layer steps; timing each step as its own graph would add a launch gap (about
    8 us on the box) to every step."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step_fn(i)
    return g


def time_chain(step_fn, n_distinct, steps, warmup):
    """Wall-clock ms per step: the steps are run eagerly once per distinct input (warm-up, and
    the library's one-time device queries), then `warmup` steps in one graph replay, then
    exactly `steps` steps in one timed graph replay, synchronized on both sides."""
    for i in range(n_distinct):
        step_fn(i)
    torch.cuda.synchronize()
    gw = capture_chain(step_fn, warmup) if warmup > 0 else None
    gt = capture_chain(step_fn, steps)
    torch.cuda.synchronize()
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gt.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del gw, gt
    return ms


def time_calls(fn, n, reps, warmup):
    """Mean device ms of one call: `reps` calls fn(i) back to back on the current stream,
    bracketed by two HIP events (the calls rotate over n inputs)."""
    for i in range(warmup):
        fn(i % n)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i % n)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def call_percentiles(fn, n, reps, warmup):
    """p10 / p50 / p90 of single calls (one HIP event pair around each call, launch stream)."""
    for i in range(warmup):
        fn(i % n)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        fn(i % n)
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    return [round(float(np.percentile(t, q)), 2) for q in (10, 50, 90)]


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of nbytes, as a measured reference next to the 8 TB/s
    peak: GB/s counting the bytes read plus the bytes written."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def cpu_baseline_decode(db: DecodeBench, budget_s: float):
    """The oracle on the host cores, over the same decode batch (the cache copied back)."""
    import oracle
    s, pb = db.spec, db.pb
    kc = wl.to_numpy_bits(db.kcs[0])
    vc = None if db.vcs[0] is None else wl.to_numpy_bits(db.vcs[0])
    q = wl.to_numpy_bits(db.q)
    code = oracle.BF16 if s.dtype == "bf16" else oracle.FP32
    runs, t_total = 0, 0.0
    while t_total < budget_s:
        t0 = time.perf_counter()
        oracle.attn_decode(code, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window,
                           float(np.float32(s.scale)), float(np.float32(s.softcap)),
                           int(s.k_eq_v), q, kc, vc, pb.block_table, pb.context_lens)
        t_total += time.perf_counter() - t0
        runs += 1
    return dict(value=round(db.bytes * runs / t_total / 1e9, 4), unit="GB/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=f"{runs} full passes of the oracle's decode attention over the same "
                       f"{pb.batch}-sequence batch ({db.bytes / 1e9:.3f} GB of K/V each), "
                       f"{t_total:.1f} s total")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="cache copies rotated over steps")
    ap.add_argument("--no-extra", action="store_true", help="headline decode workload only")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    # ---- headline: soft-capped decode -------------------------------------------------
    head = DecodeBench("softcap_decode_bf16", args.copies, dev)
    nc = len(head.kcs)
    wall = time_chain(lambda i: (head.write(i), head.attend(i)), nc, args.steps, args.warmup)
    a_ms = time_calls(head.attend, nc, args.steps, args.warmup)
    w_ms = time_calls(head.write, nc, args.steps, args.warmup)
    pct = call_percentiles(head.attend, nc, max(args.steps, 20), args.warmup)
    copy_gbs = copy_bandwidth(dev)
    props = torch.cuda.get_device_properties(dev)
    value = head.bytes / (wall * 1e-3) / 1e9
    achieved = head.bytes / (a_ms * 1e-3) / 1e9
    log(f"softcap_decode: step {wall * 1e3:.1f} us ({args.steps} steps in one graph); "
        f"attention call {a_ms * 1e3:.1f} us -> {achieved:.0f} GB/s; "
        f"write call {w_ms * 1e3:.1f} us; {value:.0f} GB/s per step")
    result = {
        "metric": "decode attn KV GB/s (% HBM peak); prefill attn TFLOP/s (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "softcap_decode_bf16", "batch": head.pb.batch,
                   "context_lens": "U[512,4096] seeded", "num_q_heads": 8, "num_kv_heads": 4,
                   "head_dim": 256, "softcap": 50.0, "scale": 0.0625, "block_size": BS,
                   "step": "kv_cache_write(32 new tokens) + attn_decode; the timed steps "
                           "replayed as one HIP graph, each over the next cache copy",
                   "kv_bytes_per_step": head.bytes, "cache_copies_rotated": nc,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "attn_decode (decode_stream_kernel + "
                     "decode_merge_kernel)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "traffic_unit": "HBM bytes per attn_decode call",
                     "call_us": round(a_ms * 1e3, 2), "bytes_per_call": head.bytes,
                     "call_us_p10_p50_p90": pct,
                     "write_call_us": round(w_ms * 1e3, 2),
                     "peak_source": "MI355X published HBM3E bandwidth, 8 TB/s",
                     "measured_copy_GBps": copy_gbs,
                     "device": {"name": props.name, "compute_units": props.multi_processor_count}},
    }
    if not args.no_extra:
        extra = {}
        for name in ("sliding_decode_bf16", "kv_shared_decode_bf16",
                     "kv_shared_decode_bf16_exact"):
            exact = name.endswith("_exact")
            base = name[:-len("_exact")] if exact else name
            db = DecodeBench(base, 2 if base == "kv_shared_decode_bf16" else args.copies, dev,
                             exact=exact)
            n = len(db.kcs)
            wall_x = time_chain(lambda i: (db.write(i), db.attend(i)), n,
                                max(args.steps // 2, 5), max(args.warmup // 2, 2))
            a_x = time_calls(db.attend, n, max(args.steps // 2, 5), max(args.warmup // 2, 2))
            gbs = db.bytes / (a_x * 1e-3) / 1e9
            log(f"{name}: attention call {a_x * 1e3:.1f} us -> {gbs:.0f} GB/s "
                f"({gbs / HBM_PEAK_GBS:.1%}); step {wall_x * 1e3:.1f} us")
            extra[name] = {"attn_call_us": round(a_x * 1e3, 2), "kv_bytes": db.bytes,
                           "attn_GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                           "step_us": round(wall_x * 1e3, 2),
                           "step_GBps": round(db.bytes / (wall_x * 1e-3) / 1e9, 1)}
            del db
            torch.cuda.empty_cache()
        pf = PrefillBench(dev)
        nl = len(pf.layers)

        def stack(i):
            for li in range(nl):
                pf.write(li)
                pf.attend(li)
        wall_p = time_chain(stack, 1, max(args.steps // 5, 3), max(args.warmup // 5, 1))
        a_layers = [time_calls(lambda i, li=li: pf.attend(li), 1, 3, 1) for li in range(nl)]
        w_layers = [time_calls(lambda i, li=li: pf.write(li), 1, 3, 1) for li in range(nl)]
        attn_ms = float(sum(a_layers))
        tf = pf.flops / (attn_ms * 1e-3) / 1e12
        log(f"chunked_prefill: 6-layer attention {attn_ms:.3f} ms -> {tf:.1f} TFLOP/s "
            f"({tf / BF16_PEAK_TFLOPS:.1%}); writes {sum(w_layers):.3f} ms; step {wall_p:.3f} ms")
        extra["chunked_prefill_bf16"] = {
            "layers": nl, "attn_ms": round(attn_ms, 4), "write_ms": round(float(sum(w_layers)), 4),
            "step_ms": round(wall_p, 4), "flops": pf.flops, "attn_TFLOPs": round(tf, 2),
            "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
            "per_layer_attn_ms": [round(x, 4) for x in a_layers],
            "step_TFLOPs": round(pf.flops / (wall_p * 1e-3) / 1e12, 2)}
        gflops = prefill_flops(pf.specs[-1], pf.pb.context_lens, pf.pb.n_new)
        forms = prefill_global_kv_forms(pf, 3)
        for form, ms in forms.items():
            log(f"chunked_prefill global layer, {form}: {ms:.3f} ms -> "
                f"{gflops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        extra["chunked_prefill_bf16"]["global_layer_kv_forms_ms"] = {
            "separate_v": round(a_layers[-1], 4),
            **{f: round(ms, 4) for f, ms in forms.items()}}
        result["extra"] = extra
        del pf
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(head, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
