"""Benchmark of the paged-KV Gemma attention hot path on one MI355X.

A step is one pass of the whole path over one batch: ga_kv_cache_write of the batch's new
tokens (norm + RoPE + scatter), then the attention call over the paged cache.  The headline line
measures the largest single-GPU workload, the global-layer K=V decode (16 sequences of about 32k
tokens, 32 query / 4 kv heads, head size 512, keys reused as values, about 2.1 GB of K per
call); the same JSON line carries every other workload (the soft-capped decode, the sliding
decode, the chunked-prefill stack of 5 sliding + 1 global layer, the tiny fp32 sliding case)
with its own roofline block, its error against the CPU oracle and the oracle's time.

value = algorithmic KV bytes read by decode attention per step / wall time per step (GB/s),
with the timed steps replayed as one HIP graph of exactly that many consecutive steps (a
serving loop replays one graph per iteration over all its layers).  Inputs are resident in HBM;
the caches rotate over copies so that the 256 MB last-level cache cannot hold a step's working
set.  The roofline figure times the attention call alone: back-to-back calls between two HIP
events on the launch stream.

--only NAME runs just one workload's timed calls (for counter runs under rocprofv3);
chunked_prefill_bf16_write times the six chunk writes of the prefill stack instead of its
attention calls.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
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
HEADLINE = "kv_shared_decode_bf16"
MFMA_FLOP = 16 * 16 * 32 * 2   # one v_mfma_f32_16x16x32_bf16

# Kernel sources behind each committed counter record: a record applies only while the sha256
# of its sources is unchanged (bench.py reports null otherwise).
DECODE_SOURCES = ("decode.hip", "attn_common.hpp", "device_common.hpp", "launch.hpp")
PREFILL_SOURCES = ("prefill.hip", "prefill_common.hpp", "attn_common.hpp", "device_common.hpp",
                   "launch.hpp")
PROFILES = os.path.join(ROOT, "profiles")


def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_write_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_record(name, files):
    """The JSON record of a committed counter summary under profiles/, or None when there is
    none or its kernel sources changed since it was taken."""
    try:
        text = open(os.path.join(PROFILES, name)).read()
    except OSError:
        return None
    if "```json" not in text:
        return None
    blob = text[text.index("```json") + 7:]
    rec = json.loads(blob[:blob.index("```")])
    if rec.get("sources_sha256") != sources_sha256(files):
        return None
    return rec


def decode_traffic(workload):
    """HBM bytes per attn_decode call of a decode workload from its committed FETCH_SIZE /
    WRITE_SIZE record (each scaled by the copy-kernel calibration), or None."""
    rec = counter_record(f"decode_stream_kernel.{workload}.pmc.md", DECODE_SOURCES)
    return None if rec is None else float(rec["hbm_bytes_per_call"])


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


def params(spec, kv_norm_w=None):
    return ga.layer_params(spec.dtype, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                           window=spec.window, scale=spec.scale, softcap=spec.softcap,
                           k_eq_v=spec.k_eq_v, rope_theta=spec.rope_theta, rms_eps=spec.rms_eps,
                           rope_angles=spec.rope_angles, rope_scale=spec.rope_scale,
                           page_ring=spec.page_ring, kv_norm_w=kv_norm_w)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def f32(x):
    return float(np.float32(x))


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


def write_bytes(spec, T, with_q=True):
    """Algorithmic bytes of one ga_kv_cache_write: every row read once and written once."""
    e = 2 if spec.dtype == "bf16" else 4
    rows = (spec.num_q_heads if with_q else 0) + spec.num_kv_heads * (1 if spec.k_eq_v else 2)
    return 2 * T * rows * spec.head_dim * e


# ----------------------------------------------------------------------------- oracle ---------

def err_stats(got: torch.Tensor, ref: np.ndarray):
    g = got.float().cpu().numpy().astype(np.float64)
    e = np.abs(g - ref)
    return {"max_abs": float(f"{e.max():.4g}"), "mean_abs": float(f"{e.mean():.4g}")}


def window_pages(kc, vc, pb, spec, lens):
    """Host copies (oracle storage) of only the pages each sequence's decode query reads, with
    a block table renumbered to match; logical page indices (and so the K page layout) are
    kept, entries before the window point at compact page 0 and are never read."""
    ids, bt = [], np.zeros_like(pb.block_table)
    for b, L in enumerate(lens):
        lo = max(0, int(L) - spec.window) if spec.window > 0 else 0
        for p in range(lo // BS, (int(L) - 1) // BS + 1):
            bt[b, p] = len(ids)
            ids.append(int(pb.block_table[b, p]))
    idx = torch.tensor(ids, dtype=torch.long, device=kc.device)
    kh = wl.to_numpy_bits(kc.index_select(0, idx))
    vh = None if vc is None else wl.to_numpy_bits(vc.index_select(0, idx))
    return kh, vh, bt


def timed(fn, reps):
    """(median seconds, result of the last run) of `reps` runs of fn()."""
    ts, r = [], None
    for _ in range(reps):
        t0 = time.perf_counter()
        r = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), r


# ----------------------------------------------------------------------------- set-up ---------

class DecodeBench:
    """Caches for one decode workload, the past written by the library, `copies` copies.
    exact=True (a K=V workload): the exact K=V form instead, unrotated keys stored once with 64
    rotated pairs (Gemma-4's proportional RoPE at head size 512) and a v_norm weight."""

    def __init__(self, name, copies, dev, seed=0, exact=False):
        specs, pb = wl.workload(name)
        self.name, self.spec, self.pb, self.dev, self.exact = name, specs[0], pb, dev, exact
        s = self.spec
        if exact:
            ws = wl.norm_weights(dataclasses.replace(s, k_eq_v=False), seed)
            self.w = [ws[0].to(dev), ws[1].to(dev), None]
            self.spec = s = dataclasses.replace(s, k_eq_v=2, rope_angles=64)
            self.kvw = (self.w[1], ws[2].to(dev))
            self.p = params(s, self.kvw)
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
        chunk = 4096
        start = np.zeros(len(past), np.int64)
        while (start < past).any():
            n = np.minimum(past - start, chunk).astype(np.int32)
            cl = (start + n).astype(np.int32)
            cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
            _, k, v = wl.raw_qkv(s, int(cu[-1]), seed + 1000 + int(start.max()), device=dev)
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

    def oracle_check(self, reps):
        """The oracle's decode over the same stored q̂ and cache bytes (cache copy 0): the
        GPU output's error, and the oracle's median wall time over `reps` runs on the host's
        cores.  (The exact K=V form is checked against the oracle by the test-suite only.)"""
        import oracle
        assert self.spec.k_eq_v != 2
        s, pb = self.spec, self.pb
        self.write(0)
        self.attend(0)
        torch.cuda.synchronize()
        lens = pb.context_lens
        kc, vc, bt = window_pages(self.kcs[0], self.vcs[0], pb, s, lens)
        q = wl.to_numpy_bits(self.q)
        code = oracle.BF16 if s.dtype == "bf16" else oracle.FP32
        sec, ref = timed(lambda: oracle.attn_decode(
            code, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, f32(s.scale),
            f32(s.softcap), int(s.k_eq_v), q, kc, vc, bt, lens), reps)
        return err_stats(self.out, ref), sec


class PrefillBench:
    """The 6-layer chunked-prefill stack: per layer a write of the varlen chunk + prefill."""

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
        self.layer_flops = [prefill_flops(s, lens, news) for s in specs]
        self.flops = sum(self.layer_flops)
        self.max_q = int(news.max())

    def write(self, li):
        L = self.layers[li]
        ga.kv_cache_write(L["p"], L["q"], L["k"], L["v"], *L["w"], self.cu, self.cl, self.bt,
                          L["kc"], L["vc"])

    def attend(self, li):
        L = self.layers[li]
        ga.attn_prefill(L["p"], L["q"], self.cu, L["kc"], L["vc"], self.bt, self.cl, self.max_q,
                        out=L["out"])

    def oracle_check(self, rows_per_seq):
        """Sampled rows of the first sliding layer and of the global layer against the oracle
        over the stored bytes (q̂ and caches after the timed write): the GPU's error, and the
        oracle's wall time per row on the host's cores, which extrapolates to the whole stack
        (every row of a sliding layer sees 1024 keys; random rows sample the global layer's mix
        of key counts)."""
        import oracle
        pb = self.pb
        rng = np.random.default_rng(7)
        cu = pb.cu_seqlens
        res = {}
        for li in (0, len(self.layers) - 1):
            L, s = self.layers[li], self.layers[li]["spec"]
            # q is normalised and rotated in place by the write, so write once from the raw
            # projection again before attending
            q_raw, _, _ = wl.raw_qkv(s, pb.total_new, 600 + li, device=self.dev)
            L["q"].copy_(q_raw)
            self.write(li)
            self.attend(li)
            torch.cuda.synchronize()
            rows = np.sort(np.concatenate([
                cu[b] + rng.choice(int(pb.n_new[b]), size=rows_per_seq[li != 0], replace=False)
                for b in range(pb.batch)])).astype(np.int32)
            kc = wl.to_numpy_bits(L["kc"])
            vc = wl.to_numpy_bits(L["vc"])
            q = wl.to_numpy_bits(L["q"])
            t0 = time.perf_counter()
            ref = oracle.attention(oracle.BF16, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                   s.window, f32(s.scale), f32(s.softcap), int(s.k_eq_v), q, cu,
                                   kc, vc, pb.block_table, pb.context_lens, rows=rows)
            sec = time.perf_counter() - t0
            res["sliding" if li == 0 else "global"] = dict(
                rows=len(rows), seconds=sec, err=err_stats(L["out"][rows], ref[rows]))
        n_sl = len(self.layers) - 1
        full = (res["sliding"]["seconds"] / res["sliding"]["rows"] * pb.total_new * n_sl +
                res["global"]["seconds"] / res["global"]["rows"] * pb.total_new)
        return res, full


class TinyBench:
    """The tiny fp32 sliding case: one sequence, a 256-token prefill (write + attention), then
    16 single-token decode steps (write + attention)."""

    def __init__(self, dev, seed=1):
        specs, pb = wl.workload("tiny_sliding_fp32")
        self.spec, self.pb, self.dev = specs[0], pb, dev
        s = self.spec
        self.p = params(s)
        self.w = [x.to(dev) for x in wl.norm_weights(s, seed)]
        self.bt = i32(pb.block_table, dev)
        self.kc, self.vc = wl.empty_caches(s, pb.num_blocks, dev)
        self.q, self.k, self.v = wl.raw_qkv(s, 256, seed, device=dev)
        self.steps = [wl.raw_qkv(s, 1, 100 + i, device=dev) for i in range(16)]
        self.cu0, self.cl0 = i32([0, 256], dev), i32([256], dev)
        self.cu1 = i32([0, 1], dev)
        self.cls = [i32([257 + i], dev) for i in range(16)]
        self.qs = [None] * 16
        self.outs = [None] * 17

    def run(self):
        """The whole case once, q̂ and outputs kept for the oracle."""
        self.qp = self.q.clone()
        ga.kv_cache_write(self.p, self.qp, self.k, self.v, *self.w, self.cu0, self.cl0, self.bt,
                          self.kc, self.vc)
        self.outs[0] = ga.attn_prefill(self.p, self.qp, self.cu0, self.kc, self.vc, self.bt,
                                       self.cl0, 256)
        for i, (q, k, v) in enumerate(self.steps):
            self.qs[i] = q.clone()
            ga.kv_cache_write(self.p, self.qs[i], k, v, *self.w, self.cu1, self.cls[i], self.bt,
                              self.kc, self.vc)
            self.outs[i + 1] = ga.attn_decode(self.p, self.qs[i], self.kc, self.vc, self.bt,
                                              self.cls[i], 257 + i)

    def oracle_check(self, reps):
        """Every output against the oracle over the stored bytes (the cache after all 16 steps
        holds the same bytes at every position each call read); median oracle time of the
        whole case."""
        import oracle
        s, pb = self.spec, self.pb
        torch.cuda.synchronize()
        kc, vc = wl.to_numpy_bits(self.kc), wl.to_numpy_bits(self.vc)
        qp = wl.to_numpy_bits(self.qp)
        qs = [wl.to_numpy_bits(q) for q in self.qs]

        def case():
            r = [oracle.attention(oracle.FP32, 4, 2, 256, 128, 1.0, 0.0, 0, qp,
                                  np.array([0, 256], np.int32), kc, vc, pb.block_table,
                                  np.array([256], np.int32))]
            for i in range(16):
                r.append(oracle.attn_decode(oracle.FP32, 4, 2, 256, 128, 1.0, 0.0, 0, qs[i], kc,
                                            vc, pb.block_table, np.array([257 + i], np.int32)))
            return r
        sec, refs = timed(case, reps)
        errs = [np.abs(o.float().cpu().numpy().astype(np.float64) - r).max()
                for o, r in zip(self.outs, refs)]
        return {"max_abs": float(f"{max(errs):.4g}")}, sec


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
        p = params(s, (ws[1], ws[2]) if exact else None)
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
    8 us on MI355X) to every step."""
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


def hbm_block(nbytes, call_ms, traffic, kernel):
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per call", "bytes_per_call": nbytes,
            "call_us": round(call_ms * 1e3, 2)}


# ----------------------------------------------------------------------------- workloads -----

def run_decode(name, dev, args, copies, exact=False, oracle_reps=0):
    """Step (write + decode, graph-replayed), attention call and write call times of one decode
    workload; with oracle_reps > 0 also its error against the oracle and the oracle's time."""
    db = DecodeBench(name, copies, dev, exact=exact)
    n = len(db.kcs)
    wall = time_chain(lambda i: (db.write(i), db.attend(i)), n, args.steps, args.warmup)
    a_ms = time_calls(db.attend, n, args.steps, args.warmup)
    w_ms = time_calls(db.write, n, args.steps, args.warmup)
    pct = call_percentiles(db.attend, n, max(args.steps, 20), args.warmup)
    tag = name + ("_exact" if exact else "")
    traffic = decode_traffic(tag)
    kern = "attn_decode (decode_stream_kernel + decode_merge_kernel)"
    res = {"roofline": hbm_block(db.bytes, a_ms, traffic, kern),
           "step_us": round(wall * 1e3, 2),
           "step_GBps": round(db.bytes / (wall * 1e-3) / 1e9, 1),
           "write_call_us": round(w_ms * 1e3, 2),
           "write_GBps": round(write_bytes(db.spec, db.pb.batch) / (w_ms * 1e-3) / 1e9, 1),
           "call_us_p10_p50_p90": pct}
    log(f"{tag}: attention call {a_ms * 1e3:.1f} us -> {res['roofline']['achieved']:.0f} GB/s "
        f"({res['roofline']['frac']:.1%}); step {wall * 1e3:.1f} us; write {w_ms * 1e3:.1f} us")
    if oracle_reps and not exact:
        err, sec = db.oracle_check(oracle_reps)
        res["err_vs_oracle"] = err
        res["oracle"] = {"seconds": round(sec, 3), "GBps": round(db.bytes / sec / 1e9, 4),
                         "runs": oracle_reps, "sample": "the whole call"}
        log(f"{tag}: vs oracle max {err['max_abs']:.3e} mean {err['mean_abs']:.3e}; oracle "
            f"{sec:.2f} s")
    return db, wall, res


def run_prefill(dev, args, with_oracle):
    pf = PrefillBench(dev)
    nl = len(pf.layers)

    def stack(i):
        for li in range(nl):
            pf.write(li)
            pf.attend(li)
    wall_p = time_chain(stack, 1, max(args.steps // 5, 3), max(args.warmup // 5, 1))
    a_layers = [time_calls(lambda i, li=li: pf.attend(li), 1, 10, 3) for li in range(nl)]
    w_layers = [time_calls(lambda i, li=li: pf.write(li), 1, 10, 3) for li in range(nl)]
    attn_ms = float(sum(a_layers))
    tf = pf.flops / (attn_ms * 1e-3) / 1e12
    log(f"chunked_prefill: 6-layer attention {attn_ms:.3f} ms -> {tf:.1f} TFLOP/s "
        f"({tf / BF16_PEAK_TFLOPS:.1%}); writes {sum(w_layers):.3f} ms; step {wall_p:.3f} ms")
    rec = counter_record("prefill_tiled_kernel.chunked_prefill_bf16.pmc.md", PREFILL_SOURCES)
    wb = sum(write_bytes(s, pf.pb.total_new) for s in pf.specs)
    res = {"roofline": {"bound": "mfma", "kernel": "attn_prefill (prefill_tiled_kernel), 6 "
                        "layers", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                        "traffic": None, "flops": pf.flops,
                        "mfma_flop_ratio": None if rec is None else rec["mfma_flop_ratio"]},
           "layers": nl, "attn_ms": round(attn_ms, 4),
           "per_layer_attn_ms": [round(x, 4) for x in a_layers],
           "per_layer_TFLOPs": [round(f / (ms * 1e-3) / 1e12, 1)
                                for f, ms in zip(pf.layer_flops, a_layers)],
           "write_ms": round(float(sum(w_layers)), 4),
           "per_layer_write_ms": [round(x, 4) for x in w_layers],
           "write_GBps": round(wb / (sum(w_layers) * 1e-3) / 1e9, 1),
           "step_ms": round(wall_p, 4),
           "step_TFLOPs": round(pf.flops / (wall_p * 1e-3) / 1e12, 2),
           "chunks": {"n_new": pf.pb.n_new.tolist(), "past": pf.pb.past.tolist()}}
    gflops = pf.layer_flops[-1]
    forms = prefill_global_kv_forms(pf, 3)
    for form, ms in forms.items():
        log(f"chunked_prefill global layer, {form}: {ms:.3f} ms -> "
            f"{gflops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    res["global_layer_kv_forms_ms"] = {"separate_v": round(a_layers[-1], 4),
                                       **{f: round(ms, 4) for f, ms in forms.items()}}
    if with_oracle:
        o, full = pf.oracle_check((32, 8))
        res["err_vs_oracle"] = {k: v["err"] for k, v in o.items()}
        res["oracle"] = {"seconds_extrapolated": round(full, 1),
                         "TFLOPs": round(pf.flops / full / 1e12, 6),
                         "sample": f"{o['sliding']['rows']} random rows of a sliding layer "
                                   f"({o['sliding']['seconds']:.2f} s) and {o['global']['rows']} "
                                   f"of the global layer ({o['global']['seconds']:.2f} s), "
                                   f"scaled by rows to the whole 6-layer stack"}
        log(f"chunked_prefill vs oracle: {res['err_vs_oracle']}; oracle extrapolated "
            f"{full:.0f} s")
    del pf
    torch.cuda.empty_cache()
    return res


def run_tiny(dev, with_oracle):
    tb = TinyBench(dev)
    tb.run()
    torch.cuda.synchronize()
    s = tb.spec
    pre_ms = time_calls(lambda i: ga.attn_prefill(tb.p, tb.qp, tb.cu0, tb.kc, tb.vc, tb.bt,
                                                  tb.cl0, 256), 1, 20, 3)
    dec_ms = time_calls(lambda i: ga.attn_decode(tb.p, tb.qs[15], tb.kc, tb.vc, tb.bt,
                                                 tb.cls[15], 272), 1, 20, 3)
    res = {"prefill_call_us": round(pre_ms * 1e3, 2), "decode_call_us": round(dec_ms * 1e3, 2),
           "bound": "latency (one sequence, 256 queries then 16 single decodes)"}
    if with_oracle:
        err, sec = tb.oracle_check(3)
        res["err_vs_oracle"] = err
        res["oracle"] = {"seconds": round(sec, 4), "runs": 3,
                         "sample": "the whole case (prefill + 16 decodes)"}
    log(f"tiny_sliding_fp32: prefill {pre_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us; "
        f"{res.get('err_vs_oracle')}")
    del tb
    torch.cuda.empty_cache()
    return res


def run_only(name, dev, args):
    """Only the timed calls of one workload (for counter runs): set-up, then `steps` attention
    calls (and, for the prefill stack, writes)."""
    if name in ("chunked_prefill_bf16", "chunked_prefill_bf16_write"):
        pf = PrefillBench(dev)
        fn = pf.write if name.endswith("_write") else pf.attend
        ms = [time_calls(lambda i, li=li: fn(li), 1, args.steps, 1) for li in range(len(pf.layers))]
        return {"only": name, "per_layer_ms": [round(x, 4) for x in ms]}
    exact = name.endswith("_exact")
    db = DecodeBench(name[:-6] if exact else name, 2, dev, exact=exact)
    ms = time_calls(db.attend, len(db.kcs), args.steps, args.warmup)
    return {"only": name, "attn_call_us": round(ms * 1e3, 2), "bytes_per_call": db.bytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=2, help="cache copies rotated over steps")
    ap.add_argument("--no-extra", action="store_true", help="headline decode workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="no oracle runs (no cpu_baseline, no error figures)")
    ap.add_argument("--only", default=None, metavar="WORKLOAD",
                    help="only one workload's timed calls (counter runs)")
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
    if args.only:
        print(json.dumps(run_only(args.only, dev, args)), flush=True)
        return
    with_oracle = not args.no_cpu_baseline

    # ---- headline: the global-layer K=V decode -------------------------------------------
    head, wall, hres = run_decode(HEADLINE, dev, args, args.copies, oracle_reps=0)
    props = torch.cuda.get_device_properties(dev)
    value = head.bytes / (wall * 1e-3) / 1e9
    roof = dict(hres["roofline"])
    roof.update({"call_us_p10_p50_p90": hres["call_us_p10_p50_p90"],
                 "write_call_us": hres["write_call_us"],
                 "peak_source": "MI355X published HBM3E bandwidth, 8 TB/s",
                 "measured_copy_GBps": copy_bandwidth(dev),
                 "device": {"name": props.name, "compute_units": props.multi_processor_count}})
    pb = head.pb
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
        "config": {"workload": HEADLINE, "batch": pb.batch,
                   "context_lens": "U[29491, 36044] seeded", "num_q_heads": 32,
                   "num_kv_heads": 4, "head_dim": 512, "k_eq_v": 1, "rope_theta": 1e6,
                   "scale": 1.0, "block_size": BS,
                   "step": "kv_cache_write(16 new tokens: q/k norm + RoPE, keys stored once) + "
                           "attn_decode; the timed steps replayed as one HIP graph, each over "
                           "the next cache copy",
                   "kv_bytes_per_step": head.bytes, "cache_copies_rotated": len(head.kcs),
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if with_oracle:
        err, sec = head.oracle_check(3)
        result["config"]["err_vs_oracle"] = err
        import oracle
        result["cpu_baseline"] = {
            "value": round(head.bytes / sec / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"median of 3 full passes of the oracle's decode attention over the same "
                      f"{pb.batch}-sequence batch and stored bytes ({head.bytes / 1e9:.3f} GB of "
                      f"K per pass, {sec:.2f} s each)"}
        log(f"{HEADLINE}: vs oracle max {err['max_abs']:.3e} mean {err['mean_abs']:.3e}; "
            f"oracle {sec:.2f} s")
    del head
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = {}
        reps = 3 if with_oracle else 0
        for name, copies, exact in (("softcap_decode_bf16", 4, False),
                                    ("sliding_decode_bf16", 2, False),
                                    (HEADLINE, 2, True)):
            db, _, res = run_decode(name, dev, args, copies, exact=exact, oracle_reps=reps)
            extra[name + ("_exact" if exact else "")] = res
            del db
            torch.cuda.empty_cache()
        extra["chunked_prefill_bf16"] = run_prefill(dev, args, with_oracle)
        extra["tiny_sliding_fp32"] = run_tiny(dev, with_oracle)
        result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
