"""Shared set-up for the GPU parity tests: seeded inputs on the device, the library's calls,
and comparisons against the CPU oracle.

The oracle always reads the bytes the GPU stored (normalised q, cache pages) for the
attention-stage checks, so the attention tolerance measures the attention kernels alone; the
write stage is compared separately, element by element, against the oracle's own write.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
import paged_kv_cache_write_amd as ga
import workloads as wl
from layout import logical_k, put_k_rows, unit_elems

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3   # bf16 inputs, fp32 accumulation
FP32_MAX_ABS = 1e-4


def dtype_code(spec):
    return oracle.BF16 if spec.dtype == "bf16" else oracle.FP32


def params(spec, kv_norm_w=None) -> ga.LayerParams:
    return ga.layer_params(spec.dtype, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                           window=spec.window, scale=spec.scale, softcap=spec.softcap,
                           k_eq_v=spec.k_eq_v, rope_theta=spec.rope_theta, rms_eps=spec.rms_eps,
                           rope_angles=spec.rope_angles, rope_scale=spec.rope_scale,
                           page_ring=spec.page_ring, kv_norm_w=kv_norm_w)


def i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class PagedCase:
    """Device caches + block table of one layer, filled through ga.kv_cache_write."""

    def __init__(self, spec: wl.LayerSpec, pb: wl.PagedBatch, seed: int, device="cuda"):
        self.spec, self.pb, self.seed, self.dev = spec, pb, seed, torch.device(device)
        self.kc, self.vc = wl.empty_caches(spec, pb.num_blocks, self.dev)
        exact = spec.k_eq_v == 2  # exact K=V: the layer also has a v norm weight
        w = wl.norm_weights(dataclasses.replace(spec, k_eq_v=False) if exact else spec, seed)
        self.w_cpu = w
        self.w = [None if x is None else x.to(self.dev) for x in w]
        self.kvw = None
        if exact:
            self.kvw = (self.w[1], self.w[2])
            self.w = [self.w[0], self.w[1], None]  # the write takes no v norm
        self.p = params(spec, self.kvw)
        self.bt = i32(pb.block_table, self.dev)

    # -- writes -------------------------------------------------------------------------
    def write(self, context_lens, n_new, seed, q_scale=1.0, with_q=True, device_gen=False):
        """Write n_new[b] fresh tokens ending at context_lens[b]; returns (raw q, k, v, q after
        the call on the device, cu_seqlens, context_lens).  Raw inputs are drawn on the CPU
        (device_gen=False, so the oracle can replay them) or on the GPU (large fills)."""
        cl = np.asarray(context_lens, np.int32)
        nn = np.asarray(n_new, np.int32)
        cu = np.concatenate([[0], np.cumsum(nn)]).astype(np.int32)
        T = int(cu[-1])
        q, k, v = wl.raw_qkv(self.spec, T, seed, q_scale=q_scale,
                             device=self.dev if device_gen else "cpu")
        qd = q.to(self.dev) if with_q else None
        ga.check_metadata_host(self.p, torch.from_numpy(cu), torch.from_numpy(cl),
                               torch.from_numpy(self.pb.block_table), self.pb.num_blocks,
                               require_nonempty=False)
        ga.kv_cache_write(self.p, qd, k.to(self.dev), None if v is None else v.to(self.dev),
                          *self.w, i32(cu, self.dev), i32(cl, self.dev), self.bt, self.kc,
                          self.vc)
        return q, k, v, qd, cu, cl

    def write_all(self, lens, seed):
        """Write every position 0 .. lens[b]-1 in one call (no query)."""
        return self.write(lens, lens, seed, with_q=False)

    def host_caches(self):
        nb = wl.to_numpy_bits
        return nb(self.kc), (None if self.vc is None else nb(self.vc))

    def oracle_write(self, kc, vc, q, k, v, cu, cl):
        """Apply the oracle's write to host caches (in place); returns the oracle's q̂."""
        return oracle_write(self.spec, self.w_cpu, self.pb.block_table, kc, vc, q, k, v, cu, cl)

    # -- attention ------------------------------------------------------------------------
    def prefill(self, q_dev, cu, cl, max_q_len=None):
        return ga.attn_prefill(self.p, q_dev, i32(cu, self.dev), self.kc, self.vc, self.bt,
                               i32(cl, self.dev), int(np.diff(cu).max()) if max_q_len is None
                               else max_q_len)

    def decode(self, q_dev, cl, max_context_len=None):
        return ga.attn_decode(self.p, q_dev, self.kc, self.vc, self.bt, i32(cl, self.dev),
                              int(np.max(cl)) if max_context_len is None else max_context_len)

    def oracle_attention(self, q_dev, cu, cl, rows=None, caches=None):
        s = self.spec
        kc, vc = caches if caches is not None else self.host_caches()
        return oracle.attention(dtype_code(s), s.num_q_heads, s.num_kv_heads, s.head_dim,
                                s.window, float(np.float32(s.scale)), float(np.float32(s.softcap)),
                                int(s.k_eq_v), wl.to_numpy_bits(q_dev), cu, kc, vc,
                                self.pb.block_table, cl, rows=rows, page_ring=s.page_ring)


def oracle_write(spec, w_cpu, block_table, kc, vc, q, k, v, cu, cl):
    """The oracle's write of raw CPU tensors q (or None), k, v into host caches kc / vc
    (numpy, in place); returns the oracle's normalised and rotated q (numpy) or None."""
    nb = wl.to_numpy_bits
    qh = None if q is None else nb(q)
    wq, wk, wv = (None if x is None else x.numpy() for x in w_cpu)
    oracle.kv_cache_write(dtype_code(spec), spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                          float(np.float32(spec.rope_theta)), float(np.float32(spec.rms_eps)),
                          int(spec.k_eq_v), qh, None if k is None else nb(k),
                          None if v is None else nb(v), wq, wk, wv, cu, cl, block_table, kc, vc,
                          rope_angles=spec.rope_angles,
                          rope_scale=float(np.float32(spec.rope_scale)), page_ring=spec.page_ring)
    return qh


def assert_attn_close(got: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, what=""):
    g = got.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    mx, mean = float(err.max()), float(err.mean())
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    else:
        assert mx <= FP32_MAX_ABS, f"{what}: max {mx:.3e}"
    return mx, mean


BF16_UNIT_ROUNDOFF = 2.0 ** -8   # bf16 keeps 8 significant bits: RNE error <= 2^-8 relative


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)); normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float, cap: float) -> np.ndarray:
    """Softmax weights (fp64) of one query q [D] over the visible keys K [n, D]: used only to
    size a rounding bound, never as an expected value."""
    s = scale * (K @ q)
    if cap > 0:
        s = cap * np.tanh(s / cap)
    p = np.exp(s - s.max())
    return p / p.sum()


def weight_rounding_sigma(w: np.ndarray, V: np.ndarray, centre: np.ndarray) -> np.ndarray:
    """Standard deviation, per output dimension, of the error that rounding every weight to
    bf16 before the P.V product adds to sum_j w_j V[j]: each weight w_j picks up a relative
    error d_j, uniform in [-u, u] with u = 2^-8 and independent across keys, so the output
    moves by sum_j w_j d_j (V[j] - centre).  centre = the output itself when the row sum adds
    the same rounded weights (both moves cancel to first order), 0 when the row sum adds the
    unrounded ones."""
    return BF16_UNIT_ROUNDOFF / np.sqrt(3.0) * np.sqrt(((w[:, None] * (V - centre)) ** 2).sum(0))


def assert_within_rounding_bound(a: torch.Tensor, b: torch.Tensor, sigma: np.ndarray, z=6.0):
    """|a - b| <= ulp_bf16(max(|a|, |b|)) + z * sigma, element by element: each side rounds its
    output to bf16 once (half an ulp each), and the rest of their difference is the bf16
    rounding of the softmax weights (sigma = the two sides' standard deviations added; z = 6
    puts a false alarm below 1e-8 per element).  fp32 accumulation error (about 2^-24
    relative per term) is far below both."""
    x, y = a.float().cpu().numpy().astype(np.float64), b.float().cpu().numpy().astype(np.float64)
    tol = bf16_ulp(np.maximum(np.abs(x), np.abs(y))) + z * sigma
    bad = np.abs(x - y) > tol
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements differ by more than the "
                           f"rounding bound; worst excess {float((np.abs(x - y) - tol).max()):.3e}")


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between two arrays of bf16 (uint16) or fp32 bits;
    NaN == NaN counts as 0."""
    if a.dtype == np.uint16:
        ai, bi = a.astype(np.int64), b.astype(np.int64)
        sign = 0x8000
        nan_a = (ai & 0x7FFF) > 0x7F80
        nan_b = (bi & 0x7FFF) > 0x7F80
    else:
        ai = a.view(np.uint32).astype(np.int64)
        bi = b.view(np.uint32).astype(np.int64)
        sign = 0x80000000
        nan_a, nan_b = np.isnan(a), np.isnan(b)
    # map sign-magnitude to a monotone integer line
    ai = np.where(ai & sign, -(ai & (sign - 1)), ai)
    bi = np.where(bi & sign, -(bi & (sign - 1)), bi)
    d = np.abs(ai - bi)
    d = np.where(nan_a & nan_b, 0, d)
    d = np.where(nan_a ^ nan_b, np.iinfo(np.int64).max, d)
    return d


def exact_kv_reference_caches(spec, kc, block_table, lens, wk, wv):
    """fp32 K and V caches (the library's fp32 layouts) holding what exact-K=V stored keys C
    mean: K = RoPE(C) by the oracle's rotation (in double, then fp32) and V = C * w_v / w_k.
    kc: the stored cache as host bits / fp32; wk, wv: CPU fp32 weights."""
    D, Hkv = spec.head_dim, spec.num_kv_heads
    unit = unit_elems(spec.dtype)
    rows = logical_k(kc, block_table, lens, unit)
    if spec.dtype == "bf16":
        rows = (rows.astype(np.uint32) << 16).view(np.float32)
    blk, r, t = [], [], []
    for b, L in enumerate(lens):
        pos = np.arange(int(L))
        blk.append(block_table[b, pos // wl.BLOCK_SIZE])
        r.append(pos % wl.BLOCK_SIZE)
        t.append(pos)
    blk, r, t = (np.concatenate(x).astype(np.int64) for x in (blk, r, t))
    X = rows[blk, :, r, :].astype(np.float64)  # [N, Hkv, D]
    f = spec.rope_scale if spec.rope_scale > 0 else 1.0
    Kr = oracle.rope_rows(X.reshape(-1, D), np.repeat(t, Hkv), float(np.float32(spec.rope_theta)),
                          spec.rope_angles, float(np.float32(f))).reshape(-1, Hkv, D)
    nb = kc.shape[0]
    K = np.full((nb, Hkv, wl.BLOCK_SIZE, D), np.nan, np.float32)
    V = np.full((nb, Hkv, D, wl.BLOCK_SIZE), np.nan, np.float32)
    for g in range(Hkv):
        put_k_rows(K, blk, g, t, Kr[:, g].astype(np.float32), 4)
    ratio = wv.double().numpy() / wk.double().numpy()
    V[blk[:, None], np.arange(Hkv)[None, :], :, r[:, None]] = (X * ratio).astype(np.float32)
    return K, V


def compact_pages(case: PagedCase, seqs, lens):
    """Copy only the pages that sequences `seqs` use into compact host caches, with a block
    table renumbered to match (page gather by block id; no arithmetic on values)."""
    bt = case.pb.block_table
    ids, rows = [], []
    for b in seqs:
        npg = -(-int(lens[b]) // wl.BLOCK_SIZE)
        start = len(ids)
        ids.extend(int(x) for x in bt[b, :npg])
        rows.append(np.arange(start, start + npg))
    idx = torch.tensor(ids, dtype=torch.long, device=case.dev)
    kc = wl.to_numpy_bits(case.kc.index_select(0, idx))
    vc = None if case.vc is None else wl.to_numpy_bits(case.vc.index_select(0, idx))
    width = max(len(r) for r in rows)
    nbt = np.zeros((len(seqs), width), np.int32)
    for i, r in enumerate(rows):
        nbt[i, :len(r)] = r
        nbt[i, len(r):] = r[-1] if len(r) else 0
    return kc, vc, nbt
