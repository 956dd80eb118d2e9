"""Seeded synthetic inputs for the paged-attention library and its CPU oracle.

This module only draws random numbers and lays out pages: it holds none of the method's
arithmetic (no norm, no rotation, no attention), so both the GPU path's tests and the oracle can
take their inputs from here.  Recipes (one per workload; the numbers are the workloads' own):

* raw q / k / v ~ N(0, 1) drawn in fp32, then rounded to the storage dtype;
* RMSNorm weights 1 + 0.1 * N(0, 1) in fp32, one set per layer (q, k, v each);
* pages: ``num_blocks = sum_b ceil(L_b / 16) + spare``; a random permutation of the block ids
  is dealt to the sequences in order, so pages are non-contiguous and interleaved across
  sequences; unused table entries point at spare blocks; spare blocks are filled with NaN so a
  stray read poisons the output.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclasses.dataclass
class LayerSpec:
    """Per-layer constants of one attention layer (the library's params struct mirrors it)."""
    dtype: str                 # "fp32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int = 0            # W > 0 sliding, 0 global
    scale: float = 1.0
    softcap: float = 0.0
    k_eq_v: bool = False
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    rope_angles: int = 0       # rotated frequency pairs (0 = all D/2)
    rope_scale: float = 0.0    # linear RoPE position divisor (0 = none)
    page_ring: bool = False    # block-table rows are rings of pages (sliding layers)
    norm_q: bool = True
    norm_k: bool = True
    norm_v: bool = True

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclasses.dataclass
class PagedBatch:
    """Sequence lengths and the block table of one call."""
    context_lens: np.ndarray   # int32 [B]: tokens in each sequence after this call's write
    n_new: np.ndarray          # int32 [B]: new tokens of this call
    block_table: np.ndarray    # int32 [B, max_blocks]
    num_blocks: int
    spare_blocks: np.ndarray   # int32 ids of blocks no sequence owns (NaN-filled)

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def past(self) -> np.ndarray:
        return (self.context_lens - self.n_new).astype(np.int32)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.n_new)]).astype(np.int32)

    @property
    def total_new(self) -> int:
        return int(self.n_new.sum())


def paged_batch(context_lens: Sequence[int], n_new: Sequence[int], seed: int,
                spare: int = 64, shuffle: bool = True, extra_cols: int = 0) -> PagedBatch:
    """Deal a random permutation of block ids to the sequences (seeded, CPU)."""
    cl = np.asarray(context_lens, dtype=np.int64)
    nn = np.asarray(n_new, dtype=np.int64)
    assert cl.shape == nn.shape and (nn <= cl).all() and (nn >= 0).all()
    need = [(int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in cl]
    num_blocks = int(sum(need)) + spare
    g = torch.Generator().manual_seed(1000 + seed)
    perm = torch.randperm(num_blocks, generator=g).numpy() if shuffle else np.arange(num_blocks)
    max_blocks = max(max(need), 1) + extra_cols
    bt = np.empty((len(cl), max_blocks), dtype=np.int32)
    pos = 0
    spare_ids = perm[sum(need):]
    for b, nb in enumerate(need):
        bt[b, :nb] = perm[pos:pos + nb]
        pos += nb
        # unused entries point at spare (NaN-filled) blocks, cycling through them
        if max_blocks > nb:
            fill = spare_ids[np.arange(max_blocks - nb) % max(len(spare_ids), 1)] \
                if len(spare_ids) else np.zeros(max_blocks - nb, dtype=np.int64)
            bt[b, nb:] = fill
    return PagedBatch(cl.astype(np.int32), nn.astype(np.int32), bt, num_blocks,
                      np.asarray(spare_ids, dtype=np.int32))


def ring_batch(context_lens: Sequence[int], n_new: Sequence[int], ring: int, seed: int,
               spare: int = 16) -> PagedBatch:
    """Block table whose rows are rings of `ring` pages: each sequence owns `ring` distinct
    blocks (random, interleaved across sequences), logical page p in column p mod ring."""
    cl = np.asarray(context_lens, dtype=np.int64)
    nn = np.asarray(n_new, dtype=np.int64)
    assert cl.shape == nn.shape and (nn <= cl).all() and (nn >= 0).all() and ring >= 1
    num_blocks = len(cl) * ring + spare
    g = torch.Generator().manual_seed(2000 + seed)
    perm = torch.randperm(num_blocks, generator=g).numpy()
    bt = perm[:len(cl) * ring].reshape(len(cl), ring).astype(np.int32)
    return PagedBatch(cl.astype(np.int32), nn.astype(np.int32), bt, num_blocks,
                      np.asarray(perm[len(cl) * ring:], dtype=np.int32))


def _gen(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def raw_qkv(spec: LayerSpec, T: int, seed: int, device="cpu", q_scale: float = 1.0):
    """Raw q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D] (v None when k_eq_v), N(0,1) then cast."""
    g = _gen(seed, device)
    dt = spec.torch_dtype
    q = torch.randn(T, spec.num_q_heads, spec.head_dim, generator=g, device=device)
    k = torch.randn(T, spec.num_kv_heads, spec.head_dim, generator=g, device=device)
    v = None if spec.k_eq_v else torch.randn(T, spec.num_kv_heads, spec.head_dim, generator=g,
                                             device=device)
    if q_scale != 1.0:
        q = q * q_scale
    return q.to(dt), k.to(dt), (None if v is None else v.to(dt))


def norm_weights(spec: LayerSpec, seed: int):
    """(wq, wk, wv) fp32 [D] each, 1 + 0.1*N(0,1); None where the norm is off."""
    g = _gen(5000 + seed, "cpu")
    D = spec.head_dim
    ws = [1.0 + 0.1 * torch.randn(D, generator=g) for _ in range(3)]
    wq = ws[0] if spec.norm_q else None
    wk = ws[1] if spec.norm_k else None
    wv = ws[2] if (spec.norm_v and not spec.k_eq_v) else None
    return wq, wk, wv


def empty_caches(spec: LayerSpec, num_blocks: int, device="cpu"):
    """NaN-filled K cache [nb,Hkv,16,D] and V cache [nb,Hkv,D,16] (None when k_eq_v)."""
    shape_k = (num_blocks, spec.num_kv_heads, BLOCK_SIZE, spec.head_dim)
    shape_v = (num_blocks, spec.num_kv_heads, spec.head_dim, BLOCK_SIZE)
    kc = torch.full(shape_k, float("nan"), dtype=spec.torch_dtype, device=device)
    vc = None if spec.k_eq_v else torch.full(shape_v, float("nan"), dtype=spec.torch_dtype,
                                             device=device)
    return kc, vc


# ------------------------------------------------------------------ named workloads -------

def jittered_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(2000 + seed)
    return torch.randint(lo, hi + 1, (B,), generator=g).numpy().astype(np.int32)


def chunk_lengths(seed: int, B: int = 4, n_mean: int = 2048, n_jit: int = 256,
                  past_lo: int = 5632, past_hi: int = 6656):
    """Seeded varlen chunk shapes: new tokens n_b = n_mean + U_int[-n_jit, n_jit] with the
    last one adjusted so that sum(n_b) = B * n_mean exactly, and past_b ~ U_int[past_lo,
    past_hi].  Returns (n, past) as int32 arrays."""
    g = torch.Generator().manual_seed(3000 + seed)
    d = torch.randint(-n_jit, n_jit + 1, (B,), generator=g).numpy().astype(np.int64)
    d[-1] = -d[:-1].sum()
    n = (n_mean + d).astype(np.int32)
    past = torch.randint(past_lo, past_hi + 1, (B,), generator=g).numpy().astype(np.int32)
    return n, past


def workload(name: str):
    """(LayerSpec list, PagedBatch) of a named workload.

    tiny_sliding_fp32    1 seq, 256-token prefill then 16 decodes, W 128, 4/2 heads, D 256
    softcap_decode_bf16  32 seqs, L ~ U[512, 4096], 8/4 heads, D 256, cap 50, scale 1/16
    sliding_decode_bf16  64 seqs, L 8192, W 1024, 32/16 heads, D 256, norms, theta 1e4
    kv_shared_decode_bf16 16 seqs, L ~ U[29491, 36044], 32/4 heads, D 512, K=V, theta 1e6
    chunked_prefill_bf16 4 seqs, varlen chunks: n_b = 2048 +- up to 256 (8192 new tokens in
                         all) appended after past_b ~ U[5632, 6656] cached tokens (seeded);
                         5 sliding layers (W 1024, D 256, 32/16 heads) + 1 global layer (D 512,
                         32/4 heads, theta 1e6)
    """
    if name == "tiny_sliding_fp32":
        # the table covers the final 272 tokens (17 pages) plus 15 spare: 32 blocks in all
        spec = LayerSpec("fp32", 4, 2, 256, window=128, rope_theta=1e4)
        return [spec], paged_batch([272], [272], seed=1, spare=15)
    if name == "softcap_decode_bf16":
        spec = LayerSpec("bf16", 8, 4, 256, window=0, scale=1.0 / 16.0, softcap=50.0,
                         rope_theta=1e4, norm_q=False, norm_k=False, norm_v=False)
        L = jittered_lengths(32, 512, 4096, seed=2)
        return [spec], paged_batch(L, np.ones(32, np.int32), seed=2)
    if name == "sliding_decode_bf16":
        spec = LayerSpec("bf16", 32, 16, 256, window=1024, rope_theta=1e4)
        return [spec], paged_batch(np.full(64, 8192), np.ones(64, np.int32), seed=3)
    if name == "kv_shared_decode_bf16":
        spec = LayerSpec("bf16", 32, 4, 512, window=0, k_eq_v=True, rope_theta=1e6)
        L = jittered_lengths(16, 29491, 36044, seed=4)
        return [spec], paged_batch(L, np.ones(16, np.int32), seed=4)
    if name == "chunked_prefill_bf16":
        sliding = LayerSpec("bf16", 32, 16, 256, window=1024, rope_theta=1e4)
        glob = LayerSpec("bf16", 32, 4, 512, window=0, rope_theta=1e6)
        news, past = chunk_lengths(seed=5)
        pb = paged_batch(past + news, news, seed=5)
        return [sliding] * 5 + [glob], pb
    raise KeyError(name)


WORKLOADS = ("tiny_sliding_fp32", "softcap_decode_bf16", "sliding_decode_bf16",
             "kv_shared_decode_bf16", "chunked_prefill_bf16")


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def to_numpy_bits(t: Optional[torch.Tensor]):
    """CPU tensor -> numpy array in the oracle's storage (uint16 bits for bf16)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def from_numpy_bits(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())

