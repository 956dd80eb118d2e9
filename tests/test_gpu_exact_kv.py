"""GPU parity of the exact K=V form (k_eq_v = 2, [MNN] §6.2): the cache holds C = k_norm(x)
once, unrotated; the attention kernels rotate it for the scores and scale it by
v_norm_w / k_norm_w for the values.

Two references, both from the oracle:
  * over the stored bytes (the bar of every attention test): K = RoPE(C) by the oracle's
    rotation in double and V = C * v_norm_w / k_norm_w, in fp32 caches, through the oracle's
    ordinary attention, at the layers' score scale 1.0;
  * end to end against the plain definition: the same raw projection x fed to the oracle's
    write as both k and v (K = RoPE(k_norm(x)), V = v_norm(x), each rounded into its own
    cache).  The two sides round the cache differently (the library stores C, the definition
    stores RoPE(k_norm(x)) and v_norm(x)), and with unit-RMS q and k at scale 1.0 the scores
    of these synthetic inputs have a spread of about sqrt(D), which turns those rounding
    differences into visible output differences; so this check runs at the score scale
    1/sqrt(D)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import assert_attn_close, exact_kv_reference_caches, i32

pytestmark = pytest.mark.gpu

BS = 16


class ExactCase:
    """Device cache of an exact K=V layer and host caches of the oracle's two-tensor form."""

    def __init__(self, dtype, Hq, Hkv, D, window, theta, angles, scale_f, lens, seed,
                 softcap=0.0):
        self.spec = wl.LayerSpec(dtype, Hq, Hkv, D, window=window, scale=1.0, softcap=softcap,
                                 rope_theta=theta, rope_angles=angles, rope_scale=scale_f)
        self.pb = wl.paged_batch(lens, lens, seed=seed)
        self.dev = torch.device("cuda")
        self.w = wl.norm_weights(self.spec, seed)  # q, k and v weights (spec has k_eq_v off)
        self.wd = [w.to(self.dev) for w in self.w]
        self.p = ga.layer_params(dtype, Hq, Hkv, D, window=window, scale=1.0, softcap=softcap,
                                 k_eq_v=2, rope_theta=theta, rope_angles=angles,
                                 rope_scale=scale_f, kv_norm_w=(self.wd[1], self.wd[2]))
        self.kc, _ = wl.empty_caches(wl.LayerSpec(dtype, Hq, Hkv, D, k_eq_v=True),
                                     self.pb.num_blocks, self.dev)
        kc_o, vc_o = wl.empty_caches(self.spec, self.pb.num_blocks)
        self.kc_o, self.vc_o = wl.to_numpy_bits(kc_o), wl.to_numpy_bits(vc_o)
        self.bt = i32(self.pb.block_table, self.dev)
        self.code = oracle.BF16 if dtype == "bf16" else oracle.FP32

    def write(self, cl, n, seed, with_q=True):
        """Write n[b] tokens ending at cl[b] on both sides; returns (device q̂, oracle q̂, cu)."""
        s = self.spec
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        q, k, _ = wl.raw_qkv(wl.LayerSpec(s.dtype, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                          k_eq_v=True), int(cu[-1]), seed)
        qd = q.to(self.dev) if with_q else None
        ga.kv_cache_write(self.p, qd, k.to(self.dev), None, self.wd[0], self.wd[1], None,
                          i32(cu, self.dev), i32(cl, self.dev), self.bt, self.kc, None)
        qh = wl.to_numpy_bits(q) if with_q else None
        kb = wl.to_numpy_bits(k)
        oracle.kv_cache_write(self.code, s.num_q_heads, s.num_kv_heads, s.head_dim,
                              float(np.float32(s.rope_theta)), float(np.float32(s.rms_eps)), 0,
                              qh, kb, kb.copy(), self.w[0].numpy(), self.w[1].numpy(),
                              self.w[2].numpy(), cu, cl, self.pb.block_table, self.kc_o,
                              self.vc_o, rope_angles=s.rope_angles,
                              rope_scale=float(np.float32(s.rope_scale)))
        return qd, qh, cu

    def params(self, scale):
        s = self.spec
        return ga.layer_params(s.dtype, s.num_q_heads, s.num_kv_heads, s.head_dim,
                               window=s.window, scale=scale, softcap=s.softcap, k_eq_v=2,
                               rope_theta=s.rope_theta, rope_angles=s.rope_angles,
                               rope_scale=s.rope_scale, kv_norm_w=(self.wd[1], self.wd[2]))

    def oracle_definition(self, qh, cu, cl, scale):
        """Attention over the oracle's own two-tensor caches (the plain definition)."""
        s = self.spec
        return oracle.attention(self.code, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window,
                                float(np.float32(scale)), float(np.float32(s.softcap)), 0, qh,
                                cu, self.kc_o, self.vc_o, self.pb.block_table, cl)

    def oracle_stored(self, q_dev, cu, cl, scale):
        """Attention over what the stored keys C mean: K = RoPE(C), V = C * w_v / w_k."""
        s = self.spec
        K, V = exact_kv_reference_caches(s, wl.to_numpy_bits(self.kc), self.pb.block_table,
                                         self.pb.context_lens, self.w[1], self.w[2])
        q32 = np.ascontiguousarray(q_dev.float().cpu().numpy())
        return oracle.attention(oracle.FP32, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window,
                                float(np.float32(scale)), float(np.float32(s.softcap)), 0, q32,
                                cu, K, V, self.pb.block_table, cl)


CASES = [  # D, Hq, Hkv, theta, rope_angles, rope_scale, window
    (512, 8, 2, 1e6, 64, 8.0, 0),     # Gemma-4 global K=V layer: a quarter of the pairs
    (512, 16, 4, 1e6, 20, 0.0, 0),    # a partial unit of rotated pairs
    (256, 8, 2, 1e4, 64, 0.0, 100),
    (128, 4, 4, 1e4, 64, 0.0, 0),     # full rotation at head size 128
]


@pytest.mark.parametrize("D,Hq,Hkv,theta,angles,f,W", CASES)
def test_exact_kv_decode(D, Hq, Hkv, theta, angles, f, W):
    lens = [3000, 17, 1, 600, 2049]
    c = ExactCase("bf16", Hq, Hkv, D, W, theta, angles, f, lens, seed=70)
    past = np.asarray(lens, np.int32) - 1
    c.write(past, past, 71, with_q=False)
    cl = np.asarray(lens, np.int32)
    qd, qh, cu = c.write(cl, np.ones(len(lens), np.int32), 72)
    small = 1.0 / np.sqrt(D)
    outs = [ga.attn_decode(c.params(sc), qd, c.kc, None, c.bt, i32(cl, c.dev), int(cl.max()))
            for sc in (1.0, small)]
    torch.cuda.synchronize()
    assert_attn_close(outs[0], c.oracle_stored(qd, cu, cl, 1.0), "bf16",
                      what=f"exact K=V decode D={D}, stored keys")
    assert_attn_close(outs[1], c.oracle_definition(qh, cu, cl, small), "bf16",
                      what=f"exact K=V decode D={D}, definition")


@pytest.mark.parametrize("D,Hq,Hkv,theta,angles,f,W", CASES)
def test_exact_kv_chunked_prefill(D, Hq, Hkv, theta, angles, f, W):
    lens, news = [700, 65, 300], [200, 65, 33]
    c = ExactCase("bf16", Hq, Hkv, D, W, theta, angles, f, lens, seed=73, softcap=30.0)
    cl = np.asarray(lens, np.int32)
    past = cl - np.asarray(news, np.int32)
    c.write(past, past, 74, with_q=False)
    qd, qh, cu = c.write(cl, np.asarray(news, np.int32), 75)
    small = 1.0 / np.sqrt(D)
    outs = [ga.attn_prefill(c.params(sc), qd, i32(cu, c.dev), c.kc, None, c.bt, i32(cl, c.dev),
                            int(max(news))) for sc in (1.0, small)]
    torch.cuda.synchronize()
    assert_attn_close(outs[0], c.oracle_stored(qd, cu, cl, 1.0), "bf16",
                      what=f"exact K=V prefill D={D}, stored keys")
    assert_attn_close(outs[1], c.oracle_definition(qh, cu, cl, small), "bf16",
                      what=f"exact K=V prefill D={D}, definition")


def test_exact_kv_fp32():
    lens, news = [90, 33], [90, 5]
    c = ExactCase("fp32", 4, 2, 256, 0, 1e4, 32, 4.0, lens, seed=76)
    cl = np.asarray(lens, np.int32)
    past = cl - np.asarray(news, np.int32)
    c.write(past, past, 77, with_q=False)
    qd, qh, cu = c.write(cl, np.asarray(news, np.int32), 78)
    out = ga.attn_prefill(c.p, qd, i32(cu, c.dev), c.kc, None, c.bt, i32(cl, c.dev), 90)
    torch.cuda.synchronize()
    assert_attn_close(out, c.oracle_stored(qd, cu, cl, 1.0), "fp32", what="exact K=V fp32")
    assert_attn_close(out, c.oracle_definition(qh, cu, cl, 1.0), "fp32",
                      what="exact K=V fp32, definition")


def test_exact_kv_without_rotation_and_equal_weights_is_the_k_eq_v_form():
    """With no RoPE and v_norm_w == k_norm_w, the stored keys are the values: the exact form
    must give the same bits as k_eq_v = 1 over the same cache."""
    lens = [300, 40]
    c = ExactCase("bf16", 8, 2, 512, 0, 0.0, 0, 0.0, lens, seed=79)
    cl = np.asarray(lens, np.int32)
    qd, _, cu = c.write(cl, cl, 80)
    p_same = ga.layer_params("bf16", 8, 2, 512, k_eq_v=2, rope_theta=0.0,
                             kv_norm_w=(c.wd[1], c.wd[1]))
    p_keqv = ga.layer_params("bf16", 8, 2, 512, k_eq_v=1, rope_theta=0.0)
    outs = [ga.attn_prefill(p, qd, i32(cu, c.dev), c.kc, None, c.bt, i32(cl, c.dev), 300)
            for p in (p_same, p_keqv)]
    qlast = torch.stack([qd[cu[1] - 1], qd[cu[2] - 1]]).contiguous()
    dec = [ga.attn_decode(p, qlast, c.kc, None, c.bt, i32(cl, c.dev), 300)
           for p in (p_same, p_keqv)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(dec[0], dec[1])
