"""The GA_DEBUG_BOUNDS library on the GPU: its in-kernel metadata checks stay silent on valid
metadata, where its results are bit-identical to the regular library's, and each kind of bad
device metadata sets its bit.

Every bad input here is one that the kernels' own clamps and exits keep inside the buffers:
out-of-range block ids are clamped (attention) or the token is skipped (write), inconsistent
lengths end the affected workgroup or wave, and lengths beyond the host bound are clamped to
it.  So no case reads or writes outside its buffers, in either library."""
import numpy as np
import pytest
import torch

import paged_kv_cache_write_amd as ga
import workloads as wl
from harness import PagedCase, i32

pytestmark = pytest.mark.gpu

SPEC = wl.LayerSpec("bf16", 8, 4, 256, window=40, rope_theta=1e4)
SPEC32 = wl.LayerSpec("fp32", 4, 2, 256, window=0, rope_theta=1e4)
LENS, NEWS = [70, 33, 200], [70, 33, 64]


@pytest.fixture
def debug_lib():
    prev = ga.select_library(ga.DEBUG_LIB_PATH)
    try:
        torch.cuda.synchronize()
        ga.debug_take_error()  # start from a clear word
        yield
    finally:
        torch.cuda.synchronize()
        ga.select_library(prev)


def take():
    torch.cuda.synchronize()
    return ga.debug_take_error()


def _prefill_case(spec, seed):
    pb = wl.paged_batch(LENS, NEWS, seed=seed)
    case = PagedCase(spec, pb, seed)
    past = [L - n for L, n in zip(LENS, NEWS)]
    case.write(past, past, seed + 1, with_q=False)
    _, _, _, qd, cu, cl = case.write(LENS, NEWS, seed + 2)
    return case, qd, cu, cl


def _decode_case(spec, lens, seed):
    pb = wl.paged_batch(lens, np.ones(len(lens), np.int32), seed=seed)
    case = PagedCase(spec, pb, seed)
    past = [L - 1 for L in lens]
    case.write(past, past, seed + 1, with_q=False)
    _, _, _, qd, cu, cl = case.write(lens, [1] * len(lens), seed + 2)
    return case, qd, cl


def _run_all(spec):
    """Writes, prefill and decode on valid metadata; returns every result as host bits."""
    case, qd, cu, cl = _prefill_case(spec, 41)
    pre = case.prefill(qd, cu, cl)
    dcase, dq, dcl = _decode_case(spec, [1, 17, 300], 43)
    dec = dcase.decode(dq, dcl)
    torch.cuda.synchronize()
    nb = wl.to_numpy_bits
    return [nb(case.kc), nb(case.vc), nb(qd), nb(pre), nb(dcase.kc), nb(dq), nb(dec)]


@pytest.mark.parametrize("spec", [SPEC, SPEC32], ids=["bf16", "fp32"])
def test_checks_are_silent_and_results_identical(spec):
    ref = _run_all(spec)  # regular library
    prev = ga.select_library(ga.DEBUG_LIB_PATH)
    try:
        take()
        got = _run_all(spec)
        assert take() == 0
    finally:
        ga.select_library(prev)
    # compared as bit patterns: the caches start NaN-filled, and fp32 arrays come back as floats
    bits = lambda x: x.view(np.uint32) if x.dtype == np.float32 else x
    for a, b in zip(ref, got):
        assert np.array_equal(bits(a), bits(b))


def test_block_id_out_of_range(debug_lib):
    case, qd, cu, cl = _prefill_case(SPEC, 51)
    assert take() == 0
    nb = case.pb.num_blocks
    # prefill: a page of sequence 2 in the window of its queries points past the cache
    bad = case.bt.clone()
    bad[2, 10] = nb + 100
    ga.attn_prefill(case.p, qd, i32(cu, case.dev), case.kc, case.vc, bad, i32(cl, case.dev),
                    int(np.diff(cu).max()))
    assert take() == ga.DEBUG_BLOCK_ID
    # write: the page of a new token is negative (the token is skipped)
    q, k, v = wl.raw_qkv(SPEC, 1, 52, device=case.dev)
    bad = case.bt.clone()
    bad[0, 0] = -7
    ga.kv_cache_write(case.p, q, k, v, *case.w, i32([0, 1, 1, 1], case.dev),
                      i32([1, 33, 200], case.dev), bad, case.kc, case.vc)
    assert take() == ga.DEBUG_BLOCK_ID
    # decode: the first page of sequence 1 points past the cache
    dq = qd[:3].contiguous()
    bad = case.bt.clone()
    bad[1, 0] = nb
    ga.attn_decode(case.p, dq, case.kc, case.vc, bad, i32(LENS, case.dev), max(LENS))
    assert take() == ga.DEBUG_BLOCK_ID


def test_inconsistent_lengths(debug_lib):
    case, qd, cu, cl = _prefill_case(SPEC, 61)
    assert take() == 0
    # prefill: sequence 1 has fewer tokens than new queries (L_b < n_b)
    bad = np.array(cl, np.int32)
    bad[1] = NEWS[1] - 1
    ga.attn_prefill(case.p, qd, i32(cu, case.dev), case.kc, case.vc, case.bt,
                    i32(bad, case.dev), int(np.diff(cu).max()))
    assert take() == ga.DEBUG_LENGTH
    # write: 3 new tokens for a sequence of length 2
    q, k, v = wl.raw_qkv(SPEC, 3, 62, device=case.dev)
    ga.kv_cache_write(case.p, q, k, v, *case.w, i32([0, 3], case.dev), i32([2], case.dev),
                      case.bt[:1].contiguous(), case.kc, case.vc)
    assert take() == ga.DEBUG_LENGTH
    # decode: a sequence of length 0
    dq = qd[:3].contiguous()
    ga.attn_decode(case.p, dq, case.kc, case.vc, case.bt, i32([70, 0, 200], case.dev), 200)
    assert take() == ga.DEBUG_LENGTH


def test_length_beyond_host_bound(debug_lib):
    case, qd, cu, cl = _prefill_case(SPEC, 71)
    assert take() == 0
    dq = qd[:3].contiguous()
    # max_context_len = 100 while sequence 2 holds 200 tokens: read as 100, flagged
    ga.attn_decode(case.p, dq, case.kc, case.vc, case.bt, i32(LENS, case.dev), 100)
    assert take() == ga.DEBUG_BOUND


def test_token_without_owner(debug_lib):
    case, qd, cu, cl = _prefill_case(SPEC, 81)
    assert take() == 0
    # 5 new tokens, but cu_seqlens only covers 3 of them
    q, k, v = wl.raw_qkv(SPEC, 5, 82, device=case.dev)
    ga.kv_cache_write(case.p, q, k, v, *case.w, i32([0, 2, 3], case.dev),
                      i32([72, 34], case.dev), case.bt[:2].contiguous(), case.kc, case.vc)
    assert take() == ga.DEBUG_OWNER


def test_fp32_path_checks(debug_lib):
    case, dq, dcl = _decode_case(SPEC32, [5, 40], 91)
    assert take() == 0
    bad = case.bt.clone()
    bad[1, 1] = case.pb.num_blocks + 3
    ga.attn_decode(case.p, dq, case.kc, case.vc, bad, i32(dcl, case.dev), 40)
    assert take() == ga.DEBUG_BLOCK_ID
    ga.attn_decode(case.p, dq, case.kc, case.vc, case.bt, i32([0, 40], case.dev), 40)
    assert take() == ga.DEBUG_LENGTH
