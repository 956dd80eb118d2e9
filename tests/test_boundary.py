"""The C ABI on the CPU: the library loads, exports every function the header declares, and
refuses bad arguments on the host before touching the GPU (no device needed: every call here
fails validation, so nothing is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_kv_cache_write_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma_attn.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ga_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ga.load_library()
    names = declared_functions()
    assert {"ga_kv_cache_write", "ga_attn_decode", "ga_attn_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_debug_library_exports_every_declared_function():
    lib = ctypes.CDLL(ga.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert "ga_debug_take_error" in declared_functions()


def test_debug_take_error_outside_the_debug_build():
    # the regular library has no in-kernel checks: it says so without touching the device
    with pytest.raises(ga.GAError) as e:
        ga.debug_take_error()
    assert e.value.status == 2 and "GA_DEBUG_BOUNDS" in str(e.value)
    dbg = ctypes.CDLL(ga.DEBUG_LIB_PATH)
    dbg.ga_debug_take_error.restype = ctypes.c_int
    dbg.ga_debug_take_error.argtypes = [ctypes.c_void_p]
    assert dbg.ga_debug_take_error(None) == 1  # NULL flags: invalid argument


def good(**kw):
    d = dict(dtype="bf16", num_q_heads=8, num_kv_heads=4, head_dim=256, window=0, scale=1.0,
             softcap=0.0, k_eq_v=False, rope_theta=1e4, rms_eps=1e-6)
    d.update(kw)
    return ga.layer_params(d.pop("dtype"), **d)


def call_decode(p, **kw):
    lib = ga.load_library()
    a = dict(q=FAKE, k_cache=FAKE, v_cache=None if p.k_eq_v else FAKE, num_blocks=10,
             block_table=FAKE, max_blocks=4, context_lens=FAKE, batch=2, max_context_len=64,
             out=FAKE, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    st = lib.ga_attn_decode(ctypes.byref(p), a["q"], a["k_cache"], a["v_cache"],
                            a["num_blocks"], a["block_table"], a["max_blocks"],
                            a["context_lens"], a["batch"], a["max_context_len"], a["out"],
                            a["workspace"], a["workspace_bytes"], a["stream"])
    return st, lib.ga_last_error().decode()


def call_write(p, **kw):
    lib = ga.load_library()
    a = dict(q=FAKE, k=FAKE, v=None if p.k_eq_v else FAKE, wq=None, wk=None, wv=None,
             cu=FAKE, cl=FAKE, bt=FAKE, max_blocks=4, batch=2, total=3, kc=FAKE,
             vc=None if p.k_eq_v else FAKE, num_blocks=10)
    a.update(kw)
    st = lib.ga_kv_cache_write(ctypes.byref(p), a["q"], a["k"], a["v"], a["wq"], a["wk"],
                               a["wv"], a["cu"], a["cl"], a["bt"], a["max_blocks"], a["batch"],
                               a["total"], a["kc"], a["vc"], a["num_blocks"], None)
    return st, lib.ga_last_error().decode()


def call_prefill(p, **kw):
    lib = ga.load_library()
    a = dict(q=FAKE, cu=FAKE, kc=FAKE, vc=None if p.k_eq_v else FAKE, num_blocks=10, bt=FAKE,
             max_blocks=4, cl=FAKE, batch=2, total_q=5, max_q_len=4, out=FAKE)
    a.update(kw)
    st = lib.ga_attn_prefill(ctypes.byref(p), a["q"], a["cu"], a["kc"], a["vc"],
                             a["num_blocks"], a["bt"], a["max_blocks"], a["cl"], a["batch"],
                             a["total_q"], a["max_q_len"], a["out"], None)
    return st, lib.ga_last_error().decode()


INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


@pytest.mark.parametrize("kw,code,msg", [
    (dict(softcap=-1.0), INVALID, "softcap"),           # negative soft cap is refused
    (dict(softcap=float("inf")), INVALID, "softcap"),
    (dict(window=-3), INVALID, "window"),
    (dict(head_dim=192), UNSUPPORTED, "head_dim"),
    (dict(num_q_heads=6, num_kv_heads=4), INVALID, "multiple"),
    (dict(num_q_heads=64, num_kv_heads=2), UNSUPPORTED, "query heads per kv head"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(rope_theta=-1.0), INVALID, "rope_theta"),
    (dict(rms_eps=-1e-6), INVALID, "rms_eps"),
    (dict(rope_angles=-1), INVALID, "rope_angles"),
    (dict(rope_angles=129), INVALID, "rope_angles"),     # > head_dim / 2
    (dict(rope_scale=-8.0), INVALID, "rope_scale"),
    (dict(rope_scale=float("nan")), INVALID, "rope_scale"),
    (dict(page_ring=2), INVALID, "page_ring"),
    (dict(page_ring=True, window=0), INVALID, "sliding window"),
])
def test_decode_rejects_bad_params(kw, code, msg):
    st, err = call_decode(good(**kw))
    assert st == code and msg in err


def test_block_size_must_be_16():
    p = good()
    p.block_size = 32
    st, err = call_decode(p)
    assert st == UNSUPPORTED and "block_size" in err


def test_decode_rejects_bad_arguments():
    p = good()
    assert call_decode(p, v_cache=None)[0] == INVALID                      # V missing
    assert call_decode(good(k_eq_v=True), v_cache=FAKE)[0] == INVALID      # V given with K=V
    assert call_decode(p, max_context_len=65)[0] == INVALID                # > max_blocks*16
    assert call_decode(p, max_context_len=0)[0] == INVALID
    assert call_decode(p, q=None)[0] == INVALID
    assert call_decode(p, batch=-1)[0] == INVALID
    need = ga.decode_workspace_bytes(p, 2, 64)
    assert need > 0
    st, err = call_decode(p, workspace_bytes=need - 1)
    assert st == WORKSPACE and "need" in err
    assert call_decode(p, workspace=None, workspace_bytes=need)[0] == WORKSPACE
    assert call_decode(p, workspace=ctypes.c_void_p(0x1008), workspace_bytes=need)[0] == WORKSPACE


def test_write_rejects_bad_arguments():
    p = good()
    assert call_write(p, v=None)[0] == INVALID
    assert call_write(good(k_eq_v=True), v=FAKE)[0] == INVALID
    assert call_write(good(k_eq_v=True), wv=FAKE)[0] == INVALID
    assert call_write(p, k=None)[0] == INVALID
    assert call_write(p, cu=None)[0] == INVALID
    assert call_write(p, total=-1)[0] == INVALID
    assert call_write(p, num_blocks=0)[0] == INVALID
    assert call_write(good(softcap=-2.0))[0] == INVALID
    # q-only write (a layer reading another layer's cache): k = v = None needs q, refuses
    # k/v inputs and norms
    assert call_write(p, k=None, v=FAKE)[0] == INVALID
    assert call_write(p, k=None, v=None, q=None)[0] == INVALID
    assert call_write(p, k=None, v=None, wk=FAKE)[0] == INVALID
    assert call_write(p, k=None, v=None, wv=FAKE)[0] == INVALID
    assert call_write(p, k=None, v=None, cl=None)[0] == INVALID
    assert call_write(p, k=None, v=None, batch=-1)[0] == INVALID


def test_ring_tables_are_sized_on_the_host():
    """A ring row must hold the decode window (floor((W - 1) / 16) + 2 pages) or a prefill
    chunk plus its first query's window (floor((n + W - 2) / 16) + 3); lengths stay below 2^30.
    Smaller rings are refused before anything is enqueued."""
    p = good(window=1024, page_ring=True)
    st, err = call_decode(p, max_blocks=64, max_context_len=36000)
    assert st == INVALID and "65" in err
    st, err = call_decode(p, max_blocks=65, max_context_len=1 << 30)
    assert st == INVALID and "2^30" in err
    st, err = call_prefill(p, max_blocks=78, max_q_len=256)      # needs (256+1022)//16+3 = 82
    assert st == INVALID and "82" in err
    # without the ring, a context beyond max_blocks * 16 is refused as before
    assert call_decode(good(window=1024), max_blocks=65, max_context_len=36000)[0] == INVALID


def test_exact_kv_params_are_checked():
    """k_eq_v = 2 (exact K=V): both value-factor weights or neither, at most 64 rotated pairs;
    the weights belong to that mode only."""
    assert call_decode(good(k_eq_v=3), v_cache=None)[0] == INVALID
    p = good(k_eq_v=1)
    p.kv_k_norm_w = 0x1000
    assert call_decode(p, v_cache=None)[0] == INVALID
    p = good(k_eq_v=2, head_dim=512, num_kv_heads=2, rope_theta=1e6, rope_angles=64)
    p.kv_k_norm_w = 0x1000
    st, err = call_decode(p, v_cache=None)
    assert st == INVALID and "both" in err
    p = good(k_eq_v=2, head_dim=512, num_kv_heads=2, rope_theta=1e6)  # all 256 pairs rotate
    st, err = call_decode(p, v_cache=None)
    assert st == UNSUPPORTED and "64" in err
    assert call_decode(good(k_eq_v=2, rope_theta=0.0), v_cache=FAKE)[0] == INVALID
    assert call_write(good(k_eq_v=2, rope_angles=64), v=FAKE)[0] == INVALID


def test_prefill_rejects_bad_arguments():
    p = good()
    assert call_prefill(p, cu=None)[0] == INVALID
    assert call_prefill(p, max_q_len=65)[0] == INVALID
    assert call_prefill(p, total_q=-1)[0] == INVALID
    assert call_prefill(good(window=-1))[0] == INVALID


def test_empty_batches_succeed_without_launching():
    p = good()
    assert call_write(p, batch=0, total=0)[0] == 0
    assert call_prefill(p, batch=0, total_q=0)[0] == 0
    need = ga.decode_workspace_bytes(p, 2, 64)
    assert call_decode(p, batch=0, workspace=ctypes.c_void_p(0x10000), workspace_bytes=need)[0] == 0


def test_workspace_size_is_a_pure_function_and_fp32_needs_none():
    p = good()
    assert ga.decode_workspace_bytes(p, 32, 4096) == ga.decode_workspace_bytes(p, 32, 4096)
    assert ga.decode_workspace_bytes(p, 32, 4096) >= ga.decode_workspace_bytes(p, 32, 512)
    assert ga.decode_workspace_bytes(good(dtype="fp32"), 32, 4096) == 0
    assert ga.decode_workspace_bytes(good(softcap=-1.0), 32, 4096) == 0


def _meta(lens, news, bt, nb, require=True, p=None):
    cu = torch.tensor(np.concatenate([[0], np.cumsum(news)]), dtype=torch.int32)
    ga.check_metadata_host(p or good(), cu, torch.tensor(lens, dtype=torch.int32),
                           torch.tensor(bt, dtype=torch.int32), nb, require_nonempty=require)


def test_metadata_check_host():
    bt = [[0, 1, 2], [3, 4, 5]]
    _meta([40, 16], [8, 16], bt, 6)
    with pytest.raises(ga.GAError, match="outside"):
        _meta([40, 16], [8, 16], [[0, 1, 9], [3, 4, 5]], 6)
    with pytest.raises(ga.GAError, match="new tokens"):
        _meta([4, 16], [8, 16], bt, 6)
    with pytest.raises(ga.GAError, match="max_blocks"):
        _meta([49, 16], [8, 16], bt, 6)
    with pytest.raises(ga.GAError, match="same cache slot"):
        _meta([40, 16], [8, 16], [[0, 1, 2], [2, 4, 5]], 6)   # page 2 written by both
    with pytest.raises(ga.GAError, match="< 1"):
        _meta([0, 16], [0, 16], bt, 6)
    _meta([0, 16], [0, 16], bt, 6, require=False)
    with pytest.raises(ga.GAError, match="decreases"):
        _meta([40, 16], [8, -1], bt, 6)


def test_metadata_check_host_ring_rows():
    """Ring rows (page_ring): only the pages the call reads must hold valid ids and fit the
    ring; positions may run past max_blocks * 16."""
    p = good(window=20, page_ring=True)
    # prefill chunk of 8 at L = 100: keys from 2 * ((100 - 8 - 19) // 32) = page 4 .. page 6
    _meta([100], [8], [[0, 1, 2, 3]], 4, p=p)
    with pytest.raises(ga.GAError, match="outside"):
        _meta([100], [8], [[99, 1, 2, 3]], 4, p=p)          # page 4 -> column 0
    # a chunk of 80 new tokens wraps onto itself in a ring of 4 pages (64 slots)
    with pytest.raises(ga.GAError, match="same cache slot"):
        _meta([100], [80], [[0, 1, 2, 3]], 4, p=p)
    # decode rule (no cu_seqlens): the window [80, 100) spans pages 5 and 6 only
    ga.check_metadata_host(p, None, torch.tensor([100], dtype=torch.int32),
                           torch.tensor([[99, 1, 2, 99]], dtype=torch.int32), 4)


def test_status_strings():
    lib = ga.load_library()
    assert lib.ga_status_string(0) == b"GA_OK"
    assert lib.ga_status_string(3) == b"GA_ERR_WORKSPACE"


def test_binding_refuses_host_tensors():
    p = good()
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="device"):
        ga.attn_decode(p, torch.zeros(2, 8, 256, dtype=torch.bfloat16),
                       torch.zeros(10, 4, 16, 256, dtype=torch.bfloat16),
                       torch.zeros(10, 4, 256, 16, dtype=torch.bfloat16),
                       torch.zeros(2, 4, dtype=torch.int32), cl, 64,
                       out=torch.zeros(2, 8, 256, dtype=torch.bfloat16),
                       workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def call_decode_noalloc(p, **kw):
    lib = ga.load_library()
    a = dict(q=FAKE, k_cache=FAKE, v_cache=None if p.k_eq_v else FAKE, num_blocks=10,
             block_table=FAKE, max_blocks=4, context_lens=FAKE, batch=2, max_context_len=64,
             out=FAKE, stream=None)
    a.update(kw)
    st = lib.ga_attn_decode_noalloc(ctypes.byref(p), a["q"], a["k_cache"], a["v_cache"],
                                    a["num_blocks"], a["block_table"], a["max_blocks"],
                                    a["context_lens"], a["batch"], a["max_context_len"],
                                    a["out"], a["stream"])
    return st, lib.ga_last_error().decode()


def test_decode_noalloc_refuses_shapes_beyond_its_scratch():
    """The allocation-free decode refuses a shape whose workspace exceeds the library's array,
    on the host and before the device is touched (no GPU here)."""
    p = good(num_q_heads=32, num_kv_heads=2, head_dim=512, rope_theta=1e6)
    need = ga.decode_workspace_bytes(p, 64, 60000)
    assert need > ga.DECODE_NOALLOC_SCRATCH_BYTES
    st, msg = call_decode_noalloc(p, batch=64, max_blocks=3750, max_context_len=60000)
    assert st == WORKSPACE and "allocation-free" in msg and str(need) in msg


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), INVALID, "required"),
    (dict(max_context_len=0), INVALID, "max_context_len"),
    (dict(max_context_len=65), INVALID, "max_blocks"),
])
def test_decode_noalloc_validates_like_decode(kw, code, msg):
    st, err = call_decode_noalloc(good(), **kw)
    assert st == code and msg in err
    st2, err2 = call_decode(good(), **kw)
    assert st2 == code and err2 == err


def test_decode_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GA_DECODE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ga.DECODE_NOALLOC_SCRATCH_BYTES
