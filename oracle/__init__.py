"""CPU oracle for paged Gemma-style attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library never loads it, and it shares no code with the GPU
path.  The arithmetic lives in ``ga_ref.c`` (double precision, plain loops); this module builds
that file with gcc and wraps it with ctypes over numpy arrays.

bf16 tensors cross this boundary as ``numpy.uint16`` bit patterns, fp32 as ``numpy.float32``.
Cache layouts are the library's documented ones (array shapes ``[blk][g][16][D]`` for K and
``[blk][g][D][16]`` for V):

* a K page ``[blk][g]`` holds its 16 key rows in 16-byte units: unit (row r, x) holds elements
  x*U .. x*U+U-1 of row r (U = 8 for bf16, 4 for fp32) at unit slot
  16*x + (r + 4*(lp % 2) + 4*((x // 8) % 2)) % 16, lp being the page's logical index
  (position // 16) in its sequence;
* a V page ``[blk][g]`` is transposed: element d of the key in row r sits at ``[d][r]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ga_ref.c")
_LIB = os.path.join(_HERE, "libga_ref.so")

FP32, BF16 = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile ga_ref.c into libga_ref.so (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # the sanitizer run of the CPU test-suite points this at an instrumented build
        path = os.environ.get("GA_ORACLE_LIB") or build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.ref_num_threads.restype = ctypes.c_int
        lib.ref_num_threads.argtypes = []
        lib.ref_double_to_bf16.restype = ctypes.c_uint16
        lib.ref_double_to_bf16.argtypes = [dbl]
        lib.ref_bf16_to_double.restype = dbl
        lib.ref_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.ref_slot.restype = i64
        lib.ref_slot.argtypes = [P, i32, ctypes.c_int, i32, i64, i32, P, P]
        lib.ref_rms_norm.restype = None
        lib.ref_rms_norm.argtypes = [P, P, ctypes.c_int, dbl, P]
        lib.ref_rope.restype = None
        lib.ref_rope.argtypes = [P, ctypes.c_int, dbl, dbl, ctypes.c_int, dbl, P]
        lib.ref_rope_rows.restype = None
        lib.ref_rope_rows.argtypes = [P, P, i64, ctypes.c_int, dbl, ctypes.c_int, dbl, P]
        lib.ref_kv_cache_write.restype = ctypes.c_int
        lib.ref_kv_cache_write.argtypes = [ctypes.c_int] * 5 + [dbl, ctypes.c_int, dbl, dbl,
                                                                ctypes.c_int] + [P] * 6 \
            + [P, P, P, i32, ctypes.c_int, i32, P, P]
        lib.ref_attention.restype = ctypes.c_int
        lib.ref_attention.argtypes = [ctypes.c_int] * 6 + [dbl, dbl, ctypes.c_int, P, P, P, P, P,
                                                           i32, ctypes.c_int, P, i32, i32, P,
                                                           i32, P]
        lib.ref_attn_decode.restype = ctypes.c_int
        lib.ref_attn_decode.argtypes = [ctypes.c_int] * 6 + [dbl, dbl, ctypes.c_int, P, P, P, P,
                                                             i32, ctypes.c_int, P, i32, P]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if a is None:
        return None
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected C-contiguous numpy {np.dtype(dtype)} array")
    return a


def _elem(dtype_code):
    return np.uint16 if dtype_code == BF16 else np.float32


# ------------------------------------------------------------------ scalar helpers --------

def num_threads() -> int:
    """Threads the oracle's parallel loops use (OpenMP)."""
    return int(_load().ref_num_threads())


def double_to_bf16(x: float) -> int:
    """Round one double to bf16 (nearest, ties to even); returns the 16-bit pattern."""
    return int(_load().ref_double_to_bf16(float(x)))


def bf16_to_double(h: int) -> float:
    return float(_load().ref_bf16_to_double(int(h)))


def slot(block_table: np.ndarray, req: int, pos: int, block_size: int, page_ring: bool = False):
    """(slot, block id, row in block) of token position ``pos`` of request ``req``; page_ring:
    the table row is a ring (logical page p in entry p mod row length)."""
    bt = _check(np.ascontiguousarray(block_table, dtype=np.int32), np.int32, "block_table")
    blk, off = ctypes.c_int64(), ctypes.c_int64()
    s = _load().ref_slot(_p(bt), bt.shape[1], int(bool(page_ring)), req, pos, block_size,
                         ctypes.byref(blk), ctypes.byref(off))
    return int(s), int(blk.value), int(off.value)


def rms_norm(x: np.ndarray, w: np.ndarray | None, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    y = np.empty_like(x)
    _load().ref_rms_norm(_p(x), _p(w), x.shape[-1], float(eps), _p(y))
    return y


def rope(x: np.ndarray, t: float, theta: float, angles: int = 0, pos_scale: float = 1.0) -> np.ndarray:
    """Rotate-half RoPE of one vector at position t; `angles` rotated frequency pairs (0 = all),
    position divided by `pos_scale`."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    D = x.shape[-1]
    a = angles if 0 < angles < D // 2 else D // 2
    _load().ref_rope(_p(x), D, float(t), float(theta), int(a), float(pos_scale), _p(y))
    return y


def rope_rows(x: np.ndarray, t: np.ndarray, theta: float, angles: int = 0,
              pos_scale: float = 1.0) -> np.ndarray:
    """`rope` of every row x[i] ([N][D]) at its own position t[i]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    t = np.ascontiguousarray(t, dtype=np.float64)
    assert x.ndim == 2 and t.shape == (x.shape[0],)
    D = x.shape[1]
    a = angles if 0 < angles < D // 2 else D // 2
    y = np.empty_like(x)
    _load().ref_rope_rows(_p(x), _p(t), x.shape[0], D, float(theta), int(a), float(pos_scale),
                          _p(y))
    return y


# ------------------------------------------------------------------ entry points ----------

def kv_cache_write(dtype, Hq, Hkv, D, rope_theta, rms_eps, k_eq_v, q, k, v, wq, wk, wv,
                   cu_seqlens, context_lens, block_table, k_cache, v_cache, block_size=16,
                   rope_angles=0, rope_scale=0.0, page_ring=False):
    """Norm + RoPE + scatter in double; updates q (if given), k_cache and v_cache in place.
    k = v = None: q only (a layer sharing another layer's cache); rope_angles: rotated
    frequency pairs (0 = all); rope_scale: position divisor (0 = 1); page_ring: the table rows
    are rings (logical page p in entry p mod row length)."""
    et = _elem(dtype)
    q = _check(q, et, "q")
    k = _check(k, et, "k")
    v = _check(v, et, "v")
    k_cache = _check(k_cache, et, "k_cache")
    v_cache = _check(v_cache, et, "v_cache")
    wq, wk, wv = (None if w is None else _check(np.ascontiguousarray(w, np.float32), np.float32, "w")
                  for w in (wq, wk, wv))
    cu = _check(np.ascontiguousarray(cu_seqlens, np.int32), np.int32, "cu_seqlens")
    cl = _check(np.ascontiguousarray(context_lens, np.int32), np.int32, "context_lens")
    bt = _check(np.ascontiguousarray(block_table, np.int32), np.int32, "block_table")
    rc = _load().ref_kv_cache_write(dtype, Hq, Hkv, D, block_size, float(rope_theta),
                                    int(rope_angles), float(rope_scale),
                                    float(rms_eps), int(k_eq_v), _p(q), _p(k), _p(v), _p(wq),
                                    _p(wk), _p(wv), _p(cu), _p(cl), _p(bt), bt.shape[1],
                                    int(bool(page_ring)), cl.shape[0], _p(k_cache), _p(v_cache))
    if rc:
        raise MemoryError("oracle kv_cache_write failed")


def attention(dtype, Hq, Hkv, D, window, scale, softcap, k_eq_v, q, cu_seqlens_q, k_cache,
              v_cache, block_table, context_lens, rows=None, block_size=16,
              page_ring=False) -> np.ndarray:
    """Plain softmax attention of the packed queries q [T][Hq][D] over the paged cache.

    Returns float64 [T][Hq][D]; rows not listed in ``rows`` (when given) are left as NaN."""
    et = _elem(dtype)
    q = _check(q, et, "q")
    k_cache = _check(k_cache, et, "k_cache")
    v_cache = _check(v_cache, et, "v_cache")
    cu = _check(np.ascontiguousarray(cu_seqlens_q, np.int32), np.int32, "cu_seqlens_q")
    cl = _check(np.ascontiguousarray(context_lens, np.int32), np.int32, "context_lens")
    bt = _check(np.ascontiguousarray(block_table, np.int32), np.int32, "block_table")
    total_q = int(cu[-1])
    out = np.full((total_q, Hq, D), np.nan, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = _load().ref_attention(dtype, Hq, Hkv, D, block_size, int(window), float(scale),
                               float(softcap), int(k_eq_v), _p(q), _p(cu), _p(k_cache),
                               _p(v_cache), _p(bt), bt.shape[1], int(bool(page_ring)), _p(cl),
                               cl.shape[0], total_q,
                               _p(r), 0 if r is None else r.shape[0], _p(out))
    if rc:
        raise MemoryError("oracle attention failed")
    return out


def attn_decode(dtype, Hq, Hkv, D, window, scale, softcap, k_eq_v, q, k_cache, v_cache,
                block_table, context_lens, block_size=16, page_ring=False) -> np.ndarray:
    """One query per sequence at position context_lens[b]-1; returns float64 [B][Hq][D]."""
    et = _elem(dtype)
    q = _check(q, et, "q")
    k_cache = _check(k_cache, et, "k_cache")
    v_cache = _check(v_cache, et, "v_cache")
    cl = _check(np.ascontiguousarray(context_lens, np.int32), np.int32, "context_lens")
    bt = _check(np.ascontiguousarray(block_table, np.int32), np.int32, "block_table")
    B = cl.shape[0]
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().ref_attn_decode(dtype, Hq, Hkv, D, block_size, int(window), float(scale),
                                 float(softcap), int(k_eq_v), _p(q), _p(k_cache), _p(v_cache),
                                 _p(bt), bt.shape[1], int(bool(page_ring)), _p(cl), B,
                                 _p(out))
    if rc:
        raise MemoryError("oracle decode failed")
    return out
