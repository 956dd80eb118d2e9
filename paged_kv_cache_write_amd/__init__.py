"""Python binding of libgemma_attn.so (paged KV write + Gemma-style attention on MI355X).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
torch tensors supply device memory and the current HIP stream.  The C ABI is documented in
include/gemma_attn.h; each function here has the same name without the ``ga_`` prefix.

If the shared library is missing this module raises on first use: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libgemma_attn.so")
# the same library built with the in-kernel metadata checks (GA_DEBUG_BOUNDS)
DEBUG_LIB_PATH = os.path.join(_PKG, "lib", "libgemma_attn_debug.so")

GA_FP32, GA_BF16 = 0, 1
BLOCK_SIZE = 16
STATUS = {0: "GA_OK", 1: "GA_ERR_INVALID_ARG", 2: "GA_ERR_UNSUPPORTED", 3: "GA_ERR_WORKSPACE",
          4: "GA_ERR_HIP"}


class GAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class LayerParams(ctypes.Structure):
    """Mirror of ga_layer_params."""
    _fields_ = [("dtype", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("window", ctypes.c_int32),
                ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
                ("k_eq_v", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("rope_angles", ctypes.c_int32),
                ("rope_scale", ctypes.c_float), ("page_ring", ctypes.c_int32),
                ("kv_k_norm_w", ctypes.c_void_p), ("kv_v_norm_w", ctypes.c_void_p)]


def layer_params(dtype, num_q_heads: int, num_kv_heads: int, head_dim: int, window: int = 0,
                 scale: float = 1.0, softcap: float = 0.0, k_eq_v: bool = False,
                 rope_theta: float = 10000.0, rms_eps: float = 1e-6,
                 block_size: int = BLOCK_SIZE, rope_angles: int = 0,
                 rope_scale: float = 0.0, page_ring: bool = False,
                 kv_norm_w=None) -> LayerParams:
    """dtype: torch.float32 / torch.bfloat16, or "fp32" / "bf16".  k_eq_v: 0/False separate
    K and V, 1/True one cache of rotated keys serves both, 2 exact K=V (unrotated keys stored
    once; kv_norm_w = (k_norm weight, v_norm weight) as device fp32 tensors, kept alive by the
    caller, or None when neither norm has a weight).  rope_angles: rotated frequency pairs
    (0 = all); rope_scale: linear position divisor (0 = none); page_ring: block table rows are
    rings (logical page p in column p mod max_blocks; sliding layers only)."""
    code = GA_BF16 if dtype in (torch.bfloat16, "bf16", GA_BF16) else GA_FP32
    kw = kvw = None
    if kv_norm_w is not None:
        wk, wv = kv_norm_w
        for w in (wk, wv):
            if not (isinstance(w, torch.Tensor) and w.is_cuda and w.dtype == torch.float32
                    and w.is_contiguous() and w.numel() == head_dim):
                raise TypeError("kv_norm_w: expected two contiguous fp32 device tensors [D]")
        kw, kvw = wk.data_ptr(), wv.data_ptr()
    return LayerParams(code, num_q_heads, num_kv_heads, head_dim, block_size, window, scale,
                       softcap, int(k_eq_v), rope_theta, rms_eps, rope_angles,
                       rope_scale, int(bool(page_ring)), kw, kvw)


_lib = None


def load_library():
    """Load the in-tree shared library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(LayerParams)
    lib.ga_kv_cache_write.restype = ctypes.c_int
    lib.ga_kv_cache_write.argtypes = [PP, P, P, P, P, P, P, P, P, P, i32, i32, i32, P, P, i64, P]
    lib.ga_decode_workspace_bytes.restype = sz
    lib.ga_decode_workspace_bytes.argtypes = [PP, i32, i32]
    lib.ga_attn_decode.restype = ctypes.c_int
    lib.ga_attn_decode.argtypes = [PP, P, P, P, i64, P, i32, P, i32, i32, P, P, sz, P]
    lib.ga_attn_decode_noalloc.restype = ctypes.c_int
    lib.ga_attn_decode_noalloc.argtypes = [PP, P, P, P, i64, P, i32, P, i32, i32, P, P]
    lib.ga_attn_prefill.restype = ctypes.c_int
    lib.ga_attn_prefill.argtypes = [PP, P, P, P, P, i64, P, i32, P, i32, i32, i32, P, P]
    lib.ga_check_metadata_host.restype = ctypes.c_int
    lib.ga_check_metadata_host.argtypes = [PP, P, P, P, i32, i32, i64, i32]
    lib.ga_status_string.restype = ctypes.c_char_p
    lib.ga_status_string.argtypes = [ctypes.c_int]
    lib.ga_last_error.restype = ctypes.c_char_p
    lib.ga_last_error.argtypes = []
    lib.ga_debug_take_error.restype = ctypes.c_int
    lib.ga_debug_take_error.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    _lib = lib
    return lib


def select_library(path: str) -> str:
    """Make the calls of this module go to the library at `path` (e.g. DEBUG_LIB_PATH);
    returns the previous path.  Loaded libraries stay loaded, so switching back is cheap."""
    global LIB_PATH, _lib
    prev = LIB_PATH
    LIB_PATH, _lib = path, None
    load_library()
    return prev


# bits of debug_take_error (GA_DEBUG_* of the header)
DEBUG_BLOCK_ID, DEBUG_LENGTH, DEBUG_BOUND, DEBUG_OWNER = 1, 2, 4, 8


def debug_take_error() -> int:
    """The in-kernel metadata-check bits set since the last call (debug library only; waits for
    the device and clears them).  The regular library raises GAError (GA_ERR_UNSUPPORTED)."""
    v = ctypes.c_uint32(0)
    _raise_on(load_library().ga_debug_take_error(ctypes.byref(v)))
    return int(v.value)


def _raise_on(status: int):
    if status != 0:
        raise GAError(status, load_library().ga_last_error().decode())


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, device: bool = True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _elem(p: LayerParams):
    return torch.bfloat16 if p.dtype == GA_BF16 else torch.float32


def kv_cache_write(p: LayerParams, q, k, v, q_norm_w, k_norm_w, v_norm_w, cu_seqlens,
                   context_lens, block_table, k_cache, v_cache, stream=None) -> None:
    """ga_kv_cache_write: norm + RoPE of q (in place) and k, norm of v, scatter into pages.
    k = v = None: q only (a layer reading another layer's cache; nothing is stored, and
    block_table / k_cache / v_cache may be None)."""
    lib = load_library()
    et = _elem(p)
    total = (k if k is not None else q).shape[0]
    st = lib.ga_kv_cache_write(
        ctypes.byref(p), _ptr(q, "q", et), _ptr(k, "k", et), _ptr(v, "v", et),
        _ptr(q_norm_w, "q_norm_w", torch.float32), _ptr(k_norm_w, "k_norm_w", torch.float32),
        _ptr(v_norm_w, "v_norm_w", torch.float32), _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        _ptr(context_lens, "context_lens", torch.int32),
        _ptr(block_table, "block_table", torch.int32),
        0 if block_table is None else block_table.shape[1],
        context_lens.shape[0], total, _ptr(k_cache, "k_cache", et),
        _ptr(v_cache, "v_cache", et), 0 if k_cache is None else k_cache.shape[0],
        _stream(stream))
    _raise_on(st)


def decode_workspace_bytes(p: LayerParams, batch: int, max_context_len: int) -> int:
    return int(load_library().ga_decode_workspace_bytes(ctypes.byref(p), batch, max_context_len))


def decode_workspace(p: LayerParams, batch: int, max_context_len: int, device="cuda"):
    """A device byte buffer large enough for attn_decode on this shape."""
    n = decode_workspace_bytes(p, batch, max_context_len)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def attn_decode(p: LayerParams, q, k_cache, v_cache, block_table, context_lens,
                max_context_len: int, out=None, workspace=None, stream=None):
    """ga_attn_decode: returns out [B, Hq, D]."""
    lib = load_library()
    et = _elem(p)
    B = context_lens.shape[0]
    if out is None:
        out = torch.empty((B, p.num_q_heads, p.head_dim), dtype=et, device=q.device)
    if workspace is None:
        workspace = decode_workspace(p, B, max_context_len, q.device)
    st = lib.ga_attn_decode(
        ctypes.byref(p), _ptr(q, "q", et), _ptr(k_cache, "k_cache", et),
        _ptr(v_cache, "v_cache", et), k_cache.shape[0],
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(context_lens, "context_lens", torch.int32), B, int(max_context_len),
        _ptr(out, "out", et), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _raise_on(st)
    return out


# GA_DECODE_NOALLOC_SCRATCH_BYTES of the header: the largest decode workspace that
# attn_decode_noalloc serves from the library's own device array
DECODE_NOALLOC_SCRATCH_BYTES = 48 << 20


def attn_decode_noalloc(p: LayerParams, q, k_cache, v_cache, block_table, context_lens,
                        max_context_len: int, out, stream=None):
    """ga_attn_decode_noalloc: decode into the caller's `out` [B, Hq, D] with the library's own
    scratch (no allocation by the library or by this binding).  Calls on one device share that
    scratch: calls that may overlap on one device race."""
    lib = load_library()
    et = _elem(p)
    st = lib.ga_attn_decode_noalloc(
        ctypes.byref(p), _ptr(q, "q", et), _ptr(k_cache, "k_cache", et),
        _ptr(v_cache, "v_cache", et), k_cache.shape[0],
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(context_lens, "context_lens", torch.int32), context_lens.shape[0],
        int(max_context_len), _ptr(out, "out", et), _stream(stream))
    _raise_on(st)
    return out


def attn_prefill(p: LayerParams, q, cu_seqlens_q, k_cache, v_cache, block_table, context_lens,
                 max_q_len: int, out=None, stream=None):
    """ga_attn_prefill: returns out [total_q, Hq, D]."""
    lib = load_library()
    et = _elem(p)
    if out is None:
        out = torch.empty_like(q)
    st = lib.ga_attn_prefill(
        ctypes.byref(p), _ptr(q, "q", et), _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _ptr(k_cache, "k_cache", et), _ptr(v_cache, "v_cache", et), k_cache.shape[0],
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(context_lens, "context_lens", torch.int32), context_lens.shape[0], q.shape[0],
        int(max_q_len), _ptr(out, "out", et), _stream(stream))
    _raise_on(st)
    return out


def check_metadata_host(p: LayerParams, cu_seqlens, context_lens, block_table, num_blocks: int,
                        require_nonempty: bool = True) -> None:
    """ga_check_metadata_host on host (CPU) int32 tensors; raises GAError when invalid."""
    lib = load_library()
    cu = None if cu_seqlens is None else cu_seqlens.detach().cpu().to(torch.int32).contiguous()
    cl = context_lens.detach().cpu().to(torch.int32).contiguous()
    bt = block_table.detach().cpu().to(torch.int32).contiguous()
    st = lib.ga_check_metadata_host(
        ctypes.byref(p), None if cu is None else ctypes.c_void_p(cu.data_ptr()),
        ctypes.c_void_p(cl.data_ptr()), ctypes.c_void_p(bt.data_ptr()), cl.shape[0],
        bt.shape[1], int(num_blocks), int(bool(require_nonempty)))
    _raise_on(st)


__all__ = ["LayerParams", "layer_params", "kv_cache_write", "attn_decode", "attn_prefill",
           "attn_decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES",
           "decode_workspace_bytes", "decode_workspace", "check_metadata_host", "GAError",
           "load_library", "LIB_PATH", "DEBUG_LIB_PATH", "select_library", "debug_take_error",
           "DEBUG_BLOCK_ID", "DEBUG_LENGTH", "DEBUG_BOUND", "DEBUG_OWNER", "GA_FP32", "GA_BF16",
           "BLOCK_SIZE"]
