"""paged_long_context_amd: paged GQA attention over a quantized KV cache on MI355X.

A thin ctypes binding over ``libplc.so`` (gfx950 HIP kernels behind the C ABI
declared in ``include/plc.h``).  The functions here only marshal arguments:
they check tensor shapes, dtypes and devices, pass raw device pointers and
torch's current HIP stream, and raise ``PlcError`` on a non-zero status.
Every step of the computation runs in the library's kernels.  There is no
CPU path: importing this package fails if the library is not built.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "PlcError", "KVCache", "kv_append_quant", "attn_prefill_paged", "attn_decode_paged",
    "attn_decode_append", "attn_decode_partials", "lse_merge", "decode_workspace_size", "decode_partition_tokens",
    "debug_e4m3_to_f16", "LIB_PATH", "KV_FP16", "KV_E4M3", "KV_INT8",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libplc.so")
ABI_VERSION = 3

KV_FP16, KV_E4M3, KV_INT8 = 0, 1, 2
DTYPE_CODES = {"fp16": KV_FP16, "e4m3": KV_E4M3, "int8": KV_INT8}

PLC_OK, PLC_ERR_INVALID_ARG, PLC_ERR_UNSUPPORTED, PLC_ERR_WORKSPACE, PLC_ERR_HIP = 0, -1, -2, -3, -4


class PlcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("plc status %d: %s" % (status, message))
        self.status = status


class plc_kv_cache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


if not os.path.exists(LIB_PATH):
    raise ImportError("libplc.so is not built (%s); run __graft_entry__.build() first" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_P, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_KV = ctypes.POINTER(plc_kv_cache)
_lib.plc_abi_version.restype = ctypes.c_uint32
_lib.plc_abi_version.argtypes = []
_lib.plc_last_error.restype = ctypes.c_char_p
_lib.plc_last_error.argtypes = []
_lib.plc_kv_append_quant.restype = ctypes.c_int
_lib.plc_kv_append_quant.argtypes = [_KV, _P, _P, _P, _i32, _P, _P, _i32, _i32, _P]
_lib.plc_attn_prefill_paged.restype = ctypes.c_int
_lib.plc_attn_prefill_paged.argtypes = [_P, _i32, _KV, _P, _i32, _P, _P, _i32, _i32, _i32, _i32,
                                        _f32, _P, _P, _P]
_lib.plc_decode_workspace_size.restype = _sz
_lib.plc_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.plc_decode_partition_tokens.restype = _i32
_lib.plc_decode_partition_tokens.argtypes = [_i32, _i32, _i32, _i32]
_lib.plc_attn_decode_paged.restype = ctypes.c_int
_lib.plc_attn_decode_paged.argtypes = [_P, _i32, _KV, _P, _i32, _P, _i32, _i32, _i32, _f32, _P, _P,
                                       _P, _sz, _P]
_lib.plc_attn_decode_append.restype = ctypes.c_int
_lib.plc_attn_decode_append.argtypes = [_P, _P, _P, _i32, _KV, _P, _i32, _P, _i32, _i32, _i32, _f32,
                                        _P, _P, _P, _sz, _P]
_lib.plc_attn_decode_append_noalloc.restype = ctypes.c_int
_lib.plc_attn_decode_append_noalloc.argtypes = [_P, _P, _P, _i32, _KV, _P, _i32, _P, _i32, _i32, _i32,
                                                _f32, _P, _P, _P]
_lib.plc_attn_decode_partials.restype = ctypes.c_int
_lib.plc_attn_decode_partials.argtypes = [_P, _i32, _KV, _P, _i32, _P, _i32, _i32, _i32, _f32, _P,
                                          _sz, ctypes.POINTER(_i32), ctypes.POINTER(_sz), _P]
_lib.plc_verify_workspace_size.restype = _sz
_lib.plc_verify_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.plc_attn_verify_paged.restype = ctypes.c_int
_lib.plc_attn_verify_paged.argtypes = [_P, _i32, _KV, _P, _i32, _P, _P, _i32, _i32, _i32, _i32, _i32,
                                       _f32, _P, _P, _P, _sz, _P]
_lib.plc_window_workspace_size.restype = _sz
_lib.plc_window_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.plc_attn_window_paged.restype = ctypes.c_int
_lib.plc_attn_window_paged.argtypes = [_P, _i32, _KV, _P, _i32, _P, _P, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _f32, _P, _P, _P, _sz, _P]
_lib.plc_lse_merge.restype = ctypes.c_int
_lib.plc_lse_merge.argtypes = [_P, _P, _i32, _i32, _i32, _P, _P, _P]
_lib.plc_verify_max_query_tokens.restype = _i32
_lib.plc_verify_max_query_tokens.argtypes = []
_lib.plc_debug_e4m3_to_f16.restype = ctypes.c_int
_lib.plc_debug_e4m3_to_f16.argtypes = [_P, _P, _i32, _P]

if _lib.plc_abi_version() != ABI_VERSION:
    raise ImportError("libplc ABI %d, binding expects %d: rebuild the library"
                      % (_lib.plc_abi_version(), ABI_VERSION))


def lib():
    return _lib


def _check(status: int):
    if status != PLC_OK:
        raise PlcError(status, _lib.plc_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class KVCache:
    """A paged cache in device memory: [num_blocks][Hkv][block_size][D] per K and V.

    dtype "e4m3" takes fp32 per-KV-head scales (k_scale, v_scale of shape
    [Hkv]); "int8" owns fp32 per-token scales [num_blocks][Hkv][block_size]
    that kv_append_quant writes; "fp16" has none.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, dtype: str,
                 k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None):
        if dtype not in DTYPE_CODES:
            raise ValueError("dtype must be one of %s" % list(DTYPE_CODES))
        elem = torch.float16 if dtype == "fp16" else torch.uint8
        if dtype == "int8" and k.dtype == torch.int8:
            elem = torch.int8
        _need(k, "k", elem)
        _need(v, "v", elem, k.shape)
        if k.dim() != 4:
            raise ValueError("cache must be [num_blocks][Hkv][block_size][D]")
        nb, hkv, bs, d = k.shape
        if dtype == "e4m3":
            if k_scale is None or v_scale is None:
                raise ValueError("E4M3 cache needs per-head k_scale and v_scale")
            _need(k_scale, "k_scale", torch.float32, (hkv,))
            _need(v_scale, "v_scale", torch.float32, (hkv,))
        elif dtype == "int8":
            if k_scale is None or v_scale is None:
                raise ValueError("INT8 cache needs per-token k_scale and v_scale buffers")
            _need(k_scale, "k_scale", torch.float32, (nb, hkv, bs))
            _need(v_scale, "v_scale", torch.float32, (nb, hkv, bs))
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        self.dtype = dtype
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = nb, hkv, bs, d
        self._desc = plc_kv_cache(k.data_ptr(), v.data_ptr(),
                                  None if k_scale is None else k_scale.data_ptr(),
                                  None if v_scale is None else v_scale.data_ptr(),
                                  nb, bs, hkv, d, DTYPE_CODES[dtype])

    @classmethod
    def empty(cls, num_blocks, num_kv_heads, block_size, head_dim, dtype, device="cuda",
              k_scale=None, v_scale=None):
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        elem = torch.float16 if dtype == "fp16" else torch.uint8
        k = torch.empty(shape, dtype=elem, device=device)
        v = torch.empty(shape, dtype=elem, device=device)
        if dtype == "int8":
            k_scale = torch.empty(shape[:3], dtype=torch.float32, device=device)
            v_scale = torch.empty(shape[:3], dtype=torch.float32, device=device)
        return cls(k, v, dtype, k_scale, v_scale)

    def desc(self):
        return ctypes.byref(self._desc)


def kv_append_quant(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                    block_tables: torch.Tensor, cu_new_lens: torch.Tensor, start_pos: torch.Tensor,
                    stream=None):
    """Write new tokens' K/V (fp16 [T][Hkv][D]) into their pages, quantized."""
    T = k_new.shape[0]
    _need(k_new, "k_new", torch.float16, (T, cache.num_kv_heads, cache.head_dim))
    _need(v_new, "v_new", torch.float16, (T, cache.num_kv_heads, cache.head_dim))
    _need(block_tables, "block_tables", torch.int32)
    B = block_tables.shape[0]
    _need(cu_new_lens, "cu_new_lens", torch.int32, (B + 1,))
    _need(start_pos, "start_pos", torch.int32, (B,))
    _check(_lib.plc_kv_append_quant(cache.desc(), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
                                    block_tables.shape[1], _ptr(cu_new_lens), _ptr(start_pos), B, T,
                                    _stream(stream)))


def attn_prefill_paged(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                       cu_q_lens: torch.Tensor, context_lens: torch.Tensor, max_q_len: int,
                       max_context_len: int, sm_scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       stream=None):
    """Causal chunked prefill; q fp16 [T][Hq][D] -> (out fp32 [T][Hq][D], lse fp32 [T][Hq])."""
    T, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(block_tables, "block_tables", torch.int32)
    B = block_tables.shape[0]
    _need(cu_q_lens, "cu_q_lens", torch.int32, (B + 1,))
    _need(context_lens, "context_lens", torch.int32, (B,))
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (T, Hq, D))
    _need(lse, "lse", torch.float32, (T, Hq))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    _check(_lib.plc_attn_prefill_paged(_ptr(q), Hq, cache.desc(), _ptr(block_tables),
                                       block_tables.shape[1], _ptr(cu_q_lens), _ptr(context_lens),
                                       B, T, int(max_q_len), int(max_context_len), float(sm_scale),
                                       _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def decode_partition_tokens(num_seqs, num_kv_heads, max_context_len, partition_tokens=0) -> int:
    return int(_lib.plc_decode_partition_tokens(num_seqs, num_kv_heads, max_context_len,
                                                partition_tokens))


def decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens=0) -> int:
    return int(_lib.plc_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                              partition_tokens))


def _workspace(q, num_seqs, Hq, D, max_context_len, partition_tokens, workspace):
    need = decode_workspace_size(num_seqs, Hq, D, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    return workspace


def attn_decode_paged(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, max_context_len: int, partition_tokens: int = 0,
                      sm_scale: Optional[float] = None, out=None, lse=None, workspace=None,
                      stream=None):
    """Split-KV decode; q fp16 [B][Hq][D] -> (out fp32 [B][Hq][D], lse fp32 [B][Hq])."""
    B, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    if block_tables.shape[0] != B:
        raise ValueError("block_tables rows %d != num_seqs %d" % (block_tables.shape[0], B))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq))
    workspace = _workspace(q, B, Hq, D, max_context_len, partition_tokens, workspace)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    _check(_lib.plc_attn_decode_paged(_ptr(q), Hq, cache.desc(), _ptr(block_tables),
                                      block_tables.shape[1], _ptr(context_lens), B,
                                      int(max_context_len), int(partition_tokens), float(sm_scale),
                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return out, lse


def attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: KVCache,
                       block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                       partition_tokens: int = 0, sm_scale: Optional[float] = None, out=None,
                       lse=None, workspace=None, stream=None):
    """Append each sequence's step token (k_new / v_new fp16 [B][Hkv][D], at
    position context_lens - 1) and decode; the append runs inside the partition kernel."""
    B, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(k_new, "k_new", torch.float16, (B, cache.num_kv_heads, D))
    _need(v_new, "v_new", torch.float16, (B, cache.num_kv_heads, D))
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    if block_tables.shape[0] != B:
        raise ValueError("block_tables rows %d != num_seqs %d" % (block_tables.shape[0], B))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq))
    workspace = _workspace(q, B, Hq, D, max_context_len, partition_tokens, workspace)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    _check(_lib.plc_attn_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), Hq, cache.desc(),
                                       _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                       B, int(max_context_len), int(partition_tokens),
                                       float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20   # PLC_NOALLOC_SCRATCH_BYTES


def attn_decode_append_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                               cache: KVCache, block_tables: torch.Tensor, context_lens: torch.Tensor,
                               max_context_len: int, partition_tokens: int = 0,
                               sm_scale: Optional[float] = None, out=None, lse=None, stream=None):
    """attn_decode_append without a workspace: the library's per-device scratch
    stands in (calls on one device must not overlap in time)."""
    B, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(k_new, "k_new", torch.float16, (B, cache.num_kv_heads, D))
    _need(v_new, "v_new", torch.float16, (B, cache.num_kv_heads, D))
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    if block_tables.shape[0] != B:
        raise ValueError("block_tables rows %d != num_seqs %d" % (block_tables.shape[0], B))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    _check(_lib.plc_attn_decode_append_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), Hq, cache.desc(),
                                               _ptr(block_tables), block_tables.shape[1],
                                               _ptr(context_lens), B, int(max_context_len),
                                               int(partition_tokens), float(sm_scale), _ptr(out),
                                               _ptr(lse), _stream(stream)))
    return out, lse


def attn_decode_partials(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, max_context_len: int, partition_tokens: int = 0,
                         sm_scale: Optional[float] = None, workspace=None, stream=None):
    """Per-partition (o_parts [B*Hq][nparts][D], lse_parts [B*Hq][nparts]) views of the workspace."""
    B, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    workspace = _workspace(q, B, Hq, D, max_context_len, partition_tokens, workspace)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    nparts = _i32(0)
    off = _sz(0)
    _check(_lib.plc_attn_decode_partials(_ptr(q), Hq, cache.desc(), _ptr(block_tables),
                                         block_tables.shape[1], _ptr(context_lens), B,
                                         int(max_context_len), int(partition_tokens),
                                         float(sm_scale), _ptr(workspace), workspace.numel(),
                                         ctypes.byref(nparts), ctypes.byref(off), _stream(stream)))
    n = nparts.value
    rows = B * Hq
    o = workspace[: rows * n * D * 4].view(torch.float32).view(rows, n, D)
    l = workspace[off.value: off.value + rows * n * 4].view(torch.float32).view(rows, n)
    return o, l


VERIFY_MAX_Q_LEN = 16


def verify_max_query_tokens() -> int:
    """The library's grouped-verify maximum query length (capability query)."""
    return int(_lib.plc_verify_max_query_tokens())


def verify_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads, head_dim, max_q_len,
                          max_context_len, partition_tokens=0) -> int:
    return int(_lib.plc_verify_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                                              head_dim, max_q_len, max_context_len,
                                              partition_tokens))


def window_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads, head_dim, max_q_len,
                          max_context_len, window_tokens, partition_tokens=0) -> int:
    return int(_lib.plc_window_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                                              head_dim, max_q_len, max_context_len, window_tokens,
                                              partition_tokens))


def attn_verify_paged(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                      cu_q_lens: torch.Tensor, context_lens: torch.Tensor, max_q_len: int,
                      max_context_len: int, partition_tokens: int = 0,
                      sm_scale: Optional[float] = None, out=None, lse=None, workspace=None,
                      stream=None):
    """Verification decode: a few query tokens per sequence (the last n_b
    positions), causal among themselves, split-KV and merged in the same call
    (with many rows per KV head, as prefill tiles over key partitions: 8-bit
    caches at head dims 128 and 256, FP16 at 128); q fp16 [T][Hq][D] ->
    (out fp32 [T][Hq][D], lse fp32 [T][Hq])."""
    return attn_window_paged(q, cache, block_tables, cu_q_lens, context_lens, max_q_len,
                             max_context_len, 0, partition_tokens, sm_scale, out, lse, workspace,
                             stream)


def attn_window_paged(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                      cu_q_lens: torch.Tensor, context_lens: torch.Tensor, max_q_len: int,
                      max_context_len: int, window_tokens: int, partition_tokens: int = 0,
                      sm_scale: Optional[float] = None, out=None, lse=None, workspace=None,
                      stream=None):
    """As attn_verify_paged, with the row at position pos limited to keys
    pos - window_tokens + 1 .. pos (0: no window)."""
    T, Hq, D = q.shape
    _need(q, "q", torch.float16)
    _need(block_tables, "block_tables", torch.int32)
    B = block_tables.shape[0]
    _need(cu_q_lens, "cu_q_lens", torch.int32, (B + 1,))
    _need(context_lens, "context_lens", torch.int32, (B,))
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (T, Hq, D))
    _need(lse, "lse", torch.float32, (T, Hq))
    if workspace is None:
        need = window_workspace_size(B, T, Hq, cache.num_kv_heads, D, int(max_q_len),
                                     int(max_context_len), int(window_tokens), int(partition_tokens))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    _check(_lib.plc_attn_window_paged(_ptr(q), Hq, cache.desc(), _ptr(block_tables),
                                      block_tables.shape[1], _ptr(cu_q_lens), _ptr(context_lens), B, T,
                                      int(max_q_len), int(max_context_len), int(window_tokens),
                                      int(partition_tokens), float(sm_scale), _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out=None, lse=None, stream=None):
    """Merge partial states: o_parts fp32 [rows][nparts][D], lse_parts fp32 [rows][nparts]."""
    rows, nparts, D = o_parts.shape
    _need(o_parts, "o_parts", torch.float32)
    _need(lse_parts, "lse_parts", torch.float32, (rows, nparts))
    if out is None:
        out = torch.empty((rows, D), dtype=torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _need(out, "out", torch.float32, (rows, D))
    _need(lse, "lse", torch.float32, (rows,))
    _check(_lib.plc_lse_merge(_ptr(o_parts), _ptr(lse_parts), rows, nparts, D, _ptr(out), _ptr(lse),
                              _stream(stream)))
    return out, lse


def debug_e4m3_to_f16(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """The kernels' E4M3 -> fp16 conversion of uint8 codes (fp16 result)."""
    _need(codes, "codes", torch.uint8)
    out = torch.empty(codes.shape, dtype=torch.int16, device=codes.device)
    _check(_lib.plc_debug_e4m3_to_f16(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)))
    return out.view(torch.float16)
