"""Python access to the CPU oracle (``plc_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg are the only callers.  The GPU library never imports
this package, and this package never imports the GPU library.

All arrays are numpy; fp16 data travels as its raw uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "plc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KV_FP16, KV_E4M3, KV_INT8 = 0, 1, 2
_DTYPE_CODES = {"fp16": KV_FP16, "e4m3": KV_E4M3, "int8": KV_INT8}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no hand vectorization."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_f16_value.restype = f64
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = f64
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_int8_encode_row.restype = None
        L.orc_int8_encode_row.argtypes = [P, ctypes.c_int, P, P]
        L.orc_kv_append.restype = ctypes.c_int
        L.orc_kv_append.argtypes = [i32, P, P, P, i32, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.orc_attention.restype = ctypes.c_int
        L.orc_attention.argtypes = [P, i32, i32, P, P, P, P, i32, i32, i32, i32, P, i32, P, P, i32,
                                    f64, P, i64, i64, i64, i64, P, P, i32]
        L.orc_lse_merge.restype = None
        L.orc_lse_merge.argtypes = [P, P, i64, i32, i32, P, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else _c(a, np.uint16)


# ---------------------------------------------------------------- formats

def f16_value(bits: int) -> float:
    return lib().orc_f16_value(bits)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(x)


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    f = lib().orc_e4m3_encode
    flat = np.asarray(x, np.float32).reshape(-1)
    return np.array([f(float(v)) for v in flat], np.uint8).reshape(np.shape(x))


def int8_encode_row(x_f16: np.ndarray):
    x = _bits(x_f16)
    codes = np.zeros(x.shape[-1], np.int8)
    sigma = np.zeros(1, np.float32)
    lib().orc_int8_encode_row(_p(x), x.shape[-1], _p(codes), _p(sigma))
    return codes, float(sigma[0])


# ---------------------------------------------------------------- cache

class HostCache:
    """Oracle-side paged cache: codes [nb][Hkv][bs][D] (+ per-token INT8 scales)."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype: str,
                 k_scale_head=None, v_scale_head=None, poison=True):
        import synthetic
        self.dtype = dtype
        self.code = _DTYPE_CODES[dtype]
        self.num_blocks, self.num_kv_heads = int(num_blocks), int(num_kv_heads)
        self.block_size, self.head_dim = int(block_size), int(head_dim)
        k, v, ks, vs = synthetic.empty_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype)
        if dtype == "int8":
            k, v = k.view(np.int8), v.view(np.int8)
        self.k, self.v = k, v
        self.k_tok_scale, self.v_tok_scale = ks, vs
        self.k_scale_head = None if k_scale_head is None else _c(k_scale_head, np.float32)
        self.v_scale_head = None if v_scale_head is None else _c(v_scale_head, np.float32)

    def scales(self):
        if self.dtype == "e4m3":
            return self.k_scale_head, self.v_scale_head
        if self.dtype == "int8":
            return self.k_tok_scale, self.v_tok_scale
        return None, None

    def append(self, k_new, v_new, block_tables, cu_new_lens, start_pos):
        bt = _c(block_tables, np.int32)
        cu = _c(cu_new_lens, np.int32)
        sp = _c(start_pos, np.int32)
        kb, vb = _bits(k_new), _bits(v_new)
        rc = lib().orc_kv_append(
            self.code, _p(kb), _p(vb), _p(bt), bt.shape[1], _p(cu), _p(sp), len(sp),
            self.num_kv_heads, self.head_dim, self.block_size, self.num_blocks,
            _p(self.k_scale_head), _p(self.v_scale_head), _p(self.k), _p(self.v),
            _p(self.k_tok_scale), _p(self.v_tok_scale))
        if rc != 0:
            raise ValueError("orc_kv_append: block table entry outside the pool")


# ---------------------------------------------------------------- attention

def attention(q, num_q_heads, cache: HostCache, block_tables, cu_q_lens, context_lens,
              sm_scale, rows=None, key_begin=0, key_end=2**62, window=0, nthreads=0):
    """Attention for query rows (row id = token * Hq + head).  window > 0
    limits the query at position pos to keys pos - window + 1 .. pos.

    Returns (out [T][Hq][D] fp32, lse [T][Hq] fp32); rows not listed stay NaN.
    """
    qb = _bits(q)
    T = qb.shape[0]
    D = cache.head_dim
    out = np.full((T, num_q_heads, D), np.nan, np.float32)
    lse = np.full((T, num_q_heads), np.nan, np.float32)
    bt = _c(block_tables, np.int32)
    cu = _c(cu_q_lens, np.int32)
    cl = _c(context_lens, np.int32)
    if rows is None:
        rows_a, n = None, T * num_q_heads
    else:
        rows_a = _c(rows, np.int64)
        n = rows_a.shape[0]
    ks, vs = cache.scales()
    rc = lib().orc_attention(
        _p(qb), num_q_heads, cache.code, _p(cache.k), _p(cache.v), _p(ks), _p(vs),
        cache.num_blocks, cache.block_size, cache.num_kv_heads, D, _p(bt), bt.shape[1],
        _p(cu), _p(cl), len(cl), float(sm_scale), _p(rows_a), n, int(key_begin), int(key_end),
        int(window), _p(out), _p(lse), int(nthreads))
    if rc != 0:
        raise ValueError("orc_attention failed (%d)" % rc)
    return out, lse


def lse_merge(o_parts, lse_parts):
    """o_parts [rows][nparts][D], lse_parts [rows][nparts] -> (out [rows][D], lse [rows])."""
    o = _c(o_parts, np.float32)
    l = _c(lse_parts, np.float32)
    rows, nparts, D = o.shape
    out = np.zeros((rows, D), np.float32)
    lo = np.zeros(rows, np.float32)
    lib().orc_lse_merge(_p(o), _p(l), rows, nparts, D, _p(out), _p(lo))
    return out, lo
