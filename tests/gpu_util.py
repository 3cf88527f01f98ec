"""Helpers for the GPU parity tests: device caches built through the library's
own kv_append_quant, and the tolerance checks of the parity bar."""
import math

import numpy as np
import torch

import synthetic

O_ATOL = 2e-3          # max |o_gpu - o_ref| on fp32 outputs
LSE_RTOL = 1e-4        # |lse_gpu - lse_ref| <= 1e-4 * max(1, |lse_ref|)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def device_cache(plc, w: synthetic.Workload, dtype: str, upto: str = "all"):
    """Poisoned device cache holding w's tokens, written by plc.kv_append_quant.

    upto = "all": every token of every sequence; "prefix": only the tokens
    before each sequence's new chunk.
    """
    s = w.spec
    k, v, ks, vs = synthetic.empty_cache(w.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, dtype)
    kt, vt = dev(k), dev(v)
    if dtype == "fp16":
        kt, vt = kt.view(torch.float16), vt.view(torch.float16)
    if dtype == "e4m3":
        cache = plc.KVCache(kt, vt, dtype, dev(w.k_scale_head), dev(w.v_scale_head))
    elif dtype == "int8":
        cache = plc.KVCache(kt, vt, dtype, dev(ks), dev(vs))
    else:
        cache = plc.KVCache(kt, vt, dtype)
    bt = dev(w.block_tables)
    if upto == "all":
        kn, vn = w.k, w.v
        cu = w.cu_kv.astype(np.int32)
        sp = np.zeros(s.num_seqs, np.int32)
    else:
        kn, vn, cu, sp = w.prefix_kv()
    if kn.shape[0]:
        plc.kv_append_quant(cache, dev(kn), dev(vn), bt, dev(cu), dev(sp))
    return cache, bt


def append_new(plc, cache, w: synthetic.Workload, bt):
    kn, vn = w.new_kv()
    plc.kv_append_quant(cache, dev(kn), dev(vn), bt, dev(w.cu_q_lens), dev(w.start_pos))


def host(t):
    return t.detach().cpu().numpy()


def assert_close(o, lse, ro, rl, rows=None, what=""):
    """Parity bar: max |o - ro| <= 2e-3 and |lse - rl| <= 1e-4 * max(1, |rl|).

    o, ro: [..., D]; lse, rl: matching leading shape.  rows selects flattened
    rows (e.g. a subsample) when given."""
    D = np.shape(ro)[-1]
    o = np.asarray(o, np.float64).reshape(-1, D)
    ro = np.asarray(ro, np.float64).reshape(-1, D)
    lse = np.asarray(lse, np.float64).reshape(-1)
    rl = np.asarray(rl, np.float64).reshape(-1)
    if rows is not None:
        o, ro, lse, rl = o[rows], ro[rows], lse[rows], rl[rows]
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    err = float(np.abs(o - ro).max()) if o.size else 0.0
    # a row that sees no key has lse -inf on both sides; it must match exactly
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), "%s: empty rows differ" % what
    assert np.all(np.isfinite(lse[~empty])), "%s: non-finite lse" % what
    lerr = float((np.abs(lse[~empty] - rl[~empty]) / np.maximum(1.0, np.abs(rl[~empty]))).max()) \
        if np.any(~empty) else 0.0
    assert err <= O_ATOL, "%s: max |do| = %.3g" % (what, err)
    assert lerr <= LSE_RTOL, "%s: max rel dlse = %.3g" % (what, lerr)
    return err, lerr


def sm_scale(d=128):
    return 1.0 / math.sqrt(d)
