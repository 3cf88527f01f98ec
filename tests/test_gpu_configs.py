"""GPU: the five workloads at full size against the oracle.

Decode workloads are checked on every output row; the chunked prefill (8,192
queries after a 122,880-token prefix) on a seeded subsample of query
positions that always includes the first and last positions and positions on
both sides of tile edges.  The launch configurations are the ones bench.py
times.
"""
import functools
import time

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import cases
from tests.gpu_util import append_new, assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu

SPECS = synthetic.named_specs()


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=None)
def workload(name):
    """Each full-size workload is drawn once per test session (the draws are
    seeded, so every test sees the same inputs)."""
    return synthetic.generate(SPECS[name])


def decode_config(plc, name, dtype, partition):
    t0 = time.time()
    w = workload(name)
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    append_new(plc, cache, w, bt)              # the step's own token
    o, l = plc.attn_decode_paged(dev(w.q), cache, bt, dev(w.context_lens),
                                 int(w.context_lens.max()), partition, sm_scale())
    torch.cuda.synchronize()
    o, l = host(o), host(l)
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale())
    err = assert_close(o, l, ro, rl, what="%s %s" % (name, dtype))
    log("%s %s: max|do| %.2e  rel dlse %.2e  (%.1fs)" % (name, dtype, err[0], err[1], time.time() - t0))


def test_c1_prefill_then_decode(plc):
    w = synthetic.c1_workload()
    k, v, _, _ = synthetic.empty_cache(w.num_blocks, 1, 16, 128, "e4m3")
    cache = plc.KVCache(dev(k), dev(v), "e4m3", dev(w.k_scale_head), dev(w.v_scale_head))
    bt = dev(w.block_tables)
    cu1 = np.array([0, 512], np.int32)
    plc.kv_append_quant(cache, dev(w.k[:512]), dev(w.v[:512]), bt, dev(cu1), dev(np.zeros(1, np.int32)))
    o, l = plc.attn_prefill_paged(dev(w.q[:512]), cache, bt, dev(cu1), dev(np.array([512], np.int32)),
                                  512, 512, sm_scale())
    plc.kv_append_quant(cache, dev(w.k[512:]), dev(w.v[512:]), bt, dev(np.array([0, 1], np.int32)),
                        dev(np.array([512], np.int32)))
    od, ld = plc.attn_decode_paged(dev(w.q[512:]), cache, bt, dev(np.array([513], np.int32)), 513, 0,
                                   sm_scale())
    torch.cuda.synchronize()
    ref = cases.oracle_cache(w, "e4m3")
    assert np.array_equal(host(cache.k), ref.k) and np.array_equal(host(cache.v), ref.v)
    ro, rl = oracle.attention(w.q[:512], 8, ref, w.block_tables, cu1, np.array([512], np.int32),
                              sm_scale())
    assert_close(host(o), host(l), ro, rl, what="c1 prefill")
    ro, rl = oracle.attention(w.q[512:], 8, ref, w.block_tables, np.array([0, 1], np.int32),
                              np.array([513], np.int32), sm_scale())
    assert_close(host(od), host(ld), ro, rl, what="c1 decode")


def test_c2_decode_batch8_32k(plc):
    decode_config(plc, "c2", "e4m3", 2048)


def test_c4_long_decode_mixed(plc):
    decode_config(plc, "c4", "e4m3", 0)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_c5_ragged_dtype_sweep(plc, dtype):
    decode_config(plc, "c5", dtype, 0)


def test_c3_chunked_prefill_subsample(plc):
    t0 = time.time()
    w = synthetic.generate(SPECS["c3"])
    cache, bt = device_cache(plc, w, "e4m3", upto="prefix")
    append_new(plc, cache, w, bt)
    o, l = plc.attn_prefill_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens),
                                  8192, 131072, sm_scale())
    torch.cuda.synchronize()
    o, l = host(o), host(l)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    # 512 positions x 8 heads: the first and last 8, both sides of every
    # 128-position tile edge, 16 edge pairs of the kernel's 32-position
    # workgroups, the rest uniform
    rows = synthetic.subsample_rows(8192, 8, 512, seed=0xC3, tile=32, every_edge=128)
    assert len(rows) == 4096
    ref = cases.oracle_cache(w, "e4m3")
    ro, rl = cases.oracle_attention(w, ref, sm_scale(), rows=rows)
    err = assert_close(o, l, ro, rl, rows=rows, what="c3")
    log("c3: %d rows, max|do| %.2e  rel dlse %.2e  (%.1fs)" % (len(rows), err[0], err[1], time.time() - t0))


# The call bench.py times for a decode step: plc_attn_decode_append (the
# step's token appended inside the partition kernel, then the merge) at full size
# in the partition bench.py resolves (2,048 for the 8 x 32K batch, automatic
# otherwise), for every KV dtype.
STEP_CASES = [("c2", 2048, dt) for dt in ("fp16", "e4m3", "int8")] + \
             [("c4", 0, dt) for dt in ("fp16", "e4m3", "int8")] + \
             [("c5", 0, dt) for dt in ("fp16", "e4m3", "int8")]


@pytest.mark.parametrize("name,partition,dtype", STEP_CASES)
def test_decode_step_full_size(plc, name, partition, dtype):
    t0 = time.time()
    w = workload(name)
    s = w.spec
    maxc = int(w.context_lens.max())
    P = plc.decode_partition_tokens(s.num_seqs, s.num_kv_heads, maxc, partition)
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    kn, vn = w.new_kv()
    q, ctx = dev(w.q), dev(w.context_lens)
    o, l = plc.attn_decode_append(q.view(s.num_seqs, s.num_q_heads, s.head_dim), dev(kn), dev(vn), cache, bt,
                                  ctx, maxc, P, sm_scale())
    # the same cache decoded again by the two-launch form's decode call
    o2, l2 = plc.attn_decode_paged(q.view(s.num_seqs, s.num_q_heads, s.head_dim), cache, bt, ctx, maxc, P,
                                   sm_scale())
    torch.cuda.synchronize()
    o, l, o2, l2 = host(o), host(l), host(o2), host(l2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), "fused step != decode of the appended cache"
    ref = cases.oracle_cache(w, dtype)
    # every slot of the cache, the appended tokens and the untouched poison included
    assert np.array_equal(host(cache.k).view(np.uint8), ref.k.view(np.uint8)), "%s %s K" % (name, dtype)
    assert np.array_equal(host(cache.v).view(np.uint8), ref.v.view(np.uint8)), "%s %s V" % (name, dtype)
    if dtype == "int8":
        for a, b in ((cache.k_scale, ref.k_tok_scale), (cache.v_scale, ref.v_tok_scale)):
            assert np.array_equal(host(a).view(np.uint32), b.view(np.uint32)), "%s int8 scales" % name
    ro, rl = cases.oracle_attention(w, ref, sm_scale())
    err = assert_close(o, l, ro, rl, what="%s %s step" % (name, dtype))
    log("%s %s step (P=%d): max|do| %.2e  rel dlse %.2e  (%.1fs)" % (name, dtype, P, err[0], err[1],
                                                                    time.time() - t0))
