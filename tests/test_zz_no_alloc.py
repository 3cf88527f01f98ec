"""GPU: the no-allocation decode step (plc_attn_decode_append_noalloc) against
the workspace form (plc_attn_decode_append) and the oracle, on two calls in
a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import synthetic
from tests import cases
from tests.gpu_util import assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def clone_cache(plc, c):
    ks = None if c.k_scale is None else c.k_scale.clone()
    vs = None if c.v_scale is None else c.v_scale.clone()
    return plc.KVCache(c.k.clone(), c.v.clone(), c.dtype, ks, vs)


def one_step(plc, w, dtype, partition):
    s = w.spec
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    twin = clone_cache(plc, cache)
    kn, vn = w.new_kv()
    q, k, v, ctx = dev(w.q), dev(kn), dev(vn), dev(w.context_lens)
    maxc = int(w.context_lens.max())
    o1, l1 = plc.attn_decode_append(q, k, v, cache, bt, ctx, maxc, partition, sm_scale(s.head_dim))
    o2, l2 = plc.attn_decode_append_noalloc(q, k, v, twin, bt, ctx, maxc, partition, sm_scale(s.head_dim))
    torch.cuda.synchronize()
    # same kernels, same inputs: identical results and identical caches
    assert np.array_equal(host(o1), host(o2)) and np.array_equal(host(l1), host(l2))
    assert np.array_equal(host(cache.k).view(np.uint8), host(twin.k).view(np.uint8))
    assert np.array_equal(host(cache.v).view(np.uint8), host(twin.v).view(np.uint8))
    if dtype == "int8":
        assert np.array_equal(host(cache.v_scale).view(np.uint32), host(twin.v_scale).view(np.uint32))
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale(s.head_dim))
    assert_close(host(o2), host(l2), ro, rl, what="no-alloc %s" % dtype)


@pytest.mark.parametrize("dtype", ["e4m3", "int8", "fp16"])
def test_no_alloc_step_twice_then_smaller(plc, dtype):
    big = synthetic.generate(cases.spec([32768] * 8, [1] * 8, hq=8, hkv=1, seed=901))
    small = synthetic.generate(cases.spec([4100, 17, 2049], [1, 1, 1], hq=16, hkv=4, seed=902))
    one_step(plc, big, dtype, 2048)           # the decode batch's shape, partitions of 2048
    one_step(plc, small, dtype, 0)            # then fewer, shorter sequences, automatic partition


def test_no_alloc_head_dim_256(plc):
    w = synthetic.generate(cases.spec([3000, 2049, 5], [1, 1, 1], hq=12, hkv=2, d=256, seed=903))
    one_step(plc, w, "e4m3", 512)
    one_step(plc, synthetic.generate(cases.spec([40], [1], hq=6, hkv=1, d=256, seed=904)), "e4m3", 0)
