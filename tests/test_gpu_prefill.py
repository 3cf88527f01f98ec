"""GPU: chunked causal prefill against the oracle."""
import numpy as np
import pytest
import torch

import synthetic
from tests import cases
from tests.gpu_util import append_new, assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def run_prefill(plc, w, dtype, cache=None, bt=None):
    """Cache the prefix, append the chunk with kv_append_quant, then prefill."""
    if cache is None:
        cache, bt = device_cache(plc, w, dtype, upto="prefix")
        append_new(plc, cache, w, bt)
    ql = np.diff(w.cu_q_lens)
    o, l = plc.attn_prefill_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens),
                                  int(ql.max()), int(w.context_lens.max()), sm_scale())
    torch.cuda.synchronize()
    return host(o), host(l)


def oracle_prefill(w, dtype):
    return cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale())


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_prefill_from_empty(plc, dtype):
    w = synthetic.generate(cases.spec([512], [512], hq=8, hkv=1, seed=301))
    o, l = run_prefill(plc, w, dtype)
    ro, rl = oracle_prefill(w, dtype)
    assert_close(o, l, ro, rl, what="prefill 512 %s" % dtype)


@pytest.mark.parametrize("chunk", [1, 2, 15, 16, 17, 63, 64, 65])
@pytest.mark.parametrize("prefix", [0, 1, 15, 16, 17, 2047, 2048, 2049])
def test_prefill_short_chunks_after_prefix(plc, chunk, prefix):
    w = synthetic.generate(cases.spec([prefix + chunk], [chunk], hq=8, hkv=1, seed=302 + chunk))
    o, l = run_prefill(plc, w, "e4m3")
    ro, rl = oracle_prefill(w, "e4m3")
    assert_close(o, l, ro, rl, what="chunk %d prefix %d" % (chunk, prefix))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (4, 2), (16, 4), (32, 4), (16, 1)])
@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_prefill_group_sizes_and_ragged_batch(plc, hq, hkv, dtype):
    w = synthetic.generate(cases.spec([300, 77, 1000], [300, 20, 150], hq=hq, hkv=hkv, seed=303))
    o, l = run_prefill(plc, w, dtype)
    ro, rl = oracle_prefill(w, dtype)
    assert_close(o, l, ro, rl, what="prefill G=%d %s" % (hq // hkv, dtype))


def test_prefill_chunked_equals_one_shot(plc):
    w = synthetic.generate(cases.spec([640], [640], hq=8, hkv=1, seed=304))
    cache, bt = device_cache(plc, w, "e4m3")
    o_all, l_all = run_prefill(plc, w, "e4m3", cache, bt)
    ro, rl = oracle_prefill(w, "e4m3")
    assert_close(o_all, l_all, ro, rl, what="one shot")
    for a in range(0, 640, 160):
        wc = synthetic.Workload(**{**w.__dict__, "q": w.q[a:a + 160],
                                   "cu_q_lens": np.array([0, 160], np.int32),
                                   "context_lens": np.array([a + 160], np.int32),
                                   "start_pos": np.array([a], np.int32)})
        o, l = run_prefill(plc, wc, "e4m3", cache, bt)
        assert_close(o, l, ro[a:a + 160], rl[a:a + 160], what="chunk at %d" % a)


def test_prefill_rows_match_decode(plc):
    w = synthetic.generate(cases.spec([300], [300], hq=8, hkv=1, seed=305))
    cache, bt = device_cache(plc, w, "e4m3")
    o, l = run_prefill(plc, w, "e4m3", cache, bt)
    i = 211                                        # prefill row i == decode at context i + 1
    od, ld = plc.attn_decode_paged(dev(w.q[i:i + 1]), cache, bt, dev(np.array([i + 1], np.int32)),
                                   i + 1, 0, sm_scale())
    assert np.abs(host(od)[0] - o[i]).max() <= 2e-3
    assert np.abs(host(ld)[0] - l[i]).max() <= 1e-4 * max(1.0, np.abs(l[i]).max())


def test_prefill_deterministic_and_placement_independent(plc):
    w = synthetic.generate(cases.spec([900, 130], [500, 130], hq=8, hkv=1, seed=306))
    cache, bt = device_cache(plc, w, "e4m3")
    o1, l1 = run_prefill(plc, w, "e4m3", cache, bt)
    o2, l2 = run_prefill(plc, w, "e4m3", cache, bt)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(2).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = synthetic.Workload(**{**w.__dict__, "block_tables": bt2})
    cache2, bt2d = device_cache(plc, w2, "e4m3")
    o3, l3 = run_prefill(plc, w2, "e4m3", cache2, bt2d)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_prefill_overflowing_logits_and_dominant_keys(plc):
    w = synthetic.generate(cases.spec([700], [200], hq=8, hkv=1, seed=307, q_scale=900.0,
                                      v_dist="uniform"))
    o, l = run_prefill(plc, w, "e4m3")
    ro, rl = oracle_prefill(w, "e4m3")
    assert np.abs(rl).max() > 1000
    assert_close(o, l, ro, rl, what="overflow")
    w = synthetic.generate(cases.spec([1000], [300], hq=8, hkv=1, seed=308, v_dist="uniform"))
    for j in [0, 63, 64, 699, 700, 701, 999]:      # tile edges, the chunk start, the last key
        w.k[j, 0, :] = np.sign(w.q[-1, 0].astype(np.float32)).astype(np.float16) * np.float16(2.0)
    w.k_scale_head[:] = synthetic.e4m3_head_scales(w.k)
    o, l = run_prefill(plc, w, "e4m3")
    ro, rl = oracle_prefill(w, "e4m3")
    assert_close(o, l, ro, rl, what="dominant keys")
