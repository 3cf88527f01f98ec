"""GPU: verification decode (a few causal query tokens per sequence, split-KV)
against the oracle, and against one-token decode where the two coincide."""
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


def run_verify(plc, w, dtype, partition=0, cache=None, bt=None, max_q_len=None):
    """Cache the prefix, append the sequences' new tokens, then verify."""
    if cache is None:
        cache, bt = device_cache(plc, w, dtype, upto="prefix")
        append_new(plc, cache, w, bt)
    ql = np.diff(w.cu_q_lens)
    if max_q_len is None:
        max_q_len = max(1, int(ql.max()))
    o, l = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens),
                                 max_q_len, int(w.context_lens.max()), partition, sm_scale())
    torch.cuda.synchronize()
    return host(o), host(l)


def oracle_verify(w, dtype, rows=None):
    return cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale(), rows=rows)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 7, 10, 16])
def test_verify_widths(plc, dtype, n):
    # contexts at and around page and partition edges; the new tokens straddle them
    ctx = [n, 17, 33, 100, 2047, 2049, 5000]
    w = synthetic.generate(cases.spec(ctx, [n] * len(ctx), hq=8, hkv=1, seed=400 + n))
    for P in [0, 16, 512]:
        o, l = run_verify(plc, w, dtype, P)
        ro, rl = oracle_verify(w, dtype)
        assert_close(o, l, ro, rl, what="verify n=%d %s P=%d" % (n, dtype, P))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 4), (16, 1), (32, 4)])
def test_verify_group_sizes(plc, hq, hkv):
    # G = 1..16: rows per (sequence, KV head) = n * G, in 16-row groups
    w = synthetic.generate(cases.spec([700, 3000, 64], [5, 3, 16], hq=hq, hkv=hkv, seed=410))
    for dtype in ["e4m3", "int8"]:
        o, l = run_verify(plc, w, dtype, 512)
        ro, rl = oracle_verify(w, dtype)
        assert_close(o, l, ro, rl, what="verify G=%d %s" % (hq // hkv, dtype))


def test_verify_ragged_widths_and_empty_sequences(plc):
    # sequences with no query token produce nothing and disturb nothing
    ctx = [4096, 50, 1, 777, 2048, 16]
    ql = [7, 0, 1, 4, 0, 16]
    w = synthetic.generate(cases.spec(ctx, ql, hq=8, hkv=1, seed=411))
    for dtype in ["fp16", "e4m3"]:
        o, l = run_verify(plc, w, dtype, 1024, max_q_len=16)
        ro, rl = oracle_verify(w, dtype)
        assert_close(o, l, ro, rl, what="verify ragged %s" % dtype)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_verify_one_token_equals_decode(plc, dtype):
    # n_b = 1 everywhere: the same kernel path as one-token decode, bit for bit
    lengths = [1, 31, 2048, 2049, 6000]
    w = synthetic.generate(cases.spec(lengths, [1] * len(lengths), hq=8, hkv=1, seed=412))
    cache, bt = device_cache(plc, w, dtype)
    ov, lv = run_verify(plc, w, dtype, 1024, cache, bt)
    od, ld = plc.attn_decode_paged(dev(w.q), cache, bt, dev(w.context_lens), 6000, 1024, sm_scale())
    torch.cuda.synchronize()
    assert np.array_equal(ov, host(od)) and np.array_equal(lv, host(ld))


def test_verify_causal_edge_keys(plc):
    # a dominant key at each new position: row j must see the ones at
    # positions <= L - n + j and none after
    L, n = 3000, 8
    w = synthetic.generate(cases.spec([L], [n], hq=8, hkv=1, seed=413, v_dist="uniform"))
    for j in range(n):
        w.k[L - n + j, 0, :] = np.sign(w.q[j, 0].astype(np.float32)).astype(np.float16) * np.float16(2.0)
    w.k_scale_head[:] = synthetic.e4m3_head_scales(w.k)
    for dtype in ["fp16", "e4m3"]:
        o, l = run_verify(plc, w, dtype, 1024)
        ro, rl = oracle_verify(w, dtype)
        assert_close(o, l, ro, rl, what="causal edge %s" % dtype)


@pytest.mark.parametrize("n", [4, 16])
def test_verify_overflowing_logits(plc, n):
    # 4 drafts x 8 heads: the decode kernel; 16: the tiles (every dtype)
    w = synthetic.generate(cases.spec([3000, 40], [n, n], hq=8, hkv=1, seed=414, q_scale=900.0,
                                      v_dist="uniform"))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_verify(plc, w, dtype, 1024)
        ro, rl = oracle_verify(w, dtype)
        assert np.abs(rl).max() > 1000
        assert_close(o, l, ro, rl, what="verify overflow %s n=%d" % (dtype, n))


@pytest.mark.parametrize("dtype,ql", [("e4m3", [4, 9]), ("fp16", [16, 11])])
def test_verify_is_deterministic_and_placement_independent(plc, dtype, ql):
    w = synthetic.generate(cases.spec([5000, 1234], ql, hq=8, hkv=1, seed=415))
    cache, bt = device_cache(plc, w, dtype)
    n = max(ql)
    o1, l1 = run_verify(plc, w, dtype, 1024, cache, bt)
    o2, l2 = run_verify(plc, w, dtype, 1024, cache, bt)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(2).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = synthetic.Workload(**{**w.__dict__, "block_tables": bt2})
    cache2, bt2d = device_cache(plc, w2, dtype)
    o3, l3 = run_verify(plc, w2, dtype, 1024, cache2, bt2d)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3), "n=%d" % n


def test_verify_full_decode_shape_sampled(plc):
    # the decode batch at full size (8 x 32768 context, 8 q / 1 kv heads,
    # partitions of 2048) with 4 drafted tokens per sequence; the oracle
    # checks a seeded sample of rows, spread over every sequence
    ctx = [32768] * 8
    w = synthetic.generate(cases.spec(ctx, [4] * 8, hq=8, hkv=1, seed=416))
    rows = np.sort(np.random.default_rng(416).choice(32 * 8, 40, replace=False))
    o, l = run_verify(plc, w, "e4m3", 2048)
    ro, rl = oracle_verify(w, "e4m3", rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="verify 8x32768 n=4")


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_verify_tiles_edges(plc, dtype):
    # 16 drafts x 8 heads = 128 rows per (sequence, KV head): the 128-row
    # tiles over key partitions, then the merge.  The first sequence is given
    # 10 keys on the device for its 16 query tokens (rows before position 0
    # see no key: out 0, lse -inf); one sequence has 9 query tokens (a part-
    # filled tile), one has none; partitions explicit (32, 48 -> 64 keys,
    # 1024) and automatic
    ctx = [40, 300, 64, 5000, 33, 777]
    ql = [16, 16, 16, 16, 9, 0]
    w = synthetic.generate(cases.spec(ctx, ql, hq=8, hkv=1, seed=417))
    cache, bt = device_cache(plc, w, dtype)
    dctx = w.context_lens.copy()
    dctx[0] = 10
    w2 = synthetic.Workload(**{**w.__dict__, "context_lens": dctx})
    ro, rl = oracle_verify(w2, dtype)
    for P in [0, 32, 48, 1024]:
        o, l = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(dctx), 16, 5000, P,
                                     sm_scale())
        torch.cuda.synchronize()
        o, l = host(o), host(l)
        assert np.isneginf(l[:6]).all() and np.all(o[:6] == 0.0)
        assert_close(o, l, ro, rl, what="verify tiles %s P=%d" % (dtype, P))


def test_verify_tiles_two_row_tiles_per_head(plc):
    # G = 16: 16 drafts x 16 heads = 256 rows per KV head, two tiles each,
    # two KV heads; mixed draft counts leave the second tile part-filled
    w = synthetic.generate(cases.spec([3000, 129, 2100], [16, 12, 5], hq=32, hkv=2, seed=418))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_verify(plc, w, dtype, 0, max_q_len=16)
        ro, rl = oracle_verify(w, dtype)
        assert_close(o, l, ro, rl, what="verify G=16 tiles %s" % dtype)


@pytest.mark.parametrize("dtype", ["e4m3", "fp16"])
def test_verify16_full_shape_sampled(plc, dtype):
    # the bench's 16-draft calls at full size: 8 x 32768 context, 8 q / 1 kv,
    # automatic partitions (128-row tiles over 32 partitions of 1,024 keys);
    # the oracle checks a seeded sample of rows spread over every sequence
    ctx = [32768] * 8
    w = synthetic.generate(cases.spec(ctx, [16] * 8, hq=8, hkv=1, seed=419))
    rows = np.sort(np.random.default_rng(419).choice(128 * 8, 48, replace=False))
    o, l = run_verify(plc, w, dtype, 0)
    ro, rl = oracle_verify(w, dtype, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="verify 8x32768 n=16 %s" % dtype)
