"""GPU: head dim 256 (Split-D) KV append, one-token decode, verification and
sliding-window attention against the oracle.

The group sizes include six query heads per KV head, the packing the pages
describe for their D256 attention."""
import numpy as np
import pytest
import torch

import synthetic
from tests import cases
from tests.gpu_util import append_new, assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu

SM = sm_scale(256)
LENGTHS = [1, 15, 16, 17, 33, 100, 2047, 2048, 2049, 5000]


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def spec(ctx, hq=12, hkv=2, seed=601, **kw):
    return cases.spec(ctx, [1] * len(ctx), hq=hq, hkv=hkv, d=256, seed=seed, **kw)


def run_decode(plc, w, dtype, partition=0, cache=None, bt=None):
    if cache is None:
        cache, bt = device_cache(plc, w, dtype)
    o, l = plc.attn_decode_paged(dev(w.q), cache, bt, dev(w.context_lens), int(w.context_lens.max()),
                                 partition, SM)
    torch.cuda.synchronize()
    return host(o), host(l)


def oracle_decode(w, dtype, rows=None):
    return cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM, rows=rows)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_d256_append_codes_match_oracle(plc, dtype):
    w = synthetic.generate(spec([37, 16, 100], seed=602))
    cache, _ = device_cache(plc, w, dtype)
    torch.cuda.synchronize()
    ref = cases.oracle_cache(w, dtype)
    assert np.array_equal(host(cache.k).view(np.uint8), ref.k.view(np.uint8))
    assert np.array_equal(host(cache.v).view(np.uint8), ref.v.view(np.uint8))
    if dtype == "int8":
        ks, vs = ref.scales()
        assert np.array_equal(host(cache.k_scale), ks, equal_nan=True)
        assert np.array_equal(host(cache.v_scale), vs, equal_nan=True)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("partition", [0, 16, 512, 2048])
def test_d256_decode_lengths(plc, dtype, partition):
    w = synthetic.generate(spec(LENGTHS, seed=603))
    o, l = run_decode(plc, w, dtype, partition)
    ro, rl = oracle_decode(w, dtype)
    assert_close(o, l, ro, rl, what="d256 decode %s P=%d" % (dtype, partition))


@pytest.mark.parametrize("hq,hkv", [(6, 1), (8, 1), (16, 1), (4, 4), (24, 4), (3, 1)])
@pytest.mark.parametrize("dtype", ["e4m3", "int8"])
def test_d256_group_sizes(plc, hq, hkv, dtype):
    w = synthetic.generate(spec([700, 33, 4096], hq=hq, hkv=hkv, seed=604))
    o, l = run_decode(plc, w, dtype, 512)
    ro, rl = oracle_decode(w, dtype)
    assert_close(o, l, ro, rl, what="d256 G=%d %s" % (hq // hkv, dtype))


def test_d256_partials_then_merge_equals_decode(plc):
    w = synthetic.generate(spec([3000, 900, 17], seed=605))
    cache, bt = device_cache(plc, w, "e4m3")
    o1, l1 = run_decode(plc, w, "e4m3", 512, cache, bt)
    op, lp = plc.attn_decode_partials(dev(w.q), cache, bt, dev(w.context_lens), 3000, 512, SM)
    o2, l2 = plc.lse_merge(op, lp)
    torch.cuda.synchronize()
    assert np.array_equal(host(o2).reshape(o1.shape), o1)
    assert np.array_equal(host(l2).reshape(l1.shape), l1)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_d256_decode_append_equals_append_then_decode(plc, dtype):
    lengths = [1, 17, 2048, 2049, 4096, 33]
    w = synthetic.generate(spec(lengths, seed=606))
    ca, bt = device_cache(plc, w, dtype, upto="prefix")
    kn, vn = w.new_kv()
    plc.kv_append_quant(ca, dev(kn), dev(vn), bt, dev(w.cu_q_lens), dev(w.start_pos))
    oa, la = plc.attn_decode_paged(dev(w.q), ca, bt, dev(w.context_lens), 4096, 2048, SM)
    cb, bt2 = device_cache(plc, w, dtype, upto="prefix")
    ob, lb = plc.attn_decode_append(dev(w.q), dev(kn), dev(vn), cb, bt2, dev(w.context_lens), 4096,
                                    2048, SM)
    torch.cuda.synchronize()
    assert np.array_equal(host(ca.k).view(np.uint8), host(cb.k).view(np.uint8))
    assert np.array_equal(host(ca.v).view(np.uint8), host(cb.v).view(np.uint8))
    if dtype == "int8":
        assert np.array_equal(host(ca.k_scale), host(cb.k_scale), equal_nan=True)
        assert np.array_equal(host(ca.v_scale), host(cb.v_scale), equal_nan=True)
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    ro, rl = oracle_decode(w, dtype)
    assert_close(host(ob), host(lb), ro, rl, what="d256 decode_append %s" % dtype)


def test_d256_overflowing_logits_and_poison(plc):
    w = synthetic.generate(spec([3000, 40, 5], seed=607, q_scale=900.0, v_dist="uniform"))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_decode(plc, w, dtype, 1024)
        ro, rl = oracle_decode(w, dtype)
        assert np.abs(rl).max() > 1000
        assert_close(o, l, ro, rl, what="d256 overflow %s" % dtype)


def test_d256_is_deterministic_and_placement_independent(plc):
    w = synthetic.generate(spec([5000, 1234], seed=608))
    cache, bt = device_cache(plc, w, "e4m3")
    o1, l1 = run_decode(plc, w, "e4m3", 1024, cache, bt)
    o2, l2 = run_decode(plc, w, "e4m3", 1024, cache, bt)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(6).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = synthetic.Workload(**{**w.__dict__, "block_tables": bt2})
    o3, l3 = run_decode(plc, w2, "e4m3", 1024)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_d256_full_decode_step(plc, dtype):
    # the bench workload (8 x 32,768 context, 12 q / 2 kv heads, head dim 256,
    # partitions of 2,048) in the bench's call: append each sequence's step
    # token and attend, one call; every row against the oracle
    w = synthetic.generate(synthetic.named_specs()["d256"])
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    kn, vn = w.new_kv()
    o, l = plc.attn_decode_append(dev(w.q), dev(kn), dev(vn), cache, bt, dev(w.context_lens), 32768,
                                  2048, SM)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w, dtype)
    assert_close(host(o), host(l), ro, rl, what="d256 step 8x32768 G=6 %s" % dtype)


def run_mq(plc, w, dtype, window=0, partition=0):
    """Cache the prefix, append the new tokens, then verify (window 0) or attend
    through the window."""
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    append_new(plc, cache, w, bt)
    mq = max(1, int(np.diff(w.cu_q_lens).max()))
    o, l = plc.attn_window_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), mq,
                                 int(w.context_lens.max()), window, partition, SM)
    torch.cuda.synchronize()
    return host(o), host(l)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("n", [2, 4, 7, 16])
def test_d256_verify(plc, dtype, n):
    # drafted tokens causal among themselves; rows = n * 6 per KV head, split
    # into groups of 16 that do not align with tokens
    ctx = [n, 17, 33, 2047, 2049, 5000]
    w = synthetic.generate(cases.spec(ctx, [n] * len(ctx), hq=12, hkv=2, d=256, seed=620 + n))
    for P in [0, 16, 512]:
        o, l = run_mq(plc, w, dtype, 0, P)
        ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM)
        assert_close(o, l, ro, rl, what="d256 verify n=%d %s P=%d" % (n, dtype, P))


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("window", [1, 17, 2048])
def test_d256_window(plc, dtype, window):
    ctx = [8, 50, 2048, 4103, 5000]
    w = synthetic.generate(cases.spec(ctx, [8] * len(ctx), hq=12, hkv=2, d=256, seed=640 + window))
    for P in [0, 512]:
        o, l = run_mq(plc, w, dtype, window, P)
        ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM, window=window)
        assert_close(o, l, ro, rl, what="d256 window %d %s P=%d" % (window, dtype, P))


def test_d256_verify_one_token_equals_decode(plc):
    w = synthetic.generate(spec([3000, 17, 2049], seed=650))
    cache, bt = device_cache(plc, w, "e4m3")
    od, ld = run_decode(plc, w, "e4m3", 512, cache, bt)
    ov, lv = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), 1,
                                   3000, 512, SM)
    torch.cuda.synchronize()
    assert np.array_equal(host(ov).reshape(od.shape), od) and np.array_equal(host(lv).reshape(ld.shape), ld)


def test_d256_verify_ragged_and_group_sizes(plc):
    for hq, hkv in [(6, 1), (16, 1), (3, 3), (24, 4)]:
        w = synthetic.generate(cases.spec([700, 3000, 64, 5], [5, 3, 16, 0], hq=hq, hkv=hkv, d=256,
                                          seed=660 + hq))
        for dtype in ["e4m3", "int8"]:
            o, l = run_mq(plc, w, dtype, 0, 512)
            ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM)
            assert_close(o, l, ro, rl, what="d256 verify G=%d %s" % (hq // hkv, dtype))


# ---------------------------------------------------------------- prefill

def run_prefill(plc, w, dtype):
    cache, bt = device_cache(plc, w, dtype, upto="prefix")
    append_new(plc, cache, w, bt)
    ql = np.diff(w.cu_q_lens)
    o, l = plc.attn_prefill_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens),
                                  max(1, int(ql.max())), int(w.context_lens.max()), SM)
    torch.cuda.synchronize()
    return host(o), host(l)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_d256_prefill_from_empty(plc, dtype):
    w = synthetic.generate(cases.spec([512], [512], hq=12, hkv=2, d=256, seed=670))
    o, l = run_prefill(plc, w, dtype)
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM)
    assert_close(o, l, ro, rl, what="d256 prefill 512 %s" % dtype)


@pytest.mark.parametrize("chunk", [1, 2, 11, 16, 17, 64, 65])
@pytest.mark.parametrize("prefix", [0, 1, 31, 32, 33, 2049])
def test_d256_prefill_short_chunks_after_prefix(plc, chunk, prefix):
    # wave tiles of 32 rows = 5 1/3 positions at six heads: tiles cut positions
    w = synthetic.generate(cases.spec([prefix + chunk], [chunk], hq=6, hkv=1, d=256, seed=671 + chunk))
    o, l = run_prefill(plc, w, "e4m3")
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "e4m3"), SM)
    assert_close(o, l, ro, rl, what="d256 chunk %d prefix %d" % (chunk, prefix))


@pytest.mark.parametrize("hq,hkv", [(6, 1), (12, 2), (16, 1), (4, 4), (3, 1)])
@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_d256_prefill_group_sizes_and_ragged_batch(plc, hq, hkv, dtype):
    w = synthetic.generate(cases.spec([300, 77, 1000, 5], [300, 20, 150, 0], hq=hq, hkv=hkv, d=256,
                                      seed=680))
    o, l = run_prefill(plc, w, dtype)
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM)
    assert_close(o, l, ro, rl, what="d256 prefill G=%d %s" % (hq // hkv, dtype))


def test_d256_prefill_last_row_matches_decode(plc):
    # the last row of a prefill agrees with a one-token decode over the same keys
    w = synthetic.generate(cases.spec([700], [700], hq=12, hkv=2, d=256, seed=690))
    o, l = run_prefill(plc, w, "e4m3")
    cache, bt = device_cache(plc, w, "e4m3")
    q_last = w.q[-1:]
    od, ld = plc.attn_decode_paged(dev(q_last), cache, bt, dev(w.context_lens), 700, 0, SM)
    torch.cuda.synchronize()
    assert np.abs(host(od)[0] - o[-1]).max() <= 2e-3     # both within the parity bar of the oracle
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "e4m3"), SM)
    assert_close(o, l, ro, rl, what="d256 prefill 700")


def test_d256_prefill_overflowing_logits(plc):
    w = synthetic.generate(cases.spec([1500], [300], hq=6, hkv=1, d=256, seed=691, q_scale=900.0,
                                      v_dist="uniform"))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_prefill(plc, w, dtype)
        ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, dtype), SM)
        assert_close(o, l, ro, rl, what="d256 prefill overflow %s" % dtype)


def test_d256_prefill_full_size_subsample(plc):
    # the bench workload: 8,192 new tokens after 122,880 cached, 12 q / 2 kv
    # heads, head dim 256, E4M3, on a seeded subsample of 96 query positions
    # (first and last 8, tile-edge pairs) x all 12 heads
    w = synthetic.generate(synthetic.named_specs()["d256_prefill"])
    o, l = run_prefill(plc, w, "e4m3")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    rows = synthetic.subsample_rows(8192, 12, 96, seed=0xD2, tile=32)
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "e4m3"), SM, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="d256 prefill 8192 after 122880")


@pytest.mark.parametrize("dtype", ["e4m3", "int8"])
def test_d256_verify_tiles_edges(plc, dtype):
    # 16 drafts x 6 heads = 96 rows per KV head: the 128-row tiles over key
    # partitions, then the merge.  The first sequence is given 7 keys on the
    # device for its 16 query tokens (rows before position 0 see no key:
    # out 0, lse -inf); one sequence has 6 query tokens, one none
    ctx = [30, 600, 4100, 33, 77]
    ql = [16, 16, 16, 6, 0]
    w = synthetic.generate(cases.spec(ctx, ql, hq=12, hkv=2, d=256, seed=680))
    cache, bt = device_cache(plc, w, dtype)
    dctx = w.context_lens.copy()
    dctx[0] = 7
    w2 = synthetic.Workload(**{**w.__dict__, "context_lens": dctx})
    ro, rl = cases.oracle_attention(w2, cases.oracle_cache(w2, dtype), SM)
    for P in [0, 32, 1024]:
        o, l = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(dctx), 16, 4100, P, SM)
        torch.cuda.synchronize()
        o, l = host(o), host(l)
        assert np.isneginf(l[:9]).all() and np.all(o[:9] == 0.0)
        assert_close(o, l, ro, rl, what="d256 verify tiles %s P=%d" % (dtype, P))


def test_d256_verify16_full_shape_sampled(plc):
    # the bench's head dim 256 verification at full size: 8 x 32768 context,
    # 12 q / 2 kv, 16 drafts (96 rows per KV head: tiles over key partitions),
    # automatic partitions; a seeded sample of rows against the oracle
    ctx = [32768] * 8
    w = synthetic.generate(cases.spec(ctx, [16] * 8, hq=12, hkv=2, d=256, seed=681))
    rows = np.sort(np.random.default_rng(681).choice(16 * 12 * 8, 40, replace=False))
    o, l = run_mq(plc, w, "e4m3", 0, 0)
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "e4m3"), SM, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="d256 verify 8x32768 n=16")
