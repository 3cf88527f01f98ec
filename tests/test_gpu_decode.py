"""GPU: split-KV paged decode and the LSE merge against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import cases
from tests.gpu_util import assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def run_decode(plc, w, dtype, partition=0, cache=None, bt=None):
    if cache is None:
        cache, bt = device_cache(plc, w, dtype)
    o, l = plc.attn_decode_paged(dev(w.q), cache, bt, dev(w.context_lens),
                                 int(w.context_lens.max()), partition, sm_scale())
    torch.cuda.synchronize()
    return host(o), host(l)


def oracle_decode(w, dtype):
    return cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale())


LENGTHS = [1, 15, 16, 17, 31, 32, 33, 100, 2047, 2048, 2049, 5000]


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("partition", [0, 16, 48, 512, 2048])
def test_decode_lengths(plc, dtype, partition):
    w = synthetic.generate(cases.spec(LENGTHS, [1] * len(LENGTHS), hq=8, hkv=1, seed=201))
    o, l = run_decode(plc, w, dtype, partition)
    ro, rl = oracle_decode(w, dtype)
    assert_close(o, l, ro, rl, what="decode %s P=%d" % (dtype, partition))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (4, 2), (16, 4), (32, 4), (16, 1)])
@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_decode_group_sizes(plc, hq, hkv, dtype):
    w = synthetic.generate(cases.spec([700, 33, 4096], [1, 1, 1], hq=hq, hkv=hkv, seed=202))
    o, l = run_decode(plc, w, dtype, 512)
    ro, rl = oracle_decode(w, dtype)
    assert_close(o, l, ro, rl, what="decode G=%d %s" % (hq // hkv, dtype))


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_decode_single_partition_writes_output_directly(plc, dtype):
    # every context fits one 256-token partition (below the 512 the
    # two-workgroup split needs): the partition kernel writes out / lse
    # itself and no merge runs.  The last sequence is given length 0 on the
    # device: out 0, lse -inf.
    lens = [1, 17, 255, 256, 200]
    w = synthetic.generate(cases.spec(lens, [1] * len(lens), hq=8, hkv=1, seed=207))
    cache, bt = device_cache(plc, w, dtype)
    ctx = w.context_lens.copy()
    ctx[-1] = 0
    o, l = plc.attn_decode_paged(dev(w.q), cache, bt, dev(ctx), 256, 256, sm_scale())
    torch.cuda.synchronize()
    o, l = host(o), host(l)
    ro, rl = oracle_decode(w, dtype)
    assert_close(o[:-1], l[:-1], ro[:-1], rl[:-1], what="single-partition decode %s" % dtype)
    assert np.all(o[-1] == 0.0) and np.all(np.isneginf(l[-1]))


@pytest.mark.parametrize("lens,partition", [([4096] * 8, 1024), ([32768] * 8, 2048), ([5000, 17, 2049], 256),
                                            ([3000] * 40, 1024)])
def test_bench_kernel_partition_is_the_steps(plc, lens, partition):
    # bench.py times the step's partition kernel alone as a partials call at
    # step_kernel_partition(): that call plus the merge must reproduce the
    # merged decode bit for bit (same partitions, same arithmetic)
    import bench
    w = synthetic.generate(cases.spec(lens, [1] * len(lens), hq=8, hkv=1, seed=209))
    cache, bt = device_cache(plc, w, "e4m3")
    maxc = int(w.context_lens.max())
    o1, l1 = run_decode(plc, w, "e4m3", partition, cache, bt)
    kp = bench.step_kernel_partition(w.spec, maxc, partition)
    op, lp = plc.attn_decode_partials(dev(w.q), cache, bt, dev(w.context_lens), maxc, kp, sm_scale())
    o2, l2 = plc.lse_merge(op, lp)
    torch.cuda.synchronize()
    assert np.array_equal(host(o2).reshape(o1.shape), o1)
    assert np.array_equal(host(l2).reshape(l1.shape), l1)


def test_verify_single_partition_writes_output_directly(plc):
    from tests.test_gpu_verify import oracle_verify, run_verify
    ctx = [40, 256, 100, 3]
    ql = [3, 4, 0, 3]
    w = synthetic.generate(cases.spec(ctx, ql, hq=8, hkv=1, seed=208))
    o, l = run_verify(plc, w, "e4m3", 256, max_q_len=4)
    ro, rl = oracle_verify(w, "e4m3")
    assert_close(o, l, ro, rl, what="single-partition verify")


def test_decode_partials_then_merge_equals_decode(plc):
    w = synthetic.generate(cases.spec([3000, 900, 17], [1, 1, 1], hq=8, hkv=1, seed=203))
    cache, bt = device_cache(plc, w, "e4m3")
    o1, l1 = run_decode(plc, w, "e4m3", 512, cache, bt)
    op, lp = plc.attn_decode_partials(dev(w.q), cache, bt, dev(w.context_lens), 3000, 512, sm_scale())
    o2, l2 = plc.lse_merge(op, lp)
    torch.cuda.synchronize()
    # the fused step may stream each partition with two workgroups (halves)
    # and merges in its own fixed grouping: equal up to fp32 rounding of the
    # different groupings, and both within the parity bar of the oracle
    assert np.abs(host(o2).reshape(o1.shape) - o1).max() <= 1e-4
    assert np.abs(host(l2).reshape(l1.shape) - l1).max() <= 1e-5
    ro_all, rl_all = oracle_decode(w, "e4m3")
    assert_close(host(o2), host(l2), ro_all, rl_all, what="partials + lse_merge")
    # each partial against the oracle over its key window
    c = cases.oracle_cache(w, "e4m3")
    opn, lpn = host(op), host(lp)
    for k in range(opn.shape[1]):
        ro, rl = cases.oracle_attention(w, c, sm_scale(), key_begin=512 * k, key_end=512 * (k + 1))
        ro = ro.reshape(-1, 128)
        rl = rl.reshape(-1)
        live = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lpn[:, k]), live)
        assert np.all(opn[~live, k] == 0)
        if live.any():
            assert_close(opn[live, k], lpn[live, k], ro[live], rl[live], what="part %d" % k)


def test_lse_merge_against_oracle(plc):
    # head dims 128 and 256 take the one-wave-per-row kernel (parts in batches
    # of 32, even and odd parts per lane half), other widths the generic one
    rng = np.random.default_rng(204)
    for rows, nparts, d in [(5, 1, 128), (64, 16, 128), (7, 300, 128), (3, 5, 64), (2, 9, 256),
                            (4, 33, 128), (6, 31, 128), (3, 64, 256), (4, 2, 128), (5, 97, 256),
                            (3, 40, 200)]:
        o = rng.standard_normal((rows, nparts, d)).astype(np.float32)
        l = (rng.standard_normal((rows, nparts)) * 30).astype(np.float32)
        l[rng.random((rows, nparts)) < 0.2] = -np.inf
        l[0, :] = -np.inf                      # an all-empty row
        if nparts > 32:
            l[1, :32] = -np.inf                # a first batch with no visible part
            l[1, -1] = 2.0
            l[2, 32:64] = -np.inf              # an empty batch between visible ones
            l[2, 0] = 1.0
        if rows > 3:
            l[3, :-1] = -np.inf                # only the last part visible
            l[3, -1] = 5.0
        ro, rl = oracle.lse_merge(o, l)
        # aligned arrays, then o_parts and out 4 bytes off a 16-byte boundary
        # (views one float into larger buffers: the generic kernel takes them)
        ob = torch.empty(o.size + 1, dtype=torch.float32, device="cuda")
        ob[1:] = dev(o).reshape(-1)
        outb = torch.empty(rows * d + 1, dtype=torch.float32, device="cuda")
        for src, dst in [(dev(o), None), (ob[1:].view(rows, nparts, d), outb[1:].view(rows, d))]:
            go, gl = plc.lse_merge(src, dev(l), out=dst)
            go, gl = host(go), host(gl)
            empty = np.isneginf(rl)            # row 0, and any row the random -inf emptied
            assert empty[0] and np.array_equal(np.isneginf(gl), empty) and np.all(go[empty] == 0)
            assert np.abs(go[~empty] - ro[~empty]).max() <= 1e-5
            assert (np.abs(gl[~empty] - rl[~empty]) / np.maximum(1, np.abs(rl[~empty]))).max() <= 1e-6


def test_decode_is_deterministic_and_placement_independent(plc):
    w = synthetic.generate(cases.spec([5000, 1234], [1, 1], hq=8, hkv=1, seed=205))
    cache, bt = device_cache(plc, w, "e4m3")
    o1, l1 = run_decode(plc, w, "e4m3", 1024, cache, bt)
    o2, l2 = run_decode(plc, w, "e4m3", 1024, cache, bt)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(1).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = synthetic.Workload(**{**w.__dict__, "block_tables": bt2})
    o3, l3 = run_decode(plc, w2, "e4m3", 1024)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_decode_overflowing_logits(plc):
    # logits far beyond fp16 range: q scaled so |s| reaches ~1e4
    w = synthetic.generate(cases.spec([3000, 64], [1, 1], hq=8, hkv=1, seed=206, q_scale=900.0,
                                      v_dist="uniform"))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_decode(plc, w, dtype, 1024)
        ro, rl = oracle_decode(w, dtype)
        assert np.abs(rl).max() > 1000
        assert_close(o, l, ro, rl, what="overflow %s" % dtype)


@pytest.mark.parametrize("where", ["last", "block_edge", "partition_start", "first"])
def test_decode_dominant_key(plc, where):
    L = 4100
    w = synthetic.generate(cases.spec([L], [1], hq=8, hkv=1, seed=207, v_dist="uniform"))
    j = {"last": L - 1, "block_edge": 16 * 100 - 1, "partition_start": 2048, "first": 0}[where]
    w.k[j, 0, :] = np.sign(w.q[0, 0].astype(np.float32)).astype(np.float16) * np.float16(2.0)
    for dtype in ["fp16", "e4m3"]:
        w.k_scale_head[:] = synthetic.e4m3_head_scales(w.k)
        o, l = run_decode(plc, w, dtype, 1024)
        ro, rl = oracle_decode(w, dtype)
        assert_close(o, l, ro, rl, what="dominant %s %s" % (where, dtype))


def test_decode_poison_does_not_leak(plc):
    w = synthetic.generate(cases.spec([37, 5, 16], [1, 1, 1], hq=8, hkv=1, seed=208))
    for dtype in ["fp16", "e4m3", "int8"]:
        o, l = run_decode(plc, w, dtype, 0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
def test_decode_append_equals_append_then_decode(plc, dtype):
    # the step token lands at a page start, mid-page, a partition start (2049)
    # and a partition end (2048, 4096)
    lengths = [1, 17, 2048, 2049, 4096, 33]
    w = synthetic.generate(cases.spec(lengths, [1] * len(lengths), hq=8, hkv=1, seed=209))
    ca, bt = device_cache(plc, w, dtype, upto="prefix")
    kn, vn = w.new_kv()
    plc.kv_append_quant(ca, dev(kn), dev(vn), bt, dev(w.cu_q_lens), dev(w.start_pos))
    oa, la = plc.attn_decode_paged(dev(w.q), ca, bt, dev(w.context_lens), 4096, 2048, sm_scale())
    cb, bt2 = device_cache(plc, w, dtype, upto="prefix")
    ob, lb = plc.attn_decode_append(dev(w.q), dev(kn), dev(vn), cb, bt2, dev(w.context_lens), 4096,
                                    2048, sm_scale())
    torch.cuda.synchronize()
    assert np.array_equal(host(ca.k).view(np.uint8), host(cb.k).view(np.uint8))
    assert np.array_equal(host(ca.v).view(np.uint8), host(cb.v).view(np.uint8))
    if dtype == "int8":
        assert np.array_equal(host(ca.k_scale), host(cb.k_scale), equal_nan=True)
        assert np.array_equal(host(ca.v_scale), host(cb.v_scale), equal_nan=True)
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    ro, rl = oracle_decode(w, dtype)
    assert_close(host(ob), host(lb), ro, rl, what="decode_append %s" % dtype)


def test_decode_append_group_sizes_and_auto_partition(plc):
    w = synthetic.generate(cases.spec([5000, 64, 1, 777], [1] * 4, hq=32, hkv=4, seed=210))
    cb, bt = device_cache(plc, w, "e4m3", upto="prefix")
    kn, vn = w.new_kv()
    ob, lb = plc.attn_decode_append(dev(w.q), dev(kn), dev(vn), cb, bt, dev(w.context_lens), 5000, 0,
                                    sm_scale())
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w, "e4m3")
    assert_close(host(ob), host(lb), ro, rl, what="decode_append G=8 Hkv=4")
