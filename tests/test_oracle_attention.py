"""Pins for the oracle's attention, paging, append and merge (CPU only).

Each check ties the oracle to something other than itself: torch's float64
scaled_dot_product_attention on gathered-dense tensors, closed forms of
softmax attention, invariants that hold in exact arithmetic (split + merge,
block-table permutation, chunking, poison), and scipy's logsumexp.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import cases, refs

DTYPES = ["fp16", "e4m3", "int8"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [
    # (context_lens, q_lens, hq, hkv, d)
    ([5], [5], 2, 1, 8),
    ([37, 64, 17], [37, 3, 1], 4, 2, 8),
    ([50, 33], [1, 20], 8, 1, 128),
    ([19], [19], 8, 8, 16),
    ([300], [40], 8, 1, 128),
    # head dim 256 with a group of six query heads per KV head
    ([40, 17], [1, 1], 12, 2, 256),
    ([70], [6], 6, 1, 256),
])
def test_paged_oracle_matches_dense_sdpa(dtype, shape):
    ctx, ql, hq, hkv, d = shape
    w = synthetic.generate(cases.spec(ctx, ql, hq=hq, hkv=hkv, d=d, seed=11 + d))
    c = cases.oracle_cache(w, dtype)
    sm = 1.0 / math.sqrt(d)
    out, lse = cases.oracle_attention(w, c, sm)
    kd, vd = refs.dequant_cache(c)
    ro, rl = refs.sdpa_reference(w.q, hq, kd, vd, w.block_tables, w.cu_q_lens, w.context_lens,
                                 w.spec.block_size, sm)
    # the oracle rounds to fp32 at the end; the reference stays in float64
    assert np.max(np.abs(out - ro)) <= 1e-6 * max(1.0, np.max(np.abs(ro)))
    assert np.max(np.abs(lse - rl)) <= 1e-6 * max(1.0, np.max(np.abs(rl)))


def test_kv_append_places_codes_like_torch_encoding():
    w = synthetic.generate(cases.spec([21, 40], [21, 40], hq=2, hkv=2, d=16, seed=5))
    c = cases.oracle_cache(w, "e4m3")
    bs = w.spec.block_size
    owned = np.zeros(c.k.shape[:3], bool)
    for b in range(2):
        kb, vb = w.seq_kv(b)
        for j in range(kb.shape[0]):
            blk, slot = w.block_tables[b, j // bs], j % bs
            owned[blk, :, slot] = True
            for h in range(2):
                for src, dst, s in ((kb, c.k, w.k_scale_head), (vb, c.v, w.v_scale_head)):
                    x = src[j, h].astype(np.float32) / np.float32(s[h])
                    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                    assert np.array_equal(dst[blk, h, slot], ref)
    assert np.all(c.k[~owned] == synthetic.POISON_CODE_8BIT)
    assert np.all(c.v[~owned] == synthetic.POISON_CODE_8BIT)


def test_kv_append_fp16_and_int8_layout():
    w = synthetic.generate(cases.spec([18], [18], hq=1, hkv=1, d=8, seed=6))
    c16 = cases.oracle_cache(w, "fp16")
    c8 = cases.oracle_cache(w, "int8")
    for j in range(18):
        blk, slot = w.block_tables[0, j // 16], j % 16
        assert np.array_equal(c16.k[blk, 0, slot], w.k[j, 0].view(np.uint16))
        assert np.array_equal(c16.v[blk, 0, slot], w.v[j, 0].view(np.uint16))
        x = w.k[j, 0].astype(np.float32)
        sig = np.float32(np.abs(x).max()) / np.float32(127)
        assert c8.k_tok_scale[blk, 0, slot] == sig
        assert np.array_equal(c8.k[blk, 0, slot], np.clip(np.rint(x / sig), -127, 127).astype(np.int8))


def test_append_in_two_steps_equals_one_step():
    w = synthetic.generate(cases.spec([45, 30], [45, 30], hq=2, hkv=1, d=8, seed=8))
    one = cases.oracle_cache(w, "int8")
    two = oracle.HostCache(w.num_blocks, 1, 16, 8, "int8")
    cut = [13, 16]
    for lo_hi in (0, 1):
        ks, vs, cu, sp = [], [], [0], []
        for b in range(2):
            kb, vb = w.seq_kv(b)
            a, e = (0, cut[b]) if lo_hi == 0 else (cut[b], kb.shape[0])
            ks.append(kb[a:e]); vs.append(vb[a:e]); cu.append(cu[-1] + e - a); sp.append(a)
        two.append(np.concatenate(ks), np.concatenate(vs), w.block_tables, cu, sp)
    assert np.array_equal(one.k, two.k) and np.array_equal(one.v, two.v)
    assert np.array_equal(one.k_tok_scale, two.k_tok_scale, equal_nan=True)


# ------------------------------------------------------------ closed forms

def _single_seq(L, n, d=8, hq=2, hkv=1, seed=21, v_dist="normal"):
    return synthetic.generate(cases.spec([L], [n], hq=hq, hkv=hkv, d=d, seed=seed, v_dist=v_dist))


def test_all_keys_equal_gives_mean_of_values():
    w = _single_seq(40, 4)
    w.k[:] = w.k[0]
    c = cases.oracle_cache(w, "fp16")
    sm = 0.3
    out, lse = cases.oracle_attention(w, c, sm)
    for i in range(4):
        pos = 36 + i
        vis = w.v[:pos + 1, 0].astype(np.float64)
        for h in range(2):
            assert np.allclose(out[i, h], vis.mean(0), atol=1e-6)
            s = sm * float(np.dot(w.q[i, h].astype(np.float64), w.k[0, 0].astype(np.float64)))
            assert abs(lse[i, h] - (s + math.log(pos + 1))) < 1e-5


def test_single_visible_key():
    w = _single_seq(10, 10)
    c = cases.oracle_cache(w, "fp16")
    out, lse = cases.oracle_attention(w, c, 0.7)
    for h in range(2):
        assert np.array_equal(out[0, h], w.v[0, 0].astype(np.float32))
        s = 0.7 * float(np.dot(w.q[0, h].astype(np.float64), w.k[0, 0].astype(np.float64)))
        assert abs(lse[0, h] - s) < 1e-6


def test_zero_query_gives_uniform_weights():
    w = _single_seq(25, 1)
    w.q[:] = 0
    c = cases.oracle_cache(w, "fp16")
    out, lse = cases.oracle_attention(w, c, 1.0)
    assert np.allclose(out[0, 0], w.v[:25, 0].astype(np.float64).mean(0), atol=1e-6)
    assert abs(lse[0, 0] - math.log(25)) < 1e-6


def test_constant_values_and_one_hot_rows():
    w = _single_seq(70, 3, d=16)
    w.v[:] = np.float16(0.375)
    c = cases.oracle_cache(w, "fp16")
    out, _ = cases.oracle_attention(w, c, 0.25)
    assert np.allclose(out, 0.375, atol=1e-7)
    w.v[:] = 0
    for j in range(70):
        w.v[j, 0, j % 16] = 1
    c = cases.oracle_cache(w, "fp16")
    out, _ = cases.oracle_attention(w, c, 0.25)
    assert np.allclose(out.sum(-1), 1.0, atol=1e-6)


def test_dominant_key_picks_its_value():
    w = _single_seq(200, 1, d=16, v_dist="uniform")
    w.q[0, :] = np.float16(1.0)
    w.k[:] = 0
    w.k[123, 0] = np.float16(8.0)
    c = cases.oracle_cache(w, "fp16")
    out, _ = cases.oracle_attention(w, c, 1.0)     # score gap 128: weight of others ~ e^-128
    assert np.allclose(out[0, 0], w.v[123, 0].astype(np.float32), atol=1e-6)


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("part", [16, 48, 64, 1000])
def test_split_then_merge_equals_unsplit(dtype, part):
    w = synthetic.generate(cases.spec([333, 64, 1], [1, 1, 1], hq=4, hkv=2, d=16, seed=31))
    c = cases.oracle_cache(w, dtype)
    full_o, full_l = cases.oracle_attention(w, c, 0.25)
    nparts = math.ceil(333 / part)
    T, Hq, D = w.q.shape
    op = np.zeros((T * Hq, nparts, D), np.float32)
    lp = np.zeros((T * Hq, nparts), np.float32)
    for k in range(nparts):
        o, l = cases.oracle_attention(w, c, 0.25, key_begin=k * part, key_end=(k + 1) * part)
        op[:, k] = o.reshape(T * Hq, D)
        lp[:, k] = l.reshape(T * Hq)
    mo, ml = oracle.lse_merge(op, lp)
    assert np.max(np.abs(mo - full_o.reshape(T * Hq, D))) < 1e-6
    assert np.max(np.abs(ml - full_l.reshape(-1))) < 1e-5


def test_permuted_block_table_is_bitwise_identical():
    w = synthetic.generate(cases.spec([100, 47], [5, 47], hq=4, hkv=1, d=16, seed=41))
    c = cases.oracle_cache(w, "e4m3")
    o1, l1 = cases.oracle_attention(w, c)
    # move every block to a new physical slot
    perm = np.random.default_rng(0).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = synthetic.Workload(**{**w.__dict__, "block_tables": bt2})
    c2 = cases.oracle_cache(w2, "e4m3")
    o2, l2 = cases.oracle_attention(w2, c2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_chunked_prefill_equals_one_shot_and_decode_rows():
    w = synthetic.generate(cases.spec([96], [96], hq=2, hkv=1, d=16, seed=51))
    c = cases.oracle_cache(w, "e4m3")
    o_all, l_all = cases.oracle_attention(w, c)
    for chunk in range(4):                       # 4 chunks of 24 against the same cache
        a = 24 * chunk
        wc = synthetic.Workload(**{**w.__dict__, "q": w.q[a:a + 24],
                                   "cu_q_lens": np.array([0, 24], np.int32),
                                   "context_lens": np.array([a + 24], np.int32)})
        o, l = cases.oracle_attention(wc, c)
        assert np.array_equal(o, o_all[a:a + 24]) and np.array_equal(l, l_all[a:a + 24])
    i = 57                                       # prefill row i == decode with context i+1
    wd = synthetic.Workload(**{**w.__dict__, "q": w.q[i:i + 1],
                               "cu_q_lens": np.array([0, 1], np.int32),
                               "context_lens": np.array([i + 1], np.int32)})
    o, l = cases.oracle_attention(wd, c)
    assert np.array_equal(o[0], o_all[i]) and np.array_equal(l[0], l_all[i])


@pytest.mark.parametrize("dtype", DTYPES)
def test_poison_values_do_not_matter(dtype):
    w = synthetic.generate(cases.spec([29, 3], [2, 3], hq=2, hkv=1, d=8, seed=61))
    c = cases.oracle_cache(w, dtype)
    o1, l1 = cases.oracle_attention(w, c)
    owned = np.zeros(c.k.shape[:3], bool)
    for b in range(2):
        for j in range(int(w.context_lens[b])):
            owned[w.block_tables[b, j // 16], :, j % 16] = True
    fill = {"fp16": np.uint16(0x3C00), "e4m3": np.uint8(0x01), "int8": np.int8(-5)}[dtype]
    c.k[~owned] = fill
    c.v[~owned] = fill
    if dtype == "int8":
        c.k_tok_scale[~owned] = 3.0
        c.v_tok_scale[~owned] = 3.0
    o2, l2 = cases.oracle_attention(w, c)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------ merge

def test_merge_matches_scipy_logsumexp():
    rng = np.random.default_rng(71)
    o = rng.standard_normal((9, 7, 32)).astype(np.float32)
    l = (rng.standard_normal((9, 7)) * 20).astype(np.float32)
    l[2, 3] = -np.inf
    l[5, :6] = -np.inf
    mo, ml = oracle.lse_merge(o, l)
    ro, rl = refs.merge_reference(o, l)
    assert np.max(np.abs(mo - ro)) < 1e-6
    assert np.max(np.abs(ml - rl)) < 1e-5


def test_merge_closed_forms():
    o = np.array([[[1.0, 2.0], [3.0, 6.0]]], np.float32)
    mo, ml = oracle.lse_merge(o, np.array([[0.5, 0.5]], np.float32))
    assert np.allclose(mo, [[2.0, 4.0]]) and abs(ml[0] - (0.5 + math.log(2))) < 1e-6
    mo, ml = oracle.lse_merge(o, np.array([[-np.inf, 1.25]], np.float32))
    assert np.array_equal(mo, [[3.0, 6.0]]) and ml[0] == np.float32(1.25)
    mo, ml = oracle.lse_merge(o, np.array([[-np.inf, -np.inf]], np.float32))
    assert np.array_equal(mo, [[0.0, 0.0]]) and ml[0] == -np.inf


def test_empty_key_window_gives_zero_and_minus_inf():
    w = _single_seq(40, 2)
    c = cases.oracle_cache(w, "fp16")
    o, l = cases.oracle_attention(w, c, key_begin=39, key_end=40)   # row 0 sits at pos 38
    assert np.all(o[0] == 0) and np.all(l[0] == -np.inf)
    assert np.all(np.isfinite(l[1]))


# ---- sliding window (1Cat-vLLM README, "DFlash2 Long-Context Decay")

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,window", [
    (([40], [40], 2, 1, 8), 1),
    (([40], [40], 2, 1, 8), 7),
    (([37, 64, 17], [37, 3, 1], 4, 2, 8), 16),
    (([300, 90], [8, 8], 8, 1, 128), 33),
    (([300], [40], 8, 1, 128), 100),
])
def test_windowed_oracle_matches_dense_sdpa(dtype, shape, window):
    ctx, ql, hq, hkv, d = shape
    w = synthetic.generate(cases.spec(ctx, ql, hq=hq, hkv=hkv, d=d, seed=31 + window))
    c = cases.oracle_cache(w, dtype)
    sm = 1.0 / math.sqrt(d)
    out, lse = cases.oracle_attention(w, c, sm, window=window)
    kd, vd = refs.dequant_cache(c)
    ro, rl = refs.sdpa_reference(w.q, hq, kd, vd, w.block_tables, w.cu_q_lens, w.context_lens,
                                 w.spec.block_size, sm, window=window)
    assert np.max(np.abs(out - ro)) <= 1e-6 * max(1.0, np.max(np.abs(ro)))
    assert np.max(np.abs(lse - rl)) <= 1e-6 * max(1.0, np.max(np.abs(rl)))


def test_window_of_one_is_the_own_token():
    # each query sees only its own key: out = its value, lse = its score
    w = _single_seq(30, 6)
    c = cases.oracle_cache(w, "fp16")
    out, lse = cases.oracle_attention(w, c, 0.5, window=1)
    for i in range(6):
        pos = 24 + i
        for h in range(2):
            assert np.array_equal(out[i, h], w.v[pos, 0].astype(np.float32))
            s = 0.5 * float(np.dot(w.q[i, h].astype(np.float64), w.k[pos, 0].astype(np.float64)))
            assert abs(lse[i, h] - s) < 1e-6


def test_window_covering_the_context_changes_nothing():
    w = synthetic.generate(cases.spec([200, 77], [5, 77], hq=4, hkv=2, d=16, seed=33))
    c = cases.oracle_cache(w, "e4m3")
    o0, l0 = cases.oracle_attention(w, c, 0.25)
    o1, l1 = cases.oracle_attention(w, c, 0.25, window=200)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_equals_key_range_per_row():
    # for one query token, the window is the key range [pos - W + 1, pos]
    w = synthetic.generate(cases.spec([500], [1], hq=8, hkv=1, d=128, seed=34))
    c = cases.oracle_cache(w, "int8")
    o1, l1 = cases.oracle_attention(w, c, 0.088, window=64)
    o2, l2 = cases.oracle_attention(w, c, 0.088, key_begin=500 - 64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("dtype", DTYPES)
def test_row_subset_equals_full_evaluation(dtype):
    """The rows= path (used by the long-chunk parity tests) writes, at every
    listed row, exactly what a full evaluation writes there, and leaves every
    other row untouched (NaN).  The subset is unsorted, skips rows, crosses
    sequences and heads, and includes the first and last rows, so a mix-up
    of the listed row id with its list index fails."""
    w = synthetic.generate(cases.spec([37, 64, 17], [37, 3, 5], hq=4, hkv=2, d=16, seed=23))
    c = cases.oracle_cache(w, dtype)
    full_o, full_l = cases.oracle_attention(w, c)
    n = w.total_q * 4
    rows = np.array([n - 1, 0, 7, 150, 3, 101, 41, 42, 168, n - 2], np.int64)
    assert len(set(rows.tolist())) == len(rows) and rows.max() < n
    for nthreads in (1, 3):
        o, l = cases.oracle_attention(w, c, rows=rows, nthreads=nthreads)
        fo, fl = o.reshape(n, -1), l.reshape(n)
        assert np.array_equal(fo[rows], full_o.reshape(n, -1)[rows])
        assert np.array_equal(fl[rows], full_l.reshape(n)[rows])
        others = np.setdiff1d(np.arange(n), rows)
        assert np.all(np.isnan(fo[others])) and np.all(np.isnan(fl[others]))
