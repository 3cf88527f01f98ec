"""GPU: sliding-window attention of a few query tokens per sequence (the draft
model's attention) against the oracle's windowed attention."""
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


def run_window(plc, w, dtype, window, partition=0, cache=None, bt=None, max_q_len=None):
    """Cache the prefix, append the sequences' new tokens, then attend."""
    if cache is None:
        cache, bt = device_cache(plc, w, dtype, upto="prefix")
        append_new(plc, cache, w, bt)
    ql = np.diff(w.cu_q_lens)
    if max_q_len is None:
        max_q_len = max(1, int(ql.max()))
    o, l = plc.attn_window_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens),
                                 max_q_len, int(w.context_lens.max()), window, partition, sm_scale())
    torch.cuda.synchronize()
    return host(o), host(l)


def oracle_window(w, dtype, window, rows=None):
    return cases.oracle_attention(w, cases.oracle_cache(w, dtype), sm_scale(), rows=rows,
                                  window=window)


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("window", [1, 16, 17, 100, 2048])
def test_window_sizes(plc, dtype, window):
    # contexts shorter than, equal to and far beyond the window; 4103 puts
    # row 0's first key (4103 - 8 - 2048 + 1 = 2048) on a partition edge
    ctx = [8, 50, 2048, 2100, 4103, 5000]
    w = synthetic.generate(cases.spec(ctx, [8] * len(ctx), hq=8, hkv=1, seed=500 + window))
    for P in [0, 16, 512]:
        o, l = run_window(plc, w, dtype, window, P)
        ro, rl = oracle_window(w, dtype, window)
        assert_close(o, l, ro, rl, what="window %d %s P=%d" % (window, dtype, P))


@pytest.mark.parametrize("n", [1, 2, 4, 16])
def test_window_draft_widths(plc, n):
    w = synthetic.generate(cases.spec([3000, 777, 40], [n] * 3, hq=8, hkv=1, seed=510 + n))
    for window in [64, 1000]:
        o, l = run_window(plc, w, "e4m3", window, 256)
        ro, rl = oracle_window(w, "e4m3", window)
        assert_close(o, l, ro, rl, what="window %d n=%d" % (window, n))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 4), (16, 1)])
def test_window_group_sizes_and_ragged(plc, hq, hkv):
    w = synthetic.generate(cases.spec([2500, 60, 1300, 16], [8, 0, 3, 16], hq=hq, hkv=hkv, seed=520))
    for dtype in ["fp16", "int8"]:
        o, l = run_window(plc, w, dtype, 512, 0, max_q_len=16)
        ro, rl = oracle_window(w, dtype, 512)
        assert_close(o, l, ro, rl, what="window G=%d %s" % (hq // hkv, dtype))


def test_window_covering_the_context_equals_verify(plc):
    # same kernel, partitions and chunk order: bit for bit (up to 8 drafts x 8
    # heads = 64 rows per KV head, where verification keeps the decode kernel)
    w = synthetic.generate(cases.spec([5000, 1234, 70], [4, 8, 2], hq=8, hkv=1, seed=530))
    cache, bt = device_cache(plc, w, "e4m3")
    ow, lw = run_window(plc, w, "e4m3", 10 ** 6, 1024, cache, bt)
    ov, lv = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), 8,
                                   5000, 1024, sm_scale())
    torch.cuda.synchronize()
    assert np.array_equal(ow, host(ov)) and np.array_equal(lw, host(lv))


def test_window_ignores_keys_before_it(plc):
    # a dominant key just outside every row's window and one just inside the
    # last row's: only the inside one may matter
    L, n, W = 3000, 8, 256
    w = synthetic.generate(cases.spec([L], [n], hq=8, hkv=1, seed=531, v_dist="uniform"))
    out_key, in_key = L - n - W, L - W
    for j in (out_key, in_key):
        w.k[j, 0, :] = np.sign(w.q[-1, 0].astype(np.float32)).astype(np.float16) * np.float16(2.0)
    w.k_scale_head[:] = synthetic.e4m3_head_scales(w.k)
    for dtype in ["fp16", "e4m3"]:
        o, l = run_window(plc, w, dtype, W, 512)
        ro, rl = oracle_window(w, dtype, W)
        assert_close(o, l, ro, rl, what="window edge %s" % dtype)


def test_window_long_context(plc):
    # the drafter's shape: 8-token blocks and a 2048-token window over long
    # contexts; every row is checked (the oracle reads only the window)
    w = synthetic.generate(cases.spec([262144, 131072, 70001], [8, 8, 8], hq=8, hkv=1, seed=532))
    o, l = run_window(plc, w, "e4m3", 2048)
    ro, rl = oracle_window(w, "e4m3", 2048)
    assert_close(o, l, ro, rl, what="window 2048 long context")
