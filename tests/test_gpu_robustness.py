"""GPU: value ranges at the edge of fp16, workspace reuse across shapes, and
the one-GPU half of decode context parallelism (key shards merged by LSE)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import cases
from tests.gpu_util import LSE_RTOL, O_ATOL, assert_close, dev, device_cache, host, sm_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def big_values(w, seed, lo=40000.0, hi=65504.0):
    """Rescale every V row (token, head) of w in place so that its largest
    magnitude is drawn from [lo, hi], with some rows at exactly fp16's largest
    finite value: INT8 then stores sigma_v up to 65504 / 127."""
    g = np.random.default_rng(seed)
    v = w.v.astype(np.float32)
    m = np.abs(v).max(axis=-1, keepdims=True)
    target = g.uniform(lo, hi, size=m.shape).astype(np.float32)
    target[g.random(m.shape) < 0.25] = 65504.0
    x = np.clip(v / np.maximum(m, 1e-6) * target, -65504.0, 65504.0).astype(np.float16)
    assert np.all(np.isfinite(x))
    w.v[...] = x
    return float(np.abs(x.astype(np.float32)).max())


def assert_close_scaled(o, l, ro, rl, vmax, what):
    """The parity bar with V's range folded out: attention is linear in V, so
    max|do| <= 2e-3 * max|V| is the 2e-3 bound for V in [-1, 1]."""
    o = np.asarray(o, np.float64)
    ro = np.asarray(ro, np.float64)
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    err = float(np.abs(o - ro).max())
    assert err <= O_ATOL * vmax, "%s: max|do| %.4g > %.4g" % (what, err, O_ATOL * vmax)
    lerr = float((np.abs(np.asarray(l, np.float64) - rl) / np.maximum(1.0, np.abs(rl))).max())
    assert lerr <= LSE_RTOL, "%s: rel dlse %.3g" % (what, lerr)
    return err / vmax


@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 1), (128, 16, 4), (256, 12, 2)])
@pytest.mark.parametrize("partition", [0, 512])
def test_int8_decode_with_fp16_extreme_values(plc, d, hq, hkv, partition):
    w = synthetic.generate(cases.spec([3000, 2049, 17, 700], [1, 1, 1, 1], hq=hq, hkv=hkv, d=d,
                                      seed=801 + d))
    vmax = big_values(w, 17)
    cache, bt = device_cache(plc, w, "int8", upto="prefix")
    kn, vn = w.new_kv()
    s = w.spec
    # the one-launch step (append inside the decode), then the plain decode
    o, l = plc.attn_decode_append(dev(w.q), dev(kn), dev(vn), cache, bt, dev(w.context_lens),
                                  3000, partition, sm_scale(d))
    o2, l2 = plc.attn_decode_paged(dev(w.q), cache, bt, dev(w.context_lens), 3000, partition,
                                   sm_scale(d))
    torch.cuda.synchronize()
    ref = cases.oracle_cache(w, "int8")
    assert float(ref.v_tok_scale[np.isfinite(ref.v_tok_scale)].max()) > 500.0   # sigma_v near 65504/127
    ro, rl = cases.oracle_attention(w, ref, sm_scale(d))
    assert np.array_equal(host(o), host(o2))
    e = assert_close_scaled(host(o), host(l), ro, rl, vmax, "int8 decode d%d extreme V" % d)
    print("int8 decode d%d G=%d P=%d: max|do|/max|V| %.2e" % (d, hq // hkv, partition, e), flush=True)


@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 1), (256, 6, 1)])
def test_int8_prefill_with_fp16_extreme_values(plc, d, hq, hkv):
    w = synthetic.generate(cases.spec([700, 300], [200, 300], hq=hq, hkv=hkv, d=d, seed=811 + d))
    vmax = big_values(w, 18)
    cache, bt = device_cache(plc, w, "int8", upto="prefix")
    kn, vn = w.new_kv()
    plc.kv_append_quant(cache, dev(kn), dev(vn), bt, dev(w.cu_q_lens), dev(w.start_pos))
    o, l = plc.attn_prefill_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), 300,
                                  700, sm_scale(d))
    torch.cuda.synchronize()
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "int8"), sm_scale(d))
    e = assert_close_scaled(host(o), host(l), ro, rl, vmax, "int8 prefill d%d extreme V" % d)
    print("int8 prefill d%d: max|do|/max|V| %.2e" % (d, e), flush=True)


@pytest.mark.parametrize("d,hq,hkv,n", [(128, 8, 1, 4), (128, 8, 1, 16), (256, 12, 2, 16)])
def test_int8_verify_with_fp16_extreme_values(plc, d, hq, hkv, n):
    # 4 drafts x 8 heads keeps the decode kernel; 16 drafts run as prefill
    # tiles over key partitions (both head dims)
    w = synthetic.generate(cases.spec([3000, 2049, 40], [n, n, n], hq=hq, hkv=hkv, d=d, seed=821 + d + n))
    vmax = big_values(w, 19)
    cache, bt = device_cache(plc, w, "int8")
    o, l = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), n, 3000, 0,
                                 sm_scale(d))
    torch.cuda.synchronize()
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "int8"), sm_scale(d))
    e = assert_close_scaled(host(o), host(l), ro, rl, vmax, "int8 verify d%d n=%d extreme V" % (d, n))
    print("int8 verify d%d n=%d: max|do|/max|V| %.2e" % (d, n, e), flush=True)


def rising_scores(w, seed, bits_per_key=1.0 / 64):
    """Overwrite Q and K in place so that every query row's score rises by
    about bits_per_key (log2 units) per key position: each KV head gets a unit
    direction u, its query rows are 8u and key t is beta * t * u.  A row's
    running maximum then grows by about half a bit per 32-key subtile, so a
    lazily kept reference maximum lags the true one by whatever slack the
    kernel allows."""
    s = w.spec
    g = np.random.default_rng(seed)
    G = s.num_q_heads // s.num_kv_heads
    u = g.standard_normal((s.num_kv_heads, s.head_dim))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    amp = 8.0
    beta = bits_per_key / (amp * sm_scale(s.head_dim) * np.log2(np.e))
    for h in range(s.num_kv_heads):
        w.q[:, h * G:(h + 1) * G, :] = (amp * u[h]).astype(np.float16)
    for b in range(s.num_seqs):
        a, e = int(w.cu_kv[b]), int(w.cu_kv[b + 1])
        t = np.arange(e - a, dtype=np.float64)[:, None, None]
        w.k[a:e] = (beta * t * u[None]).astype(np.float16)


@pytest.mark.parametrize("call,d,hq,hkv,n,part", [
    ("verify", 128, 8, 1, 16, 0), ("verify", 128, 8, 1, 16, 1024), ("verify", 256, 12, 2, 16, 0),
    ("prefill", 256, 12, 2, 300, 0)])
def test_int8_tiles_rising_maximum_with_fp16_extreme_values(plc, call, d, hq, hkv, n, part):
    """The prefill tiles keep a lazy reference maximum.  INT8's P operand
    carries 64 sigma_v, so with sigma_v near 65504 / 127 the slack must shrink
    to about one bit or P overflows fp16; here every row's maximum keeps
    rising through the keys, which is where a lagging reference would let P
    grow.  16 drafts (and a 300-token chunk at head dim 256) run as tiles."""
    q_lens = [n, n, min(n, 40)]
    w = synthetic.generate(cases.spec([3000, 1500, 40], q_lens, hq=hq, hkv=hkv, d=d, seed=851 + d + n))
    rising_scores(w, 852 + d)
    vmax = big_values(w, 853)
    cache, bt = device_cache(plc, w, "int8")
    if call == "verify":
        o, l = plc.attn_verify_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), n, 3000,
                                     part, sm_scale(d))
    else:
        o, l = plc.attn_prefill_paged(dev(w.q), cache, bt, dev(w.cu_q_lens), dev(w.context_lens), n, 3000,
                                      sm_scale(d))
    torch.cuda.synchronize()
    ro, rl = cases.oracle_attention(w, cases.oracle_cache(w, "int8"), sm_scale(d))
    e = assert_close_scaled(host(o), host(l), ro, rl, vmax, "int8 %s d%d rising max" % (call, d))
    print("int8 %s d%d P=%d rising max: max|do|/max|V| %.2e" % (call, d, part, e), flush=True)


@pytest.mark.parametrize("dtype", ["e4m3", "int8"])
def test_workspace_reused_across_shapes(plc, dtype):
    """One workspace, never initialized (filled with NaN bytes here), serves
    decode and verification calls of different shapes and partitions in
    turn: every call writes the partials it reads."""
    wa = synthetic.generate(cases.spec([5000, 17, 2049], [1, 1, 1], hq=8, hkv=1, seed=821))
    wb = synthetic.generate(cases.spec([900, 4100, 33, 70, 16], [3, 4, 1, 2, 2], hq=16, hkv=4,
                                       seed=822))
    # 16 drafts x 8 heads: verification as prefill tiles over key partitions
    wc = synthetic.generate(cases.spec([3000, 700, 20], [16, 16, 9], hq=8, hkv=1, seed=823))
    ca, bta = device_cache(plc, wa, dtype)
    cb, btb = device_cache(plc, wb, dtype)
    cc, btc = device_cache(plc, wc, dtype)
    ws = torch.full((1 << 26,), 0xFF, dtype=torch.uint8, device="cuda")
    ref_a = cases.oracle_attention(wa, cases.oracle_cache(wa, dtype), sm_scale())
    ref_b = cases.oracle_attention(wb, cases.oracle_cache(wb, dtype), sm_scale())
    ref_c = cases.oracle_attention(wc, cases.oracle_cache(wc, dtype), sm_scale())
    for it, part in enumerate([512, 0, 48]):
        o, l = plc.attn_decode_paged(dev(wa.q), ca, bta, dev(wa.context_lens), 5000, part, sm_scale(),
                                     workspace=ws)
        ob, lb = plc.attn_verify_paged(dev(wb.q), cb, btb, dev(wb.cu_q_lens), dev(wb.context_lens), 4,
                                       4100, 16 * (it + 1), sm_scale(), workspace=ws)
        oc, lc = plc.attn_verify_paged(dev(wc.q), cc, btc, dev(wc.cu_q_lens), dev(wc.context_lens), 16,
                                       3000, part, sm_scale(), workspace=ws)
        torch.cuda.synchronize()
        assert_close(host(o), host(l), *ref_a, what="decode call %d" % it)
        assert_close(host(ob), host(lb), *ref_b, what="verify call %d" % it)
        assert_close(host(oc), host(lc), *ref_c, what="verify tiles call %d" % it)


def shard_tables(w, ranks, interleave):
    """Split each sequence's pages over `ranks` key shards: page j goes to
    shard j % ranks (interleaved) or to contiguous runs.  Returns per shard
    (block_tables, context_lens) describing that shard's keys as a sequence
    of its own pages in logical order; the last logical page (partial) is
    always the last page of its shard."""
    bs = w.spec.block_size
    out = []
    for r in range(ranks):
        rows, lens = [], []
        for b in range(w.spec.num_seqs):
            L = int(w.context_lens[b])
            npg = (L + bs - 1) // bs
            if interleave:
                mine = [j for j in range(npg) if j % ranks == r]
            else:
                per = (npg + ranks - 1) // ranks
                mine = list(range(r * per, min(npg, (r + 1) * per)))
            rows.append([int(w.block_tables[b, j]) for j in mine])
            lens.append(sum(min(bs, L - j * bs) for j in mine))
        width = max(1, max(len(x) for x in rows))
        bt = np.full((w.spec.num_seqs, width), -1, np.int32)
        for b, x in enumerate(rows):
            bt[b, :len(x)] = x
        out.append((bt, np.array(lens, np.int32)))
    return out


@pytest.mark.parametrize("interleave", [True, False])
@pytest.mark.parametrize("ranks", [2, 3])
def test_key_shards_merged_by_lse(plc, interleave, ranks):
    """Decode context parallelism on one GPU: each virtual rank computes the
    split-KV partials of its key shard, the partials of every rank are
    gathered along the part axis (what the exchange would deliver) and
    plc_lse_merge combines them; the result is attention over all keys."""
    w = synthetic.generate(cases.spec([5000, 2049, 33, 17], [1, 1, 1, 1], hq=8, hkv=1, seed=831))
    cache, _ = device_cache(plc, w, "e4m3")
    ref = cases.oracle_cache(w, "e4m3")
    q = dev(w.q)
    o_all, l_all = [], []
    for bt, lens in shard_tables(w, ranks, interleave):
        maxc = max(1, int(lens.max()))
        op, lp = plc.attn_decode_partials(q, cache, dev(bt), dev(lens), maxc, 512, sm_scale())
        o_all.append(op.clone())
        l_all.append(lp.clone())
        # each shard's own merged result is attention over its keys
        os_, ls_ = plc.lse_merge(op, lp)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(w.q, 8, ref, bt, w.cu_q_lens, lens, sm_scale())
        assert_close(host(os_), host(ls_), ro.reshape(-1, 128), rl.reshape(-1), what="shard")
    o, l = plc.lse_merge(torch.cat(o_all, dim=1).contiguous(), torch.cat(l_all, dim=1).contiguous())
    torch.cuda.synchronize()
    ro, rl = cases.oracle_attention(w, ref, sm_scale())
    assert_close(host(o), host(l), ro.reshape(-1, 128), rl.reshape(-1), what="merged shards")
