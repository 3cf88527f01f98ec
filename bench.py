#!/usr/bin/env python3
"""Bench: paged GQA decode / prefill attention over an E4M3 KV cache on one MI355X.

Headline step (the workload the metric is quoted on): a decode step of a batch
of 8 sequences with 32,768-token contexts, 8 query heads over 1 KV head,
head_dim 128, E4M3 KV with fp32 per-head scales, 16-token pages scattered by a
seeded permutation, split-KV partitions of 2,048 tokens merged by log-sum-exp.
One step = one launch of the decode kernel, which appends the step's new K/V
token per sequence, runs every split-KV partition and merges the partials in
the last workgroup of each (sequence, KV head).  Eight copies of the cache (537 MB, twice
the 256 MB Infinity Cache) are rotated so every step reads its keys from HBM.
Steps are captured in a HIP graph and replayed, so host launch overhead is
not timed.

Also reported on the same JSON line: the 8,192-token chunked causal prefill
after a 122,880-token prefix (TFLOP/s of useful causal QK/PV work), the long
mixed decode (2 x 524,288 + 4 x 262,144) and the ragged 32-sequence decode in
FP16 / E4M3 / INT8, and the CPU oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu]

Further lines: verification of drafted tokens and draft-window attention at
the decode batch's shape, and head dim 256 (groups of six query heads) decode
in FP16 / E4M3 / INT8 and chunked prefill.

Profiling aids (no bench line): --prefill-only runs and times just the chunked
prefill; --verify-only just the verification and draft-window attention;
--d256-only just the head dim 256 workloads;
--copy-calibration runs a plain 256 MiB device copy five times, the
known-size kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
F16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, published
METRIC = "decode attn HBM GB/s; causal prefill attn TFLOP/s; % of MI355X roofline"
DECODE_KERNEL = "paged_decode_kernel"
PREFILL_KERNEL = "prefill_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_c2_traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="cache copies rotated in the C2 step")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="time only the headline step (no per-part graphs), e.g. under a profiler")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill workload (for profiling)")
    ap.add_argument("--d256-only", action="store_true",
                    help="only the head dim 256 workloads (decode, prefill)")
    ap.add_argument("--verify-only", action="store_true",
                    help="run only the verification-decode workload (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 256 MiB device copy 5 times and exit (counter calibration)")
    return ap.parse_args()


def kv_elem_bytes(dtype):
    return 2 if dtype == "fp16" else 1


def decode_bytes(w, dtype, with_outputs=True):
    """Algorithmic HBM bytes of one decode call: every visible K/V element once,
    INT8 per-token scales, E4M3 per-head scales, one block-table entry per page,
    the queries, and (with_outputs) the final outputs and LSEs."""
    s = w.spec
    L = w.context_lens.astype(np.int64)
    b = int(L.sum()) * s.num_kv_heads * s.head_dim * 2 * kv_elem_bytes(dtype)
    if dtype == "int8":
        b += int(L.sum()) * s.num_kv_heads * 2 * 4
    if dtype == "e4m3":
        b += s.num_kv_heads * 2 * 4
    b += int(((L + s.block_size - 1) // s.block_size).sum()) * 4
    b += s.num_seqs * s.num_q_heads * s.head_dim * 2
    if with_outputs:
        b += s.num_seqs * s.num_q_heads * (s.head_dim + 1) * 4
    return b


def append_bytes(w, dtype):
    """Algorithmic bytes of appending the step's new tokens."""
    s = w.spec
    T = int(w.cu_q_lens[-1])
    b = T * s.num_kv_heads * s.head_dim * 2 * 2                          # fp16 K, V in
    b += T * s.num_kv_heads * s.head_dim * 2 * kv_elem_bytes(dtype)      # codes out
    if dtype == "int8":
        b += T * s.num_kv_heads * 2 * 4
    b += (3 * s.num_seqs + 1) * 4                                         # cu, start, table
    return b


def verify_bytes(w, dtype):
    """Algorithmic HBM bytes of one verification call: decode_bytes's keys,
    values, scales and table entries, every query token's row read, its
    output row and LSE written, and cu_q_lens."""
    s = w.spec
    T = int(w.cu_q_lens[-1])
    b = decode_bytes(w, dtype, with_outputs=False) - s.num_seqs * s.num_q_heads * s.head_dim * 2
    b += T * s.num_q_heads * s.head_dim * 2 + T * s.num_q_heads * (s.head_dim + 1) * 4
    return b + (s.num_seqs + 1) * 4


def bench_verify(plc, synthetic, specs, K, widths=(4, 16)):
    """Verification decode at the decode batch's shape (8 x 32768, E4M3,
    partitions of 2048), 8 rotated cache copies, for a few draft widths."""
    import dataclasses
    res = {}
    for n in widths:
        sp = dataclasses.replace(specs["verify"], q_lens=[n] * len(specs["verify"].context_lens))
        log("generating verify n=%d" % n)
        w = synthetic.generate(sp)
        s = w.spec
        caches, bt = build_cache(plc, w, "e4m3", 8)
        kn, vn = w.new_kv()
        kn, vn = to_dev(kn), to_dev(vn)
        cu, start, ctx = to_dev(w.cu_q_lens), to_dev(w.start_pos), to_dev(w.context_lens)
        for c in caches:
            plc.kv_append_quant(c, kn, vn, bt, cu, start)
        q = to_dev(w.q)
        T = int(w.cu_q_lens[-1])
        maxc = int(w.context_lens.max())
        P = s.partition_tokens
        ws = torch.zeros(plc.verify_workspace_size(s.num_seqs, T, s.num_q_heads, s.num_kv_heads,
                                                   s.head_dim, n, maxc, P),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, s.num_q_heads), dtype=torch.float32, device="cuda")
        sm = 1.0 / math.sqrt(s.head_dim)

        def f(i):
            plc.attn_verify_paged(q, caches[i % len(caches)], bt, cu, ctx, n, maxc, P, sm, out=out,
                                  lse=lse, workspace=ws)
        for i in range(3):
            f(i)
        _, ev = graph_time(f, max(5, min(50, K // 4)), reps=2)
        vb = verify_bytes(w, "e4m3")
        L = w.context_lens.astype(np.int64)
        visible = int(sum(n * (int(l) - n) + n * (n + 1) // 2 for l in L))
        fl = 4 * s.head_dim * s.num_q_heads * visible
        res["n%d" % n] = {
            "drafted_tokens": n, "gbs": round(vb / ev / 1e9, 1), "unit": "GB/s",
            "us_per_call": round(ev * 1e6, 2), "bytes": vb,
            "frac_of_hbm_peak": round(vb / ev / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / ev / 1e12, 2),
        }
        log("verify n=%d: %.2f us = %.0f GB/s (%.1f%% of HBM), %.1f TFLOP/s"
            % (n, ev * 1e6, vb / ev / 1e9, 100 * vb / ev / 1e9 / HBM_PEAK_GBS, fl / ev / 1e12))
        del caches, ws, out, lse, q
        torch.cuda.empty_cache()
    res["workload"] = specs["verify"].description + "; widths as listed"
    return res


def bench_window(plc, synthetic, specs, K, window=2048):
    """Draft attention (8-token blocks, sliding window) at the long-context
    batch's contexts and at 32K, and the same calls without a window."""
    import dataclasses
    res = {}
    base = specs["draft"]
    for tag, ctx in (("ctx32k", [32768] * len(base.context_lens)), ("long", base.context_lens)):
        sp = dataclasses.replace(base, context_lens=list(ctx))
        log("generating draft %s" % tag)
        w = synthetic.generate(sp)
        s = w.spec
        caches, bt = build_cache(plc, w, "e4m3", 8)
        kn, vn = w.new_kv()
        kn, vn = to_dev(kn), to_dev(vn)
        cu, start, ctxd = to_dev(w.cu_q_lens), to_dev(w.start_pos), to_dev(w.context_lens)
        for c in caches:
            plc.kv_append_quant(c, kn, vn, bt, cu, start)
        q = to_dev(w.q)
        T = int(w.cu_q_lens[-1])
        n = max(s.q_lens)
        maxc = int(w.context_lens.max())
        out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, s.num_q_heads), dtype=torch.float32, device="cuda")
        sm = 1.0 / math.sqrt(s.head_dim)
        entry = {}
        for wt in (window, 0):
            ws = torch.zeros(plc.window_workspace_size(s.num_seqs, T, s.num_q_heads, s.num_kv_heads,
                                                       s.head_dim, n, maxc, wt, 0),
                             dtype=torch.uint8, device="cuda")

            def f(i):
                plc.attn_window_paged(q, caches[i % len(caches)], bt, cu, ctxd, n, maxc, wt, 0, sm,
                                      out=out, lse=lse, workspace=ws)
            for i in range(3):
                f(i)
            _, ev = graph_time(f, max(5, min(50, K // 4)), reps=2)
            entry["window_%d_us" % wt if wt else "no_window_us"] = round(ev * 1e6, 2)
            log("draft %s window %d: %.2f us" % (tag, wt, ev * 1e6))
            del ws
        res[tag] = dict(entry, context_lens=sorted(set(int(x) for x in ctx)), tokens_per_block=n)
        del caches, out, lse, q
        torch.cuda.empty_cache()
    res["workload"] = base.description + "; the same blocks at 32,768-token contexts; eight " \
        "rotated cache copies (the windows' 3 MB per call stay cache-resident, so these are " \
        "latency figures, not HBM-bound ones)"
    return res


def bench_d256(plc, synthetic, specs, K):
    """Head dim 256 decode step (append + partitions + merge) at the decode
    batch's shape with groups of six query heads, for each KV dtype."""
    log("generating d256 (8 x 32768, 12 q / 2 kv, head dim 256)")
    w = synthetic.generate(specs["d256"])
    res = {"workload": specs["d256"].description}
    for dt in ["fp16", "e4m3", "int8"]:
        # rotated copies: 268 MB (8-bit) / 537 MB (fp16) each, over twice the Infinity Cache
        c = DecodeCase(plc, w, dt, w.spec.partition_tokens, copies=2 if dt == "fp16" else 4)
        for i in range(3):
            c.step(i)
        n = max(5, min(50, K // 4))
        sw, se = graph_time(c.step, n, reps=2)
        _, ke = graph_time(c.partials, n, reps=2)
        sb = decode_bytes(w, dt) + append_bytes(w, dt)
        kb = decode_bytes(w, dt, with_outputs=False)
        res[dt] = {"gbs": round(sb / sw / 1e9, 1), "unit": "GB/s", "us_per_step": round(sw * 1e6, 2),
                   "step_bytes": sb, "frac_of_hbm_peak": round(sb / sw / 1e9 / HBM_PEAK_GBS, 4),
                   "partitions_kernel_us": round(ke * 1e6, 2),
                   "partitions_kernel_gbs": round(kb / ke / 1e9, 1)}
        log("d256 %s: step %.1f us = %.0f GB/s; partitions %.1f us" % (dt, sw * 1e6, sb / sw / 1e9, ke * 1e6))
        del c
        torch.cuda.empty_cache()
    return res


def bench_d256_prefill(plc, synthetic, specs, K):
    """Head dim 256 chunked prefill: 8,192 new tokens after 122,880 cached, groups of six."""
    log("generating d256_prefill (8192 new after 122880 cached, 12 q / 2 kv, head dim 256)")
    w = synthetic.generate(specs["d256_prefill"])
    s = w.spec
    caches, bt = build_cache(plc, w, "e4m3", 1)
    cache = caches[0]
    q = to_dev(w.q)
    cu, ctx = to_dev(w.cu_q_lens), to_dev(w.context_lens)
    kn, vn = w.new_kv()
    plc.kv_append_quant(cache, to_dev(kn), to_dev(vn), bt, cu, to_dev(w.start_pos))
    T = int(w.cu_q_lens[-1])
    out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, s.num_q_heads), dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(s.head_dim)

    def pre(i):
        plc.attn_prefill_paged(q, cache, bt, cu, ctx, T, int(w.context_lens.max()), sm, out=out, lse=lse)
    pre(0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all()), "d256 prefill output"
    pw, pe = graph_time(pre, 3, reps=2)
    fl = prefill_flops(w)
    tf = fl / pe / 1e12
    log("d256 prefill %.1f us, %.1f TFLOP/s" % (pe * 1e6, tf))
    del caches, cache, q, out, lse
    torch.cuda.empty_cache()
    return {"workload": s.description, "tflops": round(tf, 2), "unit": "TFLOP/s",
            "us_per_call": round(pe * 1e6, 1), "useful_flops": fl,
            "frac_of_f16_mfma_peak": round(tf / F16_MFMA_PEAK_TFLOPS, 4)}


def prefill_flops(w):
    """Useful causal QK and PV flops: 4 * D * Hq per visible (query, key) pair."""
    s = w.spec
    n = np.diff(w.cu_q_lens).astype(np.int64)
    P = w.context_lens.astype(np.int64) - n
    pairs = int((n * P + n * (n + 1) // 2).sum())
    return 4 * s.head_dim * s.num_q_heads * pairs


DECODE_SOURCES = ("decode.hip", "plc_device.h", "plc_internal.h")


def source_hash(names):
    """First 16 hex digits of the SHA-256 of the named kernel sources, concatenated."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_long_context_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stream_ptr():
    return torch.cuda.current_stream().cuda_stream


class DecodeCase:
    """A decode workload on the device with `copies` rotated caches."""

    def __init__(self, plc, w, dtype, partition, copies=1):
        self.plc, self.w, self.dtype = plc, w, dtype
        s = w.spec
        self.caches, self.bt = build_cache(plc, w, dtype, copies)
        self.q = to_dev(w.q)
        kn, vn = w.new_kv()
        self.k_new, self.v_new = to_dev(kn), to_dev(vn)
        self.cu = to_dev(w.cu_q_lens)
        self.start = to_dev(w.start_pos)
        self.ctx = to_dev(w.context_lens)
        self.max_ctx = int(w.context_lens.max())
        self.partition = plc.decode_partition_tokens(s.num_seqs, s.num_kv_heads, self.max_ctx,
                                                     partition)
        # zero-filled: the fused merge's completion counters start at zero
        self.ws = torch.zeros(plc.decode_workspace_size(s.num_seqs, s.num_q_heads, s.head_dim,
                                                        self.max_ctx, self.partition),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty((s.num_seqs, s.num_q_heads, s.head_dim), dtype=torch.float32,
                               device="cuda")
        self.lse = torch.empty((s.num_seqs, s.num_q_heads), dtype=torch.float32, device="cuda")
        self.sm = 1.0 / math.sqrt(s.head_dim)
        self.parts = None

    def append(self, i):
        self.plc.kv_append_quant(self.caches[i % len(self.caches)], self.k_new, self.v_new, self.bt,
                                 self.cu, self.start)

    def partials(self, i):
        self.parts = self.plc.attn_decode_partials(self.q, self.caches[i % len(self.caches)], self.bt,
                                                   self.ctx, self.max_ctx, self.partition, self.sm,
                                                   workspace=self.ws)

    def merge(self):
        o, l = self.parts
        self.plc.lse_merge(o, l, out=self.out.view(-1, self.out.shape[-1]), lse=self.lse.view(-1))

    def decode(self, i):
        self.plc.attn_decode_paged(self.q, self.caches[i % len(self.caches)], self.bt, self.ctx,
                                   self.max_ctx, self.partition, self.sm, out=self.out, lse=self.lse,
                                   workspace=self.ws)

    def step(self, i):
        """One decode step in one launch: append the step's token, attend, merge."""
        self.plc.attn_decode_append(self.q, self.k_new, self.v_new, self.caches[i % len(self.caches)],
                                    self.bt, self.ctx, self.max_ctx, self.partition, self.sm,
                                    out=self.out, lse=self.lse, workspace=self.ws)

    def step_two_launches(self, i):
        self.append(i)
        self.decode(i)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def build_cache(plc, w, dtype, copies):
    """Device caches (poison-filled, then the prefix appended by kv_append_quant),
    `copies` independent copies, and the device block table."""
    import synthetic
    s = w.spec
    shape = (w.num_blocks, s.num_kv_heads, s.block_size, s.head_dim)
    if dtype == "fp16":
        k = torch.full(shape, synthetic.POISON_F16, dtype=torch.int32, device="cuda").to(torch.int16)
        k = k.view(torch.float16)
    else:
        k = torch.full(shape, synthetic.POISON_CODE_8BIT, dtype=torch.uint8, device="cuda")
    v = k.clone()
    ks = vs = None
    if dtype == "e4m3":
        ks, vs = to_dev(w.k_scale_head), to_dev(w.v_scale_head)
    elif dtype == "int8":
        ks = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        vs = ks.clone()
    cache = plc.KVCache(k, v, dtype, ks, vs)
    bt = to_dev(w.block_tables)
    kp, vp, cup, spp = w.prefix_kv()
    if kp.shape[0]:
        plc.kv_append_quant(cache, to_dev(kp), to_dev(vp), bt, to_dev(cup), to_dev(spp))
    caches = [cache]
    for _ in range(copies - 1):
        k2, v2 = cache.k.clone(), cache.v.clone()
        if dtype == "int8":
            caches.append(plc.KVCache(k2, v2, dtype, cache.k_scale.clone(), cache.v_scale.clone()))
        else:
            caches.append(plc.KVCache(k2, v2, dtype, ks, vs))
    torch.cuda.synchronize()
    return caches, bt


def graph_time(fn, n, reps=3):
    """Capture n calls fn(i) in one HIP graph; replay; best-of-reps seconds per call
    by host clock and by events on the replay stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)                                   # prime allocator-free state on this stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    g.replay()                                  # first replay is not timed
    torch.cuda.synchronize()
    best_wall, best_ev = float("inf"), float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        best_wall = min(best_wall, (t1 - t0) / n)
        best_ev = min(best_ev, e0.elapsed_time(e1) * 1e-3 / n)
    del g
    return best_wall, best_ev


def cpu_baseline(w, dtype):
    """The oracle, as it stands, on the headline step: append the step's tokens
    into an oracle cache holding the prefix, then attention for every row."""
    import oracle
    s = w.spec
    kp, vp, cup, spp = w.prefix_kv()
    cache = oracle.HostCache(w.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, dtype,
                             w.k_scale_head, w.v_scale_head)
    cache.append(kp, vp, w.block_tables, cup, spp)
    kn, vn = w.new_kv()
    threads = os.cpu_count() or 1
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        cache.append(kn, vn, w.block_tables, w.cu_q_lens, w.start_pos)
        oracle.attention(w.q, s.num_q_heads, cache, w.block_tables, w.cu_q_lens, w.context_lens,
                         1.0 / math.sqrt(s.head_dim), nthreads=threads)
    dt = (time.perf_counter() - t0) / reps
    return dt, threads


def bench_prefill(plc, synthetic, specs, K):
    """The 8,192-token chunked causal prefill after a 122,880-token prefix."""
    # ---------------- C3 chunked prefill ----------------
    log("generating c3 (8192 new after 122880 cached)")
    w3 = synthetic.generate(specs["c3"])
    caches, bt = build_cache(plc, w3, "e4m3", 1)
    cache = caches[0]
    q = to_dev(w3.q)
    cu, ctx = to_dev(w3.cu_q_lens), to_dev(w3.context_lens)
    kn, vn = w3.new_kv()                       # the chunk's own K/V, appended first
    plc.kv_append_quant(cache, to_dev(kn), to_dev(vn), bt, cu, to_dev(w3.start_pos))
    out = torch.empty((8192, 8, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((8192, 8), dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(128)

    def pre(i):
        plc.attn_prefill_paged(q, cache, bt, cu, ctx, 8192, 131072, sm, out=out, lse=lse)
    pre(0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all()), "c3 prefill output"
    n3 = max(3, min(20, K // 10))
    pw, pe = graph_time(pre, n3, reps=2)
    fl = prefill_flops(w3)
    tf = fl / pe / 1e12
    res = {
        "workload": "c3: 8192 new tokens after a 122880-token cached prefix, 8 q / 1 kv, E4M3",
        "tflops": round(tf, 2), "unit": "TFLOP/s", "us_per_call": round(pe * 1e6, 1),
        "useful_flops": fl,
        "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL, "achieved": round(tf, 2),
                     "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4)},
    }
    log("c3 prefill %.1f us, %.1f TFLOP/s" % (pe * 1e6, tf))
    del caches, cache, q, out, lse
    torch.cuda.empty_cache()
    return res


def read_traffic(launch_bytes):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current decode kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(DECODE_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    global torch
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_long_context_amd as plc
    import synthetic
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    specs = synthetic.named_specs()
    K, W = args.steps, args.warmup
    if args.copy_calibration:
        x = torch.full((256 << 20,), 1, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log("copied 5 x 256 MiB")
        return
    if args.prefill_only:
        print(json.dumps({"c3_prefill": bench_prefill(plc, synthetic, specs, K)}), flush=True)
        return
    if args.d256_only:
        print(json.dumps({"d256_decode": bench_d256(plc, synthetic, specs, K),
                          "d256_prefill": bench_d256_prefill(plc, synthetic, specs, K)}), flush=True)
        return
    if args.verify_only:
        print(json.dumps({"verify_e4m3": bench_verify(plc, synthetic, specs, K),
                          "draft_window_e4m3": bench_window(plc, synthetic, specs, K)}), flush=True)
        return

    # ---------------- headline: C2 decode step ----------------
    log("generating c2 (8 x 32768, e4m3)")
    w2 = synthetic.generate(specs["c2"])
    c2 = DecodeCase(plc, w2, "e4m3", 2048, copies=args.copies)
    for i in range(W):
        c2.step(i)
    torch.cuda.synchronize()
    log("timing %d steps in a graph" % K)
    wall, ev = graph_time(c2.step, K)
    step_bytes = decode_bytes(w2, "e4m3") + append_bytes(w2, "e4m3")
    value = step_bytes / wall / 1e9
    # The step is one launch of the decode kernel (append + partitions + merge),
    # so the events around the replayed graph give that kernel's average
    # duration; the partitions alone and the two-launch form are reported too.
    achieved = step_bytes / ev / 1e9
    pk_ev = two_ev = app_ev = float("nan")
    if not args.no_breakdown:
        _, pk_ev = graph_time(c2.partials, K)
        _, two_ev = graph_time(c2.step_two_launches, K)
        _, app_ev = graph_time(c2.append, K)
    log("c2 step %.2f us (events %.2f us) = %.0f GB/s; partitions only %.2f us; "
        "append + decode as two launches %.2f us; append alone %.2f us"
        % (wall * 1e6, ev * 1e6, value, pk_ev * 1e6, two_ev * 1e6, app_ev * 1e6))
    traffic = read_traffic(step_bytes)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "c2 decode: 8 seqs x 32768-token context, 8 q / 1 kv heads, head_dim 128, "
                        "E4M3 KV (fp32 per-head scales), 16-token pages, split-KV partitions of "
                        "2048 + LSE merge; step = append 1 token/seq + decode, one launch",
            "kv_dtype": "e4m3", "batch": 8, "context": 32768, "num_q_heads": 8,
            "num_kv_heads": 1, "head_dim": 128, "block_size": 16, "partition_tokens": 2048,
            "cache_copies_rotated": args.copies, "timing": "HIP graph replay, host clock",
            "step_bytes": step_bytes,
        },
        "roofline": {
            "bound": "hbm", "kernel": DECODE_KERNEL, "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "bytes_per_launch": step_bytes,
            "avg_launch_us": round(ev * 1e6, 3),
        },
    }
    if not args.no_breakdown:
        result["step_breakdown_us"] = {"step_one_launch": round(ev * 1e6, 3),
                                       "partitions_only": round(pk_ev * 1e6, 3),
                                       "append_then_decode_two_launches": round(two_ev * 1e6, 3),
                                       "append_alone": round(app_ev * 1e6, 3)}
    del c2
    torch.cuda.empty_cache()

    if not args.headline_only:
        extra = {}
        extra["c3_prefill"] = bench_prefill(plc, synthetic, specs, K)
        # ---------------- C4 / C5 decode ----------------
        for name, dtypes in (("c4", ["e4m3"]), ("c5", ["fp16", "e4m3", "int8"])):
            log("generating %s" % name)
            w = synthetic.generate(specs[name])
            for dt in dtypes:
                c = DecodeCase(plc, w, dt, 0, copies=1)
                for i in range(3):
                    c.step(i)
                n = max(5, min(50, K // 4))
                sw, se = graph_time(c.step, n, reps=2)
                kw_, ke = graph_time(c.partials, n, reps=2)
                sb = decode_bytes(w, dt) + append_bytes(w, dt)
                kb = decode_bytes(w, dt, with_outputs=False)
                extra["%s_decode_%s" % (name, dt)] = {
                    "gbs": round(sb / sw / 1e9, 1), "unit": "GB/s", "us_per_step": round(sw * 1e6, 2),
                    "partition_tokens": c.partition, "step_bytes": sb,
                    "kernel_gbs": round(kb / ke / 1e9, 1), "kernel_us": round(ke * 1e6, 2),
                    "frac_of_hbm_peak": round(sb / sw / 1e9 / HBM_PEAK_GBS, 4),
                }
                log("%s %s: step %.1f us = %.0f GB/s; kernel %.1f us = %.0f GB/s"
                    % (name, dt, sw * 1e6, sb / sw / 1e9, ke * 1e6, kb / ke / 1e9))
                del c
                torch.cuda.empty_cache()
        extra["verify_e4m3"] = bench_verify(plc, synthetic, specs, K)
        extra["draft_window_e4m3"] = bench_window(plc, synthetic, specs, K)
        extra["d256_decode"] = bench_d256(plc, synthetic, specs, K)
        extra["d256_prefill"] = bench_d256_prefill(plc, synthetic, specs, K)
        result["other_workloads"] = extra

    if not args.no_cpu:
        log("timing the CPU oracle on the headline step")
        dt, threads = cpu_baseline(w2, "e4m3")
        result["cpu_baseline"] = {
            "value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_step": round(dt, 3),
            "sample": "the whole c2 step (append 8 tokens + all 64 query rows over 32768 keys), "
                      "mean of 3 runs; the oracle's prefix cache is built outside the timing",
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
