#!/usr/bin/env python3
"""Bench: paged GQA decode / prefill attention over an E4M3 KV cache on one MI355X.

Headline step (the workload the metric is quoted on): a decode step of a batch
of 8 sequences with 32,768-token contexts, 8 query heads over 1 KV head,
head_dim 128, E4M3 KV with fp32 per-head scales, 16-token pages scattered by a
seeded permutation, split-KV partitions of 2,048 tokens merged by log-sum-exp.
One step = the decode kernel, which appends the step's new K/V token per
sequence and runs every split-KV partition (1,024-token halves of the 2,048
partitions, two workgroups each, to fill the chip), then the LSE merge kernel
over the partials.  Eight copies of the cache
(537 MB, twice the 256 MB Infinity Cache) are rotated so every step reads its
keys from HBM.  Steps are captured in a HIP graph and replayed, so host launch
overhead is not timed.

`value` is the headline step's throughput over exactly --steps replayed steps
by the host clock; `roofline.achieved` divides the same bytes by the events'
average launch time.  Every workload also gets a distribution: at least 50
back-to-back graph replays, each bracketed by events, reported as median and
p10/p90 per step, with the GPU clocks and power read by amd-smi while the
replays run.

Also reported on the same JSON line: the tiny prefill + decode, the 8,192-token
chunked causal prefill after a 122,880-token prefix (TFLOP/s of useful causal
QK/PV work), the long mixed decode (2 x 524,288 + 4 x 262,144) and the ragged
32-sequence decode in FP16 / E4M3 / INT8; for each of these five the GPU
result's max|do| and relative dlse against the oracle (checked after the
timing) and the oracle itself timed on the host cores (the prefill on a
4,096-row subsample, also extrapolated to all rows).  Then verification of
drafted tokens, draft-window attention, head dim 256, a device-copy bandwidth
ceiling, and the pages' V100 operator record as context.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu]

Profiling aids (no bench line): --only NAME runs one workload (c2, c3, c4,
c5_fp16, c5_e4m3, c5_int8, verify, window, d256, d256_prefill); --prefill-only,
--verify-only and --d256-only are the older spellings of three of them;
--copy-calibration runs a plain 256 MiB device copy five times, the
known-size kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters.
"""
import argparse
import hashlib
import json
import math
import os
import subprocess
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
MIN_SAMPLES = 50
O_ATOL, LSE_RTOL = 2e-3, 1e-4
PAGES_RECORD = {
    "tflops": {"tp4": 71.111, "tp2": 70.221, "tp1": 69.982},
    "hardware": "one V100-SXM2-32GB",
    "what": "useful causal QK/PV attention, FP32 QK/PV accumulation, local head layouts of TP4/TP2/TP1",
    "source": "1Cat-vLLM README, 'Performance First' -> 'Long-Context Attention'",
    "role": "context from other hardware, not the target",
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="cache copies rotated in the C2 step")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle (CPU baseline and accuracy)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="time only the headline step (no per-part graphs), e.g. under a profiler")
    ap.add_argument("--only", default="", help="run one workload only (profiling)")
    ap.add_argument("--prefill-only", action="store_true", help="= --only c3")
    ap.add_argument("--d256-only", action="store_true", help="= --only d256 and d256_prefill")
    ap.add_argument("--verify-only", action="store_true", help="= --only verify and window")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 256 MiB device copy 5 times and exit (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ accounting

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


def read_traffic(name):
    """HBM bytes per decode launch of workload `name` from its committed
    rocprofv3 counter summary (profiles/decode_<name>_traffic.json), if that
    was taken on the current decode kernel source; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "decode_%s_traffic.json" % name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(DECODE_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ run record

def gpu_identity():
    p = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"gpu": p.name, "gfx_arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hbm_bytes": p.total_memory,
            "rocm": rocm, "torch_hip": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu, "host_threads_used": host_threads()}


def _flatten(x, prefix="", out=None):
    if out is None:
        out = {}
    if isinstance(x, dict):
        if "value" in x and not isinstance(x["value"], (dict, list)):
            out[prefix.rstrip(".")] = x["value"]
            return out
        for k, v in x.items():
            _flatten(v, prefix + str(k) + ".", out)
    elif isinstance(x, list):
        for i, v in enumerate(x):
            _flatten(v, prefix + str(i) + ".", out)
    elif isinstance(x, (int, float)) or (isinstance(x, str) and x and x != "N/A"):
        out[prefix.rstrip(".")] = x
    return out


def _profiled():
    """Under rocprofv3 a child process inherits the profiler's preload, which
    initialises the GPU before the smi tools' launchers re-exec themselves;
    the clock and power readings are skipped there."""
    return any(k.startswith("ROCPROF") for k in os.environ)


def _smi(args, timeout=20):
    if _profiled():
        return None, "skipped under a profiler"
    try:
        r = subprocess.run(["amd-smi"] + args + ["--json"], capture_output=True, text=True,
                           timeout=timeout)
        return json.loads(r.stdout), None
    except Exception as e:          # recorded, never fatal
        return None, "%s: %s" % (type(e).__name__, str(e)[:200])


SMI_KEYS = ("clk", "clock", "freq", "power", "cap", "limit")


def smi_filter(data):
    """Current clocks and power of an `amd-smi metric --clock --power` reading
    (min/max clock bounds and non-numeric fields dropped)."""
    flat = _flatten(data)
    keep = {}
    for k, v in flat.items():
        kl = k.lower()
        if isinstance(v, str) or kl.endswith(("min_clk", "max_clk")):
            continue
        if any(t in kl for t in SMI_KEYS):
            keep[k.replace("gpu_data.0.", "")] = v
    return dict(list(keep.items())[:60])


def smi_static():
    """Board identity and clock levels (amd-smi static) and the power cap (rocm-smi)."""
    out = {}
    d, err = _smi(["static", "-g", "0"])
    if d is None:
        out["amd_smi_static_error"] = err
    else:
        flat = _flatten(d)
        for k, v in flat.items():
            kl = k.lower()
            if kl.endswith(("market_name", "product_name")) or ".ifwi.name" in kl or \
                    (".clock." in kl and ("frequency_levels" in kl) and (".sys." in kl or ".mem." in kl)):
                out[k] = v
    try:
        if _profiled():
            raise RuntimeError("skipped under a profiler")
        r = subprocess.run(["rocm-smi", "--showmaxpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        j = json.loads(r.stdout)
        out.update({"rocm_smi." + k: v for k, v in _flatten(j).items() if "power" in k.lower()})
    except Exception as e:
        out["rocm_smi_error"] = "%s: %s" % (type(e).__name__, str(e)[:200])
    return out


def smi_under_load(replay, readings=3, max_s=8.0, warm_s=0.3):
    """GPU clocks and power read by amd-smi `readings` times while `replay`
    keeps the GPU busy (up to 16 replays queued between synchronizations, and
    busy for warm_s before the first reading, so the clocks have ramped).
    Returns the fields of the reading with the highest socket power (a
    reading can fall between two queued replays and show the idle clock)
    plus, per clock/power field, the list of all readings."""
    if _profiled():
        return {"error": "skipped under a profiler"}
    n = 0

    def spin(until, p=None):
        nonlocal n
        while time.time() < until and (p is None or p.poll() is None):
            replay()
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()

    spin(time.time() + warm_s)
    got = []
    for _ in range(readings):
        try:
            p = subprocess.Popen(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"],
                                 stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        except Exception as e:
            torch.cuda.synchronize()
            return {"error": "%s: %s" % (type(e).__name__, e)}
        spin(time.time() + max_s, p)
        try:
            out, _ = p.communicate(timeout=10)
            got.append(smi_filter(json.loads(out)))
        except Exception as e:
            p.kill()
            got.append({"error": "%s: %s" % (type(e).__name__, str(e)[:200])})
    torch.cuda.synchronize()

    def power(g):
        v = g.get("power.socket_power")
        return v if isinstance(v, (int, float)) else -1

    res = dict(max(got, key=power))
    keys = [k for k in res if k.startswith("clock.gfx_0") or k.startswith("clock.mem_0") or k.startswith("power")]
    res["readings"] = {k: [g.get(k) for g in got] for k in keys}
    return res


# ------------------------------------------------------------------ timing

class GraphTimer:
    """`steps` calls fn(i) captured in one HIP graph, replayed on torch's
    current stream."""

    def __init__(self, fn, steps):
        self.steps = steps
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
        g.replay()                              # first replay is not timed
        torch.cuda.synchronize()
        self.g = g

    def once(self):
        """(host-clock s, event s) per call over one replay."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        self.g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) / self.steps, e0.elapsed_time(e1) * 1e-3 / self.steps

    def samples(self, n):
        """Per-call seconds of n back-to-back replays, each between two events."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(n):
            self.g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)]) * 1e-3 / self.steps


def timed(fn, call_s_guess, smi=True, n=MIN_SAMPLES):
    """Distribution of fn's per-call time: graph replays of about 2 ms each
    (at least one call, at most 64), n of them back to back.  The GPU waits
    8-13 us between two replays for the next graph's launch (rocprofv3 kernel
    traces: no gap between kernels inside a replay), so a replay holds enough
    calls that this launch cost stays near 1 % of a call.  Returns (stats
    dict in us, GraphTimer)."""
    steps = max(1, min(64, int(math.ceil(2e-3 / max(call_s_guess, 1e-7)))))
    gt = GraphTimer(fn, steps)
    x = gt.samples(n) * 1e6
    st = {"median_us": round(float(np.median(x)), 3), "p10_us": round(float(np.percentile(x, 10)), 3),
          "p90_us": round(float(np.percentile(x, 90)), 3), "mean_us": round(float(x.mean()), 3),
          "min_us": round(float(x.min()), 3), "max_us": round(float(x.max()), 3),
          "samples": n, "calls_per_sample": steps}
    if smi:
        st["gpu_under_load"] = smi_under_load(gt.g.replay)
    return st, gt


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ------------------------------------------------------------------ device data

def stream_ptr():
    return torch.cuda.current_stream().cuda_stream


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


def step_kernel_partition(spec, max_context_len, partition):
    """The partition the decode step's partition kernel streams: half of
    `partition` when the library runs each partition as two workgroups (a
    one-token decode at head dim 128 whose grid, 8 ceil(units / 8) x nparts
    workgroups, would fill at most half of the 256 compute units; the
    partition a multiple of 64 and at least 512), else `partition`.  A
    partials call at this partition launches the step's partition kernel
    without the fused append (tests/test_gpu_decode.py checks the two give
    bitwise-equal merged outputs)."""
    units = spec.num_seqs * spec.num_kv_heads
    nparts = -(-max_context_len // partition) if max_context_len > 0 else 1
    if (spec.head_dim == 128 and ((units + 7) // 8) * 8 * nparts * 2 <= 256 and partition % 64 == 0
            and partition >= 512):
        return partition // 2
    return partition


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
        self.ws = torch.zeros(plc.decode_workspace_size(s.num_seqs, s.num_q_heads, s.head_dim,
                                                        self.max_ctx, self.partition),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty((s.num_seqs, s.num_q_heads, s.head_dim), dtype=torch.float32,
                               device="cuda")
        self.lse = torch.empty((s.num_seqs, s.num_q_heads), dtype=torch.float32, device="cuda")
        self.sm = 1.0 / math.sqrt(s.head_dim)
        self.parts = None
        self.kernel_partition = step_kernel_partition(s, self.max_ctx, self.partition)
        self.kws = torch.empty(plc.decode_workspace_size(s.num_seqs, s.num_q_heads, s.head_dim,
                                                         self.max_ctx, self.kernel_partition),
                               dtype=torch.uint8, device="cuda")
        self.mout = torch.empty((s.num_seqs * s.num_q_heads, s.head_dim), dtype=torch.float32,
                                device="cuda")
        self.mlse = torch.empty((s.num_seqs * s.num_q_heads,), dtype=torch.float32, device="cuda")

    def append(self, i):
        self.plc.kv_append_quant(self.caches[i % len(self.caches)], self.k_new, self.v_new, self.bt,
                                 self.cu, self.start)

    def partials(self, i):
        self.parts = self.plc.attn_decode_partials(self.q, self.caches[i % len(self.caches)], self.bt,
                                                   self.ctx, self.max_ctx, self.partition, self.sm,
                                                   workspace=self.ws)

    def kernel(self, i):
        """The step's partition kernel alone (no fused append, no merge)."""
        self.kparts = self.plc.attn_decode_partials(self.q, self.caches[i % len(self.caches)], self.bt,
                                                    self.ctx, self.max_ctx, self.kernel_partition,
                                                    self.sm, workspace=self.kws)

    def merge(self, i):
        """The step's merge kernel alone, over the partials of kernel()."""
        self.plc.lse_merge(*self.kparts, out=self.mout, lse=self.mlse)

    def decode(self, i):
        self.plc.attn_decode_paged(self.q, self.caches[i % len(self.caches)], self.bt, self.ctx,
                                   self.max_ctx, self.partition, self.sm, out=self.out, lse=self.lse,
                                   workspace=self.ws)

    def step(self, i):
        """One decode step: append the step's token and attend (one kernel), merge."""
        self.plc.attn_decode_append(self.q, self.k_new, self.v_new, self.caches[i % len(self.caches)],
                                    self.bt, self.ctx, self.max_ctx, self.partition, self.sm,
                                    out=self.out, lse=self.lse, workspace=self.ws)

    def step_two_launches(self, i):
        self.append(i)
        self.decode(i)


# ------------------------------------------------------------------ oracle legs

def oracle_step(w, dtype, rows=None):
    """The oracle as it stands, on one step of workload w: its cache holds the
    prefix (built before the clock starts); timed are the append of the
    step's new tokens and attention for every row (or the listed rows).
    Returns (out, lse, append_s, attention_s, threads)."""
    import oracle
    s = w.spec
    kp, vp, cup, spp = w.prefix_kv()
    cache = oracle.HostCache(w.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, dtype,
                             w.k_scale_head, w.v_scale_head)
    if kp.shape[0]:
        cache.append(kp, vp, w.block_tables, cup, spp)
    kn, vn = w.new_kv()
    threads = host_threads()
    t0 = time.perf_counter()
    cache.append(kn, vn, w.block_tables, w.cu_q_lens, w.start_pos)
    t1 = time.perf_counter()
    ro, rl = oracle.attention(w.q, s.num_q_heads, cache, w.block_tables, w.cu_q_lens,
                              w.context_lens, 1.0 / math.sqrt(s.head_dim), rows=rows, nthreads=threads)
    t2 = time.perf_counter()
    return ro, rl, t1 - t0, t2 - t1, threads


def accuracy(o, l, ro, rl, rows=None):
    """max|do| and max |dlse| / max(1, |lse|) over the rows (all when None)."""
    D = ro.shape[-1]
    o = np.asarray(o, np.float64).reshape(-1, D)
    ro = np.asarray(ro, np.float64).reshape(-1, D)
    l = np.asarray(l, np.float64).reshape(-1)
    rl = np.asarray(rl, np.float64).reshape(-1)
    if rows is not None:
        o, ro, l, rl = o[rows], ro[rows], l[rows], rl[rows]
    do = float(np.abs(o - ro).max()) if o.size else 0.0
    dl = float((np.abs(l - rl) / np.maximum(1.0, np.abs(rl))).max()) if l.size else 0.0
    ok = bool(np.all(np.isfinite(o)) and do <= O_ATOL and dl <= LSE_RTOL)
    return {"rows_checked": int(o.shape[0]), "max_abs_do": do, "max_rel_dlse": dl,
            "within_tolerance": ok, "tolerance": {"abs_o": O_ATOL, "rel_lse": LSE_RTOL}}


def decode_oracle_leg(w, dtype, out, lse, step_bytes):
    ro, rl, ta, tt, th = oracle_step(w, dtype)
    acc = accuracy(out, lse, ro, rl)
    t = ta + tt
    cpu = {"value": round(step_bytes / t / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
           "seconds_per_step": round(t, 3), "append_s": round(ta, 4), "attention_s": round(tt, 3),
           "sample": "the whole step (append the step's tokens + every query row over its whole "
                     "context); the oracle's prefix cache is built outside the timing"}
    return acc, cpu


# ------------------------------------------------------------------ workloads

def bench_c1(plc, synthetic, cpu):
    """Tiny prefill of 512 tokens, then one decode step over 513: the
    correctness workload (launch-bound; not judged against a roofline)."""
    w = synthetic.c1_workload()
    k, v, _, _ = synthetic.empty_cache(w.num_blocks, 1, 16, 128, "e4m3")
    cache = plc.KVCache(to_dev(k), to_dev(v), "e4m3", to_dev(w.k_scale_head), to_dev(w.v_scale_head))
    bt = to_dev(w.block_tables)
    cu1, ctx1 = to_dev(np.array([0, 512], np.int32)), to_dev(np.array([512], np.int32))
    cud, ctxd = to_dev(np.array([0, 1], np.int32)), to_dev(np.array([513], np.int32))
    q = to_dev(w.q)
    kn, vn = to_dev(w.k), to_dev(w.v)
    sp0, sp512 = to_dev(np.zeros(1, np.int32)), to_dev(np.array([512], np.int32))
    sm = 1.0 / math.sqrt(128)
    out = torch.empty((512, 8, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((512, 8), dtype=torch.float32, device="cuda")
    outd = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
    lsed = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    ws = torch.zeros(plc.decode_workspace_size(1, 8, 128, 513, 0), dtype=torch.uint8, device="cuda")

    def run(i):
        plc.kv_append_quant(cache, kn[:512], vn[:512], bt, cu1, sp0)
        plc.attn_prefill_paged(q[:512], cache, bt, cu1, ctx1, 512, 512, sm, out=out, lse=lse)
        plc.attn_decode_append(q[512:], kn[512:], vn[512:], cache, bt, ctxd, 513, 0, sm, out=outd,
                               lse=lsed, workspace=ws)
    run(0)
    torch.cuda.synchronize()
    st, _ = timed(run, 50e-6, smi=False)
    res = {"workload": "c1: prefill 512 tokens (append + attention), then one decode step over 513 "
                       "(append fused into the attention kernel); 8 q / 1 kv, E4M3",
           "timing": st, "note": "launch-bound correctness workload; no roofline"}
    if cpu:
        import oracle
        ref = oracle.HostCache(w.num_blocks, 1, 16, 128, "e4m3", w.k_scale_head, w.v_scale_head)
        ref.append(w.k, w.v, w.block_tables, np.array([0, 513], np.int32), np.zeros(1, np.int32))
        ro, rl = oracle.attention(w.q[:512], 8, ref, w.block_tables, np.array([0, 512], np.int32),
                                  np.array([512], np.int32), sm)
        rdo, rdl = oracle.attention(w.q[512:], 8, ref, w.block_tables, np.array([0, 1], np.int32),
                                    np.array([513], np.int32), sm)
        res["accuracy_prefill"] = accuracy(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
        res["accuracy_decode"] = accuracy(outd.cpu().numpy(), lsed.cpu().numpy(), rdo, rdl)
        res["codes_bit_exact"] = bool(np.array_equal(cache.k.cpu().numpy(), ref.k) and
                                      np.array_equal(cache.v.cpu().numpy(), ref.v))
    return res


def bench_c2(plc, synthetic, specs, args):
    """The headline decode step.  Returns (result line without the extras, DecodeCase, w)."""
    K, W = args.steps, args.warmup
    log("generating c2 (8 x 32768, e4m3)")
    w2 = synthetic.generate(specs["c2"])
    c2 = DecodeCase(plc, w2, "e4m3", 2048, copies=args.copies)
    for i in range(W):
        c2.step(i)
    torch.cuda.synchronize()
    log("timing %d steps in a graph" % K)
    head = GraphTimer(c2.step, K)
    wall, ev = head.once()
    step_bytes = decode_bytes(w2, "e4m3") + append_bytes(w2, "e4m3")
    value = step_bytes / wall / 1e9
    del head
    dist, _ = timed(c2.step, ev, smi=not args.no_breakdown)
    # the dominant kernel: the step's partition kernel, launched alone at the
    # partition the step streams; its algorithmic bytes are the keys, values,
    # scales, table entries and queries it reads
    for i in range(3):
        c2.kernel(i)
    kst, _ = timed(c2.kernel, ev, smi=False)
    mst, _ = timed(c2.merge, 3e-6, smi=False)
    kbytes = decode_bytes(w2, "e4m3", with_outputs=False)
    achieved = kbytes / (kst["mean_us"] * 1e-6) / 1e9
    pk = two = app = None
    if not args.no_breakdown:
        pk, _ = timed(c2.partials, ev, smi=False)
        two, _ = timed(c2.step_two_launches, ev, smi=False)
        app, _ = timed(c2.append, 3e-6, smi=False)
    log("c2 step %.2f us (events %.2f us; median %.2f, p10 %.2f, p90 %.2f) = %.0f GB/s; partition kernel "
        "%.2f us = %.0f GB/s, merge kernel %.2f us"
        % (wall * 1e6, ev * 1e6, dist["median_us"], dist["p10_us"], dist["p90_us"], value, kst["mean_us"],
           achieved, mst["mean_us"]))
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
                        "2048 + LSE merge; step = append 1 token/seq fused into the partition kernel, then "
                        "the merge kernel",
            "kv_dtype": "e4m3", "batch": 8, "context": 32768, "num_q_heads": 8,
            "num_kv_heads": 1, "head_dim": 128, "block_size": 16, "partition_tokens": 2048,
            "cache_copies_rotated": args.copies, "timing": "HIP graph replay of --steps steps, host clock",
            "step_bytes": step_bytes,
        },
        "roofline": {
            "bound": "hbm", "kernel": DECODE_KERNEL, "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("c2"), "bytes_per_launch": kbytes,
            "avg_launch_us": kst["mean_us"],
            "launch": "the step's partition kernel alone (partials call at partition %d, the %d "
                      "partitions of %d each streamed as two workgroups), graph replays of %d "
                      "back-to-back launches between HIP events (per-launch time includes the "
                      "launch gap)" % (c2.kernel_partition, 32768 // 2048, 2048,
                                       kst["calls_per_sample"]),
            "merge_kernel_avg_us": mst["mean_us"],
            "step_avg_us_events": round(ev * 1e6, 3),
            "step_frac_of_hbm_peak": round(step_bytes / ev / 1e9 / HBM_PEAK_GBS, 4),
        },
        "timing": dict(dist, frac_of_hbm_peak_at_median=round(step_bytes / dist["median_us"] / 1e3 /
                                                               HBM_PEAK_GBS, 4)),
    }
    if pk is not None:
        result["step_breakdown_us"] = {"step_median": dist["median_us"],
                                       "partition_kernel_median": kst["median_us"],
                                       "merge_kernel_median": mst["median_us"],
                                       "partials_at_2048_unsplit_median": pk["median_us"],
                                       "append_then_decode_median": two["median_us"],
                                       "append_alone_median": app["median_us"]}
    return result, c2, w2, step_bytes


def bench_prefill(plc, synthetic, specs, cpu):
    """The 8,192-token chunked causal prefill after a 122,880-token prefix."""
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
    st, _ = timed(pre, 4e-3)
    fl = prefill_flops(w3)
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    res = {
        "workload": "c3: 8192 new tokens after a 122880-token cached prefix, 8 q / 1 kv, E4M3",
        "tflops": round(tf, 2), "unit": "TFLOP/s", "us_per_call": st["median_us"],
        "useful_flops": fl, "timing": st,
        "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL, "achieved": round(tf, 2),
                     "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4),
                     "p10_p90_frac": [round(fl / (st["p90_us"] * 1e-6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
                                      round(fl / (st["p10_us"] * 1e-6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)]},
    }
    log("c3 prefill median %.1f us (p10 %.1f, p90 %.1f), %.1f TFLOP/s"
        % (st["median_us"], st["p10_us"], st["p90_us"], tf))
    if cpu:
        o_h, l_h = out.cpu().numpy(), lse.cpu().numpy()
        rows = synthetic.subsample_rows(8192, 8, 512, seed=0xC3, tile=32, every_edge=128)
        log("oracle on the c3 subsample (%d rows)" % len(rows))
        ro, rl, ta, tt, th = oracle_step(w3, "e4m3", rows=rows)
        res["accuracy"] = accuracy(o_h, l_h, ro, rl, rows=rows)
        scale = 8192 * 8 / len(rows)
        sub_fl = fl * len(rows) / (8192 * 8)
        res["cpu_baseline"] = {
            "value": round(sub_fl / (ta + tt) / 1e12, 6), "unit": "TFLOP/s", "cores": th,
            "kind": "oracle", "seconds_subsample": round(ta + tt, 3),
            "seconds_all_rows_extrapolated_x%d" % round(scale): round(ta + tt * scale, 2),
            "sample": "append of the 8,192-token chunk + attention for a seeded subsample of "
                      "%d of the 65,536 query rows (512 positions x 8 heads); value = the "
                      "subsample's useful flops / its time (flops pro rata by rows)" % len(rows)}
    del caches, cache, q, out, lse
    torch.cuda.empty_cache()
    return res


def bench_decode_config(plc, synthetic, specs, name, dtypes, cpu, w=None):
    out = {}
    if w is None:
        log("generating %s" % name)
        w = synthetic.generate(specs[name])
    for dt in dtypes:
        c = DecodeCase(plc, w, dt, 0, copies=1)
        for i in range(3):
            c.step(i)
        torch.cuda.synchronize()
        one = GraphTimer(c.step, 1).once()[1]
        st, _ = timed(c.step, one)
        for i in range(3):
            c.kernel(i)
        kst, _ = timed(c.kernel, one, smi=False)
        mst, _ = timed(c.merge, 3e-6, smi=False)
        c.step(0)
        torch.cuda.synchronize()
        o_h, l_h = c.out.cpu().numpy(), c.lse.cpu().numpy()
        sb = decode_bytes(w, dt) + append_bytes(w, dt)
        kb = decode_bytes(w, dt, with_outputs=False)
        med = st["median_us"] * 1e-6
        gbs = sb / med / 1e9
        kg = kb / (kst["mean_us"] * 1e-6) / 1e9
        r = {"gbs": round(gbs, 1), "unit": "GB/s", "us_per_step": st["median_us"],
             "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
             "p10_p90_frac": [round(sb / (st["p90_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                              round(sb / (st["p10_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)],
             "partition_tokens": c.partition, "step_bytes": sb, "timing": st,
             "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL, "achieved": round(kg, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kg / HBM_PEAK_GBS, 4),
                          "p10_p90_frac": [round(kb / (kst["p90_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                           round(kb / (kst["p10_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)],
                          "traffic": read_traffic("%s_%s" % (name, dt)), "bytes_per_launch": kb,
                          "avg_launch_us": kst["mean_us"],
                          "launch": "the step's partition kernel alone (partials call at partition %d), "
                                    "graph replays between HIP events" % c.kernel_partition,
                          "merge_kernel_avg_us": mst["mean_us"]}}
        log("%s %s: step median %.1f us (p10 %.1f, p90 %.1f) = %.0f GB/s (%.1f%%); partition kernel "
            "%.1f us = %.1f%%; merge %.1f us"
            % (name, dt, st["median_us"], st["p10_us"], st["p90_us"], gbs, 100 * gbs / HBM_PEAK_GBS,
               kst["mean_us"], 100 * kg / HBM_PEAK_GBS, mst["mean_us"]))
        del c
        torch.cuda.empty_cache()
        if cpu:
            log("oracle on %s %s" % (name, dt))
            r["accuracy"], r["cpu_baseline"] = decode_oracle_leg(w, dt, o_h, l_h, sb)
        out["%s_decode_%s" % (name, dt)] = r
    return out


def bench_verify(plc, synthetic, specs, widths=(4, 16), spec_name="verify", dtype="e4m3"):
    """Verification decode at the decode batch's shape (8 x 32768, E4M3 unless
    dtype says otherwise, automatic partitions), 8 rotated cache copies, for a
    few draft widths; spec_name "d256" takes the head dim 256 batch (12 q / 2
    kv) instead."""
    import dataclasses
    res = {}
    for n in widths:
        sp = dataclasses.replace(specs[spec_name], q_lens=[n] * len(specs[spec_name].context_lens))
        tag = ("verify" if spec_name == "verify" else spec_name + " verify") + ("" if dtype == "e4m3" else " " + dtype)
        log("generating %s n=%d" % (tag, n))
        w = synthetic.generate(sp)
        s = w.spec
        caches, bt = build_cache(plc, w, dtype, 8)
        kn, vn = w.new_kv()
        kn, vn = to_dev(kn), to_dev(vn)
        cu, start, ctx = to_dev(w.cu_q_lens), to_dev(w.start_pos), to_dev(w.context_lens)
        for c in caches:
            plc.kv_append_quant(c, kn, vn, bt, cu, start)
        q = to_dev(w.q)
        T = int(w.cu_q_lens[-1])
        maxc = int(w.context_lens.max())
        P = 0                                   # the library's own partition choice
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
        st, _ = timed(f, 30e-6, smi=False)
        ev = st["median_us"] * 1e-6
        vb = verify_bytes(w, dtype)
        L = w.context_lens.astype(np.int64)
        visible = int(sum(n * (int(l) - n) + n * (n + 1) // 2 for l in L))
        fl = 4 * s.head_dim * s.num_q_heads * visible
        res["n%d" % n] = {
            "drafted_tokens": n, "gbs": round(vb / ev / 1e9, 1), "unit": "GB/s",
            "us_per_call": st["median_us"], "bytes": vb, "timing": st,
            "frac_of_hbm_peak": round(vb / ev / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / ev / 1e12, 2),
        }
        log("%s n=%d: %.2f us = %.0f GB/s (%.1f%% of HBM), %.1f TFLOP/s"
            % (tag, n, ev * 1e6, vb / ev / 1e9, 100 * vb / ev / 1e9 / HBM_PEAK_GBS, fl / ev / 1e12))
        del caches, ws, out, lse, q
        torch.cuda.empty_cache()
    res["workload"] = specs[spec_name].description + "; widths as listed" + \
        ("" if dtype == "e4m3" else "; %s cache" % dtype.upper())
    return res


def bench_window(plc, synthetic, specs, window=2048):
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
            st, _ = timed(f, 20e-6, smi=False)
            key = "window_%d" % wt if wt else "no_window"
            entry[key + "_us"] = st["median_us"]
            entry[key + "_p10_p90_us"] = [st["p10_us"], st["p90_us"]]
            log("draft %s window %d: %.2f us" % (tag, wt, st["median_us"]))
            del ws
        res[tag] = dict(entry, context_lens=sorted(set(int(x) for x in ctx)), tokens_per_block=n)
        del caches, out, lse, q
        torch.cuda.empty_cache()
    res["workload"] = base.description + "; the same blocks at 32,768-token contexts; eight " \
        "rotated cache copies (the windows' 3 MB per call stay cache-resident, so these are " \
        "latency figures, not HBM-bound ones)"
    return res


def bench_d256(plc, synthetic, specs):
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
        st, _ = timed(c.step, 60e-6, smi=False)
        kst, _ = timed(c.partials, 60e-6, smi=False)
        sb = decode_bytes(w, dt) + append_bytes(w, dt)
        kb = decode_bytes(w, dt, with_outputs=False)
        sw, ke = st["median_us"] * 1e-6, kst["median_us"] * 1e-6
        res[dt] = {"gbs": round(sb / sw / 1e9, 1), "unit": "GB/s", "us_per_step": st["median_us"],
                   "step_p10_p90_us": [st["p10_us"], st["p90_us"]],
                   "step_bytes": sb, "frac_of_hbm_peak": round(sb / sw / 1e9 / HBM_PEAK_GBS, 4),
                   "partitions_kernel_us": kst["median_us"],
                   "partitions_kernel_gbs": round(kb / ke / 1e9, 1)}
        log("d256 %s: step %.1f us = %.0f GB/s; partitions %.1f us" % (dt, sw * 1e6, sb / sw / 1e9, ke * 1e6))
        del c
        torch.cuda.empty_cache()
    return res


def bench_d256_prefill(plc, synthetic, specs):
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
    st, _ = timed(pre, 20e-3, smi=False, n=20)
    fl = prefill_flops(w)
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    log("d256 prefill %.1f us, %.1f TFLOP/s" % (st["median_us"], tf))
    del caches, cache, q, out, lse
    torch.cuda.empty_cache()
    return {"workload": s.description, "tflops": round(tf, 2), "unit": "TFLOP/s",
            "us_per_call": st["median_us"], "timing": st, "useful_flops": fl,
            "frac_of_f16_mfma_peak": round(tf / F16_MFMA_PEAK_TFLOPS, 4)}


def copy_ceiling():
    """Device-to-device copy of 1 GiB (torch's copy, a plain copy kernel):
    read + written bytes over the median time of 20 copies."""
    n = 1 << 30
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ts = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.median(ts))
    del x, y
    torch.cuda.empty_cache()
    return {"what": "device copy of 1 GiB (read 1 GiB + write 1 GiB), median of 20",
            "gbs": round(2 * n / t / 1e9, 1), "frac_of_hbm_peak": round(2 * n / t / 1e9 / HBM_PEAK_GBS, 4),
            "us": round(t * 1e6, 1)}


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
    cpu = not args.no_cpu
    if args.copy_calibration:
        x = torch.full((256 << 20,), 1, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log("copied 5 x 256 MiB")
        return
    only = args.only
    if args.prefill_only:
        only = "c3"
    if args.d256_only:
        only = "d256,d256_prefill"
    if args.verify_only:
        only = "verify,window"
    if only and only != "c2":
        res = {}
        for name in only.split(","):
            if name == "c3":
                res["c3_prefill"] = bench_prefill(plc, synthetic, specs, cpu)
            elif name == "c4":
                res.update(bench_decode_config(plc, synthetic, specs, "c4", ["e4m3"], cpu))
            elif name.startswith("c5_"):
                res.update(bench_decode_config(plc, synthetic, specs, "c5", [name[3:]], cpu))
            elif name == "verify":
                res["verify_e4m3"] = bench_verify(plc, synthetic, specs)
            elif name == "verify_d256":
                res["verify_d256_e4m3"] = bench_verify(plc, synthetic, specs, widths=(16,), spec_name="d256")
            elif name == "verify_fp16":
                res["verify_fp16"] = bench_verify(plc, synthetic, specs, widths=(16,), dtype="fp16")
            elif name == "window":
                res["draft_window_e4m3"] = bench_window(plc, synthetic, specs)
            elif name == "d256":
                res["d256_decode"] = bench_d256(plc, synthetic, specs)
            elif name == "d256_prefill":
                res["d256_prefill"] = bench_d256_prefill(plc, synthetic, specs)
            else:
                raise SystemExit("unknown workload %r" % name)
        print(json.dumps(res), flush=True)
        return

    # ---------------- headline: C2 decode step ----------------
    run = {"identity": gpu_identity(), "power_limits": smi_static() if not args.no_breakdown else None}
    result, c2, w2, step_bytes = bench_c2(plc, synthetic, specs, args)
    c2.step(0)
    torch.cuda.synchronize()
    o2, l2 = c2.out.cpu().numpy(), c2.lse.cpu().numpy()
    del c2
    torch.cuda.empty_cache()
    if cpu:
        log("oracle on the headline step")
        result["accuracy"], result["cpu_baseline"] = decode_oracle_leg(w2, "e4m3", o2, l2, step_bytes)
    result["run"] = run

    if not args.headline_only and only != "c2":
        extra = {}
        extra["c1_tiny"] = bench_c1(plc, synthetic, cpu)
        extra["c3_prefill"] = bench_prefill(plc, synthetic, specs, cpu)
        extra.update(bench_decode_config(plc, synthetic, specs, "c4", ["e4m3"], cpu))
        extra.update(bench_decode_config(plc, synthetic, specs, "c5", ["fp16", "e4m3", "int8"], cpu))
        extra["verify_e4m3"] = bench_verify(plc, synthetic, specs)
        extra["verify_d256_e4m3"] = bench_verify(plc, synthetic, specs, widths=(16,), spec_name="d256")
        extra["verify_fp16"] = bench_verify(plc, synthetic, specs, widths=(16,), dtype="fp16")
        extra["draft_window_e4m3"] = bench_window(plc, synthetic, specs)
        extra["d256_decode"] = bench_d256(plc, synthetic, specs)
        extra["d256_prefill"] = bench_d256_prefill(plc, synthetic, specs)
        extra["copy_ceiling"] = copy_ceiling()
        extra["pages_operator_record"] = PAGES_RECORD
        result["other_workloads"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
