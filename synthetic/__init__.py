"""Seeded synthetic inputs for paged GQA attention over a quantized KV cache.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``paged_long_context_amd``).  It draws inputs and lays out block tables;
it holds none of the attention arithmetic and none of the KV codecs.

Workloads follow the operator shapes the pages measure (1Cat-vLLM README,
"Long-Context Attention" and "128-bit Loads"; ReVolta README, opening summary
and "Weight and KV formats"): fp16 queries, fp16 K/V that the cache stores as
FP8 E4M3, INT8 or FP16, 16-token pages, block tables that scatter logical
blocks over a shared physical pool.

Random numbers come from numpy's Philox counter-based generator keyed by
``(seed, stream << 32 | sequence)``, so a sequence's values depend only on the
seed, the stream and the sequence index, never on batch order or chunking.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# Stream identifiers for the counter-based generator.
STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_LENGTHS = 4
STREAM_PERM = 5
STREAM_SUBSAMPLE = 6

KV_FP16 = "fp16"
KV_E4M3 = "e4m3"
KV_INT8 = "int8"
KV_DTYPES = (KV_FP16, KV_E4M3, KV_INT8)

# Largest finite E4M3 magnitude; the per-head scale maps max|x| onto it.
E4M3_MAX = 448.0

# Byte patterns that fill cache slots no sequence owns (and padded table
# entries), so that any read of them shows up in the output.
POISON_CODE_8BIT = 0x7F          # E4M3 NaN; INT8 +127
POISON_F16 = 0x7E00              # fp16 quiet NaN
POISON_SCALE = float("nan")      # INT8 per-token scale of an unowned slot
POISON_TABLE = -1                # padded block-table entry

BASE_SEED = 0x504C43


def rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    """Philox generator for (seed, stream, index); independent per triple."""
    key = np.array([seed & (2**64 - 1), ((stream & 0xFFFFFFFF) << 32) | (index & 0xFFFFFFFF)],
                   dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal_f16(seed: int, stream: int, index: int, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) drawn in fp32, rounded to fp16 (round-to-nearest-even)."""
    x = rng(seed, stream, index).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x.astype(np.float16)


def uniform_f16(seed: int, stream: int, index: int, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    x = rng(seed, stream, index).uniform(lo, hi, size=shape).astype(np.float32)
    return x.astype(np.float16)


@dataclasses.dataclass
class Spec:
    """Shape of one workload.

    context_lens[b] counts every token of sequence b after the step's new
    tokens are appended; q_lens[b] of them are new (and carry queries).
    """
    name: str
    context_lens: List[int]
    q_lens: List[int]
    num_q_heads: int = 8
    num_kv_heads: int = 1
    head_dim: int = 128
    block_size: int = 16
    partition_tokens: int = 0
    kv_dtypes: Sequence[str] = (KV_E4M3,)
    seed: int = BASE_SEED
    v_dist: str = "normal"         # "normal" | "uniform"
    q_scale: float = 1.0
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclasses.dataclass
class Workload:
    """Host arrays for one workload (all numpy, C-contiguous)."""
    spec: Spec
    q: np.ndarray               # f16 [Tq][Hq][D]           new query tokens, sequence-major
    k: np.ndarray               # f16 [Tkv][Hkv][D]         every token of every sequence
    v: np.ndarray               # f16 [Tkv][Hkv][D]
    cu_kv: np.ndarray           # int64 [B+1] offsets of sequences in k/v
    cu_q_lens: np.ndarray       # int32 [B+1]
    context_lens: np.ndarray    # int32 [B]
    start_pos: np.ndarray       # int32 [B] = context_lens - q_lens
    block_tables: np.ndarray    # int32 [B][max_blocks], POISON_TABLE padded
    num_blocks: int
    k_scale_head: np.ndarray    # f32 [Hkv]  E4M3 per-KV-head scale (max|k|/448)
    v_scale_head: np.ndarray    # f32 [Hkv]

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    def seq_kv(self, b: int):
        a, e = int(self.cu_kv[b]), int(self.cu_kv[b + 1])
        return self.k[a:e], self.v[a:e]

    def new_kv(self):
        """K/V of the new tokens only, packed [Tq][Hkv][D] (append input)."""
        ks, vs = [], []
        for b in range(self.spec.num_seqs):
            kb, vb = self.seq_kv(b)
            s = int(self.start_pos[b])
            ks.append(kb[s:])
            vs.append(vb[s:])
        return np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs))

    def prefix_kv(self):
        """K/V of the already-cached tokens, packed, with matching cu/start arrays."""
        ks, vs, cu = [], [], [0]
        for b in range(self.spec.num_seqs):
            kb, vb = self.seq_kv(b)
            s = int(self.start_pos[b])
            ks.append(kb[:s])
            vs.append(vb[:s])
            cu.append(cu[-1] + s)
        shape = (0,) + self.k.shape[1:]
        k = np.concatenate(ks) if ks else np.zeros(shape, np.float16)
        v = np.concatenate(vs) if vs else np.zeros(shape, np.float16)
        return (np.ascontiguousarray(k), np.ascontiguousarray(v),
                np.asarray(cu, np.int32), np.zeros(self.spec.num_seqs, np.int32))


def e4m3_head_scales(x: np.ndarray) -> np.ndarray:
    """fp32 scale per KV head chosen so that max|x| / scale == 448 (x: [T][H][D])."""
    h = x.shape[1]
    if x.shape[0] == 0:
        return np.ones(h, np.float32)
    m = np.abs(x.astype(np.float32)).max(axis=(0, 2)).astype(np.float32)
    s = (m / np.float32(E4M3_MAX)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    return s


def make_block_tables(context_lens: Sequence[int], block_size: int, seed: int):
    """Scatter each sequence's logical blocks over a shared, permuted physical pool.

    The pool holds sum(ceil(L_b / block_size)) owned blocks plus one spare that
    no sequence owns.  A seeded permutation of the pool is dealt to the
    sequences in order, so sequences interleave physically.
    """
    nbs = [(int(L) + block_size - 1) // block_size for L in context_lens]
    owned = sum(nbs)
    num_blocks = owned + 1
    perm = rng(seed, STREAM_PERM).permutation(num_blocks).astype(np.int32)
    max_blocks = max(1, max(nbs) if nbs else 1)
    bt = np.full((len(nbs), max_blocks), POISON_TABLE, np.int32)
    off = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    return bt, num_blocks


def generate(spec: Spec) -> Workload:
    B, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    assert Hq % Hkv == 0
    ctx = np.asarray(spec.context_lens, np.int64)
    ql = np.asarray(spec.q_lens, np.int64)
    assert np.all(ql <= ctx) and np.all(ql >= 0)
    cu_kv = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    k = np.empty((int(cu_kv[-1]), Hkv, D), np.float16)
    v = np.empty_like(k)
    q = np.empty((int(cu_q[-1]), Hq, D), np.float16)
    for b in range(B):
        a, e = int(cu_kv[b]), int(cu_kv[b + 1])
        k[a:e] = normal_f16(spec.seed, STREAM_K, b, (e - a, Hkv, D))
        if spec.v_dist == "uniform":
            v[a:e] = uniform_f16(spec.seed, STREAM_V, b, (e - a, Hkv, D))
        else:
            v[a:e] = normal_f16(spec.seed, STREAM_V, b, (e - a, Hkv, D))
        qa, qe = int(cu_q[b]), int(cu_q[b + 1])
        q[qa:qe] = normal_f16(spec.seed, STREAM_Q, b, (qe - qa, Hq, D), spec.q_scale)
    bt, nblocks = make_block_tables(spec.context_lens, spec.block_size, spec.seed)
    return Workload(
        spec=spec, q=q, k=k, v=v, cu_kv=cu_kv, cu_q_lens=cu_q,
        context_lens=ctx.astype(np.int32), start_pos=(ctx - ql).astype(np.int32),
        block_tables=bt, num_blocks=nblocks,
        k_scale_head=e4m3_head_scales(k), v_scale_head=e4m3_head_scales(v))


def c5_lengths(seed: int, n: int = 32, lo: int = 1024, hi: int = 131072) -> List[int]:
    """Context lengths log-uniform in [lo, hi] (seeded)."""
    u = rng(seed, STREAM_LENGTHS).random(n)
    return [int(min(hi, math.floor(math.exp(math.log(lo) + x * math.log(hi / lo))))) for x in u]


def named_specs() -> Dict[str, Spec]:
    """The five operator workloads (one GPU's share of heads), plus the
    verification-decode workload at the decode batch's shape."""
    s = {}
    s["c1_prefill"] = Spec(
        name="c1_prefill", context_lens=[512], q_lens=[512], seed=BASE_SEED + 1,
        description="tiny causal prefill: 1 x 512 tokens, 8 q / 1 kv heads, E4M3 KV")
    s["c1_decode"] = Spec(
        name="c1_decode", context_lens=[513], q_lens=[1], seed=BASE_SEED + 1,
        description="one decode step after the tiny prefill (context 513)")
    s["c2"] = Spec(
        name="c2", context_lens=[32768] * 8, q_lens=[1] * 8, partition_tokens=2048,
        seed=BASE_SEED + 2,
        description="decode batch 8 x 32,768 context, 8 q / 1 kv, E4M3, partitions of 2,048")
    s["c3"] = Spec(
        name="c3", context_lens=[131072], q_lens=[8192], seed=BASE_SEED + 3,
        description="chunked causal prefill: 8,192 new tokens after a 122,880-token cached prefix")
    s["c4"] = Spec(
        name="c4", context_lens=[524288] * 2 + [262144] * 4, q_lens=[1] * 6, seed=BASE_SEED + 4,
        description="long-context decode: 2 x 524,288 + 4 x 262,144, 8 q / 1 kv, E4M3")
    c5_seed = BASE_SEED + 5
    s["c5"] = Spec(
        name="c5", context_lens=c5_lengths(c5_seed), q_lens=[1] * 32, num_q_heads=32,
        num_kv_heads=4, kv_dtypes=(KV_FP16, KV_E4M3, KV_INT8), seed=c5_seed,
        description="ragged decode: 32 sequences, log-uniform [1,024, 131,072], 32 q / 4 kv, "
                    "FP16 / E4M3 / INT8 KV")
    # beyond the five: verification of drafted tokens at the decode batch's shape
    s["verify"] = Spec(
        name="verify", context_lens=[32768] * 8, q_lens=[4] * 8, partition_tokens=2048,
        seed=BASE_SEED + 6,
        description="verification decode: 8 x 32,768 context, 4 drafted tokens per sequence "
                    "(causal among themselves), 8 q / 1 kv, E4M3, partitions of 2,048")
    # and the draft model's attention: 8-token blocks over the long-context
    # batch's contexts, attending through a 2,048-token sliding window
    s["draft"] = Spec(
        name="draft", context_lens=[524288] * 2 + [262144] * 4, q_lens=[8] * 6, seed=BASE_SEED + 7,
        description="draft attention: 2 x 524,288 + 4 x 262,144 context, 8-token blocks, "
                    "2,048-token sliding window, 8 q / 1 kv, E4M3")
    # and the wide head: head dim 256 with six query heads per KV head, at the
    # decode batch's shape
    s["d256"] = Spec(
        name="d256", context_lens=[32768] * 8, q_lens=[1] * 8, num_q_heads=12, num_kv_heads=2,
        head_dim=256, partition_tokens=2048, kv_dtypes=(KV_FP16, KV_E4M3, KV_INT8), seed=BASE_SEED + 8,
        description="head dim 256 decode: 8 x 32,768 context, 12 q / 2 kv heads (groups of six), "
                    "FP16 / E4M3 / INT8 KV, partitions of 2,048")
    s["d256_prefill"] = Spec(
        name="d256_prefill", context_lens=[131072], q_lens=[8192], num_q_heads=12, num_kv_heads=2,
        head_dim=256, seed=BASE_SEED + 9,
        description="head dim 256 chunked causal prefill: 8,192 new tokens after a 122,880-token "
                    "cached prefix, 12 q / 2 kv heads (groups of six), E4M3 KV")
    return s


def c1_workload() -> Workload:
    """Tiny workload: one sequence of 513 tokens; the first 512 are the
    prefill chunk, token 512 is the decode step's new token."""
    spec = Spec(name="c1", context_lens=[513], q_lens=[513], seed=BASE_SEED + 1)
    return generate(spec)


def subsample_rows(n_q: int, num_q_heads: int, count: int, seed: int, tile: int = 128,
                   every_edge: int = 0) -> np.ndarray:
    """Seeded subsample of query positions of a long chunk (row ids t*Hq+h).

    Always keeps the first 8 and last 8 positions, both sides of 16 randomly
    chosen edges of `tile`-position tiles, and (every_edge > 0) both sides of
    every edge of `every_edge`-position tiles; the rest are uniform without
    replacement, up to `count` positions.
    """
    keep = set(range(min(8, n_q))) | set(range(max(0, n_q - 8), n_q))
    if every_edge > 0:
        for e in range(every_edge, n_q, every_edge):
            keep |= {e - 1, e}
    edges = []
    for e in range(tile, n_q, tile):
        edges += [e - 1, e]
    g = rng(seed, STREAM_SUBSAMPLE)
    if edges:
        pick = g.choice(len(edges) // 2, size=min(16, len(edges) // 2), replace=False)
        for p in pick:
            keep |= {edges[2 * p], edges[2 * p + 1]}
    rest = np.setdiff1d(np.arange(n_q), np.fromiter(keep, np.int64))
    need = max(0, count - len(keep))
    if need and len(rest):
        keep |= set(g.choice(rest, size=min(need, len(rest)), replace=False).tolist())
    pos = np.array(sorted(keep), np.int64)
    return (pos[:, None] * num_q_heads + np.arange(num_q_heads)[None, :]).reshape(-1)


def empty_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str):
    """Host cache arrays filled with poison: (k, v, k_tok_scale, v_tok_scale)."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    if dtype == KV_FP16:
        k = np.full(shape, POISON_F16, np.uint16)
        return k, k.copy(), None, None
    k = np.full(shape, POISON_CODE_8BIT, np.uint8)
    if dtype == KV_INT8:
        s = np.full(shape[:3], POISON_SCALE, np.float32)
        return k, k.copy(), s, s.copy()
    return k, k.copy(), None, None
