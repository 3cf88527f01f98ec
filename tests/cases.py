"""Small workload builders shared by the oracle pins and the GPU parity tests."""
import math

import numpy as np

import oracle
import synthetic

SM_SCALE_128 = 1.0 / math.sqrt(128.0)


def spec(context_lens, q_lens, hq=8, hkv=1, d=128, seed=1234, v_dist="normal", q_scale=1.0,
         bs=16, name="case"):
    return synthetic.Spec(name=name, context_lens=list(context_lens), q_lens=list(q_lens),
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                          seed=seed, v_dist=v_dist, q_scale=q_scale)


def oracle_cache(w: synthetic.Workload, dtype: str) -> oracle.HostCache:
    """Oracle cache holding every token of every sequence of w."""
    s = w.spec
    c = oracle.HostCache(w.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, dtype,
                         w.k_scale_head, w.v_scale_head)
    c.append(w.k, w.v, w.block_tables, w.cu_kv.astype(np.int32), np.zeros(s.num_seqs, np.int32))
    return c


def oracle_attention(w: synthetic.Workload, cache, sm_scale=None, rows=None, **kw):
    s = w.spec
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(s.head_dim)
    return oracle.attention(w.q, s.num_q_heads, cache, w.block_tables, w.cu_q_lens,
                            w.context_lens, sm_scale, rows=rows, **kw)
