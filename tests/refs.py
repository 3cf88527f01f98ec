"""Independent references used to pin the oracle (CPU, float64).

Nothing here calls the oracle's arithmetic: dequantization goes through
torch's float8_e4m3fn and numpy's float16, attention through torch's
scaled_dot_product_attention, and merging through scipy's logsumexp.
"""
import numpy as np
import torch
from scipy.special import logsumexp


def dequant_cache(cache):
    """Dequantized K, V as float64 [nb][Hkv][bs][D] from an oracle HostCache."""
    if cache.dtype == "fp16":
        k = cache.k.view(np.float16).astype(np.float64)
        v = cache.v.view(np.float16).astype(np.float64)
    elif cache.dtype == "e4m3":
        def dq(c, s):
            x = torch.from_numpy(c.view(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            return x * s.astype(np.float64)[None, :, None, None]
        k = dq(cache.k, cache.k_scale_head)
        v = dq(cache.v, cache.v_scale_head)
    else:
        k = cache.k.astype(np.float64) * cache.k_tok_scale.astype(np.float64)[..., None]
        v = cache.v.astype(np.float64) * cache.v_tok_scale.astype(np.float64)[..., None]
    return k, v


def gather_dense(kd, block_tables, b, length, block_size):
    """Sequence b's first `length` tokens through its block table: [length][Hkv][D]."""
    j = np.arange(length)
    blk = block_tables[b, j // block_size]
    return kd[blk, :, j % block_size, :]


def sdpa_reference(q_f16, num_q_heads, kd, vd, block_tables, cu_q_lens, context_lens,
                   block_size, sm_scale, window=0):
    """Gathered-dense causal GQA attention through torch SDPA in float64;
    window > 0 also hides keys more than window - 1 positions back.

    Returns out [T][Hq][D], lse [T][Hq] (natural log, from an explicit
    masked score matrix and scipy.special.logsumexp)."""
    T = q_f16.shape[0]
    D = q_f16.shape[-1]
    out = np.zeros((T, num_q_heads, D))
    lse = np.zeros((T, num_q_heads))
    Hkv = kd.shape[1]
    G = num_q_heads // Hkv
    for b in range(len(context_lens)):
        a, e = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        n, L = e - a, int(context_lens[b])
        if n == 0:
            continue
        K = gather_dense(kd, block_tables, b, L, block_size)      # [L][Hkv][D]
        V = gather_dense(vd, block_tables, b, L, block_size)
        Q = q_f16[a:e].astype(np.float64)                        # [n][Hq][D]
        pos = L - n + np.arange(n)
        mask = np.arange(L)[None, :] <= pos[:, None]             # [n][L]
        if window > 0:
            mask &= np.arange(L)[None, :] > pos[:, None] - window
        qt = torch.from_numpy(Q).permute(1, 0, 2)                # [Hq][n][D]
        kt = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2).contiguous()
        vt = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=sm_scale)
        out[a:e] = o.permute(1, 0, 2).numpy()
        s = np.einsum("nhd,lhd->hnl", Q, np.repeat(K, G, axis=1)) * sm_scale
        s = np.where(mask[None], s, -np.inf)
        lse[a:e] = logsumexp(s, axis=-1).T
    return out, lse


def merge_reference(o_parts, lse_parts):
    """Merge via scipy.special.logsumexp weights (float64)."""
    lp = lse_parts.astype(np.float64)
    tot = logsumexp(lp, axis=1)
    w = np.exp(lp - tot[:, None])
    w[~np.isfinite(lp)] = 0.0
    out = np.einsum("rk,rkd->rd", w, o_parts.astype(np.float64))
    return out, tot
