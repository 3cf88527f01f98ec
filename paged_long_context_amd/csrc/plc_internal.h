// Host-side launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace plc {

struct KvView {
    const void* k;          // [num_blocks][Hkv][block_size][D] elements
    const void* v;
    const float* k_scale;   // E4M3: [Hkv]; INT8: [num_blocks][Hkv][block_size]
    const float* v_scale;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;       // 128, or 256 (KV append and one-token decode only)
    int32_t dtype;
};

// Decode: per-partition normalized partial outputs and natural-log LSEs.
struct DecodeParams {
    const void* q;              // f16 [B][Hq][D]
    KvView kv;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t max_context_len;    // device lengths are clamped to it
    int32_t partition_tokens;   // multiple of 16
    int32_t nparts;
    float qk_scale_log2;        // sm_scale * log2(e)
    float* o_parts;             // [B*Hq][nparts][D]
    float* lse_parts;           // [B*Hq][nparts]
    // merge != 0: the merged output is wanted in out fp32 [rows][D] and lse
    // fp32 [rows] (the partitions, then the merge kernel over the partials);
    // 0: partials only
    int32_t merge;
    float* out;
    float* lse;
    // fused append of each sequence's step token (position context_len - 1):
    // f16 [B][Hkv][D] each, or NULL
    const void* k_new;
    const void* v_new;
    // Several query tokens per sequence (verification of drafted tokens), or
    // NULL for one.  cu_q_lens int32 [B+1]: sequence b's n_b query tokens are
    // its last n_b positions (n_b clamped to max_q_len); q, out, lse and the
    // partials are indexed by row (cu_q_lens[b] + j) * Hq + head.  Without
    // cu_q_lens, row b * Hq + head.  The rows of one (sequence, KV head) are
    // split into ncg groups of 16 (position-major), one workgroup column each.
    const int32_t* cu_q_lens;
    int32_t max_q_len;
    int32_t ncg;
    // with cu_q_lens: > 0 limits the row at position pos to keys
    // pos - window + 1 .. pos, and partition k of a sequence is then the k-th
    // one from the partition holding its first query's first key
    int32_t window;
    // query tokens in the call (rows = total_q_tokens * num_q_heads): num_seqs
    // for a one-token decode, cu_q_lens[num_seqs] with cu_q_lens
    int32_t total_q_tokens;
    // set by the launcher: workgroup columns per (sequence, KV head), each
    // taking groups_per_workgroup() row groups of 16
    int32_t ncgw;
    // set by the launcher: one-dimensional grid that keeps each group's
    // partitions on one XCD (used when the whole grid is resident at once)
    int32_t xcd_local;
    // set by the launcher: merge requested and a single partition per
    // sequence, so the partition kernel writes out and lse itself
    int32_t direct;
    // set by the caller: the workspace holds partials for twice nparts, so
    // the launcher may stream each partition with two workgroups (halves)
    // when a merged call's grid would otherwise leave compute units idle
    int32_t may_split;
};

// Row groups of 16 query rows that one workgroup of the 128-wide decode
// kernel takes in a call with several query tokens per sequence (ncg groups
// per (sequence, KV head)) and partitions of partition_tokens: two groups
// share each converted chunk of keys and values when partitions are at least
// 512 tokens (measured: 16 drafts over 8 x 32K, 68 -> 56 us); shorter
// partitions (sliding windows) keep one group per workgroup, whose extra
// workgroups hide latency.  1 for a one-token decode and at head dim 256.  An
// FP16 cache takes one group per workgroup (wider operands: two groups spill
// registers); sizing the workspace with this value is then conservative.
inline int32_t groups_per_workgroup(int32_t head_dim, bool multi_token, int32_t ncg, int32_t partition_tokens) {
    return (head_dim == 128 && multi_token && ncg >= 2 && partition_tokens >= 512) ? 2 : 1;
}

hipError_t launch_decode_partials(const DecodeParams& p, hipStream_t s);

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t rows,
                            int32_t nparts, int32_t head_dim, float* out, float* lse_out,
                            hipStream_t s);

struct AppendParams {
    KvView kv;                  // k/v/scales written through const_cast by the kernel
    const void* k_new;          // f16 [T][Hkv][D]
    const void* v_new;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* cu_new_lens;
    const int32_t* start_pos;
    int32_t num_seqs;
    int32_t total_new_tokens;
};

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);

struct PrefillParams {
    const void* q;              // f16 [T][Hq][D]
    KvView kv;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* cu_q_lens;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t max_q_len;
    int32_t max_context_len;    // device lengths are clamped to it
    float qk_scale_log2;
    float* out;                 // f32 [T][Hq][D]
    float* lse;                 // f32 [T][Hq]
    // 0: one pass over every visible key into out and lse.  > 0 (a multiple
    // of 32, tiles of 8-bit caches only): partition k of a sequence is keys
    // [k P, (k+1) P); each writes normalized partials of its rows to
    // o_parts [T*Hq][nparts][D] and natural-log LSEs to lse_parts
    // [T*Hq][nparts] (0 and -inf where a row sees none of its keys), and a
    // sequence's n query tokens are its last n positions even when n exceeds
    // its length (the rows before position 0 see no key)
    int32_t partition_tokens;
    int32_t nparts;
    float* o_parts;
    float* lse_parts;
};

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill256(const PrefillParams& p, hipStream_t s);   // head dim 256
// tiles of 128 query rows over 8-bit caches whose codes reach LDS by DMA
// (head dim 128 or 256), with or without key partitions
hipError_t launch_prefill_dma(const PrefillParams& p, hipStream_t s);

hipError_t launch_debug_e4m3(const uint8_t* codes, uint16_t* out, int32_t n, hipStream_t s);

}  // namespace plc
