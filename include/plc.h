/*
 * plc.h -- C ABI of libplc: paged grouped-query attention over a quantized
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The problem is the one the pages state for long-context serving: K and V
 * live in fixed-size pages reached through per-sequence block tables
 * (1Cat-vLLM README, "FlashAttention-V100", Layer 1 "Move KV Cache Correctly,
 * Wide, and Once"); the cache holds FP8 E4M3 with calibrated per-layer
 * scales, FP16, or INT8 with scales computed per token and head at run time
 * (ReVolta README, "Weight and KV formats": "E4M3 KV", "INT8 KV"); prefill
 * runs in chunks after an already-cached prefix (ReVolta README, "Quick
 * start"; 1Cat-vLLM README, Layer 2, "Prefix / Causal-Tail Separation"); long
 * decode splits the keys into partitions whose fp32 partial states are merged
 * (Layer 2, "Split-KV3"); QK and PV accumulate in fp32 ("Performance First").
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are HIP device pointers; the library only reads
 *    or writes them from kernels.  Pointers marked (host) are read on the
 *    host before the call returns.  The caller owns every buffer; the library
 *    allocates nothing and keeps no device state.
 *  - fp16 data is IEEE binary16 passed as its 16-bit pattern.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work on it and return; device faults surface at the caller's next
 *    synchronization.
 *  - Return value: PLC_OK, or a negative PLC_ERR_* code after which nothing
 *    was enqueued (except PLC_ERR_HIP, a launch failure).  plc_last_error()
 *    gives the message (thread-local).  All checks use host-visible arguments
 *    only; values read from device memory (block tables, lengths, scales) are
 *    trusted within the bounds the host arguments state.
 *  - Supported shapes: head_dim 128, block_size 16, num_q_heads a multiple of
 *    num_kv_heads with a group size G = Hq/Hkv of 1, 2, 4, 8 or 16.
 *  - head_dim 256 (1Cat-vLLM README, Layer 2 "D256 Split-D": the head is
 *    processed as two 128-wide halves; "GQA Multi-Head Packing": six query
 *    heads per KV head) is taken by every entry point, with any group size G
 *    from 1 to 16.  There the decode family (plc_attn_decode_partials,
 *    plc_attn_decode_paged, plc_attn_decode_append, plc_attn_verify_paged,
 *    plc_attn_window_paged) writes partials and merges them in a second
 *    kernel (the one of plc_lse_merge), as it does at head_dim 128.
 *  - fp32 outputs `out` of the decode family and every workspace start on a
 *    16-byte boundary (PLC_ERR_INVALID_ARG otherwise; any hipMalloc'ed
 *    buffer does).
 */
#ifndef PLC_H
#define PLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLC_ABI_VERSION 3u

/*
 * Every decode-family workspace (plc_attn_decode_paged / _append / _partials,
 * plc_attn_verify_paged, plc_attn_window_paged) holds the partial outputs fp32
 * [rows][nparts][head_dim] at offset 0, then the partial LSEs fp32
 * [rows][nparts] at the next 256-byte boundary.  Its contents need no
 * initialization and are scratch between calls; calls that share a
 * workspace must not overlap in time.  The merged calls run two kernels on
 * `stream`: the partitions, then the merge of plc_lse_merge, which the kernel
 * boundary orders after every partial is written.
 */

/* KV storage types. */
#define PLC_KV_FP16 0 /* fp16 values as is */
#define PLC_KV_E4M3 1 /* OCP E4M3FN codes; value = decode(code) * scale[kv_head] */
#define PLC_KV_INT8 2 /* int8 codes; value = code * scale[block][kv_head][slot] */

/* Status codes. */
#define PLC_OK 0
#define PLC_ERR_INVALID_ARG (-1) /* null pointer, bad size, inconsistent shape */
#define PLC_ERR_UNSUPPORTED (-2) /* dtype / head_dim / block_size / group size not built */
#define PLC_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define PLC_ERR_HIP (-4)         /* a kernel launch failed */

/*
 * A paged KV cache (the struct itself is read on the host).
 *  k_cache, v_cache (device): [num_blocks][num_kv_heads][block_size][head_dim]
 *      elements of 1 byte (E4M3, INT8) or 2 bytes (FP16).
 *  k_scale, v_scale (device):
 *      E4M3: fp32 [num_kv_heads], read-only, strictly required (no implied 1.0);
 *      INT8: fp32 [num_blocks][num_kv_heads][block_size], written by
 *            plc_kv_append_quant and read by attention;
 *      FP16: unused, may be NULL.
 *  Slots no sequence owns may hold anything (NaN included): no result depends
 *  on them.
 */
typedef struct plc_kv_cache {
    void* k_cache;
    void* v_cache;
    float* k_scale;
    float* v_scale;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
} plc_kv_cache;

/* ABI version the library was built with; bindings refuse a mismatch. */
uint32_t plc_abi_version(void);

/* Message for the last non-zero status returned on this thread. */
const char* plc_last_error(void);

/*
 * Append new tokens' K and V to the cache, quantizing to kv->dtype (ReVolta
 * README, "Weight and KV formats"; 1Cat-vLLM README, Layer 1).
 *  k_new, v_new (device): fp16 [total_new_tokens][num_kv_heads][head_dim];
 *      tokens packed sequence after sequence.
 *  block_tables (device): int32 [num_seqs][max_blocks] physical block ids.
 *  cu_new_lens (device): int32 [num_seqs + 1] prefix sums of new tokens;
 *      cu_new_lens[num_seqs] must equal total_new_tokens.
 *  start_pos (device): int32 [num_seqs] tokens already cached per sequence.
 * Token t of sequence b (cu_new_lens[b] <= t < cu_new_lens[b+1]) goes to
 * position p = start_pos[b] + t - cu_new_lens[b], i.e. block
 * block_tables[b][p / block_size], slot p % block_size.
 * E4M3: code = nearest E4M3FN value to x / k_scale[h] (fp32 division), ties to
 *       even, magnitudes above 448 saturate to 448, NaN stays NaN.
 * INT8: sigma = max_d |x_d| / 127 per (token, head); code = clamp(rint(x /
 *       sigma), -127, 127) in fp32 (ties to even); sigma stored in the scale
 *       array at the token's slot; an all-zero row stores sigma 0, codes 0.
 *       Attention folds 64 * sigma_v into the fp16 probability operand, so
 *       every finite fp16 value row (sigma <= 65504/127) stays in fp16 range
 *       (64 * 515.8 < 65504); a scale array written by other means must keep
 *       sigma <= 1023 for the same reason.
 * FP16: copied.  A block id outside [0, num_blocks) skips that write.
 */
int plc_kv_append_quant(const plc_kv_cache* kv, const void* k_new, const void* v_new,
                        const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* cu_new_lens, const int32_t* start_pos,
                        int32_t num_seqs, int32_t total_new_tokens, void* stream);

/*
 * Causal prefill over the paged cache, in chunks after a cached prefix
 * (1Cat-vLLM README, Layer 2: "N32 Online Softmax", "GQA Multi-Head
 * Packing", "Wide QK / PV", "Prefix / Causal-Tail Separation").
 *  q (device): fp16 [total_q_tokens][num_q_heads][head_dim], packed by sequence.
 *  cu_q_lens (device): int32 [num_seqs + 1]; context_lens (device): int32
 *      [num_seqs] = cached + new tokens.  The new tokens' K/V must already be
 *      appended.  Query row i of sequence b sits at position
 *      context_lens[b] - n_b + i and attends to keys 0 .. that position.
 *  max_q_len (host): bound on n_b; max_context_len (host): bound on
 *      context_lens[b]; it must not exceed max_blocks * block_size.
 *  out (device): fp32 [total_q_tokens][num_q_heads][head_dim];
 *  lse (device): fp32 [total_q_tokens][num_q_heads], natural-log
 *      log-sum-exp of sm_scale * q . k over the visible keys.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
int plc_attn_prefill_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* cu_q_lens, const int32_t* context_lens,
                           int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                           int32_t max_context_len, float sm_scale, float* out, float* lse,
                           void* stream);

/*
 * Workspace bytes plc_attn_decode_paged / _append / _partials need: partial
 * outputs fp32 [num_seqs * num_q_heads][nparts][head_dim] and partial LSEs
 * fp32 [num_seqs * num_q_heads][nparts] (nparts = ceil(max_context_len /
 * partition); twice that when the grid would fit in half the chip, which
 * then streams each partition with two workgroups), each region 256-byte
 * aligned.
 * partition_tokens = 0 picks the default partition for max_context_len
 * (plc_decode_partition_tokens).
 */
size_t plc_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);

/* The partition size partition_tokens = 0 resolves to. */
int32_t plc_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_context_len, int32_t partition_tokens);

/*
 * Split-KV decode for one new query token per sequence (1Cat-vLLM README,
 * "128-bit Loads"; Layer 2 "Split-KV3").
 *  q (device): fp16 [num_seqs][num_q_heads][head_dim].
 *  context_lens (device): int32 [num_seqs], the query token's own K/V
 *      included (append first); the query attends to every cached token.
 *  partition_tokens: keys per split partition, a multiple of block_size;
 *      partitions start at multiples of it; 0 = default.
 *  out (device): fp32 [num_seqs][num_q_heads][head_dim]; lse (device): fp32
 *      [num_seqs][num_q_heads].  A sequence of length 0 gives out 0, lse -inf.
 *  workspace (device): at least plc_decode_workspace_size(...) bytes.  Calls
 *      that share a workspace must not overlap in time.
 * Two kernels: each partition writes its partial state, then the merge
 * combines them into out / lse.  With a single partition per sequence the
 * partition kernel writes out / lse itself and no merge runs.
 */
int plc_attn_decode_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * One decode step: append each sequence's step token and attend, the append
 * fused into the partition kernel.
 * Same result, bit for bit, as plc_kv_append_quant of k_new / v_new at
 * position context_lens[b] - 1 (one token per sequence) followed by
 * plc_attn_decode_paged with the same arguments.
 *  k_new, v_new (device): fp16 [num_seqs][num_kv_heads][head_dim], the K/V of
 *      the token each query belongs to.  A sequence with context 0 appends
 *      nothing.
 * The partition that holds position context_lens[b] - 1 writes the token
 * before reading its pages; no other partition reads that page.
 */
int plc_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                           int32_t num_q_heads, const plc_kv_cache* kv,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * plc_attn_decode_append for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without a workspace.  The
 * library's own device scratch of PLC_NOALLOC_SCRATCH_BYTES stands in for it
 * (held by every device the library runs on until the process ends); its
 * address is looked up on the first call on each device.  The call allocates
 * nothing, and the scratch needs no initialization.
 *  A call that needs more than PLC_NOALLOC_SCRATCH_BYTES
 *      (plc_decode_workspace_size > it) returns PLC_ERR_WORKSPACE.
 *  Every call on one device shares that device's scratch: calls that overlap
 *      in time on one device (other streams, other threads) race and give
 *      wrong results; serialize them.
 */
#define PLC_NOALLOC_SCRATCH_BYTES (16 << 20)
int plc_attn_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                   int32_t num_q_heads, const plc_kv_cache* kv,
                                   const int32_t* block_tables, int32_t max_blocks,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                                   float* out, float* lse, void* stream);

/*
 * Verification decode (speculative decoding: the target model scores several
 * drafted tokens per sequence in one step; ReVolta 0.1.2 release notes, the
 * DFlash2 settings that verify 3, 4 or 7 drafts per request; 1Cat-vLLM README,
 * installation check of the grouped-verify maximum query length).  Each
 * sequence b has n_b = cu_q_lens[b+1] - cu_q_lens[b] query tokens, in
 * [0, max_q_len], already appended as its last n_b positions; row j of b
 * attends causally to keys 0 .. context_lens[b] - n_b + j (the chunked-prefill
 * rule of plc_attn_prefill_paged), computed split-KV over partition_tokens
 * and merged as plc_attn_decode_paged does.  With n_b = 1
 * for every b it computes what plc_attn_decode_paged computes.
 *  q (device): fp16 [total_q_tokens][num_q_heads][head_dim], sequence b's
 *      tokens at rows cu_q_lens[b] ..; out fp32 [total_q_tokens][num_q_heads]
 *      [head_dim], lse fp32 [total_q_tokens][num_q_heads].
 *  cu_q_lens (device): int32 [num_seqs + 1], nondecreasing, cu_q_lens[0] = 0,
 *      cu_q_lens[num_seqs] = total_q_tokens (trusted, like context_lens).
 *  max_q_len (host): bound on every n_b, 1 .. PLC_VERIFY_MAX_Q_LEN (larger
 *      counts are a prefill: PLC_ERR_INVALID_ARG); n_b above it is clamped.
 *  partition_tokens: as for plc_attn_decode_paged (0 = automatic).
 *  workspace: plc_verify_workspace_size bytes.
 * With more than 64 rows per (sequence, KV head) (max_q_len x the group
 * size) of an E4M3 or INT8 cache, more than 32 at head_dim 256, or more than
 * 32 of an FP16 cache at head_dim 128, the rows run as 128-row tiles of the
 * prefill kernel over key partitions (an explicit
 * partition_tokens is rounded up to a multiple of 32; 0 sizes them for
 * about one workgroup per compute unit), merged as above; the results obey
 * the same bounds.
 * A row whose causal range holds no key (n_b > context_lens[b]) gets out 0
 * and lse -inf.  Calls that share a workspace must not overlap.
 */
#define PLC_VERIFY_MAX_Q_LEN 16
/* Capability query: the largest max_q_len plc_attn_verify_paged and
 * plc_attn_window_paged take (PLC_VERIFY_MAX_Q_LEN of the built library; the
 * pages' installation check prints the grouped-verify maximum query length,
 * 1Cat-vLLM README, "Installation"). */
int32_t plc_verify_max_query_tokens(void);
size_t plc_verify_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                                 int32_t max_context_len, int32_t partition_tokens);
int plc_attn_verify_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                          const int32_t* context_lens, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t partition_tokens,
                          float sm_scale, float* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Sliding-window attention of a few query tokens per sequence (the draft
 * model's attention: 1Cat-vLLM README, "DFlash2 Long-Context Decay", whose
 * loop starts at the first tile the window uses; ReVolta 0.1.2 release notes,
 * the DFlash2 drafter's 8-token blocks and 2048-token window).  Arguments and
 * results as plc_attn_verify_paged, except that the row at position pos
 * attends to keys max(0, pos - window_tokens + 1) .. pos only (window_tokens
 * 0: no window, which is plc_attn_verify_paged).  Only the partitions that
 * hold a row's window are computed, so the cost follows the window, not the
 * context; the automatic partition size follows the window too.
 *  workspace: plc_window_workspace_size bytes.
 */
size_t plc_window_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                                 int32_t max_context_len, int32_t window_tokens,
                                 int32_t partition_tokens);
int plc_attn_window_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                          const int32_t* context_lens, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t window_tokens,
                          int32_t partition_tokens, float sm_scale, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * First half of plc_attn_decode_paged: per-partition normalized outputs and
 * LSEs into the workspace, laid out as plc_lse_merge reads them (o_parts at
 * offset 0, lse_parts at *lse_parts_offset bytes, nparts in *nparts).
 * Partitions past a sequence's end hold o = 0, lse = -inf.  Lets a caller
 * merge partials from several sources (e.g. key shards on other devices).
 */
int plc_attn_decode_partials(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                             const int32_t* block_tables, int32_t max_blocks,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                             void* workspace, size_t workspace_bytes, int32_t* nparts,
                             size_t* lse_parts_offset, void* stream);

/*
 * Merge partial attention states of the same rows computed over disjoint key
 * sets (1Cat-vLLM README, Layer 2: "Split-KV3", "Prefix / Causal-Tail
 * Separation"): M = max_k lse_k, w_k = exp(lse_k - M),
 * out = sum_k w_k o_k / sum_k w_k, lse_out = M + ln sum_k w_k; parts with
 * lse = -inf carry no weight; all-empty rows give out 0, lse -inf.  Parts are
 * summed in index order.
 *  o_parts (device): fp32 [rows][nparts][head_dim]; lse_parts (device): fp32
 *  [rows][nparts]; out (device): fp32 [rows][head_dim]; lse_out (device):
 *  fp32 [rows].  head_dim 1..512, nparts >= 1.
 */
int plc_lse_merge(const float* o_parts, const float* lse_parts, int32_t rows, int32_t nparts,
                  int32_t head_dim, float* out, float* lse_out, void* stream);

/*
 * Diagnostic: the kernels' E4M3 -> fp16 conversion applied to n codes.
 *  codes (device): uint8 [n]; out (device): fp16 bits [n].  Exact: every
 *  finite E4M3FN value is an fp16 value.
 */
int plc_debug_e4m3_to_f16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PLC_H */
