// C ABI of libplc: host-side validation and dispatch.  Every check runs on the
// host before anything is enqueued and uses host-visible arguments only; the
// library refuses rather than guesses (a missing E4M3 scale is an error, not
// an implied 1.0: ReVolta README, "E4M3 KV"; a context longer than the block
// table can hold is rejected: ReVolta README, "Performance" and "Support and
// limits").
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/plc.h"
#include "plc_internal.h"

// Device scratch of plc_attn_decode_append_noalloc: the decode workspace
// (partial outputs, partial LSEs) for callers that cannot
// allocate one.  Every device the library runs on holds its own copy until
// the process ends.  In host code this name is only a handle for
// hipGetSymbolAddress; kernels get the device address it returns.
static __device__ __align__(256) unsigned char scratch[PLC_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

constexpr int kHeadDim = 128;       // every entry point
constexpr int kHeadDimWide = 256;   // KV append and one-token decode (split in two 128 halves)
constexpr int kBlockSize = 16;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_cache(const plc_kv_cache* kv) {
    if (!kv) return fail(PLC_ERR_INVALID_ARG, "kv cache descriptor is NULL");
    if (kv->dtype != PLC_KV_FP16 && kv->dtype != PLC_KV_E4M3 && kv->dtype != PLC_KV_INT8)
        return fail(PLC_ERR_UNSUPPORTED, "kv dtype %d is not one of FP16(0), E4M3(1), INT8(2)",
                    kv->dtype);
    if (kv->head_dim != kHeadDim && kv->head_dim != kHeadDimWide)
        return fail(PLC_ERR_UNSUPPORTED, "head_dim %d: kernels are built for %d and %d", kv->head_dim,
                    kHeadDim, kHeadDimWide);
    if (kv->block_size != kBlockSize)
        return fail(PLC_ERR_UNSUPPORTED, "block_size %d: kernels are built for %d", kv->block_size,
                    kBlockSize);
    if (kv->num_blocks <= 0 || kv->num_kv_heads <= 0)
        return fail(PLC_ERR_INVALID_ARG, "num_blocks %d / num_kv_heads %d must be positive",
                    kv->num_blocks, kv->num_kv_heads);
    if (!kv->k_cache || !kv->v_cache) return fail(PLC_ERR_INVALID_ARG, "k_cache / v_cache is NULL");
    if (kv->dtype != PLC_KV_FP16 && (!kv->k_scale || !kv->v_scale))
        return fail(PLC_ERR_INVALID_ARG,
                    "%s cache without %s scales: scales are required, never assumed 1.0",
                    kv->dtype == PLC_KV_E4M3 ? "E4M3" : "INT8",
                    kv->dtype == PLC_KV_E4M3 ? "per-head" : "per-token");
    return PLC_OK;
}

int check_heads(int32_t num_q_heads, const plc_kv_cache* kv) {
    if (num_q_heads <= 0 || num_q_heads % kv->num_kv_heads != 0)
        return fail(PLC_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    num_q_heads, kv->num_kv_heads);
    const int G = num_q_heads / kv->num_kv_heads;
    if (kv->head_dim == kHeadDimWide) {
        // the wide decode packs the group into one 16-column MFMA tile
        if (G > 16) return fail(PLC_ERR_UNSUPPORTED, "GQA group size %d: head_dim 256 supports 1..16", G);
        return PLC_OK;
    }
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(PLC_ERR_UNSUPPORTED, "GQA group size %d: supported are 1, 2, 4, 8, 16", G);
    return PLC_OK;
}


int check_lengths(int32_t num_seqs, int32_t max_blocks, int32_t max_context_len, int32_t block_size) {
    if (num_seqs <= 0) return fail(PLC_ERR_INVALID_ARG, "num_seqs %d must be positive", num_seqs);
    if (max_blocks <= 0) return fail(PLC_ERR_INVALID_ARG, "max_blocks %d must be positive", max_blocks);
    if (max_context_len < 0)
        return fail(PLC_ERR_INVALID_ARG, "max_context_len %d is negative", max_context_len);
    if ((int64_t)max_context_len > (int64_t)max_blocks * block_size)
        return fail(PLC_ERR_INVALID_ARG,
                    "max_context_len %d exceeds the block table's capacity %lld (%d blocks of %d)",
                    max_context_len, (long long)max_blocks * block_size, max_blocks, block_size);
    return PLC_OK;
}

plc::KvView view(const plc_kv_cache* kv) {
    plc::KvView v;
    v.k = kv->k_cache;
    v.v = kv->v_cache;
    v.k_scale = kv->k_scale;
    v.v_scale = kv->v_scale;
    v.num_blocks = kv->num_blocks;
    v.num_kv_heads = kv->num_kv_heads;
    v.head_dim = kv->head_dim;
    v.dtype = kv->dtype;
    return v;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(PLC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return PLC_OK;
}

// Workspace layout of the decode family: the partial outputs, then the
// partial LSEs.
void set_workspace(plc::DecodeParams* p, void* ws, size_t rows, int32_t nparts, int32_t head_dim) {
    char* base = static_cast<char*>(ws);
    const size_t o_bytes = align_up(rows * nparts * head_dim * sizeof(float));
    p->o_parts = reinterpret_cast<float*>(base);
    p->lse_parts = reinterpret_cast<float*>(base + o_bytes);
}

size_t partial_bytes(size_t rows, int64_t nparts, int32_t head_dim) {
    return align_up(rows * nparts * head_dim * sizeof(float)) + align_up(rows * nparts * sizeof(float));
}

// A merged launch of at most this many workgroup slots (rounded units of
// eight (sequence, KV head) groups x workgroup columns x partitions) leaves
// compute units idle on the 256-CU chip; the launcher then streams each
// partition with two workgroups, and the workspace holds partials for 2 nparts.
bool may_split_partitions(int64_t units, int32_t ncgw, int64_t nparts, int32_t partition_tokens) {
    return ((units + 7) / 8) * 8 * ncgw * nparts * 2 <= 256 && partition_tokens % 64 == 0 &&
           partition_tokens >= 512;
}

// Partial bytes of a decode-family call: doubled partitions when the launch
// may split them.
size_t decode_partial_bytes(size_t rows, int64_t units, int32_t ncgw, int64_t nparts, int32_t partition_tokens,
                            int32_t head_dim) {
    const bool split = may_split_partitions(units, ncgw, nparts, partition_tokens);
    return partial_bytes(rows, split ? 2 * nparts : nparts, head_dim);
}

// the kernels store 16-byte vectors to out and the workspace
int check_aligned(const void* ptr, const char* what) {
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
        return fail(PLC_ERR_INVALID_ARG, "%s at %p is not 16-byte aligned", what, ptr);
    return PLC_OK;
}

int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t partition_tokens, int32_t min_tokens = 512) {
    if (partition_tokens > 0) return partition_tokens;
    // The shortest power of two in [min_tokens, 8192] that keeps the grid
    // within about one workgroup per compute unit (256 CUs): each workgroup
    // then streams a long run of pages, and the merge reads few partials.
    const int64_t groups = (int64_t)num_seqs * num_kv_heads;
    int32_t p = min_tokens;
    while (p < 8192 && groups * ((max_context_len + p - 1) / p) > 256) p *= 2;
    return p;
}

int decode_setup(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                 const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                 int32_t num_seqs, int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                 void* workspace, size_t workspace_bytes, plc::DecodeParams* out) {
    int rc;
    if ((rc = check_cache(kv))) return rc;
    if ((rc = check_heads(num_q_heads, kv))) return rc;
    if ((rc = check_lengths(num_seqs, max_blocks, max_context_len, kv->block_size))) return rc;
    if (!q || !block_tables || !context_lens)
        return fail(PLC_ERR_INVALID_ARG, "q / block_tables / context_lens is NULL");
    if (partition_tokens < 0 || partition_tokens % kv->block_size != 0)
        return fail(PLC_ERR_INVALID_ARG, "partition_tokens %d must be 0 or a multiple of block_size %d",
                    partition_tokens, kv->block_size);
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(PLC_ERR_INVALID_ARG, "sm_scale must be positive and finite");
    const int32_t P = resolve_partition(num_seqs, kv->num_kv_heads, max_context_len, partition_tokens);
    const size_t need = plc_decode_workspace_size(num_seqs, num_q_heads, kv->head_dim,
                                                  max_context_len, P);
    if (!workspace || workspace_bytes < need)
        return fail(PLC_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                    workspace_bytes, workspace, need);
    if ((rc = check_aligned(workspace, "workspace"))) return rc;
    const int32_t nparts = max_context_len > 0 ? (max_context_len + P - 1) / P : 1;
    const size_t rows = (size_t)num_seqs * num_q_heads;
    plc::DecodeParams& p = *out;
    p.q = q;
    p.kv = view(kv);
    p.block_tables = block_tables;
    p.max_blocks = max_blocks;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.max_context_len = max_context_len;
    p.partition_tokens = P;
    p.nparts = nparts;
    p.qk_scale_log2 = sm_scale * 1.4426950408889634f;
    set_workspace(&p, workspace, rows, nparts, kv->head_dim);
    p.may_split = workspace_bytes >= partial_bytes(rows, 2 * (int64_t)nparts, kv->head_dim) ? 1 : 0;
    if (p.may_split) set_workspace(&p, workspace, rows, 2 * nparts, kv->head_dim);
    p.merge = 0;
    p.direct = 0;
    p.xcd_local = 0;
    p.out = nullptr;
    p.lse = nullptr;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.cu_q_lens = nullptr;
    p.max_q_len = 1;
    p.ncg = 1;
    p.window = 0;
    p.total_q_tokens = num_seqs;
    return PLC_OK;
}

// rows of one (sequence, KV head) in groups of 16, one workgroup column each
int32_t verify_row_groups(int32_t num_q_heads, int32_t num_kv_heads, int32_t max_q_len) {
    return (max_q_len * (num_q_heads / num_kv_heads) + 15) / 16;
}

// Partition size and partitions per sequence for a few-query-token call.
// Without a window the keys are the whole context.  With one, a sequence's
// rows need at most window + max_q_len - 1 keys, which touch at most one
// partition more than they fill; the default size follows that span.
void mq_partitions(int32_t groups, int32_t num_kv_heads, int32_t max_q_len, int32_t max_context_len,
                   int32_t window, int32_t partition_tokens, int32_t* P, int32_t* nparts) {
    const int64_t span = window > 0 ? std::min<int64_t>(max_context_len, (int64_t)window + max_q_len - 1)
                                    : max_context_len;
    // a window's few thousand keys: partitions down to 256 tokens, measured
    // 20 % faster than 512 for 8-token blocks over a 2048-token window
    *P = resolve_partition(groups, num_kv_heads, (int32_t)span, partition_tokens, window > 0 ? 256 : 512);
    const int64_t all = max_context_len > 0 ? (max_context_len + *P - 1) / *P : 1;
    *nparts = (int32_t)(window > 0 ? std::min<int64_t>(all, (span + *P - 1) / *P + 1) : all);
    if (*nparts < 1) *nparts = 1;
}

// Calls with a few query tokens per sequence whose rows of one (sequence, KV
// head) (drafted positions x heads) exceed a few 16-row groups run as the
// 128-row tiles of the prefill DMA kernel over key partitions, merged
// afterwards: a tile shares each K and V subtile among 128 rows where a
// decode workgroup shares it among 16 or 32.  Calls without a window, 8-bit
// caches at head dims 128 and 256, FP16 at 128 (windows, and FP16 at 256,
// keep the decode kernel).  The row counts above which tiles win, measured
// over 8 x 32K contexts:
// - E4M3, head dim 128 (G = 8): 64 rows 28.9 us by the decode kernel against
//   34.3 by tiles, 80 rows 42.8 against 35.3, 128 rows 43.8 against 38.1;
// - E4M3, head dim 256 (G = 6): 24 rows 69 against 89, 48 rows 123 against
//   94, 96 rows 227 against 98;
// - FP16, head dim 128 (G = 8): 24 rows 34.6 against 38.8, 32 rows 34.9
//   against 38.0, 48 rows 51.9 against 38.3, 64 rows 51.3 against 38.9, 128
//   rows 87.7 against 42.7.
constexpr int32_t kTileRows = 128;

int64_t tile_row_threshold(int32_t dtype, int32_t head_dim) {
    if (head_dim == kHeadDimWide) return dtype == PLC_KV_FP16 ? INT64_MAX : 32;
    return dtype == PLC_KV_FP16 ? 32 : 64;
}

bool tile_eligible(int32_t dtype, int32_t head_dim, int32_t window, int32_t max_q_len, int32_t group) {
    return window == 0 && (int64_t)max_q_len * group > tile_row_threshold(dtype, head_dim);
}

// Key partitions of the tile path: an explicit size rounded up to whole
// 32-key subtiles, else the shortest multiple of 32 keys (at least 256) that
// keeps the grid within about one workgroup per compute unit (measured at 16
// drafts over 8 x 32K: 37.8 us with 1024-key partitions and one workgroup
// per CU, 40.4 with 512 and two: two tiles on a CU share its SIMDs no faster
// than one, and the partials double).
void tile_partitions(int64_t tiles, int32_t max_context_len, int32_t partition_tokens, int32_t* P,
                     int32_t* nparts) {
    int64_t p;
    if (partition_tokens > 0) {
        p = ((int64_t)partition_tokens + 31) / 32 * 32;
    } else {
        const int64_t want = std::max<int64_t>(1, (256 + tiles - 1) / tiles);
        p = std::max<int64_t>(256, ((max_context_len + want - 1) / want + 31) / 32 * 32);
    }
    *P = (int32_t)p;
    *nparts = max_context_len > 0 ? (int32_t)((max_context_len + p - 1) / p) : 1;
}

// (sequence, KV head, 128-row tile) units of a tile-path call
int64_t tile_units(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_q_len) {
    const int64_t G = num_q_heads / num_kv_heads;
    return (int64_t)num_seqs * num_kv_heads * ((max_q_len * G + kTileRows - 1) / kTileRows);
}

// Per-device address of `scratch`, looked up on the first call on each
// device, with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PLC_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                       "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PLC_OK;
}

}  // namespace

extern "C" {

uint32_t plc_abi_version(void) { return PLC_ABI_VERSION; }

const char* plc_last_error(void) { return g_err; }

int plc_kv_append_quant(const plc_kv_cache* kv, const void* k_new, const void* v_new,
                        const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* cu_new_lens, const int32_t* start_pos, int32_t num_seqs,
                        int32_t total_new_tokens, void* stream) {
    int rc;
    if ((rc = check_cache(kv))) return rc;
    if (num_seqs <= 0) return fail(PLC_ERR_INVALID_ARG, "num_seqs %d must be positive", num_seqs);
    if (max_blocks <= 0) return fail(PLC_ERR_INVALID_ARG, "max_blocks %d must be positive", max_blocks);
    if (total_new_tokens < 0)
        return fail(PLC_ERR_INVALID_ARG, "total_new_tokens %d is negative", total_new_tokens);
    if (total_new_tokens == 0) return PLC_OK;
    if (!k_new || !v_new || !block_tables || !cu_new_lens || !start_pos)
        return fail(PLC_ERR_INVALID_ARG, "k_new / v_new / block_tables / cu_new_lens / start_pos is NULL");
    if ((int64_t)total_new_tokens * kv->num_kv_heads * 2 * 16 > ((int64_t)1 << 40))
        return fail(PLC_ERR_INVALID_ARG, "total_new_tokens %d too large", total_new_tokens);
    plc::AppendParams p;
    p.kv = view(kv);
    p.k_new = k_new;
    p.v_new = v_new;
    p.block_tables = block_tables;
    p.max_blocks = max_blocks;
    p.cu_new_lens = cu_new_lens;
    p.start_pos = start_pos;
    p.num_seqs = num_seqs;
    p.total_new_tokens = total_new_tokens;
    return hip_status(plc::launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv_append_quant launch");
}

int plc_attn_prefill_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* cu_q_lens, const int32_t* context_lens,
                           int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                           int32_t max_context_len, float sm_scale, float* out, float* lse,
                           void* stream) {
    int rc;
    if ((rc = check_cache(kv))) return rc;
    if ((rc = check_heads(num_q_heads, kv))) return rc;
    if ((rc = check_lengths(num_seqs, max_blocks, max_context_len, kv->block_size))) return rc;
    if (total_q_tokens < 0 || max_q_len < 0)
        return fail(PLC_ERR_INVALID_ARG, "total_q_tokens %d / max_q_len %d is negative",
                    total_q_tokens, max_q_len);
    if (max_q_len > max_context_len)
        return fail(PLC_ERR_INVALID_ARG, "max_q_len %d exceeds max_context_len %d", max_q_len,
                    max_context_len);
    if (total_q_tokens == 0 || max_q_len == 0) return PLC_OK;
    if (!q || !block_tables || !cu_q_lens || !context_lens || !out || !lse)
        return fail(PLC_ERR_INVALID_ARG, "q / block_tables / cu_q_lens / context_lens / out / lse is NULL");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(PLC_ERR_INVALID_ARG, "sm_scale must be positive and finite");
    plc::PrefillParams p;
    p.q = q;
    p.kv = view(kv);
    p.block_tables = block_tables;
    p.max_blocks = max_blocks;
    p.cu_q_lens = cu_q_lens;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.max_q_len = max_q_len;
    p.max_context_len = max_context_len;
    p.qk_scale_log2 = sm_scale * 1.4426950408889634f;
    p.out = out;
    p.lse = lse;
    p.partition_tokens = 0;
    p.nparts = 1;
    p.o_parts = nullptr;
    p.lse_parts = nullptr;
    if (kv->head_dim == kHeadDimWide)
        return hip_status(plc::launch_prefill256(p, static_cast<hipStream_t>(stream)), "prefill launch");
    return hip_status(plc::launch_prefill(p, static_cast<hipStream_t>(stream)), "prefill launch");
}

int32_t plc_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                    int32_t partition_tokens) {
    return resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_tokens);
}

size_t plc_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
    // the default partition shrinks as (sequence, KV head) groups get fewer;
    // sizing with one KV head gives the shortest partition, so the bound holds
    // for every head count
    const int32_t P = partition_tokens > 0
                          ? partition_tokens
                          : resolve_partition(num_seqs, 1, max_context_len, 0);
    const int64_t nparts = max_context_len > 0 ? (max_context_len + P - 1) / P : 1;
    const size_t rows = (size_t)num_seqs * num_q_heads;
    // partial outputs and partial LSEs; sized for one KV
    // head (the fewest units, so the split partitions whenever they may occur)
    return decode_partial_bytes(rows, num_seqs, 1, nparts, P, head_dim);
}

int plc_attn_decode_partials(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                             const int32_t* block_tables, int32_t max_blocks,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                             void* workspace, size_t workspace_bytes, int32_t* nparts,
                             size_t* lse_parts_offset, void* stream) {
    plc::DecodeParams p;
    int rc = decode_setup(q, num_q_heads, kv, block_tables, max_blocks, context_lens, num_seqs,
                          max_context_len, partition_tokens, sm_scale, workspace, workspace_bytes, &p);
    if (rc) return rc;
    if (nparts) *nparts = p.nparts;
    if (lse_parts_offset)
        *lse_parts_offset = (size_t)(reinterpret_cast<char*>(p.lse_parts) - static_cast<char*>(workspace));
    return hip_status(plc::launch_decode_partials(p, static_cast<hipStream_t>(stream)),
                      "decode partition launch");
}

int plc_attn_decode_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                          int32_t partition_tokens, float sm_scale, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
    plc::DecodeParams p;
    int rc = decode_setup(q, num_q_heads, kv, block_tables, max_blocks, context_lens, num_seqs,
                          max_context_len, partition_tokens, sm_scale, workspace, workspace_bytes, &p);
    if (rc) return rc;
    if (!out || !lse) return fail(PLC_ERR_INVALID_ARG, "out / lse is NULL");
    if ((rc = check_aligned(out, "out"))) return rc;
    p.merge = 1;
    p.out = out;
    p.lse = lse;
    return hip_status(plc::launch_decode_partials(p, static_cast<hipStream_t>(stream)),
                      "decode launch");
}

int plc_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                           int32_t num_q_heads, const plc_kv_cache* kv,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t partition_tokens, float sm_scale, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
    plc::DecodeParams p;
    int rc = decode_setup(q, num_q_heads, kv, block_tables, max_blocks, context_lens, num_seqs,
                          max_context_len, partition_tokens, sm_scale, workspace, workspace_bytes, &p);
    if (rc) return rc;
    if (!out || !lse) return fail(PLC_ERR_INVALID_ARG, "out / lse is NULL");
    if (!k_new || !v_new) return fail(PLC_ERR_INVALID_ARG, "k_new / v_new is NULL");
    if ((rc = check_aligned(out, "out"))) return rc;
    p.merge = 1;
    p.out = out;
    p.lse = lse;
    p.k_new = k_new;
    p.v_new = v_new;
    return hip_status(plc::launch_decode_partials(p, static_cast<hipStream_t>(stream)),
                      "decode-append launch");
}

int plc_attn_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                   int32_t num_q_heads, const plc_kv_cache* kv,
                                   const int32_t* block_tables, int32_t max_blocks,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t partition_tokens, float sm_scale,
                                   float* out, float* lse, void* stream) {
    if (!kv) return fail(PLC_ERR_INVALID_ARG, "kv cache descriptor is NULL");
    const size_t need = plc_decode_workspace_size(num_seqs, num_q_heads, kv->head_dim, max_context_len,
                                                  partition_tokens);
    if (need == 0) return fail(PLC_ERR_INVALID_ARG, "num_seqs %d / num_q_heads %d / max_context_len %d",
                               num_seqs, num_q_heads, max_context_len);
    if (need > (size_t)PLC_NOALLOC_SCRATCH_BYTES)
        return fail(PLC_ERR_WORKSPACE,
                    "this decode needs %zu bytes of scratch; the no-allocation entry point has %d "
                    "(use plc_attn_decode_append with a workspace)",
                    need, PLC_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const int rc = scratch_for_current_device(&ws);
    if (rc) return rc;
    return plc_attn_decode_append(q, k_new, v_new, num_q_heads, kv, block_tables, max_blocks, context_lens,
                                  num_seqs, max_context_len, partition_tokens, sm_scale, out, lse, ws,
                                  PLC_NOALLOC_SCRATCH_BYTES, stream);
}

size_t plc_window_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                                 int32_t max_context_len, int32_t window_tokens,
                                 int32_t partition_tokens) {
    if (num_seqs <= 0 || total_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_q_len < 1 ||
        max_q_len > PLC_VERIFY_MAX_Q_LEN || max_context_len < 0 || window_tokens < 0 ||
        partition_tokens < 0)
        return 0;
    const int32_t ncg = verify_row_groups(num_q_heads, num_kv_heads, max_q_len);
    int32_t P = 0, nparts = 0;
    mq_partitions(num_seqs * ncg, num_kv_heads, max_q_len, max_context_len, window_tokens,
                  partition_tokens, &P, &nparts);
    const size_t rows = (size_t)total_q_tokens * num_q_heads;
    // partial outputs and LSEs per query row
    // workgroup columns per (sequence, KV head): the launcher's grid
    const int32_t rg = plc::groups_per_workgroup(head_dim, true, ncg, P);
    size_t need = decode_partial_bytes(rows, (int64_t)num_seqs * num_kv_heads, (ncg + rg - 1) / rg, nparts,
                                       P, head_dim);
    // the cache's dtype is not an argument: room for the tile path of any dtype
    const int32_t group = num_q_heads / num_kv_heads;
    if (tile_eligible(PLC_KV_FP16, head_dim, window_tokens, max_q_len, group) ||
        tile_eligible(PLC_KV_E4M3, head_dim, window_tokens, max_q_len, group)) {
        int32_t Pt = 0, npt = 0;
        tile_partitions(tile_units(num_seqs, num_q_heads, num_kv_heads, max_q_len), max_context_len,
                        partition_tokens, &Pt, &npt);
        need = std::max(need, partial_bytes(rows, npt, head_dim));
    }
    return need;
}

size_t plc_verify_workspace_size(int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                                 int32_t max_context_len, int32_t partition_tokens) {
    return plc_window_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads, head_dim,
                                     max_q_len, max_context_len, 0, partition_tokens);
}

int plc_attn_window_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                          const int32_t* context_lens, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t window_tokens,
                          int32_t partition_tokens, float sm_scale, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int rc;
    if ((rc = check_cache(kv))) return rc;
    if ((rc = check_heads(num_q_heads, kv))) return rc;
    if ((rc = check_lengths(num_seqs, max_blocks, max_context_len, kv->block_size))) return rc;
    if (total_q_tokens < 0)
        return fail(PLC_ERR_INVALID_ARG, "total_q_tokens %d is negative", total_q_tokens);
    if (max_q_len < 1 || max_q_len > PLC_VERIFY_MAX_Q_LEN)
        return fail(PLC_ERR_INVALID_ARG, "max_q_len %d outside [1, %d]: longer chunks are prefill",
                    max_q_len, PLC_VERIFY_MAX_Q_LEN);
    if (max_q_len > max_context_len)
        return fail(PLC_ERR_INVALID_ARG, "max_q_len %d exceeds max_context_len %d", max_q_len,
                    max_context_len);
    if (window_tokens < 0)
        return fail(PLC_ERR_INVALID_ARG, "window_tokens %d is negative (0: no window)", window_tokens);
    if (total_q_tokens == 0) return PLC_OK;
    if (!q || !block_tables || !cu_q_lens || !context_lens || !out || !lse)
        return fail(PLC_ERR_INVALID_ARG, "q / block_tables / cu_q_lens / context_lens / out / lse is NULL");
    if (partition_tokens < 0 || partition_tokens % kv->block_size != 0)
        return fail(PLC_ERR_INVALID_ARG, "partition_tokens %d must be 0 or a multiple of block_size %d",
                    partition_tokens, kv->block_size);
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(PLC_ERR_INVALID_ARG, "sm_scale must be positive and finite");
    const size_t rows = (size_t)total_q_tokens * num_q_heads;
    if (tile_eligible(kv->dtype, kv->head_dim, window_tokens, max_q_len, num_q_heads / kv->num_kv_heads)) {
        int32_t Pt = 0, npt = 0;
        tile_partitions(tile_units(num_seqs, num_q_heads, kv->num_kv_heads, max_q_len), max_context_len,
                        partition_tokens, &Pt, &npt);
        const size_t need = partial_bytes(rows, npt, kv->head_dim);
        if (!workspace || workspace_bytes < need)
            return fail(PLC_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                        workspace_bytes, workspace, need);
        if ((rc = check_aligned(workspace, "workspace")) || (rc = check_aligned(out, "out"))) return rc;
        plc::PrefillParams t;
        t.q = q;
        t.kv = view(kv);
        t.block_tables = block_tables;
        t.max_blocks = max_blocks;
        t.cu_q_lens = cu_q_lens;
        t.context_lens = context_lens;
        t.num_seqs = num_seqs;
        t.num_q_heads = num_q_heads;
        t.max_q_len = max_q_len;
        t.max_context_len = max_context_len;
        t.qk_scale_log2 = sm_scale * 1.4426950408889634f;
        t.out = nullptr;
        t.lse = nullptr;
        t.partition_tokens = Pt;
        t.nparts = npt;
        char* base = static_cast<char*>(workspace);
        t.o_parts = reinterpret_cast<float*>(base);
        t.lse_parts = reinterpret_cast<float*>(base + align_up(rows * npt * kv->head_dim * sizeof(float)));
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if ((rc = hip_status(plc::launch_prefill_dma(t, s), "verify tile launch"))) return rc;
        return hip_status(plc::launch_lse_merge(t.o_parts, t.lse_parts, (int32_t)rows, npt, kv->head_dim, out,
                                                lse, s),
                          "verify merge launch");
    }
    const int32_t ncg = verify_row_groups(num_q_heads, kv->num_kv_heads, max_q_len);
    int32_t P = 0, nparts = 0;
    mq_partitions(num_seqs * ncg, kv->num_kv_heads, max_q_len, max_context_len, window_tokens,
                  partition_tokens, &P, &nparts);
    const int32_t rg = plc::groups_per_workgroup(kv->head_dim, true, ncg, P);
    const size_t need = decode_partial_bytes(rows, (int64_t)num_seqs * kv->num_kv_heads, (ncg + rg - 1) / rg,
                                             nparts, P, kv->head_dim);
    if (!workspace || workspace_bytes < need)
        return fail(PLC_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                    workspace_bytes, workspace, need);
    if ((rc = check_aligned(workspace, "workspace")) || (rc = check_aligned(out, "out"))) return rc;
    plc::DecodeParams p;
    p.q = q;
    p.kv = view(kv);
    p.block_tables = block_tables;
    p.max_blocks = max_blocks;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.max_context_len = max_context_len;
    p.partition_tokens = P;
    p.nparts = nparts;
    p.qk_scale_log2 = sm_scale * 1.4426950408889634f;
    set_workspace(&p, workspace, rows, nparts, kv->head_dim);
    p.may_split = workspace_bytes >= partial_bytes(rows, 2 * (int64_t)nparts, kv->head_dim) ? 1 : 0;
    if (p.may_split) set_workspace(&p, workspace, rows, 2 * nparts, kv->head_dim);
    p.merge = 1;
    p.direct = 0;
    p.xcd_local = 0;
    p.out = out;
    p.lse = lse;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.cu_q_lens = cu_q_lens;
    p.max_q_len = max_q_len;
    p.ncg = ncg;
    p.window = window_tokens;
    p.total_q_tokens = total_q_tokens;
    return hip_status(plc::launch_decode_partials(p, static_cast<hipStream_t>(stream)),
                      window_tokens > 0 ? "window launch" : "verify launch");
}

int plc_attn_verify_paged(const void* q, int32_t num_q_heads, const plc_kv_cache* kv,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                          const int32_t* context_lens, int32_t num_seqs, int32_t total_q_tokens,
                          int32_t max_q_len, int32_t max_context_len, int32_t partition_tokens,
                          float sm_scale, float* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return plc_attn_window_paged(q, num_q_heads, kv, block_tables, max_blocks, cu_q_lens, context_lens,
                                 num_seqs, total_q_tokens, max_q_len, max_context_len, 0,
                                 partition_tokens, sm_scale, out, lse, workspace, workspace_bytes,
                                 stream);
}

int plc_lse_merge(const float* o_parts, const float* lse_parts, int32_t rows, int32_t nparts,
                  int32_t head_dim, float* out, float* lse_out, void* stream) {
    if (rows < 0 || nparts < 1 || head_dim < 1 || head_dim > 512)
        return fail(PLC_ERR_INVALID_ARG, "rows %d / nparts %d / head_dim %d out of range", rows,
                    nparts, head_dim);
    if (rows == 0) return PLC_OK;
    if (!o_parts || !lse_parts || !out || !lse_out)
        return fail(PLC_ERR_INVALID_ARG, "o_parts / lse_parts / out / lse_out is NULL");
    return hip_status(plc::launch_lse_merge(o_parts, lse_parts, rows, nparts, head_dim, out, lse_out,
                                            static_cast<hipStream_t>(stream)),
                      "lse merge launch");
}

int32_t plc_verify_max_query_tokens(void) { return PLC_VERIFY_MAX_Q_LEN; }

int plc_debug_e4m3_to_f16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream) {
    if (n < 0) return fail(PLC_ERR_INVALID_ARG, "n %d is negative", n);
    if (n == 0) return PLC_OK;
    if (!codes || !out) return fail(PLC_ERR_INVALID_ARG, "codes / out is NULL");
    return hip_status(plc::launch_debug_e4m3(codes, out, n, static_cast<hipStream_t>(stream)),
                      "debug e4m3 launch");
}

}  // extern "C"
