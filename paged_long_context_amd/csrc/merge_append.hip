// LSE merge of partial attention states, KV append with quantization, and the
// E4M3 conversion diagnostic, for gfx950.
#include "plc_device.h"
#include "plc_internal.h"

namespace plc {
namespace {

// ------------------------------------------------------------------ merge
//
// One wave per (row, 64-column slice); lane l owns column 64 * slice + l.
// Parts are visited in index order (1Cat-vLLM README, Layer 2 "Split-KV3": the
// fp32 partial states of the partitions are combined), so the result does not
// depend on how the rows are scheduled.  Parts come in batches of up to 64:
// lane k loads part k's LSE while every part's value of the batch is loaded
// in the same round trip; lane k then computes part k's weight against the
// batch maximum and readlane hands it to every lane.  A later batch (more
// than 64 parts) rescales the running sums to its larger maximum.
// one wave per workgroup: a step's few hundred merge rows spread over as many
// compute units (measured faster than four waves per workgroup)
constexpr int kMergeWavesPerBlock = 1;

template <int KB>
__device__ __forceinline__ void merge_batch(const float* lp, const float* op, int kb, int kn, int D,
                                            int lane, float& M, float& acc, float& wsum) {
    const float NEG = -__builtin_inff();
    float ov[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) ov[u] = op[(int64_t)(kb + (u < kn ? u : 0)) * D];
    const float lk = lane < kn ? lp[kb + lane] : NEG;
    // all of the batch's loads in one round trip: without this the compiler
    // sinks the value loads behind the LSE reduction
#pragma unroll
    for (int u = 0; u < KB; ++u) pin(ov[u]);
    float mb = lk;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, shfl_xor(mb, off));
    mb = fmaxf(mb, M);
    if (mb == NEG) return;                             // nothing visible yet
    const float sc = (M == NEG) ? 0.0f : fast_exp2((M - mb) * kLog2e);
    acc *= sc;
    wsum *= sc;
    const float wl = (lk == NEG) ? 0.0f : fast_exp2((lk - mb) * kLog2e);
#pragma unroll
    for (int u = 0; u < KB; ++u)
        if (u < kn) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), u));
            wsum += w;
            acc += w * ov[u];
        }
    M = mb;
}

__global__ __launch_bounds__(64 * kMergeWavesPerBlock) void lse_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int rows, int nparts,
    int D, float* __restrict__ out, float* __restrict__ lse_out) {
    const int lane = threadIdx.x & 63;
    const int nslice = (D + 63) / 64;
    const int wv = blockIdx.x * kMergeWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = wv / nslice, slice = wv - row * nslice;
    if (row >= rows) return;
    const int d = 64 * slice + lane;
    const bool dv = d < D;
    const float* lp = lse_parts + (int64_t)row * nparts;
    const float* op = o_parts + (int64_t)row * nparts * D + (dv ? d : 0);
    float M = -__builtin_inff(), acc = 0.0f, wsum = 0.0f;
    for (int kb = 0; kb < nparts; kb += 64) {
        const int kn = min(64, nparts - kb);
        if (kn > 32) merge_batch<64>(lp, op, kb, kn, D, lane, M, acc, wsum);
        else if (kn > 16) merge_batch<32>(lp, op, kb, kn, D, lane, M, acc, wsum);
        else merge_batch<16>(lp, op, kb, kn, D, lane, M, acc, wsum);
    }
    const bool empty = !(wsum > 0.0f);
    if (dv) out[(int64_t)row * D + d] = empty ? 0.0f : acc / wsum;
    if (slice == 0 && lane == 0) lse_out[row] = empty ? -__builtin_inff() : M + __builtin_logf(wsum);
}

// Head dims 128 and 256: one wave per row.  Lane (h, c) = (l / 32, l % 32)
// takes the parts of parity h and columns 4c + 128s + [0,4) (s < D / 128),
// so one load instruction moves the pieces of two adjacent parts (contiguous
// in o_parts) and a batch of 32 parts is 16 such loads per column block, all
// in one round trip.  Lane k (mod 32) loads part k's LSE and computes its
// weight against the batch maximum; readlane hands the weights of parts 2j
// and 2j + 1 to every lane, which keeps its parity's.  The even and odd
// parities are summed separately, each in index order, and added at the end.
template <int D>
__global__ __launch_bounds__(64) void lse_merge_rows_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int rows, int nparts,
    float* __restrict__ out, float* __restrict__ lse_out) {
    constexpr int NS = D / 128;
    constexpr int KB = 32;                             // parts per batch
    const int lane = threadIdx.x, h = lane >> 5, c = lane & 31;
    const int row = blockIdx.x;
    if (row >= rows) return;
    const float NEG = -__builtin_inff();
    const float* lp = lse_parts + (int64_t)row * nparts;
    const float* op = o_parts + (int64_t)row * nparts * D + 4 * c;
    float M = NEG, wsum = 0.0f;
    f32x4 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < nparts; kb += KB) {
        const int kn = min(KB, nparts - kb);
        // this lane's parts kb + 2j + h (a part past the batch reads part kb
        // and gets weight 0)
        f32x4 ov[KB / 2][NS];
#pragma unroll
        for (int j = 0; j < KB / 2; ++j) {
            const int k = (2 * j + h < kn) ? kb + 2 * j + h : kb;
#pragma unroll
            for (int s = 0; s < NS; ++s) ov[j][s] = *reinterpret_cast<const f32x4*>(op + (int64_t)k * D + 128 * s);
        }
        const float lk = c < kn ? lp[kb + c] : NEG;
        // all of the batch's loads in one round trip
#pragma unroll
        for (int j = 0; j < KB / 2; ++j)
#pragma unroll
            for (int s = 0; s < NS; ++s) pin(ov[j][s]);
        float mb = lk;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) mb = fmaxf(mb, shfl_xor(mb, off));
        mb = fmaxf(mb, M);
        if (mb == NEG) continue;                       // nothing visible yet
        const float sc = (M == NEG) ? 0.0f : fast_exp2((M - mb) * kLog2e);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s] *= sc;
        wsum *= sc;
        const float wl = (lk == NEG) ? 0.0f : fast_exp2((lk - mb) * kLog2e);
#pragma unroll
        for (int j = 0; j < KB / 2; ++j)
            if (2 * j < kn) {
                const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), 2 * j));
                const float w1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), 2 * j + 1));
                const float w = (2 * j + h < kn) ? (h ? w1 : w0) : 0.0f;
                wsum += w;
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s] += w * ov[j][s];
            }
        M = mb;
    }
    // the two parities' sums, even first (every lane takes part in each
    // exchange: a permute reads nothing from lanes outside the exec mask)
    const float wother = shfl_xor(wsum, 32);
    const float wtot = h ? wother + wsum : wsum + wother;
    const bool empty = !(wtot > 0.0f);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float other = shfl_xor(acc[s][e], 32);
            o[e] = h ? other + acc[s][e] : acc[s][e] + other;
        }
        if (h == 0) *reinterpret_cast<f32x4*>(out + (int64_t)row * D + 128 * s + 4 * c) = empty ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : o / wtot;
    }
    if (lane == 0) lse_out[row] = empty ? NEG : M + __builtin_logf(wtot);
}

// ------------------------------------------------------------------ append
//
// D / 8 lanes (16 for head dim 128, 32 for 256) per (token, KV head, K-or-V)
// row of D fp16 values, eight values per lane (one 16-byte load).  E4M3 divides by the head's scale in
// IEEE fp32 and rounds to nearest-even; INT8 takes the row's absolute maximum
// across the row's lanes first (ReVolta README, "INT8 KV": scales per token
// and head at run time).
constexpr int kAppendThreads = 256;

template <int KV, int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
    constexpr int BS = 16, LPR = D / 8, LSH = (D == 256) ? 5 : 4;
    static_assert(LPR == 1 << LSH, "lanes per row");
    const int64_t gid = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int Hkv = p.kv.num_kv_heads;
    const int64_t row = gid >> LSH;               // (token, head, kv) row
    const int part = (int)(gid & (LPR - 1));      // 8-value slice of the row
    const int64_t nrows = (int64_t)p.total_new_tokens * Hkv * 2;
    const bool live = row < nrows;
    const int64_t r = live ? row : 0;
    const int which = (int)(r & 1);               // 0: K, 1: V
    const int h = (int)((r >> 1) % Hkv);
    const int t = (int)((r >> 1) / Hkv);

    // sequence of token t: last b with cu_new_lens[b] <= t
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu_new_lens[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int pos = p.start_pos[b] + (t - p.cu_new_lens[b]);
    const int lb = pos / BS;
    int blk = (lb >= 0 && lb < p.max_blocks) ? p.block_tables[(int64_t)b * p.max_blocks + lb] : -1;
    const bool ok = live && blk >= 0 && blk < p.kv.num_blocks && pos >= 0;
    const int slot = pos - lb * BS;

    const f16* src = static_cast<const f16*>(which ? p.v_new : p.k_new) +
                     ((int64_t)t * Hkv + h) * D + 8 * part;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
    const f16x8 x = __builtin_bit_cast(f16x8, raw);
    const int64_t crow = ((int64_t)(ok ? blk : 0) * Hkv + h) * BS + slot;

    if constexpr (KV == KV_FP16) {
        if (ok) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(const_cast<void*>(
                    which ? p.kv.v : p.kv.k)) + crow * D + 8 * part) = raw;
    } else {
        float s = 1.0f, sigma = 0.0f;
        if constexpr (KV == KV_E4M3) s = (which ? p.kv.v_scale : p.kv.k_scale)[h];
        const u32x2 w = quantize_slice<KV, LPR>(x, s, sigma);
        if (ok) {
            *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(const_cast<void*>(
                which ? p.kv.v : p.kv.k)) + crow * D + 8 * part) = w;
            if constexpr (KV == KV_INT8)
                if (part == 0) const_cast<float*>(which ? p.kv.v_scale : p.kv.k_scale)[crow] = sigma;
        }
    }
}

__global__ void debug_e4m3_kernel(const uint8_t* codes, uint16_t* out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const f16x2 v = e4m3x2_to_f16x2<false>((uint32_t)codes[i]);
    out[i] = __builtin_bit_cast(uint16_t, v[0]);
}

}  // namespace

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t rows,
                            int32_t nparts, int32_t head_dim, float* out, float* lse_out,
                            hipStream_t s) {
    if (rows == 0) return hipSuccess;
    // the one-wave-per-row kernel moves 16-byte pieces: taken when both
    // value arrays are 16-byte aligned (every workspace and decode-family
    // output is; plc_lse_merge callers may pass any float pointers)
    const bool aligned = ((reinterpret_cast<uintptr_t>(o_parts) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    if (aligned && (head_dim == 128 || head_dim == 256)) {
        if (head_dim == 128)
            hipLaunchKernelGGL((lse_merge_rows_kernel<128>), dim3(rows), dim3(64), 0, s, o_parts, lse_parts, rows,
                               nparts, out, lse_out);
        else
            hipLaunchKernelGGL((lse_merge_rows_kernel<256>), dim3(rows), dim3(64), 0, s, o_parts, lse_parts, rows,
                               nparts, out, lse_out);
        return hipGetLastError();
    }
    const int64_t waves = (int64_t)rows * ((head_dim + 63) / 64);
    dim3 grid((unsigned)((waves + kMergeWavesPerBlock - 1) / kMergeWavesPerBlock));
    hipLaunchKernelGGL(lse_merge_kernel, grid, dim3(64 * kMergeWavesPerBlock), 0, s, o_parts, lse_parts, rows,
                       nparts, head_dim, out, lse_out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_kv_append_d(const AppendParams& p, hipStream_t s) {
    const int64_t threads = (int64_t)p.total_new_tokens * p.kv.num_kv_heads * 2 * (D / 8);
    if (threads == 0) return hipSuccess;
    dim3 grid((unsigned)((threads + kAppendThreads - 1) / kAppendThreads));
    switch (p.kv.dtype) {
    case KV_FP16: hipLaunchKernelGGL((kv_append_kernel<KV_FP16, D>), grid, dim3(kAppendThreads), 0, s, p); break;
    case KV_E4M3: hipLaunchKernelGGL((kv_append_kernel<KV_E4M3, D>), grid, dim3(kAppendThreads), 0, s, p); break;
    case KV_INT8: hipLaunchKernelGGL((kv_append_kernel<KV_INT8, D>), grid, dim3(kAppendThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
    switch (p.kv.head_dim) {
    case 128: return launch_kv_append_d<128>(p, s);
    case 256: return launch_kv_append_d<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_debug_e4m3(const uint8_t* codes, uint16_t* out, int32_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(debug_e4m3_kernel, dim3((n + 255) / 256), dim3(256), 0, s, codes, out, n);
    return hipGetLastError();
}

}  // namespace plc
