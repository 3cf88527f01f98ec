// Chunked causal prefill over the paged KV cache, for gfx950.
//
// Workgroup = 8 waves = 256 query rows of one KV head; a row is a (query
// position, query head) pair, positions outer, so the G query heads that read
// one KV head share every K/V tile (1Cat-vLLM README, Layer 2 "GQA Multi-Head
// Packing").  Each wave owns one 32-row MFMA tile and keeps its Q operands and
// O accumulators in registers for the whole key loop; at about 210 VGPRs two
// waves share each SIMD, so one wave's softmax overlaps the other's MFMAs.
//
// Keys are walked in tiles of 64 (four 16-token pages).  Per tile four of the
// waves gather the pages' codes with 16- and 8-byte loads (one page id per
// page), convert them to fp16 exactly and write K as [key][d] (two LDS
// buffers) and V already transposed as [d][key] (three); the next tile's loads are
// in flight while the current tile is computed (Layer 1 and the
// "Software-Reconstructed Async" section describe the same goals with V100
// means).  Each wave then forms S^T = K Q^T on 32x32x16 f16 MFMA with fp32
// accumulation, runs the online softmax per query row in fp32 (Layer 2 "N32
// Online Softmax"; "Performance First": fp32 QK/PV), and accumulates
// O^T = V^T P^T on MFMA ("Wide QK / PV").  Tiles wholly below the chunk's first
// position skip the causal mask; only the tiles at the diagonal apply it
// (Layer 2 "Prefix / Causal-Tail Separation").
#include <type_traits>

#include "plc_device.h"
#include "plc_internal.h"

namespace plc {
namespace {

constexpr int D = 128;
constexpr int BS = 16;
constexpr int KT = 64;                  // keys per tile
constexpr int KSTR = D;                 // K row stride in LDS (halves), swizzled
constexpr int VSTR = KT + 8;            // V^T row stride in LDS (halves)
constexpr int KBUF = KT * KSTR;         // halves
constexpr int VBUF = D * VSTR;          // halves

// Which key MFMA row rho of S^T holds (within a 64-key tile): the swap of
// bits 2 and 3 makes the eight keys a lane owns for one PV step consecutive.
// K is stored in LDS in MFMA row order, so LDS row rho holds key
// key_of_row(rho) (the map is its own inverse).
__device__ __forceinline__ int key_of_row(int rho) {
    return (rho & 0x33) | ((rho & 0x8) >> 1) | ((rho & 0x4) << 1);
}

// K rows are 256 bytes without padding; the 16-byte chunk c of row rho lives
// at chunk slot c ^ 2(c >> 3) ^ (rho & 15).  Operand reads (lanes = 16
// consecutive rows, one chunk) and staging writes (lanes = 4 rows x 4 chunks
// 4q + i) then touch 16 distinct slots, so neither conflicts on LDS banks.
__device__ __forceinline__ int k_slot(int c, int rho) { return c ^ (2 * (c >> 3)) ^ (rho & 15); }

// Staging: the first half of the workgroup's threads gathers a tile's K, the
// second half its V, 256 threads each.  A K thread holds key t>>2,
// d = 32(t&3) + [0,32); a V thread holds keys 4(t&15) + [0,4), d = 8(t>>4) + [0,8)
// (t = thread index within its half).  Either way a thread carries 32 codes.
template <int KV>
struct Stage {
    // K: raw[j] = d chunk j (16 B each).  V: FP16 raw[e] = key e; 8-bit codes
    // raw[e>>1] holds key e in dwords 2(e&1) + [0,2).
    u32x4 raw[(KV == KV_FP16) ? 4 : 2];
    float sc[4];                                     // INT8 scales: K sc[0], V sc[0..3]
};

// The page id the thread's first key lives on, or -1 past the visible keys.
__device__ __forceinline__ int stage_page(const int32_t* bt, bool is_k, int k0, int kend, int t) {
    const int key = k0 + (is_k ? (t >> 2) : 4 * (t & 15));
    return key < kend ? bt[key / BS] : -1;
}

template <int KV>
__device__ __forceinline__ void stage_load(Stage<KV>& st, const PrefillParams& p, bool is_k, int kvh,
                                           int k0, int kend, int pg, int t) {
    constexpr int EB = (KV == KV_FP16) ? 2 : 1;
    const int Hkv = p.kv.num_kv_heads;
    const bool pgok = pg >= 0 && pg < p.kv.num_blocks;
    const int64_t pb = pgok ? pg : 0;
    if (is_k) {
        const int key = k0 + (t >> 2);
        const bool ok = pgok && key < kend;
        const int64_t row = (pb * Hkv + kvh) * BS + (key & (BS - 1));
        const uint8_t* src = static_cast<const uint8_t*>(p.kv.k) + (row * D + 32 * (t & 3)) * EB;
#pragma unroll
        for (int j = 0; j < ((KV == KV_FP16) ? 4 : 2); ++j)
            st.raw[j] = ok ? *reinterpret_cast<const u32x4*>(src + 16 * j) : u32x4{0, 0, 0, 0};
        if constexpr (KV == KV_INT8) st.sc[0] = ok ? p.kv.k_scale[row] : 0.0f;
    } else {
        // four consecutive keys share one page (4 | 16)
        const int key0 = k0 + 4 * (t & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = key0 + e;
            const bool ok = pgok && key < kend;
            const int64_t row = (pb * Hkv + kvh) * BS + (key & (BS - 1));
            const uint8_t* src = static_cast<const uint8_t*>(p.kv.v) + (row * D + 8 * (t >> 4)) * EB;
            if constexpr (KV == KV_FP16) {
                st.raw[e] = ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
            } else {
                const u32x2 c = ok ? *reinterpret_cast<const u32x2*>(src) : u32x2{0, 0};
                st.raw[e >> 1][2 * (e & 1)] = c[0];
                st.raw[e >> 1][2 * (e & 1) + 1] = c[1];
            }
            if constexpr (KV == KV_INT8) st.sc[e] = ok ? p.kv.v_scale[row] : 0.0f;
        }
    }
}

template <int KV>
__device__ __forceinline__ void stage_store(const Stage<KV>& st, bool is_k, f16* lk, f16* lv,
                                            float* lks, float* lvs, int t) {
    if (is_k) {   // K -> LDS row key_of_row(key), chunks 4q + [0,4) at their swizzled slots
        const int rho = key_of_row(t >> 2), q = t & 3;
        f16* dst = lk + rho * KSTR;
        if constexpr (KV == KV_FP16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x4*>(dst + 8 * k_slot(4 * q + j, rho)) = st.raw[j];
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<f16x8*>(dst + 8 * k_slot(4 * q + 2 * j, rho)) =
                    codes8_to_f16x8<KV>(st.raw[j][0], st.raw[j][1]);
                *reinterpret_cast<f16x8*>(dst + 8 * k_slot(4 * q + 2 * j + 1, rho)) =
                    codes8_to_f16x8<KV>(st.raw[j][2], st.raw[j][3]);
            }
        }
        if constexpr (KV == KV_INT8)
            if ((t & 3) == 0) lks[t >> 2] = st.sc[0];
    } else {      // V -> [d][key]: row 8(t>>4) + col, keys 4(t&15) + [0,4); the 16 lanes
                  // of a write cover one row's 64 keys, so the writes do not conflict
        f16* dst = lv + (8 * (t >> 4)) * VSTR + 4 * (t & 15);
        if constexpr (KV == KV_FP16) {
#pragma unroll
            for (int col = 0; col < 8; ++col) {
                const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
                u32x2 r;
                r[0] = __builtin_amdgcn_perm(st.raw[1][col >> 1], st.raw[0][col >> 1], sel);
                r[1] = __builtin_amdgcn_perm(st.raw[3][col >> 1], st.raw[2][col >> 1], sel);
                *reinterpret_cast<u32x2*>(dst + col * VSTR) = r;
            }
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f16x2 pr[2][4];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    // keys 2pp and 2pp + 1, dword hf of each
                    const uint32_t a = st.raw[pp][2 + hf], b = st.raw[pp][hf];
                    const uint32_t p01 = __builtin_amdgcn_perm(a, b, 0x05010400u);
                    const uint32_t p23 = __builtin_amdgcn_perm(a, b, 0x07030602u);
                    pr[pp][0] = codes2_to_f16x2<KV, false>(p01);
                    pr[pp][1] = codes2_to_f16x2<KV, true>(p01);
                    pr[pp][2] = codes2_to_f16x2<KV, false>(p23);
                    pr[pp][3] = codes2_to_f16x2<KV, true>(p23);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f16x4*>(dst + (4 * hf + c) * VSTR) =
                        f16x4{pr[0][c][0], pr[0][c][1], pr[1][c][0], pr[1][c][1]};
            }
        }
        if constexpr (KV == KV_INT8)
            if ((t >> 4) == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lvs[4 * (t & 15) + e] = st.sc[e];
            }
    }
}

// RT 32-row MFMA tiles per wave, NWAVE waves: 32 * RT * NWAVE query rows per
// workgroup.
template <int KV, int RT, int NWAVE>
__global__ __launch_bounds__(64 * NWAVE) void prefill_kernel(PrefillParams p) {
    constexpr int ROWS = 32 * RT * NWAVE;
    constexpr int NT = 64 * NWAVE;                   // threads
    // K double-buffered, V triple-buffered: the last subtile's PV of tile j
    // runs in iteration j + 1, while tile j + 2 is being staged
    __shared__ __attribute__((aligned(16))) f16 s_k[2][KBUF];
    __shared__ __attribute__((aligned(16))) f16 s_v[3][VBUF];
    __shared__ float s_ks[2][KT], s_vs[3][KT];

    const int tile = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = p.num_q_heads, G = Hq / p.kv.num_kv_heads;
    const int qa = p.cu_q_lens[b];
    // lengths beyond the host-stated bounds are clamped so that no page id
    // outside the table is ever read
    const int L = max(0, min(p.context_lens[b], p.max_context_len));
    const int n = min(min(p.cu_q_lens[b + 1] - qa, p.max_q_len), L);
    const int ppw = ROWS / G;                        // positions per workgroup
    const int q0 = tile * ppw;
    if (q0 >= n) return;
    const int base = L - n;                          // position of the chunk's first token
    const int qlast = min(q0 + ppw, n) - 1;
    const int kend = base + qlast + 1;               // keys [0, kend) are visible to someone
    const int kfull = base + q0 + 1;                 // keys [0, kfull) are visible to every row
    const int ntiles = (kend + KT - 1) / KT;
    const int nfull = kfull / KT;                    // tiles needing no mask
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;

    // ---- Q operands: lane holds row l%32 of row-tile rt, d = 16kc + 8(l/32) + [0,8)
    const int h32 = lane >> 5, r32 = lane & 31;
    f16x8 qop[RT][8];
    int rowpos[RT];
    int64_t rowid[RT];
    bool rowok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 32 * RT * wave + 32 * rt + r32;
        const int po = q0 + r / G;
        rowok[rt] = po < n;
        const int poc = rowok[rt] ? po : qlast;
        rowpos[rt] = base + poc;
        rowid[rt] = (int64_t)(qa + poc) * Hq + kvh * G + (r % G);
        const f16* q = static_cast<const f16*>(p.q) + rowid[rt] * D + 8 * h32;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) qop[rt][kc] = *reinterpret_cast<const f16x8*>(q + 16 * kc);
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / 256.0f;

    float m_ref[RT], l_run[RT];                       // raw-score units
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_ref[rt] = -__builtin_inff();
        l_run[rt] = 0.0f;
    }
    const float grow_raw = (KV == KV_INT8) ? 0.0f : 8.0f / cscale;
    f32x16 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rt][dt][r] = 0.0f;

    // waves 0-3 stage K, waves 4-7 stage V
    static_assert(NT == 512, "staging assumes 256 K threads and 256 V threads");
    const bool is_k = wave < NWAVE / 2;
    const int st_t = tid & 255;
    Stage<KV> st;
    int pg_next = stage_page(bt, is_k, 0, kend, st_t);
    stage_load<KV>(st, p, is_k, kvh, 0, kend, pg_next, st_t);
    if (ntiles > 1) pg_next = stage_page(bt, is_k, KT, kend, st_t);
    stage_store<KV>(st, is_k, s_k[0], s_v[0], s_ks[0], s_vs[0], st_t);
    for (int x = tid; x < VBUF / 8; x += NT)          // the zeroed V buffer the first PV reads
        reinterpret_cast<f16x8*>(s_v[2])[x] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    __syncthreads();

    // Subtile pipeline: for each 32-key subtile, QK^T first, then the PV of
    // the previous subtile (its MFMAs run while this subtile's softmax runs on
    // the vector unit), then the softmax.  The previous subtile's P operands
    // and V buffer are carried across iterations; before the first subtile
    // they are zeros and a zeroed V buffer, so the PV step has no branch.
    f16x8 pprev[RT][2];                               // [rt][half] of the pending subtile
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) pprev[rt][hf] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    int pv_buf = 2, pv_ks = 0;
    auto pv = [&](int vb, int kss) __attribute__((always_inline)) {
        const f16* lv = s_v[vb];
        f16x8 va[4][2];                               // all V operands first
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                va[dt][hf] = *reinterpret_cast<const f16x8*>(lv + (32 * dt + r32) * VSTR + 8 * h32 +
                                                             32 * kss + 16 * hf);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = mfma32(va[dt][hf], pprev[rt][hf], acc[rt][dt]);
    };

    const int kslot = h32 ^ (r32 & 15);              // lane part of the K chunk slot
    // One key tile; MASKED tiles (at the diagonal) compare each key with the
    // row's position, the others skip the mask entirely.
    auto run_tile = [&](auto mtag, int j) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        const int k0 = j * KT;
        const int kb = j & 1, vb = j % 3;
        if (j + 1 < ntiles) {
            stage_load<KV>(st, p, is_k, kvh, k0 + KT, kend, pg_next, st_t);
            if (j + 2 < ntiles) pg_next = stage_page(bt, is_k, k0 + 2 * KT, kend, st_t);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // S^T[key][row] of this subtile
            f32x16 sc[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 16; ++r) sc[rt][r] = 0.0f;
            // MFMA row r32 is LDS row 32ks + r32; its chunk 2kc + h32 sits at
            // slot (2kc ^ 2(kc >> 2)) ^ h32 ^ (r32 & 15)
            const f16* krp = s_k[kb] + (32 * ks + r32) * KSTR;
            f16x8 ka[8];                              // all of the subtile's K operands first,
#pragma unroll                                        // so the LDS latency is paid once
            for (int kc = 0; kc < 8; ++kc)
                ka[kc] = *reinterpret_cast<const f16x8*>(krp + 8 * ((2 * kc ^ 2 * (kc >> 2)) ^ kslot));
#pragma unroll
            for (int kc = 0; kc < 8; ++kc)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) sc[rt] = mfma32(ka[kc], qop[rt][kc], sc[rt]);
            pv(pv_buf, pv_ks);

            f16x8 pnew[RT][2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // raw scores (INT8: times the key's scale), masked keys at -inf
                float mx = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v = sc[rt][r];
                    if constexpr (KV == KV_INT8) v *= s_ks[kb][32 * ks + 16 * (r >> 3) + 8 * h32 + (r & 7)];
                    if constexpr (MASKED) {
                        const int key = k0 + 32 * ks + 16 * (r >> 3) + 8 * h32 + (r & 7);
                        v = (key <= rowpos[rt]) ? v : -__builtin_inff();
                    }
                    sc[rt][r] = v;
                    mx = fmaxf(mx, v);
                }
                mx = fmaxf(mx, shfl_xor(mx, 32));
                // The reference maximum moves only when a row's maximum grew by
                // more than grow_raw (2^8 in probability; 0 for INT8, whose P
                // carries the value scale): the accumulators are rescaled
                // rarely, not per subtile.
                const bool grow = mx > m_ref[rt] + grow_raw;
                if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
                    const float m_new = grow ? mx : m_ref[rt];
                    const float alpha = (m_ref[rt] == -__builtin_inff())
                                            ? 0.0f
                                            : fast_exp2((m_ref[rt] - m_new) * cscale);
                    l_run[rt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) acc[rt][dt] *= alpha;
                    m_ref[rt] = m_new;
                }
                // p = 2^(c*s - c*m): one fma and one exp per score
                const float moff = (m_ref[rt] == -__builtin_inff()) ? 0.0f : -m_ref[rt] * cscale;
                // l sums the fp32 p (summing the fp16-rounded weights would
                // leave up to 2^-11 relative error in l on short rows)
                float psum = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pe = fast_exp2(__builtin_fmaf(sc[rt][r], cscale, moff));
                    psum += pe;
                    if constexpr (KV == KV_INT8)   // P carries each key's value scale
                        pe *= s_vs[vb][32 * ks + 16 * (r >> 3) + 8 * h32 + (r & 7)] * 256.0f;
                    pnew[rt][r >> 3][r & 7] = (f16)pe;
                }
                l_run[rt] += psum;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) pprev[rt][hf] = pnew[rt][hf];
            pv_buf = vb;
            pv_ks = ks;
        }
        if (j + 1 < ntiles)
            stage_store<KV>(st, is_k, s_k[kb ^ 1], s_v[(j + 1) % 3], s_ks[kb ^ 1], s_vs[(j + 1) % 3], st_t);
        __syncthreads();
    };
    const int nunmasked = min(nfull, ntiles);
    for (int j = 0; j < nunmasked; ++j) run_tile(std::false_type{}, j);
    for (int j = nunmasked; j < ntiles; ++j) run_tile(std::true_type{}, j);
    pv(pv_buf, pv_ks);

    // ---- epilogue: lanes l and l^32 hold halves of the same row's keys
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float l = l_run[rt] + shfl_xor(l_run[rt], 32);
        if (!rowok[rt]) continue;
        const float inv = vscale / l;
        float* o = p.out + rowid[rt] * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = 32 * dt + 8 * a4 + 4 * h32;
                f32x4 v = f32x4{acc[rt][dt][4 * a4 + 0], acc[rt][dt][4 * a4 + 1],
                                acc[rt][dt][4 * a4 + 2], acc[rt][dt][4 * a4 + 3]} * inv;
                *reinterpret_cast<f32x4*>(o + d) = v;
            }
        if (h32 == 0) p.lse[rowid[rt]] = (m_ref[rt] * cscale + __builtin_log2f(l)) * kLn2;
    }
}

}  // namespace

#ifndef PLC_PREFILL_RT
#define PLC_PREFILL_RT 1          // 32-row MFMA tiles per wave
#endif
#ifndef PLC_PREFILL_NWAVE
#define PLC_PREFILL_NWAVE 8       // waves per workgroup
#endif

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
    constexpr int RT = PLC_PREFILL_RT, NW = PLC_PREFILL_NWAVE;
    const int G = p.num_q_heads / p.kv.num_kv_heads;
    const int ppw = 32 * RT * NW / G;
    dim3 grid((p.max_q_len + ppw - 1) / ppw, p.kv.num_kv_heads, p.num_seqs);
    if (grid.x == 0) return hipSuccess;
    const dim3 block(64 * NW);
    switch (p.kv.dtype) {
    case KV_FP16: hipLaunchKernelGGL((prefill_kernel<KV_FP16, RT, NW>), grid, block, 0, s, p); break;
    case KV_E4M3: hipLaunchKernelGGL((prefill_kernel<KV_E4M3, RT, NW>), grid, block, 0, s, p); break;
    case KV_INT8: hipLaunchKernelGGL((prefill_kernel<KV_INT8, RT, NW>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace plc
