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

// K rows are 256 bytes without padding; the 16-byte chunk c of row rho lives
// at chunk slot h(c) ^ g(rho), h(c) = (c >> 1) | 8(c & 1),
// g(rho) = (rho & 7) | 8((rho ^ rho >> 3) & 1).  Operand reads (lanes = 16
// consecutive rows, one chunk) and staging writes (lanes = 2 rows x 8 chunks
// 2q + i) then touch 16 distinct slots, so neither conflicts on LDS banks.
__device__ __forceinline__ int k_row_key(int rho) { return (rho & 7) | (((rho ^ (rho >> 3)) & 1) << 3); }
__device__ __forceinline__ int k_slot(int c, int rho) { return ((c >> 1) | ((c & 1) << 3)) ^ k_row_key(rho); }

// V^T staging: thread group u = t >> 4 writes d rows 4 v_group(u) + [0,4); the
// permutation puts the four 16-lane groups of a wave at row offsets 0, 32,
// 16 and 48 words modulo 64, so a write covers all banks once.
__device__ __forceinline__ int v_group(int u) { return (u & ~3) | ((u & 1) << 1) | ((u >> 1) & 1); }

// Staging: every thread of the workgroup gathers 16 codes of a tile's K (key
// t>>3, d = 16(t&7) + [0,16)) and 16 of its V (keys 4(t&15) + [0,4),
// d = 4 v_group(t>>4) + [0,4)).  Keys past kend or on an invalid page are
// zeroed when written to LDS; the loads themselves are always issued (from
// page 0 when the key is not readable), so nothing waits on them early and
// the loads in flight stay countable across the key loop.
template <int KV>
struct Stage {
    static constexpr int NW = (KV == KV_FP16) ? 8 : 4;   // words of K, and of V
    uint32_t k[NW];
    uint32_t v[NW];                                  // 8-bit: v[e] = key e; fp16: v[2e + i]
    float ks, vs[4];                                 // INT8 scales
    uint32_t ok;                                     // bit 0: K key readable; bit 4 + e: V key e
};

// Per-thread constants of the staging addresses: a code's byte offset is
// page * page_bytes + the thread's offset within a page (its keys' positions
// in the page are the same for every tile, since tiles start on page bounds).
struct StageAddr {
    int64_t page_bytes;                              // Hkv * BS * D * elem bytes
    int64_t k_off, v_off;                            // byte offsets within a page
    int32_t page_rows;                               // Hkv * BS (INT8 scale rows per page)
    int32_t ks_row, vs_row;                          // scale rows within a page
};

// The table entry of key's page, read unconditionally at an index clamped to
// the visible keys and used raw: stage_load checks it against num_blocks and
// zeroes keys past kend, so nothing consumes the load before the tile is
// staged two phases later (a select on it here would wait for the load in
// the very next phase).
__device__ __forceinline__ int page_of(const int32_t* bt, int key, int kend) {
    return bt[(uint32_t)min(key, kend - 1) / BS];
}

template <int KV>
__device__ __forceinline__ void stage_load_k(Stage<KV>& st, const PrefillParams& p, const StageAddr& sa,
                                             int key, int kend, int pg) {
    const bool pgok = pg >= 0 && pg < p.kv.num_blocks;
    const int64_t pb = pgok ? pg : 0;
    const uint8_t* src = static_cast<const uint8_t*>(p.kv.k) + pb * sa.page_bytes + sa.k_off;
#pragma unroll
    for (int j = 0; j < Stage<KV>::NW / 4; ++j) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(src + 16 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.k[4 * j + i] = c[i];
    }
    if constexpr (KV == KV_INT8) st.ks = p.kv.k_scale[pb * sa.page_rows + sa.ks_row];
    st.ok = (st.ok & ~1u) | ((pgok && key < kend) ? 1u : 0u);
}

// key0 = the first of the thread's four V keys, which share one page (4 | 16)
template <int KV>
__device__ __forceinline__ void stage_load_v(Stage<KV>& st, const PrefillParams& p, const StageAddr& sa,
                                             int key0, int kend, int pg) {
    constexpr int EB = (KV == KV_FP16) ? 2 : 1;
    const bool pgok = pg >= 0 && pg < p.kv.num_blocks;
    const int64_t pb = pgok ? pg : 0;
    const uint8_t* src = static_cast<const uint8_t*>(p.kv.v) + pb * sa.page_bytes + sa.v_off;
    uint32_t okb = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (KV == KV_FP16) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(src + e * D * EB);
            st.v[2 * e] = c[0];
            st.v[2 * e + 1] = c[1];
        } else {
            st.v[e] = *reinterpret_cast<const uint32_t*>(src + e * D * EB);
        }
        if constexpr (KV == KV_INT8) st.vs[e] = p.kv.v_scale[pb * sa.page_rows + sa.vs_row + e];
        okb |= ((pgok && key0 + e < kend) ? 1u : 0u) << e;
    }
    st.ok = (st.ok & 1u) | (okb << 4);
}

// K -> LDS row key_of_row(key), chunks 2(t&7) + [0,2) at their swizzled slots
template <int KV>
__device__ __forceinline__ void stage_store_k(const Stage<KV>& st, f16* lk, float* lks, int t) {
    const int rho = key_of_row(t >> 3), c0 = 2 * (t & 7);
    const bool ok = st.ok & 1u;
    uint32_t c[Stage<KV>::NW];
#pragma unroll
    for (int i = 0; i < Stage<KV>::NW; ++i) c[i] = ok ? st.k[i] : 0u;
    f16* dst = lk + rho * KSTR;
    if constexpr (KV == KV_FP16) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<u32x4*>(dst + 8 * k_slot(c0 + j, rho)) =
                u32x4{c[4 * j], c[4 * j + 1], c[4 * j + 2], c[4 * j + 3]};
    } else {
        *reinterpret_cast<f16x8*>(dst + 8 * k_slot(c0, rho)) = codes8_to_f16x8<KV>(c[0], c[1]);
        *reinterpret_cast<f16x8*>(dst + 8 * k_slot(c0 + 1, rho)) = codes8_to_f16x8<KV>(c[2], c[3]);
    }
    if constexpr (KV == KV_INT8)
        if ((t & 7) == 0) lks[t >> 3] = ok ? st.ks : 0.0f;
}

// V -> [d][key]: rows 4 v_group(t>>4) + [0,4), keys 4(t&15) + [0,4)
template <int KV>
__device__ __forceinline__ void stage_store_v(const Stage<KV>& st, f16* lv, float* lvs, int t) {
    f16* dst = lv + (4 * v_group(t >> 4)) * VSTR + 4 * (t & 15);
    auto okey = [&](int e) { return (st.ok >> (4 + e)) & 1u; };
    if constexpr (KV == KV_FP16) {
        uint32_t w2[4][2];                           // key e's d pairs, zeroed if unreadable
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 2; ++i) w2[e][i] = okey(e) ? st.v[2 * e + i] : 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int w = c >> 1;                    // word of each key holding the d pair
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x2 r;
            r[0] = __builtin_amdgcn_perm(w2[1][w], w2[0][w], sel);
            r[1] = __builtin_amdgcn_perm(w2[3][w], w2[2][w], sel);
            *reinterpret_cast<u32x2*>(dst + c * VSTR) = r;
        }
    } else {
        f16x2 pr[2][4];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            // keys 2pp and 2pp + 1: byte c of each is d0 + c
            const uint32_t a = okey(2 * pp + 1) ? st.v[2 * pp + 1] : 0u;
            const uint32_t b = okey(2 * pp) ? st.v[2 * pp] : 0u;
            const uint32_t p01 = __builtin_amdgcn_perm(a, b, 0x05010400u);
            const uint32_t p23 = __builtin_amdgcn_perm(a, b, 0x07030602u);
            pr[pp][0] = codes2_to_f16x2<KV, false>(p01);
            pr[pp][1] = codes2_to_f16x2<KV, true>(p01);
            pr[pp][2] = codes2_to_f16x2<KV, false>(p23);
            pr[pp][3] = codes2_to_f16x2<KV, true>(p23);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<f16x4*>(dst + c * VSTR) = f16x4{pr[0][c][0], pr[0][c][1], pr[1][c][0], pr[1][c][1]};
    }
    if constexpr (KV == KV_INT8)
        if ((t >> 4) == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) lvs[4 * (t & 15) + e] = okey(e) ? st.vs[e] : 0.0f;
        }
}

// Phase barrier: every wave of the workgroup; the scheduler moves nothing
// across it, so the MFMA and VALU phases stay as written.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// 8 waves x 32 query rows.  The waves form two groups, 0-3 and 4-7, so each
// SIMD holds one wave of each.  A step is one 32-key subtile in two phases:
// the MFMA phase (the previous subtile's V operands from LDS, S = K Q^T of
// this subtile, O += V^T P^T of the previous one, and the staging of the next
// tile's K or V between those MFMAs) and the VALU phase (this subtile's online
// softmax and the next subtile's K operands from LDS).  Both groups thus read
// LDS in every phase, which a single wave per SIMD cannot saturate.  Group 4-7 starts one barrier late, so while one
// group runs its MFMA phase the other runs its VALU phase and the two waves
// of a SIMD keep the matrix core and the vector unit busy together.
//
// Global phase g is the span between the g-th and (g+1)-th barrier after the
// first tile is staged.  Group 0-3 runs the MFMA phase of step i in phase 2i
// and its VALU phase in 2i+1; group 4-7 runs them in 2i+1 and 2i+2.
template <int KV>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillParams p) {
    constexpr int ROWS = 256;
    __shared__ __attribute__((aligned(16))) f16 s_k[2][KBUF];
    __shared__ __attribute__((aligned(16))) f16 s_v[2][VBUF];
    __shared__ float s_ks[3][KT], s_vs[2][KT];     // INT8 key scales: three buffers (see below)

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
    const int nfull = min(kfull / KT, ntiles);       // tiles needing no mask
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;
    const bool late = wave >= 4;                     // group 4-7: one phase behind

    // ---- Q operands: lane holds row l%32 of the wave's tile, d = 16kc + 8(l/32) + [0,8)
    const int h32 = lane >> 5, r32 = lane & 31;
    f16x8 qop[8];
    int rowpos;
    int64_t rowid;
    bool rowok;
    {
        const int r = 32 * wave + r32;
        const int po = q0 + r / G;
        rowok = po < n;
        const int poc = rowok ? po : qlast;
        rowpos = base + poc;
        rowid = (int64_t)(qa + poc) * Hq + kvh * G + (r % G);
        const f16* q = static_cast<const f16*>(p.q) + rowid * D + 8 * h32;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) qop[kc] = *reinterpret_cast<const f16x8*>(q + 16 * kc);
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / kInt8PFold;

    float m_ref = -__builtin_inff(), l_run = 0.0f;   // raw-score units
    const float grow_raw = (KV == KV_INT8) ? 0.0f : 8.0f / cscale;
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

    // ---- staging.  K of tile T+1 is written to LDS during the MFMA phase of
    // step 2T (phases 4T and 4T+1), V of tile T+1 during that of step 2T+1
    // (4T+2, 4T+3), each interleaved with the MFMAs and followed by the loads
    // of tile T+2.  Tile T's K operands are read in phases [4T-1, 4T+2], its V
    // operands in [4T+2, 4T+5], its K and V scales (softmax) in [4T+1, 4T+4]:
    // two K and V buffers suffice, the K scales need three.  Before the loop:
    // tile 0 in LDS, tile 1 in registers, tile 2's page ids.
    const int kkey = tid >> 3, vkey = 4 * (tid & 15);   // the thread's K key / first V key
    StageAddr sa;
    {
        constexpr int EB = (KV == KV_FP16) ? 2 : 1;
        const int Hkv = p.kv.num_kv_heads;
        sa.page_rows = Hkv * BS;
        sa.page_bytes = (int64_t)sa.page_rows * D * EB;
        sa.ks_row = kvh * BS + (kkey & (BS - 1));
        sa.vs_row = kvh * BS + (vkey & (BS - 1));
        sa.k_off = ((int64_t)sa.ks_row * D + 16 * (tid & 7)) * EB;
        sa.v_off = ((int64_t)sa.vs_row * D + 4 * v_group(tid >> 4)) * EB;
    }
    Stage<KV> st;
    st.ok = 0;
    int pgk = page_of(bt, kkey, kend), pgv = page_of(bt, vkey, kend);
    stage_load_k<KV>(st, p, sa, kkey, kend, pgk);
    stage_load_v<KV>(st, p, sa, vkey, kend, pgv);
    stage_store_k<KV>(st, s_k[0], s_ks[0], tid);
    stage_store_v<KV>(st, s_v[0], s_vs[0], tid);
    pgk = page_of(bt, KT + kkey, kend);
    pgv = page_of(bt, KT + vkey, kend);
    stage_load_k<KV>(st, p, sa, KT + kkey, kend, pgk);
    stage_load_v<KV>(st, p, sa, KT + vkey, kend, pgv);
    pgk = page_of(bt, 2 * KT + kkey, kend);
    pgv = page_of(bt, 2 * KT + vkey, kend);
    __syncthreads();

    // K operands of one subtile: MFMA row r32 is LDS row 32ks + r32, whose
    // chunk 2kc + h32 sits at slot kc ^ 8 h32 ^ k_row_key(r32)
    const int kslot = (h32 << 3) ^ k_row_key(r32);
    f16x8 ka[8];
    auto load_k = [&](int kb, int ks) __attribute__((always_inline)) {
        const f16* krp = s_k[kb] + (32 * ks + r32) * KSTR;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) ka[kc] = *reinterpret_cast<const f16x8*>(krp + 8 * (kc ^ kslot));
    };
    // P and V operands of the previous subtile (zero P before the first, on
    // tile 0's V, which is finite) and its PV
    f16x8 pprev[2] = {f16x8{0, 0, 0, 0, 0, 0, 0, 0}, f16x8{0, 0, 0, 0, 0, 0, 0, 0}};
    f16x8 va[4][2];
    auto load_v = [&](int vb, int kss) __attribute__((always_inline)) {
        const f16* lv = s_v[vb];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                va[dt][hf] = *reinterpret_cast<const f16x8*>(lv + (32 * dt + r32) * VSTR + 8 * h32 +
                                                             32 * kss + 16 * hf);
    };
    auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) acc[dt] = mfma32(va[dt][hf], pprev[hf], acc[dt]);
    };

    load_k(0, 0);
    if (late) phase_barrier();

    // One step: subtile ks of tile T.  MASKED tiles (at the diagonal) compare
    // each key with the row's position; the others skip the mask.
    auto step = [&](auto mtag, auto kstag, int T) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int ks = decltype(kstag)::value;
        const int kb = T & 1;
        // ---------------- MFMA phase: S of this subtile, PV of the previous;
        // raised priority so the MFMAs win issue against the other wave's softmax
        __builtin_amdgcn_s_setprio(2);
        if constexpr (ks == 0) load_v(T > 0 ? (T - 1) & 1 : 0, 1);   // zero P before the first
        else load_v(kb, 0);
        f32x16 sc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) sc = mfma32(ka[kc], qop[kc], sc);
        pv();
        {
            // tile T+1 to LDS (past the last tile: zeros into a retired
            // buffer), then tile T+2 into registers; branch-free, so that the
            // scheduler can slot this work between the MFMAs
            if constexpr (ks == 0) {
                stage_store_k<KV>(st, s_k[kb ^ 1], s_ks[(T + 1) % 3], tid);
                stage_load_k<KV>(st, p, sa, (T + 2) * KT + kkey, kend, pgk);
                pgk = page_of(bt, (T + 3) * KT + kkey, kend);
            } else {
                stage_store_v<KV>(st, s_v[kb ^ 1], s_vs[kb ^ 1], tid);
                stage_load_v<KV>(st, p, sa, (T + 2) * KT + vkey, kend, pgv);
                pgv = page_of(bt, (T + 3) * KT + vkey, kend);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
            }
        }
        __builtin_amdgcn_s_setprio(0);
        phase_barrier();

        // ---------------- VALU phase: the next subtile's K operands, this
        // subtile's softmax, its V operands, staging
        if constexpr (ks == 0) load_k(kb, 1);
        else load_k(kb ^ 1, 0);                     // past the last subtile: a harmless reread
        const int k0 = T * KT + 32 * ks;
        float mx = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // row r of this lane's scores holds key k0 + 16(r>>3) + 8 h32 + (r&7)
            float v = sc[r];
            if constexpr (KV == KV_INT8) v *= s_ks[T % 3][32 * ks + 16 * (r >> 3) + 8 * h32 + (r & 7)];
            if constexpr (MASKED) {
                const int key = k0 + 16 * (r >> 3) + 8 * h32 + (r & 7);
                v = (key <= rowpos) ? v : -__builtin_inff();
            }
            sc[r] = v;
            mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, shfl_xor(mx, 32));
        // The reference maximum moves only when a row's maximum grew by more
        // than grow_raw (2^8 in probability; 0 for INT8, whose P carries the
        // value scale): the accumulators are rescaled rarely, not per subtile.
        const bool grow = mx > m_ref + grow_raw;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = (m_ref == -__builtin_inff()) ? 0.0f : fast_exp2((m_ref - m_new) * cscale);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
            m_ref = m_new;
        }
        // p = 2^(c*s - c*m): one fma and one exp per score; l sums the fp32 p
        // (summing the fp16-rounded weights would leave up to 2^-11 relative
        // error in l on short rows)
        const float moff = (m_ref == -__builtin_inff()) ? 0.0f : -m_ref * cscale;
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pe = fast_exp2(__builtin_fmaf(sc[r], cscale, moff));
            psum += pe;
            if constexpr (KV == KV_INT8)   // P carries each key's value scale
                pe *= s_vs[kb][32 * ks + 16 * (r >> 3) + 8 * h32 + (r & 7)] * kInt8PFold;
            pprev[r >> 3][r & 7] = (f16)pe;
        }
        l_run += psum;
        pin(pprev[0]);
        pin(pprev[1]);
        phase_barrier();
    };
    using U = std::false_type;
    using M = std::true_type;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    for (int T = 0; T < nfull; ++T) { step(U{}, S0{}, T); step(U{}, S1{}, T); }
    for (int T = nfull; T < ntiles; ++T) { step(M{}, S0{}, T); step(M{}, S1{}, T); }
    load_v((ntiles - 1) & 1, 1);
    pv();
    if (!late) phase_barrier();                      // equal barrier counts in both groups

    // ---- epilogue: lanes l and l^32 hold halves of the same row's keys
    const float l = l_run + shfl_xor(l_run, 32);
    if (rowok) {
        const float inv = vscale / l;
        float* o = p.out + rowid * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = 32 * dt + 8 * a4 + 4 * h32;
                f32x4 v = f32x4{acc[dt][4 * a4 + 0], acc[dt][4 * a4 + 1], acc[dt][4 * a4 + 2],
                                acc[dt][4 * a4 + 3]} * inv;
                *reinterpret_cast<f32x4*>(o + d) = v;
            }
        if (h32 == 0) p.lse[rowid] = (m_ref * cscale + __builtin_log2f(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
    const int G = p.num_q_heads / p.kv.num_kv_heads;
    const int ppw = 256 / G;                         // query positions per workgroup
    dim3 grid((p.max_q_len + ppw - 1) / ppw, p.kv.num_kv_heads, p.num_seqs);
    if (grid.x == 0) return hipSuccess;
    const dim3 block(512);
    switch (p.kv.dtype) {
    case KV_FP16: hipLaunchKernelGGL(prefill_kernel<KV_FP16>, grid, block, 0, s, p); break;
    case KV_E4M3: hipLaunchKernelGGL(prefill_kernel<KV_E4M3>, grid, block, 0, s, p); break;
    case KV_INT8: hipLaunchKernelGGL(prefill_kernel<KV_INT8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace plc
