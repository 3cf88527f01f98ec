// Chunked causal prefill at head dim 256 over the paged KV cache, for gfx950.
//
// The pages split a 256-wide head into two 128-wide halves on their
// hardware (1Cat-vLLM README, Layer 2 "D256 Split-D"); here the whole head
// is one MFMA contraction: S^T = K Q^T sums over all 256 dimensions in one
// 32x32 accumulator and O^T = V^T P^T keeps eight 32-dimension accumulator
// tiles.  A workgroup is 4 waves = 128 query rows of one (sequence, KV head),
// position-major rows (row r = query token r / G, head r % G, so the G heads
// of a KV head share every K/V tile: Layer 2 "GQA Multi-Head Packing"), one
// 32-row MFMA tile per wave.  Q operands (64 VGPRs) and O^T accumulators (128)
// stay in registers for the whole key loop; at about 450 registers a SIMD
// holds one wave, so each wave overlaps its own softmax with its MFMAs: the
// online softmax of 32-key subtile j runs between the MFMAs of S for subtile
// j+1, and the staging of later tiles between the MFMAs of O += V^T P^T for
// subtile j.
//
// Keys are walked in tiles of 64 (four 16-token pages).  Per tile every
// thread gathers 64 K codes and 64 V codes with 8-byte loads (16-byte for
// FP16), converts them to fp16 exactly and writes K as [key][d] (two buffers)
// and V transposed as [d][key] (two buffers), so each workgroup converts a
// tile once and its four waves read fp16 operands (Layer 1 and the
// "Software-Reconstructed Async" section give the same goals on V100).  Tiles
// wholly below the workgroup's first position skip the causal mask (Layer 2
// "Prefix / Causal-Tail Separation").
//
// The launcher takes this register-staged kernel for FP16 caches only; E4M3
// and INT8 caches go to the tile kernel whose codes reach LDS by DMA
// (prefill_dma.hip), measured faster for 8-bit codes.  The kernel stays
// written for every dtype (its INT8 and E4M3 paths are not instantiated).
#include <type_traits>

#include "plc_device.h"
#include "plc_internal.h"

namespace plc {
namespace {

constexpr int D = 256;
constexpr int BS = 16;
constexpr int KT = 64;                  // keys per tile
constexpr int KSTR = D + 8;             // K row stride in LDS (halves)
constexpr int VSTR = KT + 8;            // V^T row stride in LDS (halves)
constexpr int KBUF = KT * KSTR;         // 33 KiB
constexpr int VBUF = D * VSTR;          // 36 KiB
constexpr int ROWS = 128;               // query rows per workgroup
constexpr int PF = 4;                   // MFMA operands read from LDS this many MFMAs ahead

// LDS bank map (64 banks of 4 bytes).  K rows are 528 bytes, 4 banks apart
// modulo 256 bytes: an operand read (16 consecutive rows, one 16-byte chunk
// per lane) covers the 64 banks once, and a staging write (one row, chunks
// q = 0..15 or 16 + q) covers them once.  V^T rows are 144 bytes: 16
// consecutive rows start 36 banks apart modulo 64, distinct 4-bank groups.

// Staging of one tile.  K: thread t takes dimensions 8 (t & 15) + [0,8) and
// 128 + 8 (t & 15) + [0,8) of key 16 j + (t >> 4) on each page j.  V: keys
// 8 (t & 7) + [0,8) (one page), dimensions 8 (t >> 3) + [0,8).  Keys past the
// visible end or on an invalid page are zeroed when written to LDS; the loads
// themselves are always issued (page 0 when a page id is invalid), so the
// loads in flight stay countable across the key loop.
template <int KV>
struct Stage {
    static constexpr int KW = (KV == KV_FP16) ? 4 : 2;   // words per K half-row piece
    static constexpr int VW = (KV == KV_FP16) ? 4 : 2;   // words per V key
    uint32_t k[4][2][KW];                            // [page j][half h]
    uint32_t v[8][VW];                               // [key e]
    float ks[4];                                     // INT8: key scale on page j
    float vs[8];                                     // INT8: V key e's scale
    uint32_t ok;                                     // bit j: K key on page j; bit 8 + e: V key e
};

struct StageAddr {
    int64_t page_bytes;                              // Hkv * BS * D * elem bytes
    int64_t k_off, v_off;                            // byte offsets within a page
    int32_t page_rows;                               // Hkv * BS (INT8 scale rows per page)
    int32_t ks_row, vs_row;                          // scale rows within a page
};

// A value the compiler must treat as varying per lane, so that a load indexed
// by it is a vector load: a scalar load in flight would make every wait for
// an LDS read also wait for it (both count on the same counter, and scalar
// loads return out of order).
__device__ __forceinline__ int per_lane(int x) {
    int y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

template <int KV>
__device__ __forceinline__ void load_k_piece(Stage<KV>& st, const PrefillParams& p, const StageAddr& sa, int j,
                                             int h, int key, int kend, int pg) {
    constexpr int EB = (KV == KV_FP16) ? 2 : 1;
    const bool pgok = pg >= 0 && pg < p.kv.num_blocks;
    const int64_t pb = pgok ? pg : 0;
    const uint8_t* src = static_cast<const uint8_t*>(p.kv.k) + pb * sa.page_bytes + sa.k_off + 128 * EB * h;
    if constexpr (KV == KV_FP16) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.k[j][h][i] = c[i];
    } else {
        const u32x2 c = *reinterpret_cast<const u32x2*>(src);
        st.k[j][h][0] = c[0];
        st.k[j][h][1] = c[1];
    }
    if (h == 0) {
        if constexpr (KV == KV_INT8) st.ks[j] = p.kv.k_scale[pb * sa.page_rows + sa.ks_row];
        st.ok = (st.ok & ~(1u << j)) | (((pgok && key < kend) ? 1u : 0u) << j);
    }
}

// V key e of the thread's eight (all on page pg)
template <int KV>
__device__ __forceinline__ void load_v_key(Stage<KV>& st, const PrefillParams& p, const StageAddr& sa, int e,
                                           int key, int kend, int pg) {
    constexpr int EB = (KV == KV_FP16) ? 2 : 1;
    const bool pgok = pg >= 0 && pg < p.kv.num_blocks;
    const int64_t pb = pgok ? pg : 0;
    const uint8_t* src = static_cast<const uint8_t*>(p.kv.v) + pb * sa.page_bytes + sa.v_off + e * D * EB;
    if constexpr (KV == KV_FP16) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.v[e][i] = c[i];
    } else {
        const u32x2 c = *reinterpret_cast<const u32x2*>(src);
        st.v[e][0] = c[0];
        st.v[e][1] = c[1];
    }
    if constexpr (KV == KV_INT8) st.vs[e] = p.kv.v_scale[pb * sa.page_rows + sa.vs_row + e];
    st.ok = (st.ok & ~(1u << (8 + e))) | (((pgok && key < kend) ? 1u : 0u) << (8 + e));
}

// K piece (j, h) -> LDS row key_of_row(16 j + (t >> 4)), chunk 16 h + (t & 15)
template <int KV>
__device__ __forceinline__ void store_k_piece(const Stage<KV>& st, f16* lk, float* lks, int t, int j, int h) {
    const int key = 16 * j + (t >> 4), rho = key_of_row(key);
    const bool ok = (st.ok >> j) & 1u;
    f16* dst = lk + rho * KSTR + 8 * (16 * h + (t & 15));
    if constexpr (KV == KV_FP16) {
        const u32x4 c{ok ? st.k[j][h][0] : 0u, ok ? st.k[j][h][1] : 0u, ok ? st.k[j][h][2] : 0u,
                      ok ? st.k[j][h][3] : 0u};
        *reinterpret_cast<u32x4*>(dst) = c;
    } else {
        *reinterpret_cast<f16x8*>(dst) = codes8_to_f16x8<KV>(ok ? st.k[j][h][0] : 0u, ok ? st.k[j][h][1] : 0u);
    }
    // the 16 lanes of a key store the same scale (branch-free)
    if constexpr (KV == KV_INT8)
        if (h == 0) lks[key] = ok ? st.ks[j] : 0.0f;
}

// V -> [d][key], rows 8 (t >> 3) + 2cp + [0,2), keys 8 (t & 7) + [0,8).  Eight
// consecutive lanes write one 128-byte row segment; the next eight write the
// row 8 further on, 8 x 144 bytes = 128 bytes (mod 256) away, so 16 lanes
// cover the 64 banks once.
template <int KV>
__device__ __forceinline__ void store_v_rows(const Stage<KV>& st, f16* lv, int t, int cp) {
    f16* dst = lv + (8 * (t >> 3) + 2 * cp) * VSTR + 8 * (t & 7);
    auto okey = [&](int e) { return (st.ok >> (8 + e)) & 1u; };
    if constexpr (KV == KV_FP16) {
        // row c = 2cp + i is half i of word cp of every key
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t sel = i ? 0x07060302u : 0x05040100u;
            u32x4 r;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                r[m] = __builtin_amdgcn_perm(okey(2 * m + 1) ? st.v[2 * m + 1][cp] : 0u,
                                             okey(2 * m) ? st.v[2 * m][cp] : 0u, sel);
            *reinterpret_cast<u32x4*>(dst + i * VSTR) = r;
        }
    } else {
        // rows 2cp and 2cp + 1 are bytes 2(cp&1) and 2(cp&1) + 1 of word cp >> 1
        const int w = cp >> 1;
        const uint32_t sel = (cp & 1) ? 0x07030602u : 0x05010400u;
        f16x2 lo[4], hi[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t a = okey(2 * m + 1) ? st.v[2 * m + 1][w] : 0u;
            const uint32_t b = okey(2 * m) ? st.v[2 * m][w] : 0u;
            const uint32_t pr = __builtin_amdgcn_perm(a, b, sel);   // (b_c, a_c, b_c+1, a_c+1)
            lo[m] = codes2_to_f16x2<KV, false>(pr);
            hi[m] = codes2_to_f16x2<KV, true>(pr);
        }
        *reinterpret_cast<f16x8*>(dst) = f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1],
                                               lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
        *reinterpret_cast<f16x8*>(dst + VSTR) = f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1],
                                                      hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
    }
}

// INT8: the eight V keys' scales; the 32 threads of a key group store the
// same values (branch-free)
template <int KV>
__device__ __forceinline__ void store_vscales(const Stage<KV>& st, float* lvs, int t) {
    const int kv0 = 8 * (t & 7);
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = ((st.ok >> (8 + i)) & 1u) ? st.vs[i] : 0.0f;
        b[i] = ((st.ok >> (12 + i)) & 1u) ? st.vs[4 + i] : 0.0f;
    }
    *reinterpret_cast<f32x4*>(lvs + kv0) = a;
    *reinterpret_cast<f32x4*>(lvs + kv0 + 4) = b;
}

// Schedule of the key loop, per 32-key subtile j of tile T = j / 2, written
// out as 16 steps per part (one MFMA each, the compiler may not move work
// across steps):
//   part A: S(j+1) = K Q^T; step i reads K operand i + PF from LDS (the last
//           PF steps read the first V operands of part B) and runs a slice of
//           the online softmax of S(j);
//   (a rare branch rescales O when a row's reference maximum moved)
//   workgroup barrier
//   part B: O += V^T P(j)^T; step i reads V operand i + PF (the last PF
//           read the first K operands of subtile j+2) and a slice of the
//           staging: for j even, V of tile T+1 to LDS and V of T+2 into
//           registers; for j odd, K of T+2 (with the INT8 scales of K and V of
//           T+2) to LDS and K of T+3 into registers.
// K of tile T is read from the end of part B of 2T-2 to part A of 2T, V of T
// from the end of part A of 2T to part B of 2T+1.  The barrier of subtile
// 2T+1 separates the last read of K of T from its replacement (part B of
// 2T+1), that of 2T the last read of V of T-1 from its replacement (part B
// of 2T), and each write lies before a barrier that precedes its first
// reader (end of part B of 2T+2, end of part A of 2T+2).
template <int KV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill256_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) f16 s_k[2][KBUF];
    __shared__ __attribute__((aligned(16))) f16 s_v[2][VBUF];
    __shared__ __attribute__((aligned(16))) float s_ks[2][KT];   // INT8 scales
    __shared__ __attribute__((aligned(16))) float s_vs[2][KT];

    const int rb = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = p.num_q_heads, G = Hq / p.kv.num_kv_heads;
    const int qa = p.cu_q_lens[b];
    // lengths beyond the host-stated bounds are clamped so that no page id
    // outside the table is ever read
    const int L = max(0, min(p.context_lens[b], p.max_context_len));
    const int n = min(max(p.cu_q_lens[b + 1] - qa, 0), min(p.max_q_len, L));
    const int nrows = n * G;
    const int r0 = ROWS * rb;
    if (r0 >= nrows) return;
    const int base = L - n;                          // position of the chunk's first token
    const int rlast = min(r0 + ROWS, nrows) - 1;
    const int kend = base + rlast / G + 1;           // keys [0, kend) are visible to someone
    const int kfull = base + r0 / G + 1;             // keys [0, kfull) are visible to every row
    const int ntiles = (kend + KT - 1) / KT;
    const int nfull = min(kfull / KT, ntiles);       // tiles needing no mask
    const int plast = (kend - 1) / BS;               // last page with a visible key
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;

    // ---- this lane's query row: row l%32 of the wave's tile
    const int h32 = lane >> 5, r32 = lane & 31;
    int rowpos;
    int64_t rowid;
    bool rowok;
    {
        const int r = r0 + 32 * wave + r32;
        rowok = r < nrows;
        const int rc = rowok ? r : rlast;
        rowpos = base + rc / G;
        rowid = (int64_t)(qa + rc / G) * Hq + kvh * G + rc % G;
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / kInt8PFold;

    float m_ref = -__builtin_inff(), l_run = 0.0f;   // raw-score units
    // the reference maximum moves only when a row's maximum grew by more than
    // 2^8 in probability (0 for INT8, whose P carries the value scale): O is
    // rescaled rarely, not per subtile
    const float grow_raw = (KV == KV_INT8) ? 0.0f : 8.0f / cscale;
    f32x16 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

    // ---- staging addresses and the first tiles: tile 0 (with its INT8
    // scales) and K of 1 (with the INT8 scales of tile 1) in LDS, V of 1 and K
    // of 2 in registers, then the page ids of V of 2 (the thread's page) and
    // of K of 3 (the tile's four pages)
    const int kp = tid >> 4, vkey = 8 * (tid & 7);
    StageAddr sa;
    {
        constexpr int EB = (KV == KV_FP16) ? 2 : 1;
        const int Hkv = p.kv.num_kv_heads;
        sa.page_rows = Hkv * BS;
        sa.page_bytes = (int64_t)sa.page_rows * D * EB;
        sa.ks_row = kvh * BS + kp;
        sa.vs_row = kvh * BS + (vkey & (BS - 1));
        sa.k_off = ((int64_t)sa.ks_row * D + 8 * (tid & 15)) * EB;
        sa.v_off = ((int64_t)sa.vs_row * D + 8 * (tid >> 3)) * EB;
    }
    auto kpage = [&](int T, int j) __attribute__((always_inline)) { return bt[per_lane(min(4 * T + j, plast))]; };
    auto vpage = [&](int T) __attribute__((always_inline)) { return bt[min(4 * T + (vkey >> 4), plast)]; };
    Stage<KV> st;
    st.ok = 0;
    int pk[4];
    int pv;
    auto load_k_tile = [&](int T) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) load_k_piece<KV>(st, p, sa, j, h, T * KT + 16 * j + kp, kend, pk[j]);
    };
    auto store_k_tile = [&](f16* lk, float* lks) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) store_k_piece<KV>(st, lk, lks, tid, j, h);
    };
    auto load_v_tile = [&](int T) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) load_v_key<KV>(st, p, sa, e, T * KT + vkey + e, kend, pv);
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = kpage(0, j);
    pv = vpage(0);
    load_k_tile(0);
    load_v_tile(0);
    store_k_tile(s_k[0], s_ks[0]);
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) store_v_rows<KV>(st, s_v[0], tid, cp);
    if constexpr (KV == KV_INT8) store_vscales<KV>(st, s_vs[0], tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = kpage(1, j);
    pv = vpage(1);
    load_k_tile(1);
    load_v_tile(1);
    store_k_tile(s_k[1], s_ks[1]);
    if constexpr (KV == KV_INT8) store_vscales<KV>(st, s_vs[1], tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = kpage(2, j);
    load_k_tile(2);
    pv = vpage(2);
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = kpage(3, j);
    // Q operands, loaded after the staging prologue so that they do not share
    // its register peak: lane holds d = 16kc + 8(l/32) + [0,8) of its row
    f16x8 qop[16];
    {
        const f16* q = static_cast<const f16*>(p.q) + rowid * D + 8 * h32;
#pragma unroll
        for (int kc = 0; kc < 16; ++kc) qop[kc] = *reinterpret_cast<const f16x8*>(q + 16 * kc);
    }
    __syncthreads();

    // operand addresses: K operand kc of (buffer kb, half ks) is LDS row
    // 32ks + r32, chunk 2kc + h32; V^T operand (dt, hf) is row 32dt + r32,
    // keys 32ks + 16hf + 8h32 + [0,8)
    const f16* kbase = &s_k[0][0] + r32 * KSTR + 8 * h32;
    const f16* vbase = &s_v[0][0] + r32 * VSTR + 8 * h32;
    auto kop = [&](int kb, int ks, int kc) __attribute__((always_inline)) {
        return *reinterpret_cast<const f16x8*>(kbase + kb * KBUF + 32 * ks * KSTR + 16 * kc);
    };
    auto vop = [&](int vb, int ks, int dt, int hf) __attribute__((always_inline)) {
        return *reinterpret_cast<const f16x8*>(vbase + vb * VBUF + 32 * dt * VSTR + 32 * ks + 16 * hf);
    };

    f16x8 kq[PF], vq[PF];                            // operands in flight
    f32x16 sc;                                       // S of the current subtile
    {
#pragma unroll
        for (int kc = 0; kc < 16; ++kc) sc = mfma32(kop(0, 0, kc), qop[kc], kc ? sc : f32x16{});
#pragma unroll
        for (int kc = 0; kc < PF; ++kc) kq[kc] = kop(0, 1, kc);
    }

    // one subtile j = 2T + ks
    auto sub = [&](auto mtag, auto kstag, int T) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int ks = decltype(kstag)::value;
        constexpr int SO = (KV == KV_INT8) ? 2 : 0;  // INT8: two steps for the scale reads
        const int kb = T & 1;
        // subtile j + 1 (past the last subtile: a harmless read of a retired buffer)
        const int kbn = ks ? kb ^ 1 : kb, ksn = ks ^ 1;
        const int k0 = T * KT + 32 * ks;
        f32x16 sn;
        float mloc = -__builtin_inff(), mx = 0.0f, m_new = 0.0f, moff = 0.0f, psum = 0.0f;
        bool grow = false;
        f16x8 pp[2];
        f32x4 sks[4], svs[4];                        // INT8 scales of this subtile's keys
        // ---------------- part A
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sn = mfma32(kq[i % PF], qop[i], i ? sn : f32x16{});
            if (i < 16 - PF) kq[i % PF] = kop(kbn, ksn, i + PF);
            else vq[i - (16 - PF)] = vop(kb, ks, (i - (16 - PF)) >> 1, (i - (16 - PF)) & 1);
            if constexpr (KV == KV_INT8)
                if (i == 0) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ko = 32 * ks + 16 * (u >> 1) + 8 * h32 + 4 * (u & 1);
                        sks[u] = *reinterpret_cast<const f32x4*>(&s_ks[kb][ko]);
                        svs[u] = *reinterpret_cast<const f32x4*>(&s_vs[kb][ko]);
                    }
                }
            if (i >= SO && i < SO + 4) {
                // scores 4(i - SO) + [0,4): element r is key k0 + 16(r>>3) + 8 h32 + (r&7)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 4 * (i - SO) + rr;
                    float v = sc[r];
                    if constexpr (KV == KV_INT8) v *= sks[r >> 2][r & 3];
                    if constexpr (MASKED) {
                        const int key = k0 + 16 * (r >> 3) + 8 * h32 + (r & 7);
                        v = (key <= rowpos) ? v : -__builtin_inff();
                    }
                    sc[r] = v;
                    mloc = fmaxf(mloc, v);
                }
            }
            if (i == SO + 4) {
                mx = max_halves(mloc);
                grow = mx > m_ref + grow_raw;
                m_new = grow ? mx : m_ref;
                // p = 2^(c*s - c*m): one fma and one exp per score
                moff = (m_new == -__builtin_inff()) ? 0.0f : -m_new * cscale;
            }
            if (i >= SO + 5 && i < SO + 13) {
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = 2 * (i - SO - 5) + rr;
                    float pe = fast_exp2(__builtin_fmaf(sc[r], cscale, moff));
                    psum += pe;                      // l sums the fp32 p
                    if constexpr (KV == KV_INT8) pe *= svs[r >> 2][r & 3] * kInt8PFold;   // P carries the V scale
                    pp[r >> 3][r & 7] = (f16)pe;
                }
            }
            step_fence();
        }
        // the compiler would otherwise sink the softmax past the branch
        pin(pp[0]);
        pin(pp[1]);
        pin(psum);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
            const float alpha = (m_ref == -__builtin_inff()) ? 0.0f : fast_exp2((m_ref - m_new) * cscale);
            l_run *= alpha;
            // one accumulator tile at a time, so the rescale holds few registers
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] = scale_acc(acc[dt][r], alpha);
            // AGPR writes before an MFMA reads them as its accumulator
            asm volatile("s_nop 7" ::: "memory");
        }
        m_ref = m_new;
        l_run += psum;
        subtile_barrier();
        // ---------------- part B
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[i >> 1] = mfma32(vq[i % PF], pp[i & 1], acc[i >> 1]);
            if (i < 16 - PF) vq[i % PF] = vop(kb, ks, (i + PF) >> 1, (i + PF) & 1);
            else kq[i - (16 - PF)] = kop(kb ^ 1, ks, i - (16 - PF));   // subtile j + 2
            if constexpr (ks == 0) {
                // V of tile T+1 to LDS, V of T+2 into registers
                if (i < 4) store_v_rows<KV>(st, s_v[kb ^ 1], tid, i);
                if (i >= 4 && i < 12) load_v_key<KV>(st, p, sa, i - 4, (T + 2) * KT + vkey + i - 4, kend, pv);
                if (i == 12) pv = vpage(T + 3);
            } else {
                // K of tile T+2 (and the INT8 scales of T+2) to LDS, K of T+3
                // into registers
                if (i < 8) store_k_piece<KV>(st, s_k[kb], s_ks[kb], tid, i >> 1, i & 1);
                if constexpr (KV == KV_INT8)
                    if (i == 0) store_vscales<KV>(st, s_vs[kb], tid);
                if (i >= 8) {
                    const int j = (i - 8) >> 1, h = (i - 8) & 1;
                    load_k_piece<KV>(st, p, sa, j, h, (T + 3) * KT + 16 * j + kp, kend, pk[j]);
                    if (h == 1) pk[j] = kpage(T + 4, j);
                }
            }
            step_fence();
        }
        sc = sn;
    };
    using U = std::false_type;
    using M = std::true_type;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    for (int T = 0; T < nfull; ++T) {
        sub(U{}, S0{}, T);
        sub(U{}, S1{}, T);
    }
    for (int T = nfull; T < ntiles; ++T) {
        sub(M{}, S0{}, T);
        sub(M{}, S1{}, T);
    }

    // ---- epilogue: lanes l and l^32 hold halves of the same row's keys
    const float l = l_run + shfl_xor(l_run, 32);
    if (rowok) {
        const float inv = vscale / l;
        float* o = p.out + rowid * D;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = 32 * dt + 8 * a4 + 4 * h32;
                *reinterpret_cast<f32x4*>(o + d) = f32x4{acc[dt][4 * a4 + 0], acc[dt][4 * a4 + 1],
                                                         acc[dt][4 * a4 + 2], acc[dt][4 * a4 + 3]} * inv;
            }
        if (h32 == 0) p.lse[rowid] = (m_ref * cscale + __builtin_log2f(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill256(const PrefillParams& p, hipStream_t s) {
    if (p.kv.dtype != KV_FP16) return launch_prefill_dma(p, s);   // 8-bit codes by DMA
    const int G = p.num_q_heads / p.kv.num_kv_heads;
    dim3 grid((unsigned)(((int64_t)p.max_q_len * G + ROWS - 1) / ROWS), p.kv.num_kv_heads, p.num_seqs);
    if (grid.x == 0) return hipSuccess;
    const dim3 block(256);
    switch (p.kv.dtype) {
    case KV_FP16: hipLaunchKernelGGL(prefill256_kernel<KV_FP16>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace plc
