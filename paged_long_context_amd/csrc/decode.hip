// Split-KV paged decode for gfx950.
//
// One workgroup per (partition, KV head, sequence).  The partition's 16-token
// pages are walked two at a time (a 32-token chunk) by the workgroup's waves.
// Per chunk a wave:
//   - reads the two page ids once and moves the pages into its LDS buffer by
//     DMA in whole kilobytes, 16 bytes per lane (the page-id reuse and wide
//     loads that the 1Cat-vLLM README's "128-bit Loads" section credits for
//     its decode gain), FP16 V going to registers instead;
//   - converts K codes to fp16 and forms S^T = K * Q^T with the G query heads of
//     the KV head as the 16-wide MFMA N dimension (GQA packing, Layer 2 "GQA
//     Multi-Head Packing"); every lane therefore owns one query head;
//   - runs the online softmax in fp32 (Layer 2, "N32 Online Softmax"), with the
//     row maximum shared by the four lanes that hold the same head;
//   - transposes V bytes in registers with v_perm, converts them to fp16 and
//     accumulates O^T = V^T * P^T on MFMA, so O stays in the same head-per-lane
//     layout as the softmax state.
// Waves merge through LDS in a fixed order; the workgroup writes the
// normalized partial output and its natural-log LSE for plc_lse_merge
// (Layer 2, "Split-KV3").
#include "plc_device.h"
#include "plc_internal.h"

namespace plc {
namespace {

constexpr int D = 128;
constexpr int BS = 16;

template <int KV>
struct ElemBytes { static constexpr int value = (KV == KV_FP16) ? 2 : 1; };

// Raw registers of one 32-token chunk (two pages) for one lane.
template <int KV>
struct Chunk {
    // K: lane (row i = l%16, group g = l/16) holds, for each page, the bytes of
    // token i at d = 64h + 16g + [0, 16) for h = 0, 1.
    u32x4 k[2][(KV == KV_FP16) ? 1 : 2];            // E4M3/INT8 codes
    f16x8 kh[2][(KV == KV_FP16) ? 4 : 1];           // FP16 values, already operands
    // V: eight tokens t(g, e) = 16*(e/4) + 4g + e%4, d = 8*(l%16) + [0, 8).
    u32x4 v16[(KV == KV_FP16) ? 8 : 1];
    u32x2 v8[(KV == KV_FP16) ? 1 : 8];
    f32x4 ks[2], vs[2];             // INT8 per-token scales of tokens 4g..4g+3
    int valid_blk;                  // bit p set when page p is inside the pool
};

// DH: the cache's head dim (row length in elements).  A page of head dim 256 is
// read as two halves of 128 (Split-D), each laid out in LDS like a whole
// 128-wide page; hoff selects the half.
template <int KV, int NW, int DH = 128>
struct Decode {
    static constexpr int EB = ElemBytes<KV>::value;
    static constexpr int RB = DH * EB;              // bytes per cache row

    // ---- Pages reach a per-wave LDS buffer (two 8 KiB chunk buffers per wave,
    // ping-pong) by DMA: global_load_lds, 16 bytes per lane, every instruction
    // one contiguous kilobyte; the operands are then read from LDS.
    //  8-bit codes: K pages at 0 and 2048, V pages at 4096 and 6144.  LDS row
    //   slot s of a page holds token row swap02(s) (bits 0 and 2 swapped) with
    //   its 16-byte chunk c at chunk slot c ^ kap(s), kap(s) = (s & 7) ^ (s >> 3
    //   & 1): the K operand reads (16 rows, one chunk) and V row reads (two rows
    //   4 apart) hit every bank at most once.
    //  FP16: K pages at 0 and 4096 (256-byte rows), chunk c of row s at slot
    //   c ^ s; V (whole 256-byte rows per 16-lane group already) stays in
    //   registers.
    struct Meta {
        u32x4 v16[(KV == KV_FP16) ? 8 : 1];   // FP16 V rows, as in Chunk
        int valid_blk;
    };
    __device__ __forceinline__ static int swap02(int x) { return (x & ~5) | ((x & 1) << 2) | ((x >> 2) & 1); }
    __device__ __forceinline__ static int kap(int s) { return (s & 7) ^ ((s >> 3) & 1); }
    // DMA instructions per page (8-bit: K and V, 2 each; FP16: K, 4)
    static constexpr int kDmaPerPage = (KV == KV_FP16) ? 4 : 2;
    // lane l's source offset within a page for DMA instruction q
    __device__ __forceinline__ static int dma_src(int lane, int q) {
        if constexpr (KV == KV_FP16) {
            const int s = 4 * q + (lane >> 4);
            return s * RB + 16 * ((lane & 15) ^ s);
        } else {
            const int s = 8 * q + (lane >> 3);
            return swap02(s) * RB + 16 * ((lane & 7) ^ kap(s));
        }
    }
    // One global_load_lds_dwordx4: lane l's 16 bytes at src land at LDS
    // dst + 16 l (dst wave-uniform).  Written as asm so that the compiler does
    // not treat every later LDS read as waiting on it: the loop waits with
    // explicit vmcnt counts instead (unknown vector loads can only make the
    // compiler's own counts wait longer, never shorter).
    // M0 (the LDS base it reads at issue) is saved and restored around it.
    // The loads are non-temporal: a step reads every page once.
    __device__ __forceinline__ static void dma16(const uint8_t* src, uint8_t* dst) {
        const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %2, off nt\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "s"(base), "v"(src) : "memory");
    }
    // bit p set when page p of a chunk is inside the pool (page 1 only if the
    // chunk has a second page)
    __device__ __forceinline__ static int valid_bits(int pb0, int pb1, bool has1, int nb) {
        return ((pb0 >= 0 && pb0 < nb) ? 1 : 0) | ((has1 && pb1 >= 0 && pb1 < nb) ? 2 : 0);
    }
    __device__ __forceinline__ static void issue(Meta& m, uint8_t* lbuf, f32x4* sbuf, const DecodeParams& p,
                                                 int kvh, int pb0,
                                                 int pb1, bool has1, int lane, const int src[kDmaPerPage],
                                                 int hoff = 0, bool scales = true) {
        const int g = lane >> 4, i = lane & 15;
        m.valid_blk = valid_bits(pb0, pb1, has1, p.kv.num_blocks);
        const int pbs[2] = {(m.valid_blk & 1) ? pb0 : 0, (m.valid_blk & 2) ? pb1 : 0};
        const int Hkv = p.kv.num_kv_heads;
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            const int64_t base = ((int64_t)pbs[pg] * Hkv + kvh) * (BS * RB) + hoff;
            const uint8_t* kp = static_cast<const uint8_t*>(p.kv.k) + base;
            const uint8_t* vp = static_cast<const uint8_t*>(p.kv.v) + base;
            if constexpr (KV == KV_FP16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) dma16(kp + src[q], lbuf + 4096 * pg + 1024 * q);
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    dma16(kp + src[q], lbuf + 2048 * pg + 1024 * q);
                    dma16(vp + src[q], lbuf + 4096 + 2048 * pg + 1024 * q);
                }
            }
        }
        if constexpr (KV == KV_FP16) {
            // V: token 4g + e%4 of page e/4, d = 8i..8i+7, one 16-byte load each
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t base = ((int64_t)pbs[e >> 2] * Hkv + kvh) * (BS * RB) + hoff;
                m.v16[e] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.kv.v) + base +
                                                           (4 * g + (e & 3)) * RB + 16 * i);
            }
        }
        if constexpr (KV == KV_INT8) if (scales) {
            // the two pages' per-token scales by one more DMA: lane l (mod
            // 16) moves 16 bytes (4 tokens) of [K | V][page][4 tokens x 4]
            // into slot l of sbuf; lanes 16..63 repeat lanes 0..15 into
            // slots nothing reads
            const int sl = lane & 15, spg = (sl >> 2) & 1;
            const float* sc = ((sl >> 3) ? p.kv.v_scale : p.kv.k_scale) +
                              ((int64_t)pbs[spg] * Hkv + kvh) * BS + 4 * (sl & 3);
            dma16(reinterpret_cast<const uint8_t*>(sc), reinterpret_cast<uint8_t*>(sbuf));
        }
        (void)g;
        (void)i;
        (void)sbuf;
    }
    // vector memory operations issue() puts in flight
    static constexpr int kIssueOps = (KV == KV_FP16) ? 16 : (KV == KV_INT8) ? 9 : 8;
    // The chunk's operands from LDS.  8-bit: lane (i, g) reads token row i's
    // chunks 4h + g of K (kofs[h]) and the 8 bytes d = 8i.. of V tokens
    // 16(e>>2) + 4g + (e&3) (vofs[e&3]).  FP16: token row i's chunks
    // 8h + 2g + sub of K (kofs[2h + sub]).
    __device__ __forceinline__ static void read(Chunk<KV>& c, const Meta& m, const uint8_t* lbuf,
                                                const f32x4* sbuf, const int kofs[4], const int vofs[4],
                                                int g) {
        if constexpr (KV == KV_FP16) {
#pragma unroll
            for (int pg = 0; pg < 2; ++pg)
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    c.kh[pg][kc] = *reinterpret_cast<const f16x8*>(lbuf + 4096 * pg + kofs[kc]);
#pragma unroll
            for (int e = 0; e < 8; ++e) c.v16[e] = m.v16[e];
        } else {
#pragma unroll
            for (int pg = 0; pg < 2; ++pg)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    c.k[pg][h] = *reinterpret_cast<const u32x4*>(lbuf + 2048 * pg + kofs[h]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                c.v8[e] = *reinterpret_cast<const u32x2*>(lbuf + 4096 + 2048 * (e >> 2) + vofs[e & 3]);
        }
        if constexpr (KV == KV_INT8) {                 // scales of tokens 4g..4g+3 of each page
#pragma unroll
            for (int pg = 0; pg < 2; ++pg) {
                c.ks[pg] = sbuf[4 * pg + g];
                c.vs[pg] = sbuf[4 * (2 + pg) + g];
            }
        }
        (void)g;
        c.valid_blk = m.valid_blk;
    }

    // K of page pg as the four MFMA A operands (d-slots kc = 2h + sub).
    __device__ __forceinline__ static void k_operands(const Chunk<KV>& c, int pg, f16x8 out[4]) {
        if constexpr (KV == KV_FP16) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) out[kc] = c.kh[pg][kc];
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                out[2 * h + 0] = codes8_to_f16x8<KV>(c.k[pg][h][0], c.k[pg][h][1]);
                out[2 * h + 1] = codes8_to_f16x8<KV>(c.k[pg][h][2], c.k[pg][h][3]);
            }
        }
    }

    // V^T operands: vt[col] holds V[t(g, e)][8*(l%16) + col] for e = 0..7.
    __device__ __forceinline__ static void v_operands(const Chunk<KV>& c, f16x8 vt[8]) {
        if constexpr (KV == KV_FP16) {
            // 16-bit transpose: pair (e, e+1) of column col = perm of dword col/2.
#pragma unroll
            for (int col = 0; col < 8; ++col) {
                const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
                const int w = col >> 1;
                const u32x4 r = u32x4{__builtin_amdgcn_perm(c.v16[1][w], c.v16[0][w], sel),
                                      __builtin_amdgcn_perm(c.v16[3][w], c.v16[2][w], sel),
                                      __builtin_amdgcn_perm(c.v16[5][w], c.v16[4][w], sel),
                                      __builtin_amdgcn_perm(c.v16[7][w], c.v16[6][w], sel)};
                vt[col] = __builtin_bit_cast(f16x8, r);
            }
        } else {
            // Byte transpose: for tokens (e, e+1) and half hf, interleave their
            // bytes, then each fp8/int8 -> fp16 pair conversion yields one
            // (token e, token e+1) pair of a column.
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const uint32_t a = c.v8[2 * pr + 1][hf], b = c.v8[2 * pr][hf];
                    const uint32_t p01 = __builtin_amdgcn_perm(a, b, 0x05010400u);  // cols 0,1
                    const uint32_t p23 = __builtin_amdgcn_perm(a, b, 0x07030602u);  // cols 2,3
                    const f16x2 c0 = codes2_to_f16x2<KV, false>(p01);
                    const f16x2 c1 = codes2_to_f16x2<KV, true>(p01);
                    const f16x2 c2 = codes2_to_f16x2<KV, false>(p23);
                    const f16x2 c3 = codes2_to_f16x2<KV, true>(p23);
                    vt[4 * hf + 0][2 * pr] = c0[0]; vt[4 * hf + 0][2 * pr + 1] = c0[1];
                    vt[4 * hf + 1][2 * pr] = c1[0]; vt[4 * hf + 1][2 * pr + 1] = c1[1];
                    vt[4 * hf + 2][2 * pr] = c2[0]; vt[4 * hf + 2][2 * pr + 1] = c2[1];
                    vt[4 * hf + 3][2 * pr] = c3[0]; vt[4 * hf + 3][2 * pr + 1] = c3[1];
                }
            }
        }
    }

    // Zero V codes of tokens that must not contribute (past the end, bad
    // page): a zero weight times a NaN poison value would still be NaN (INT8:
    // the token's scale too, which may be a NaN poison).  FP16 masks the
    // operands instead (mask_vt), leaving the loaded words untouched.
    __device__ __forceinline__ static void mask_v(Chunk<KV>& c, const bool ok[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {          // selects, not branches: stays in registers
            c.v8[e][0] = ok[e] ? c.v8[e][0] : 0u;
            c.v8[e][1] = ok[e] ? c.v8[e][1] : 0u;
            if constexpr (KV == KV_INT8) c.vs[e >> 2][e & 3] = ok[e] ? c.vs[e >> 2][e & 3] : 0.0f;
        }
    }
};

// Online-softmax state of one wave: lane (i, g) owns query head i.
struct WaveState {
    float m, l;                    // running max (log2 units), lane-partial sum
    f32x4 acc[8];                  // O^T[d = 32g + 8r + c][head i] in acc[c][r]
};

// lim1: the lane's query row scores keys below lim1 = min(tok1, its causal
// limit) (tok1 itself for a one-token decode).  V validity (inside the
// partition, on a valid page) is a property of the token, shared by every
// row, and is only needed for a partial chunk; the causal limit masks scores.
// With LO, tokens below lo are excluded too (a sliding window's start).
template <bool LO>
__device__ __forceinline__ void token_ok(bool v[8], int ctok, int lo, int lim, int valid_blk, int g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int pg = e >> 2;
        const int t = ctok + 16 * pg + 4 * g + (e & 3);
        v[e] = (t < lim) && (!LO || t >= lo) && ((valid_blk >> pg) & 1);
    }
}

// One chunk for RG groups of 16 query rows (lane (i, g) holds row i of each
// group): the chunk's K and V operands are converted once and feed every
// group's MFMAs.  LO: a lane's row also ignores keys below its lo1 (its
// sliding window's start).
template <int KV, int NW, bool LO, int RG>
__device__ __forceinline__ void process_chunk(WaveState (&st)[RG], Chunk<KV>& cur, const f16x8 (&qop)[RG][4],
                                              float cscale, int ctok, int tok1, const int (&lo1)[RG],
                                              const int (&lim1)[RG], int g) {
    using Dk = Decode<KV, NW>;
    const bool partial = (ctok + 32 > tok1) || (cur.valid_blk != 3);
    if constexpr (KV != KV_FP16)
        if (partial) {
            bool vok[8];
            token_ok<false>(vok, ctok, 0, tok1, cur.valid_blk, g);
            Dk::mask_v(cur, vok);
        }

    // S^T = K Q^T per page: lane holds tokens 4g + r of page pg, head i.
    float x[RG][8];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
        f16x8 kop[4];
        Dk::k_operands(cur, pg, kop);
#pragma unroll
        for (int q = 0; q < RG; ++q) {
            f32x4 s = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) s = mfma16(kop[kc], qop[q][kc], s);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sc = cscale;
                if constexpr (KV == KV_INT8) sc *= cur.ks[pg][r];
                x[q][4 * pg + r] = s[r] * sc;
            }
        }
    }
    f16x8 pop[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        // scored tokens of the lane's eight t(g, e)
        bool ok[8];
        token_ok<LO>(ok, ctok, lo1[q], lim1[q], cur.valid_blk, g);
        float mx = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[q][e] = ok[e] ? x[q][e] : -__builtin_inff();
            mx = fmaxf(mx, x[q][e]);
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(st[q].m, mx);
        // m_new is -inf only while every key so far is masked; keep the state finite
        const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
        const float alpha = fast_exp2(st[q].m - m_use);
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float pe = fast_exp2(x[q][e] - m_use);
            psum += pe;
            if constexpr (KV == KV_INT8) pe *= cur.vs[e >> 2][e & 3] * kInt8PFold;
            pop[q][e] = (f16)pe;
        }
        st[q].l = st[q].l * alpha + psum;
        st[q].m = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < 8; ++c) st[q].acc[c] *= alpha;
        }
    }
    f16x8 vt[8];
    Dk::v_operands(cur, vt);
    if constexpr (KV == KV_FP16)
        if (partial) {
            bool vok[8];
            token_ok<false>(vok, ctok, 0, tok1, cur.valid_blk, g);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[c][e] = vok[e] ? vt[c][e] : (f16)0.0f;
        }
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
        for (int c = 0; c < 8; ++c) st[q].acc[c] = mfma16(vt[c], pop[q], st[q].acc[c]);
}

// Query rows of one workgroup column: column c is row r = cg16 + c of its
// (sequence, KV head) group, i.e. query token qa + r / G (position-major) and
// head kvh * G + r % G.
struct RowMap {
    int64_t base;                   // row of the group's first query token's first head
    int Hq, cg16, gshift;           // G = 1 << gshift (G is a power of two)
    __device__ __forceinline__ int64_t row(int c) const {
        const int r = cg16 + c;
        return base + ((r >> gshift) * Hq + (r & ((1 << gshift) - 1)));
    }
};

template <int KV, int NW, bool MQ, int RG>
__global__ __launch_bounds__(64 * NW) void paged_decode_kernel(DecodeParams p) {
    using Dk = Decode<KV, NW>;
    static_assert(MQ || RG == 1, "a one-token decode has one row group");
    // Pages stream through per-wave LDS buffers (two 8 KiB chunks per wave);
    // the wave merge reuses that space afterwards.
    __shared__ __attribute__((aligned(16))) uint8_t s_dma[NW][2][8192];
    // INT8 per-token scales of each buffer's chunk (slots 0..15 used)
    __shared__ __attribute__((aligned(16))) f32x4 s_scl[KV == KV_INT8 ? NW : 1][2][KV == KV_INT8 ? 64 : 1];
    float* smem = reinterpret_cast<float*>(&s_dma[0][0][0]);
    // Workgroup -> (partition, workgroup column of RG row groups).  The usual
    // grid is (partition, KV head x column, sequence).  When the whole grid
    // fits on the chip at once (p.xcd_local), it is one-dimensional instead:
    // the hardware deals workgroups to the eight XCDs in turn (i % 8), and
    // workgroup i takes the (sequence, KV head) unit 8 (i / 8 / (ncgw nparts))
    // + i % 8, so every partition and column of a unit runs on one XCD; within
    // the unit the columns of one partition are neighbours, so the second
    // column's page reads hit that XCD's L2.
    int part, b, kvh, cgw;
    if (p.xcd_local) {
        const int i8 = blockIdx.x & 7, rest = blockIdx.x >> 3;
        const int per_unit = p.ncgw * p.nparts;
        const int unit = 8 * (rest / per_unit) + i8;
        if (unit >= p.num_seqs * p.kv.num_kv_heads) return;       // padding of the last eight units
        const int within = rest % per_unit;
        part = within / p.ncgw;
        cgw = within % p.ncgw;
        kvh = unit % p.kv.num_kv_heads;
        b = unit / p.kv.num_kv_heads;
    } else {
        part = blockIdx.x;
        b = blockIdx.z;
        kvh = MQ ? (int)blockIdx.y / p.ncgw : (int)blockIdx.y;
        cgw = MQ ? (int)blockIdx.y - kvh * p.ncgw : 0;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Chunk c of the partition goes to the wave with cw = c mod NW, cw =
    // NW - 1 - wave: waves w and w + NW/2 share a SIMD and the second one
    // issues behind the first, so the last chunk (the step's new token in a
    // decode step) belongs to wave 0, which has slack for the append.
    const int cw = NW - 1 - wave;
    const int g = lane >> 4, i = lane & 15;
    const int Hq = p.num_q_heads, G = Hq / p.kv.num_kv_heads;
    // lengths beyond the host-stated bound are clamped so that no page id
    // outside the table is ever read
    const int P = p.partition_tokens;
    int blk0 = part * (P / BS);                                  // MQ: set once L is known
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;
    // The first segment's page ids do not depend on the sequence length:
    // fetch them now, alongside the length (entries past the end are masked
    // once the length is known; the index stays inside the table row).
    const int tb0 = 2 * (cw + (lane >> 1) * NW) + (lane & 1);
    int tbl0 = MQ ? 0 : bt[min(blk0 + tb0, p.max_blocks - 1)];
    const int L = max(0, min(p.context_lens[b], p.max_context_len));
    const int nparts = p.nparts;
    // this workgroup's query rows: NC columns of the 16-wide N tile
    int n = 1;
    int64_t qa = b;                                              // the sequence's first query token
    if constexpr (MQ) {
        qa = p.cu_q_lens[b];
        n = min(max(p.cu_q_lens[b + 1] - p.cu_q_lens[b], 0), p.max_q_len);
    }
    // the column's RG row groups: group q holds rows 16 (RG cgw + q) + [0, NC[q])
    RowMap rm[RG];
    int NC[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        rm[q] = RowMap{qa * Hq + kvh * G, Hq, 16 * (RG * cgw + q), __builtin_ctz(G)};
        NC[q] = MQ ? min(16, n * G - 16 * (RG * cgw + q)) : G;
    }
    if (MQ && NC[0] <= 0) return;                                // no rows: no partials, no merge
    // Sliding window (MQ, p.window > 0): row j sees keys from L - n + j -
    // window + 1 on, so no row needs a key below lo_min (row 0's start); the
    // workgroups' partition index counts from the partition that holds it.
    int lo_min = 0, first_part = 0;
    if constexpr (MQ)
        if (p.window > 0) {
            lo_min = max(0, L - n + 1 - p.window);
            first_part = lo_min / P;
        }
    const int nparts_b = (L + P - 1) / P - first_part;
    int tok0 = (part + first_part) * P;

    if (part >= nparts_b) {                                      // partition past the end
        // an empty partial (or, written directly, the output of a sequence
        // with no key at all)
#pragma unroll
        for (int q = 0; q < RG; ++q)
            for (int idx = tid; idx < NC[q] * D; idx += 64 * NW) {
                const int j = idx / D, d = idx % D;
                const int64_t row = rm[q].row(j);
                float* od = p.direct ? p.out + row * D : p.o_parts + (row * nparts + part) * D;
                float* ld = p.direct ? p.lse + row : p.lse_parts + row * nparts + part;
                od[d] = 0.0f;
                if (d == 0) *ld = -__builtin_inff();
            }
        return;
    }
    const int tok1 = min(tok0 + P, L);
    if constexpr (MQ) {
        // skip the chunks below every row's window, then fetch the first
        // segment's page ids (deferred until the length was known)
        tok0 += 32 * (max(0, lo_min - tok0) / 32);
        blk0 = tok0 / BS;
        tbl0 = bt[min(blk0 + tb0, p.max_blocks - 1)];
    }
    const int nblk = (tok1 - tok0 + BS - 1) / BS;
    const int nchunks = (nblk + 1) / 2;

    // Fused append: the partition that holds the step's own token (position
    // L - 1) writes it to its page, quantized exactly as plc_kv_append_quant
    // does, by the wave that owns the token's chunk (lanes 0-15: K, 16-31: V,
    // eight values each).  That wave does not wait for the stores: it keeps
    // the codes (and INT8 scales) in registers and writes them over the
    // token's row in its LDS copy of the chunk once the chunk's pages have
    // landed, so whatever the page loads saw of the row does not matter.  No
    // other wave reads that page.
    const bool appends = p.k_new != nullptr && part == (L - 1) / P;     // uniform in the workgroup
    const int tok_chunk = appends ? (L - 1 - tok0) / 32 : -1;           // chunk index in the partition
    const bool app_wave = appends && cw == tok_chunk % NW;
    u32x2 app_codes = u32x2{0, 0};                                      // 8-bit codes of the lane's slice
    f16x8 app_x = f16x8{0, 0, 0, 0, 0, 0, 0, 0};                         // FP16 values of the lane's slice
    float app_sigma = 0.0f;                                             // INT8 scale (lanes 0 and 16)
    if (app_wave && lane < 32) {
        const int which = lane >> 4, sl = lane & 15;
        const int pos = L - 1;
        const int pg = bt[pos / BS];
        app_x = *reinterpret_cast<const f16x8*>(
            static_cast<const f16*>(which ? p.v_new : p.k_new) + ((int64_t)b * p.kv.num_kv_heads + kvh) * D + 8 * sl);
        if constexpr (KV != KV_FP16) {
            float sc = 1.0f;
            if constexpr (KV == KV_E4M3) sc = (which ? p.kv.v_scale : p.kv.k_scale)[kvh];
            app_codes = quantize_slice<KV>(app_x, sc, app_sigma);
        }
        if (pg >= 0 && pg < p.kv.num_blocks) {
            const int64_t crow = ((int64_t)pg * p.kv.num_kv_heads + kvh) * BS + (pos % BS);
            void* cache = const_cast<void*>(which ? p.kv.v : p.kv.k);
            if constexpr (KV == KV_FP16) {
                *reinterpret_cast<f16x8*>(static_cast<f16*>(cache) + crow * D + 8 * sl) = app_x;
            } else {
                *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(cache) + crow * D + 8 * sl) = app_codes;
                if constexpr (KV == KV_INT8)
                    if (sl == 0) const_cast<float*>(which ? p.kv.v_scale : p.kv.k_scale)[crow] = app_sigma;
            }
        }
    }
    // the token's row inside its chunk: page tpg, row tr
    const int t_in = appends ? (L - 1) - (tok0 + 32 * tok_chunk) : 0;
    const int tpg = t_in >> 4, tr = t_in & 15;
    // FP16 V reaches registers, not LDS: every lane (i, g) takes the V slice
    // d = 8i.. from lane 16 + i, for when g holds the token's row (token 4g +
    // e%4 of page e/4 in register e)
    u32x4 app_v = u32x4{0, 0, 0, 0};
    if constexpr (KV == KV_FP16)
        if (app_wave) {
            const u32x4 xs = __builtin_bit_cast(u32x4, app_x);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                app_v[w] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 + i) << 2, (int)xs[w]);
        }

    // Q^T operand: lane (i, g) holds row (column) i, d = 64*(kc/2) + 16g +
    // 8*(kc%2) + [0, 8); its causal limit: position L - n + j sees keys below
    // L - n + j + 1 (L for a one-token decode; nothing for a spare column).
    f16x8 qop[RG][4];
    int lim1[RG], lo1[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        const bool live = i < NC[q];
        const int lim = live ? L - n + 1 + ((rm[q].cg16 + i) >> rm[q].gshift) : 0;
        lim1[q] = MQ ? min(lim, tok1) : tok1;         // and inside the partition
        lo1[q] = p.window > 0 ? lim - p.window : 0;   // the row's window start (MQ)
        const f16* qr = static_cast<const f16*>(p.q) + rm[q].row(live ? i : 0) * D;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            if (live)
                qop[q][kc] = *reinterpret_cast<const f16x8*>(qr + 64 * (kc >> 1) + 16 * g + 8 * (kc & 1));
            else
                qop[q][kc] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    // value scale applied once to the normalized output; INT8 carries its
    // per-token scale (times kInt8PFold: no fp16 overflow, few subnormals) in P
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / kInt8PFold;

    WaveState st[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        st[q].m = -__builtin_inff();
        st[q].l = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) st[q].acc[c] = f32x4{0, 0, 0, 0};
    }

    // per-lane LDS offsets of the DMA path (see Decode::issue / Decode::read)
    int dsrc[Dk::kDmaPerPage], kofs[4], vofs[4];
#pragma unroll
    for (int q = 0; q < Dk::kDmaPerPage; ++q) dsrc[q] = Dk::dma_src(lane, q);
    if constexpr (KV == KV_FP16) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kofs[kc] = i * (2 * D) + 16 * ((8 * (kc >> 1) + 2 * g + (kc & 1)) ^ i);
#pragma unroll
        for (int x = 0; x < 4; ++x) vofs[x] = 0;
    } else {
        const int sk = Dk::swap02(i);
#pragma unroll
        for (int h = 0; h < 4; ++h) kofs[h] = sk * D + 16 * ((4 * (h & 1) + g) ^ Dk::kap(sk));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int sv = Dk::swap02(4 * g + x);
            vofs[x] = sv * D + 16 * ((i >> 1) ^ Dk::kap(sv)) + 8 * (i & 1);
        }
    }

    // The wave's chunks are walked in segments of at most 32 whose 64 page ids
    // sit one per lane of a VGPR (read with readlane).  Inside a segment the
    // next chunk is always in flight: the prefetch target is clamped to the
    // segment's last chunk, so a load past the end re-reads data already
    // loaded (cache hits) and no load is conditional -- which lets the
    // compiler wait only for the chunk in use.
    // The wave's chunks are interleaved with the other waves' (chunk wave +
    // it*NW), so at any time the workgroup streams neighbouring pages.
    const int my_chunks = cw < nchunks ? (nchunks - cw + NW - 1) / NW : 0;
    for (int seg = 0; seg < my_chunks; seg += 32) {
        const int segn = min(32, my_chunks - seg);
        const int tch = cw + (seg + (lane >> 1)) * NW;        // chunk of this lane's page
        const int tb = 2 * tch + (lane & 1);
        const bool tok = lane < 2 * segn && tb < nblk;
        const int tbl = !tok ? -1 : (seg == 0 ? tbl0 : bt[blk0 + tb]);
        // two LDS buffers in ping-pong: the next chunk's DMA is in flight
        // while the current one is computed; before reading a chunk the
        // wave waits until only the next chunk's operations are pending
        // (none after the segment's last chunk, so no DMA outlives it)
        auto issue = [&](typename Dk::Meta& m, int b, int k) __attribute__((always_inline)) {
            const int ch = cw + (seg + k) * NW;
            Dk::issue(m, &s_dma[wave][b][0], &s_scl[KV == KV_INT8 ? wave : 0][b][0], p, kvh, __builtin_amdgcn_readlane(tbl, 2 * k),
                      __builtin_amdgcn_readlane(tbl, 2 * k + 1), 2 * ch + 1 < nblk, lane, dsrc);
        };
        // consume chunk k of the segment from buffer bf: the appending wave
        // first writes the step's token over its row (after the pages landed)
        Chunk<KV> c;
        auto consume = [&](typename Dk::Meta& m, int bf, int k) __attribute__((always_inline)) {
            const int ch = cw + (seg + k) * NW;
            uint8_t* lb = &s_dma[wave][bf][0];
            f32x4* sb = &s_scl[KV == KV_INT8 ? wave : 0][bf][0];
            const bool patch = app_wave && ch == tok_chunk;                 // uniform
            if (patch) {
                if constexpr (KV == KV_FP16) {
                    if (lane < 16)                      // K row tr: chunk sl at slot sl ^ tr
                        *reinterpret_cast<f16x8*>(lb + 4096 * tpg + 256 * tr + 16 * (lane ^ tr)) = app_x;
                } else {
                    const int srow = Dk::swap02(tr);
                    if (lane < 32) {
                        const int which = lane >> 4, sl = lane & 15;
                        *reinterpret_cast<u32x2*>(lb + 4096 * which + 2048 * tpg + 128 * srow +
                                                  16 * ((sl >> 1) ^ Dk::kap(srow)) + 8 * (sl & 1)) = app_codes;
                    }
                    if constexpr (KV == KV_INT8)
                        if (lane == 0 || lane == 16)    // [K | V][page][4 tokens] slots of f32x4
                            reinterpret_cast<float*>(sb)[4 * (((lane >> 4) << 3) | (tpg << 2) | (tr >> 2)) + (tr & 3)] =
                                app_sigma;
                }
            }
            Dk::read(c, m, lb, sb, kofs, vofs, g);
            if constexpr (KV == KV_FP16)
                if (patch && g == (tr >> 2)) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (e == 4 * tpg + (tr & 3)) c.v16[e] = app_v;
                }
            process_chunk<KV, NW, MQ, RG>(st, c, qop, cscale, tok0 + 32 * ch, tok1, lo1, lim1, g);
        };
        typename Dk::Meta ma, mb;
        issue(ma, 0, 0);
        for (int k = 0; k < segn; k += 2) {
            if (k + 1 < segn) {
                issue(mb, 1, k + 1);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Dk::kIssueOps) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            consume(ma, 0, k);
            if (k + 1 >= segn) break;
            if (k + 2 < segn) {
                issue(ma, 0, k + 2);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Dk::kIssueOps) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            consume(mb, 1, k + 1);
        }
    }
    // ---- merge the waves of the workgroup (fixed order), one row group at a time ----
    constexpr int AST = D + 4;                         // padded head stride (floats)
    float* s_m = smem;                                 // [NW][16]
    float* s_l = smem + NW * 16;                       // [NW][16]
    float* s_acc = smem + NW * 32;                     // [NW][16][AST]
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        __syncthreads();                               // the DMA buffers / the previous group's state
        if (NC[q] <= 0) break;                         // uniform: no rows in this group or later ones
        float l_run = st[q].l;
        l_run += shfl_xor(l_run, 16);
        l_run += shfl_xor(l_run, 32);
        if (g == 0) {
            s_m[wave * 16 + i] = st[q].m;
            s_l[wave * 16 + i] = l_run;
        }
        if (i < NC[q]) {
            float* dst = s_acc + ((int64_t)wave * 16 + i) * AST + 32 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f32x4 lo = f32x4{st[q].acc[0][r], st[q].acc[1][r], st[q].acc[2][r], st[q].acc[3][r]};
                f32x4 hi = f32x4{st[q].acc[4][r], st[q].acc[5][r], st[q].acc[6][r], st[q].acc[7][r]};
                *reinterpret_cast<f32x4*>(dst + 8 * r) = lo;
                *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = hi;
            }
        }
        __syncthreads();
        // thread t: four columns of one row per pass
        for (int e = tid; e < NC[q] * (D / 4); e += 64 * NW) {
            const int j = e / (D / 4), d = 4 * (e % (D / 4));
            // every wave's state in one LDS round trip, then no branch
            float mw[NW], lw[NW];
            f32x4 aw[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                mw[w] = s_m[w * 16 + j];
                lw[w] = s_l[w * 16 + j];
                aw[w] = *reinterpret_cast<const f32x4*>(s_acc + (w * 16 + j) * AST + d);
            }
            float M = -__builtin_inff();
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w]);
            const bool any = M != -__builtin_inff();
            float Lsum = 0.0f;
            f32x4 O = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float wt = any ? fast_exp2(mw[w] - M) : 0.0f;
                Lsum += lw[w] * wt;
                O += wt * aw[w];
            }
            const bool empty = !(Lsum > 0.0f);
            const f32x4 ov = O * (empty ? 0.0f : vscale / Lsum);
            const float lv = empty ? -__builtin_inff() : (M + __builtin_log2f(Lsum)) * kLn2;
            const int64_t row = rm[q].row(j);
            // a single partition per sequence: the normalized partial is the output
            float* od = p.direct ? p.out + row * D + d : p.o_parts + (row * nparts + part) * D + d;
            float* ld = p.direct ? p.lse + row : p.lse_parts + row * nparts + part;
            *reinterpret_cast<f32x4*>(od) = ov;
            if (d == 0) *ld = lv;
        }
    }
}

// ---------------------------------------------------------------- head dim 256
// Split-D (1Cat-vLLM README, Layer 2 "D256 Split-D"): a 256-wide head is two
// 128-wide halves.  Each 32-token chunk arrives as two half-chunks in the
// 128-wide LDS layout; the scores sum both halves' QK^T before the softmax,
// and PV runs per half into its own accumulators, so the probabilities are
// computed once for the whole row.  The GQA group (any size up to 16; the
// pages pack six heads, Layer 2 "GQA Multi-Head Packing") is the MFMA N
// dimension, as in the 128-wide kernel.  One query token per sequence;
// partials only (the merge is plc_lse_merge's kernel).
struct WaveState2 {
    float m, l;
    f32x4 acc[2][8];               // half h: O^T[d = 128h + 32g + 8r + c][head i] in acc[h][c][r]
};

// lim1 / lo1: the lane's row scores keys in [lo1, lim1) (lim1 = tok1 and no
// lower bound for a one-token decode); V is zeroed only for keys outside the
// partition or on invalid pages, since every row shares the V operands.
template <int KV, int NW, bool LO>
__device__ __forceinline__ void process_chunk_d256(WaveState2& st, Chunk<KV> cur[2], const f16x8 qop[2][4],
                                                   float cscale, int ctok, int tok1, int lo1, int lim1, int g) {
    using Dk = Decode<KV, NW, 256>;
    bool ok[8], vok[8];
    token_ok<LO>(ok, ctok, lo1, lim1, cur[0].valid_blk, g);
    token_ok<false>(vok, ctok, 0, tok1, cur[0].valid_blk, g);
    const bool partial = (ctok + 32 > tok1) || (cur[0].valid_blk != 3);
    if constexpr (KV != KV_FP16)
        if (partial) {
            Dk::mask_v(cur[0], vok);
            Dk::mask_v(cur[1], vok);
        }
    float x[8];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
        f32x4 s = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f16x8 kop[4];
            Dk::k_operands(cur[h], pg, kop);
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) s = mfma16(kop[kc], qop[h][kc], s);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sc = cscale;
            if constexpr (KV == KV_INT8) sc *= cur[0].ks[pg][r];
            x[4 * pg + r] = s[r] * sc;
        }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = ok[e] ? x[e] : -__builtin_inff();
        mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    float psum = 0.0f;
    f16x8 pop;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float pe = fast_exp2(x[e] - m_use);
        psum += pe;
        if constexpr (KV == KV_INT8) pe *= cur[0].vs[e >> 2][e & 3] * kInt8PFold;
        pop[e] = (f16)pe;
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) st.acc[h][c] *= alpha;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f16x8 vt[8];
        Dk::v_operands(cur[h], vt);
        if constexpr (KV == KV_FP16)
            if (partial) {
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) vt[c][e] = vok[e] ? vt[c][e] : (f16)0.0f;
            }
#pragma unroll
        for (int c = 0; c < 8; ++c) st.acc[h][c] = mfma16(vt[c], pop, st.acc[h][c]);
    }
}

// MQ: several query tokens per sequence (verification, sliding window), the
// rows of a (sequence, KV head) in groups of 16 as in the 128-wide kernel.
template <int KV, int NW, bool MQ>
__global__ __launch_bounds__(64 * NW) void paged_decode256_kernel(DecodeParams p) {
    using Dk = Decode<KV, NW, 256>;
    constexpr int DW = 256;
    // [wave][buffer][half]: two buffers in ping-pong, each chunk's two halves
    __shared__ __attribute__((aligned(16))) uint8_t s_dma[NW][2][2][8192];
    __shared__ __attribute__((aligned(16))) f32x4 s_scl[KV == KV_INT8 ? NW : 1][2][KV == KV_INT8 ? 64 : 1];
    float* smem = reinterpret_cast<float*>(&s_dma[0][0][0][0]);
    const int part = blockIdx.x, b = blockIdx.z;
    const int kvh = MQ ? (int)blockIdx.y / p.ncg : (int)blockIdx.y;
    const int cg = MQ ? (int)blockIdx.y - kvh * p.ncg : 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = NW - 1 - wave;
    const int g = lane >> 4, i = lane & 15;
    const int Hq = p.num_q_heads, Hkv = p.kv.num_kv_heads, G = Hq / Hkv;
    const int P = p.partition_tokens;
    int blk0 = part * (P / BS);
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;
    const int tb0 = 2 * (cw + (lane >> 1) * NW) + (lane & 1);
    int tbl0 = MQ ? 0 : bt[min(blk0 + tb0, p.max_blocks - 1)];
    const int L = max(0, min(p.context_lens[b], p.max_context_len));
    const int nparts = p.nparts;
    int n = 1;
    int64_t qa = b;                                                 // the sequence's first query token
    if constexpr (MQ) {
        qa = p.cu_q_lens[b];
        n = min(max(p.cu_q_lens[b + 1] - p.cu_q_lens[b], 0), p.max_q_len);
    }
    const int NC = MQ ? min(16, n * G - 16 * cg) : G;               // rows of this workgroup
    if (MQ && NC <= 0) return;
    // row of column c: r = 16 cg + c is query token qa + r / G, head kvh G + r % G
    auto row_of = [&](int c) __attribute__((always_inline)) {
        const int r = 16 * cg + c;
        return (qa + r / G) * Hq + (int64_t)kvh * G + r % G;
    };
    int lo_min = 0, first_part = 0;
    if constexpr (MQ)
        if (p.window > 0) {
            lo_min = max(0, L - n + 1 - p.window);
            first_part = lo_min / P;
        }
    const int nparts_b = (L + P - 1) / P - first_part;
    int tok0 = (part + first_part) * P;
    if (part >= nparts_b) {                                        // partition past the end
        for (int idx = tid; idx < NC * DW; idx += 64 * NW) {
            const int j = idx / DW, d = idx % DW;
            const int64_t row = row_of(j);
            p.o_parts[(row * nparts + part) * DW + d] = 0.0f;
            if (d == 0) p.lse_parts[row * nparts + part] = -__builtin_inff();
        }
        return;
    }
    const int tok1 = min(tok0 + P, L);
    if constexpr (MQ) {
        // skip the chunks below every row's window, then fetch the first
        // segment's page ids
        tok0 += 32 * (max(0, lo_min - tok0) / 32);
        blk0 = tok0 / BS;
        tbl0 = bt[min(blk0 + tb0, p.max_blocks - 1)];
    }
    const int nblk = (tok1 - tok0 + BS - 1) / BS;
    const int nchunks = (nblk + 1) / 2;

    if (p.k_new != nullptr && part == (L - 1) / P) {
        // fused append of the step's token (position L - 1), quantized as
        // plc_kv_append_quant does: wave 0, 32 lanes per K / V row; every
        // wave waits for the stores before it loads
        if (wave == 0) {
            const int which = lane >> 5, sl = lane & 31;
            const int pos = L - 1;
            const int pg = bt[pos / BS];
            const f16x8 x = *reinterpret_cast<const f16x8*>(
                static_cast<const f16*>(which ? p.v_new : p.k_new) + ((int64_t)b * Hkv + kvh) * DW + 8 * sl);
            const bool ok = pg >= 0 && pg < p.kv.num_blocks;
            const int64_t crow = ((int64_t)(ok ? pg : 0) * Hkv + kvh) * BS + (pos % BS);
            void* cache = const_cast<void*>(which ? p.kv.v : p.kv.k);
            if constexpr (KV == KV_FP16) {
                if (ok) *reinterpret_cast<f16x8*>(static_cast<f16*>(cache) + crow * DW + 8 * sl) = x;
            } else {
                float s = 1.0f, sigma = 0.0f;
                if constexpr (KV == KV_E4M3) s = (which ? p.kv.v_scale : p.kv.k_scale)[kvh];
                const u32x2 w = quantize_slice<KV, 32>(x, s, sigma);   // all 64 lanes take part
                if (ok) {
                    *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(cache) + crow * DW + 8 * sl) = w;
                    if constexpr (KV == KV_INT8)
                        if (sl == 0) const_cast<float*>(which ? p.kv.v_scale : p.kv.k_scale)[crow] = sigma;
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
    }

    // Q^T operands per half: lane (i, g) holds column i, d = 128h + 64*(kc/2) +
    // 16g + 8*(kc%2) + [0, 8); columns past the rows are zero.  Its causal
    // limit: position L - n + j sees keys below L - n + j + 1 (L for a
    // one-token decode), and with a window none below that minus the window.
    f16x8 qop[2][4];
    {
        const f16* q = static_cast<const f16*>(p.q) + row_of(i < NC ? i : 0) * DW;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                qop[h][kc] = i < NC ? *reinterpret_cast<const f16x8*>(q + 128 * h + 64 * (kc >> 1) + 16 * g + 8 * (kc & 1))
                                    : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int lim = i < NC ? L - n + 1 + (16 * cg + i) / G : 0;
    const int lim1 = MQ ? min(lim, tok1) : tok1;
    const int lo1 = p.window > 0 ? lim - p.window : 0;
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / kInt8PFold;

    WaveState2 st;
    st.m = -__builtin_inff();
    st.l = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) st.acc[h][c] = f32x4{0, 0, 0, 0};

    int dsrc[Dk::kDmaPerPage], kofs[4], vofs[4];
#pragma unroll
    for (int q = 0; q < Dk::kDmaPerPage; ++q) dsrc[q] = Dk::dma_src(lane, q);
    if constexpr (KV == KV_FP16) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kofs[kc] = i * (2 * D) + 16 * ((8 * (kc >> 1) + 2 * g + (kc & 1)) ^ i);
#pragma unroll
        for (int x = 0; x < 4; ++x) vofs[x] = 0;
    } else {
        const int sk = Dk::swap02(i);
#pragma unroll
        for (int h = 0; h < 4; ++h) kofs[h] = sk * D + 16 * ((4 * (h & 1) + g) ^ Dk::kap(sk));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int sv = Dk::swap02(4 * g + x);
            vofs[x] = sv * D + 16 * ((i >> 1) ^ Dk::kap(sv)) + 8 * (i & 1);
        }
    }
    // vector memory operations of one chunk (both halves; INT8 scales once)
    constexpr int kOps = 2 * Dk::kIssueOps - (KV == KV_INT8 ? 1 : 0);

    const int my_chunks = cw < nchunks ? (nchunks - cw + NW - 1) / NW : 0;
    for (int seg = 0; seg < my_chunks; seg += 32) {
        const int segn = min(32, my_chunks - seg);
        const int tch = cw + (seg + (lane >> 1)) * NW;
        const int tb = 2 * tch + (lane & 1);
        const bool tok = lane < 2 * segn && tb < nblk;
        const int tbl = !tok ? -1 : (seg == 0 ? tbl0 : bt[blk0 + tb]);
        auto issue = [&](typename Dk::Meta m[2], int bf, int k) __attribute__((always_inline)) {
            const int ch = cw + (seg + k) * NW;
            const int pb0 = __builtin_amdgcn_readlane(tbl, 2 * k), pb1 = __builtin_amdgcn_readlane(tbl, 2 * k + 1);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                Dk::issue(m[h], &s_dma[wave][bf][h][0], &s_scl[KV == KV_INT8 ? wave : 0][bf][0], p, kvh, pb0, pb1,
                          2 * ch + 1 < nblk, lane, dsrc, 128 * Dk::EB * h, h == 0);
        };
        auto consume = [&](typename Dk::Meta m[2], int bf, int k) __attribute__((always_inline)) {
            Chunk<KV> c[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                Dk::read(c[h], m[h], &s_dma[wave][bf][h][0], &s_scl[KV == KV_INT8 ? wave : 0][bf][0], kofs, vofs, g);
            process_chunk_d256<KV, NW, MQ>(st, c, qop, cscale, tok0 + 32 * (cw + (seg + k) * NW), tok1, lo1, lim1,
                                           g);
        };
        typename Dk::Meta ma[2], mb[2];
        issue(ma, 0, 0);
        for (int k = 0; k < segn; k += 2) {
            if (k + 1 < segn) {
                issue(mb, 1, k + 1);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOps) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            consume(ma, 0, k);
            if (k + 1 >= segn) break;
            if (k + 2 < segn) {
                issue(ma, 0, k + 2);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOps) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            consume(mb, 1, k + 1);
        }
    }
    __syncthreads();                                   // the merge below reuses the DMA buffers

    // ---- merge the waves of the workgroup (fixed order) ----
    float l_run = st.l;
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    constexpr int AST = DW + 4;
    float* s_m = smem;                                 // [NW][16]
    float* s_l = smem + NW * 16;                       // [NW][16]
    float* s_acc = smem + NW * 32;                     // [NW][NC][AST]
    if (g == 0) {
        s_m[wave * 16 + i] = st.m;
        s_l[wave * 16 + i] = l_run;
    }
    if (i < NC) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float* dst = s_acc + ((int64_t)wave * NC + i) * AST + 128 * h + 32 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f32x4 lo = f32x4{st.acc[h][0][r], st.acc[h][1][r], st.acc[h][2][r], st.acc[h][3][r]};
                f32x4 hi = f32x4{st.acc[h][4][r], st.acc[h][5][r], st.acc[h][6][r], st.acc[h][7][r]};
                *reinterpret_cast<f32x4*>(dst + 8 * r) = lo;
                *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = hi;
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < NC * DW; idx += 64 * NW) {
        const int j = idx / DW, d = idx % DW;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + j]);
        float Lsum = 0.0f, O = 0.0f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float wt = fast_exp2(s_m[w * 16 + j] - M);
                Lsum += s_l[w * 16 + j] * wt;
                O += s_acc[((int64_t)w * NC + j) * AST + d] * wt;
            }
        }
        const bool empty = !(Lsum > 0.0f);
        const int64_t row = row_of(j);
        p.o_parts[(row * nparts + part) * DW + d] = empty ? 0.0f : O * vscale / Lsum;
        if (d == 0) p.lse_parts[row * nparts + part] = empty ? -__builtin_inff() : (M + __builtin_log2f(Lsum)) * kLn2;
    }
}

template <int KV>
hipError_t launch_d256(const DecodeParams& p, hipStream_t s) {
    constexpr int NW = 4;
    static_assert(NW * 2 * 2 * 8192 >= 4 * NW * (32 + 16 * (256 + 4)), "merge space");
    dim3 grid(p.nparts, p.kv.num_kv_heads * p.ncg, p.num_seqs);
    if (p.cu_q_lens)
        hipLaunchKernelGGL((paged_decode256_kernel<KV, NW, true>), grid, dim3(64 * NW), 0, s, p);
    else
        hipLaunchKernelGGL((paged_decode256_kernel<KV, NW, false>), grid, dim3(64 * NW), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.merge) return e;
    // merged output requested: plc_lse_merge's kernel over the partials
    return launch_lse_merge(p.o_parts, p.lse_parts, p.total_q_tokens * p.num_q_heads, p.nparts, 256, p.out,
                            p.lse, s);
}

template <int KV, int NW, bool MQ, int RG>
hipError_t launch_mq(const DecodeParams& p, hipStream_t s) {
    // the wave-merge buffers live in the kernel's static DMA buffers
    // (NW * 16 KiB; at most NW * (32 + 16 * 132) floats are needed)
    static_assert(NW * 16384 >= 4 * NW * (32 + 16 * (D + 4)), "merge space");
    const size_t lds = 0;
    dim3 grid(p.nparts, p.kv.num_kv_heads * p.ncgw, p.num_seqs);
    if (p.xcd_local) {
        const int64_t units = (int64_t)p.num_seqs * p.kv.num_kv_heads;
        grid = dim3((unsigned)(((units + 7) / 8) * 8 * p.ncgw * p.nparts), 1, 1);
    }
    // The merged output: the partitions, then the merge kernel over their
    // partials, ordered after them by the kernel boundary (no fence inside
    // either kernel).  Measured against a merge by each group's last
    // workgroup inside the partition kernel, the second launch is the faster
    // one: that workgroup's agent-scope release (an L2 write-back per
    // workgroup) and its lone reads of the group's partials cost more than
    // the launch.
    hipLaunchKernelGGL((paged_decode_kernel<KV, NW, MQ, RG>), grid, dim3(64 * NW), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.merge || p.direct) return e;
    return launch_lse_merge(p.o_parts, p.lse_parts, p.total_q_tokens * p.num_q_heads, p.nparts, D, p.out,
                            p.lse, s);
}

// One-token decode: 4 waves for more than 8 heads per KV head, else 8.
// Several query tokens: 8 waves, with the launcher's row groups per
// workgroup (two per workgroup hold about 210 VGPRs, so two waves still share
// a SIMD); FP16 keeps one group per workgroup (its operands are twice as
// wide: two groups spill registers), 4 waves from three groups on.
template <int KV>
hipError_t launch_kv(const DecodeParams& p, hipStream_t s) {
    if (!p.cu_q_lens)
        return p.num_q_heads / p.kv.num_kv_heads > 8 ? launch_mq<KV, 4, false, 1>(p, s)
                                                     : launch_mq<KV, 8, false, 1>(p, s);
    if constexpr (KV == KV_FP16)
        return p.ncg > 2 ? launch_mq<KV, 4, true, 1>(p, s) : launch_mq<KV, 8, true, 1>(p, s);
    else
        return p.ncgw < p.ncg ? launch_mq<KV, 8, true, 2>(p, s) : launch_mq<KV, 8, true, 1>(p, s);
}

}  // namespace

hipError_t launch_decode_partials(const DecodeParams& p0, hipStream_t s) {
    // The XCD-local placement only when every workgroup is resident at once
    // (one 128 KiB-LDS workgroup per CU, 256 CUs): then the dispatch order
    // cannot delay any partition, and the row groups of a partition share
    // one XCD's L2.
    // Larger grids keep the sequence-major order, which starts a long
    // sequence's partitions together.
    DecodeParams p = p0;
    const int64_t units = (int64_t)p.num_seqs * p.kv.num_kv_heads;
    const int32_t rg = p.kv.dtype == KV_FP16 ? 1 : groups_per_workgroup(p.kv.head_dim, p.cu_q_lens != nullptr,
                                                                          p.ncg, p.partition_tokens);
    p.ncgw = (p.ncg + rg - 1) / rg;
    const int64_t slots = ((units + 7) / 8) * 8 * p.ncgw;
    // A merged call whose grid would leave half the compute units idle
    // streams each partition with two workgroups (each a half of P, both
    // merged with the rest by the LSE merge), when the workspace holds their
    // partials.
    if (p.kv.head_dim == 128 && p.merge && p.may_split && slots * p.nparts * 2 <= 256 &&
        p.partition_tokens % 64 == 0 && p.partition_tokens >= 512) {
        p.partition_tokens /= 2;
        p.nparts *= 2;
    }
    p.xcd_local = p.kv.head_dim == 128 && slots * p.nparts <= 256;
    p.direct = p.kv.head_dim == 128 && p.merge && p.nparts == 1;
    if (p.kv.head_dim == 256) {
        switch (p.kv.dtype) {
        case KV_FP16: return launch_d256<KV_FP16>(p, s);
        case KV_E4M3: return launch_d256<KV_E4M3>(p, s);
        case KV_INT8: return launch_d256<KV_INT8>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.kv.dtype) {
    case KV_FP16: return launch_kv<KV_FP16>(p, s);
    case KV_E4M3: return launch_kv<KV_E4M3>(p, s);
    case KV_INT8: return launch_kv<KV_INT8>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace plc
