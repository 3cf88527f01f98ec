// Split-KV paged decode for gfx950.
//
// One workgroup per (partition, KV head, sequence).  The partition's 16-token
// pages are walked two at a time (a 32-token chunk) by the workgroup's waves.
// Per chunk a wave:
//   - reads the two page ids once and issues 16-byte K loads and 8-byte V
//     loads straight into registers (the page-id reuse and wide loads that the
//     1Cat-vLLM README's "128-bit Loads" section credits for its decode gain);
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
    u32x4 k[2][(KV == KV_FP16) ? 4 : 2];
    // V: eight tokens t(g, e) = 16*(e/4) + 4g + e%4, d = 8*(l%16) + [0, 8).
    u32x4 v16[(KV == KV_FP16) ? 8 : 1];
    u32x2 v8[(KV == KV_FP16) ? 1 : 8];
    f32x4 ks[2], vs[2];             // INT8 per-token scales of tokens 4g..4g+3
    int valid_blk;                  // bit p set when page p is inside the pool
};

template <int KV, int NW>
struct Decode {
    static constexpr int EB = ElemBytes<KV>::value;

    __device__ static void load(Chunk<KV>& c, const DecodeParams& p, int kvh, int pb0, int pb1,
                                bool has1, int lane) {
        const int g = lane >> 4, i = lane & 15;
        const int nb = p.kv.num_blocks;
        c.valid_blk = ((pb0 >= 0 && pb0 < nb) ? 1 : 0) | ((has1 && pb1 >= 0 && pb1 < nb) ? 2 : 0);
        const int pbs[2] = {(c.valid_blk & 1) ? pb0 : 0, (c.valid_blk & 2) ? pb1 : 0};
        const int Hkv = p.kv.num_kv_heads;
        const uint8_t* kc = static_cast<const uint8_t*>(p.kv.k);
        const uint8_t* vc = static_cast<const uint8_t*>(p.kv.v);
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            const int64_t base = ((int64_t)pbs[pg] * Hkv + kvh) * (BS * D * EB);
            const uint8_t* kr = kc + base + i * (D * EB);
            if constexpr (KV == KV_FP16) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
                        c.k[pg][2 * h + sub] =
                            *reinterpret_cast<const u32x4*>(kr + (64 * h + 16 * g + 8 * sub) * 2);
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    c.k[pg][h] = *reinterpret_cast<const u32x4*>(kr + 64 * h + 16 * g);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int pg = e >> 2;
            const int slot = 4 * g + (e & 3);
            const int64_t base = ((int64_t)pbs[pg] * Hkv + kvh) * (BS * D * EB);
            const uint8_t* vr = vc + base + slot * (D * EB) + 8 * i * EB;
            if constexpr (KV == KV_FP16)
                c.v16[e] = *reinterpret_cast<const u32x4*>(vr);
            else
                c.v8[e] = *reinterpret_cast<const u32x2*>(vr);
        }
        if constexpr (KV == KV_INT8) {
#pragma unroll
            for (int pg = 0; pg < 2; ++pg) {
                const int64_t srow = ((int64_t)pbs[pg] * Hkv + kvh) * BS + 4 * g;
                c.ks[pg] = *reinterpret_cast<const f32x4*>(p.kv.k_scale + srow);
                c.vs[pg] = *reinterpret_cast<const f32x4*>(p.kv.v_scale + srow);
            }
        }
    }

    // K of page pg as the four MFMA A operands (d-slots kc = 2h + sub).
    __device__ static void k_operands(const Chunk<KV>& c, int pg, f16x8 out[4]) {
        if constexpr (KV == KV_FP16) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) out[kc] = __builtin_bit_cast(f16x8, c.k[pg][kc]);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                out[2 * h + 0] = codes8_to_f16x8<KV>(c.k[pg][h][0], c.k[pg][h][1]);
                out[2 * h + 1] = codes8_to_f16x8<KV>(c.k[pg][h][2], c.k[pg][h][3]);
            }
        }
    }

    // V^T operands: vt[col] holds V[t(g, e)][8*(l%16) + col] for e = 0..7.
    __device__ static void v_operands(const Chunk<KV>& c, f16x8 vt[8]) {
        if constexpr (KV == KV_FP16) {
            // 16-bit transpose: pair (e, e+1) of column col = perm of dword col/2.
#pragma unroll
            for (int col = 0; col < 8; ++col) {
                const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
                u32x4 r;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr)
                    r[pr] = __builtin_amdgcn_perm(c.v16[2 * pr + 1][col >> 1], c.v16[2 * pr][col >> 1], sel);
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

    // Zero V of tokens that must not contribute (past the end, bad page): a
    // zero weight times a NaN poison value would still be NaN
    // (INT8: the token's scale too, which may be a NaN poison).
    __device__ static void mask_v(Chunk<KV>& c, const bool ok[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (KV == KV_FP16) {
                if (!ok[e]) c.v16[e] = u32x4{0, 0, 0, 0};
            } else {
                if (!ok[e]) c.v8[e] = u32x2{0, 0};
            }
            if constexpr (KV == KV_INT8) {
                if (!ok[e]) c.vs[e >> 2][e & 3] = 0.0f;
            }
        }
    }
};

template <int KV, int NW>
__global__ __launch_bounds__(64 * NW) void decode_partials_kernel(DecodeParams p) {
    using Dk = Decode<KV, NW>;
    extern __shared__ float smem[];
    const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int Hq = p.num_q_heads, G = Hq / p.kv.num_kv_heads;
    // lengths beyond the host-stated bound are clamped so that no page id
    // outside the table is ever read
    const int L = min(p.context_lens[b], p.max_context_len);
    const int tok0 = part * p.partition_tokens;
    const int64_t row0 = (int64_t)b * Hq + (int64_t)kvh * G;   // first query row of the group
    const int nparts = p.nparts;

    if (tok0 >= L) {                                             // partition past the end
        for (int idx = tid; idx < G * D; idx += 64 * NW) {
            const int j = idx / D, d = idx % D;
            p.o_parts[((row0 + j) * nparts + part) * D + d] = 0.0f;
            if (d == 0) p.lse_parts[(row0 + j) * nparts + part] = -__builtin_inff();
        }
        return;
    }
    const int tok1 = min(tok0 + p.partition_tokens, L);
    const int nblk = (tok1 - tok0 + BS - 1) / BS;
    const int nchunks = (nblk + 1) / 2;
    const int blk0 = tok0 / BS;
    const int32_t* bt = p.block_tables + (int64_t)b * p.max_blocks;

    // Q^T operand: lane (i, g) holds head i, d = 64*(kc/2) + 16g + 8*(kc%2) + [0, 8).
    f16x8 qop[4];
    {
        const f16* q = static_cast<const f16*>(p.q) + (row0 + i) * D;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            if (i < G)
                qop[kc] = *reinterpret_cast<const f16x8*>(q + 64 * (kc >> 1) + 16 * g + 8 * (kc & 1));
            else
                qop[kc] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    // value scale applied once to the normalized output; INT8 carries its
    // per-token scale (times 256, to keep P away from fp16 subnormals) in P
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / 256.0f;

    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0, 0, 0, 0};

    // Page ids of this wave's chunks, 32 chunks per refill: lane 2k+pg holds
    // the page of chunk (wave + k*NW), page pg.
    int tbl = 0;
    auto refill = [&](int it0) {
        const int k = lane >> 1, pg = lane & 1;
        const int ch = wave + (it0 + k) * NW;
        const int blk = 2 * ch + pg;
        tbl = (ch < nchunks && blk < nblk) ? bt[blk0 + blk] : -1;
    };
    auto page = [&](int it, int pg) {
        return __builtin_amdgcn_readlane(tbl, 2 * (it & 31) + pg);
    };

    const int my_chunks = (wave < nchunks) ? (nchunks - wave + NW - 1) / NW : 0;
    Chunk<KV> cur, nxt;
    if (my_chunks > 0) {
        refill(0);
        const int ch = wave;
        Dk::load(cur, p, kvh, page(0, 0), page(0, 1), 2 * ch + 1 < nblk, lane);
    }
    for (int it = 0; it < my_chunks; ++it) {
        const int ch = wave + it * NW;
        if (it + 1 < my_chunks) {
            if (((it + 1) & 31) == 0) refill(it + 1);
            const int chn = ch + NW;
            Dk::load(nxt, p, kvh, page(it + 1, 0), page(it + 1, 1), 2 * chn + 1 < nblk, lane);
        }
        // validity of the lane's eight tokens t(g, e)
        bool ok[8];
        const int ctok = tok0 + 32 * ch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int pg = e >> 2;
            ok[e] = (ctok + 16 * pg + 4 * g + (e & 3) < tok1) && ((cur.valid_blk >> pg) & 1);
        }
        const bool partial = (ctok + 32 > tok1) || (cur.valid_blk != 3);
        if (partial) Dk::mask_v(cur, ok);

        // S^T = K Q^T per page: lane holds tokens 4g + r of page pg, head i.
        float x[8];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            f16x8 kop[4];
            Dk::k_operands(cur, pg, kop);
            f32x4 s = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) s = mfma16(kop[kc], qop[kc], s);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sc = cscale;
                if constexpr (KV == KV_INT8) sc *= cur.ks[pg][r];
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
        const float m_new = fmaxf(m_run, mx);
        // m_new is -inf only while every key so far is masked (cannot happen
        // for a valid page of a non-empty partition, but keep the state finite)
        const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.0f;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = fast_exp2(x[e] - m_use);
            psum += pe;
            pv[e] = pe;
            if constexpr (KV == KV_INT8) pv[e] *= cur.vs[e >> 2][e & 3] * 256.0f;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] *= alpha;
        }
        f16x8 pop;
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[e] = (f16)pv[e];

        f16x8 vt[8];
        Dk::v_operands(cur, vt);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma16(vt[c], pop, acc[c]);

        if (it + 1 < my_chunks) cur = nxt;
    }

    // ---- merge the waves of the workgroup (fixed order) ----
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    constexpr int AST = D + 4;                         // padded head stride (floats)
    float* s_m = smem;                                 // [NW][16]
    float* s_l = smem + NW * 16;                       // [NW][16]
    float* s_acc = smem + NW * 32;                     // [NW][G][AST]
    if (g == 0) {
        s_m[wave * 16 + i] = m_run;
        s_l[wave * 16 + i] = l_run;
    }
    if (i < G) {
        float* dst = s_acc + ((int64_t)wave * G + i) * AST + 32 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 lo = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
            f32x4 hi = f32x4{acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
            *reinterpret_cast<f32x4*>(dst + 8 * r) = lo;
            *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = hi;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 64 * NW) {
        const int j = idx / D, d = idx % D;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + j]);
        float Lsum = 0.0f, O = 0.0f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float wt = fast_exp2(s_m[w * 16 + j] - M);
                Lsum += s_l[w * 16 + j] * wt;
                O += s_acc[((int64_t)w * G + j) * AST + d] * wt;
            }
        }
        const bool empty = !(Lsum > 0.0f);
        p.o_parts[((row0 + j) * nparts + part) * D + d] = empty ? 0.0f : O * vscale / Lsum;
        if (d == 0)
            p.lse_parts[(row0 + j) * nparts + part] =
                empty ? -__builtin_inff() : (M + __builtin_log2f(Lsum)) * kLn2;
    }
}

template <int KV, int NW>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
    const int G = p.num_q_heads / p.kv.num_kv_heads;
    const size_t lds = sizeof(float) * (NW * 32 + (size_t)NW * G * (D + 4));
    dim3 grid(p.nparts, p.kv.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((decode_partials_kernel<KV, NW>), grid, dim3(64 * NW), lds, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partials(const DecodeParams& p, hipStream_t s) {
    // LDS holds every wave's unnormalized output: keep it within 64 KiB
    const bool wide = p.num_q_heads / p.kv.num_kv_heads > 8;
    switch (p.kv.dtype) {
    case KV_FP16: return wide ? launch_t<KV_FP16, 4>(p, s) : launch_t<KV_FP16, 8>(p, s);
    case KV_E4M3: return wide ? launch_t<KV_E4M3, 4>(p, s) : launch_t<KV_E4M3, 8>(p, s);
    case KV_INT8: return wide ? launch_t<KV_INT8, 4>(p, s) : launch_t<KV_INT8, 8>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace plc
