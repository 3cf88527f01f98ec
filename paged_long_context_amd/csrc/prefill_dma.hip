// Attention tiles of 128 query rows over paged KV caches whose rows reach LDS
// by DMA, for gfx950: 8-bit codes (E4M3, INT8) at head dims 128 and 256, and
// FP16 values at head dim 128 (rows of 256 bytes, like 256 codes).  They
// serve the chunked causal prefill at head dim 256 (8-bit), and key
// partitions of the same tiles for calls with up to 16 query tokens per
// sequence whose rows fill a tile.
//
// A workgroup is 4 waves = 128 query rows of one (sequence, KV head),
// position-major (row r = query token r / G, head r % G, so the G heads of a
// KV head share every K/V tile: 1Cat-vLLM README, Layer 2 "GQA Multi-Head
// Packing"), one 32-row MFMA tile per wave.  Q operands and the O^T
// accumulators stay in registers for the whole key loop.  S^T = K Q^T sums
// over the whole head in one 32x32 accumulator (the pages split a 256-wide
// head into halves on their hardware, Layer 2 "D256 Split-D"); O^T = V^T P^T
// keeps one 32-dimension accumulator tile per 32 dimensions; QK and PV
// accumulate in fp32 ("Performance First").  Keys are walked in subtiles of
// 32 (two 16-token pages); subtiles wholly below the tile's first position
// skip the causal mask (Layer 2 "Prefix / Causal-Tail Separation").
//
// The rows of each subtile reach LDS unconverted, by DMA (16 bytes per lane,
// one contiguous kilobyte per instruction, no registers involved), NBS
// subtiles ahead of use; each wave converts the 8-bit K and V operands it
// reads, and FP16 values are operands as they stand (the pages keep the same
// goals with register prefetch on V100: Layer 1 and "Software-Reconstructed
// Async").  V^T operands come from V stored as [key][d] through the gfx950
// transposing reads (ds_read_b64_tr_b8: within each 16 lanes, lane 8p + i
// receives byte i of the eight rows that lanes p, p + 2, ..., p + 14
// address; ds_read_b64_tr_b16 for FP16, below).
//
// Key partitions (Layer 2 "Split-KV3": partial states in fp32, merged after):
// with partition_tokens > 0 the grid holds one workgroup per (row tile,
// partition), each walking only its partition's subtiles and writing its
// rows' normalized partial output and natural-log LSE; a row that sees no key
// of the partition writes 0 and -inf.
#include <type_traits>

#include "plc_device.h"
#include "plc_internal.h"

namespace plc {
namespace {

constexpr int BS = 16;
constexpr int ROWS = 128;               // query rows per workgroup
constexpr int NBS = 6;                  // 32-key code buffers in flight
constexpr int PFV = 5;                  // V operands read this many MFMAs ahead

// all zeros: the DMA source of pages whose id is outside the pool (one
// (page, head) slice at the widest head)
__device__ __attribute__((aligned(16))) uint8_t g_zero_page[BS * 256];

// Shapes of the key loop per head dim DH and cache element bytes EB (1 for
// the 8-bit codes; 2 for FP16, at head dim 128 only).
template <int DH, int EB>
struct Geo {
    static_assert((DH == 128 || DH == 256) && (EB == 1 || (EB == 2 && DH == 128)), "head dim");
    static constexpr int RB = DH * EB;      // bytes of one K (or V) row
    static constexpr int NQ = DH / 16;      // K MFMAs per subtile = PV MFMAs = steps per part
    static constexpr int NDT = DH / 32;     // O^T accumulator tiles
    static constexpr int KPR = 2 / EB;      // K operands per 16-byte read (a code pair, or one fp16 operand)
    static constexpr int NKP = NQ / KPR;    // K reads per row
    static constexpr int PFK = EB == 1 ? 3 : 4;   // K reads issued this many reads ahead
    static constexpr int NCH = RB / 16;     // 16-byte chunks per row
    static constexpr int CB = 32 * RB;      // bytes of one subtile's K (or V) rows
    static constexpr int NDK = RB / 128;    // K (and V) DMAs per wave per subtile
    static constexpr int RPD = 1024 / RB;   // rows one DMA moves
    static constexpr int NM = DH == 256 ? 4 : 2;   // part A steps of the row maximum
    static constexpr int NE = DH == 256 ? 8 : 4;   // part A steps of the exponentials
    // chunk slot swizzles.  Chunk c (16 bytes) of K row rho sits at slot
    // c ^ kswz(rho), chunk c of V row (key) k at slot c ^ vswz(k).  A K operand
    // read (16 consecutive rows, one chunk) and a V transposing read (eight
    // rows x two adjacent chunks per 32 lanes for 8-bit codes; four rows x
    // four adjacent chunks for fp16) then touch distinct banks: 256-byte rows
    // all start on bank 0, so 16 distinct slots cover the 64 banks; 128-byte
    // rows alternate between banks 0 and 32, so the slot of rows of one
    // parity must differ.
    __device__ static int kswz(int rho) { return RB == 256 ? (rho & 15) : ((rho >> 1) & 7); }
    __device__ static int vswz(int k) {
        if (EB == 2) return 4 * (k & 3);
        return DH == 256 ? (((k & 7) << 1) | ((k >> 3) & 1)) : (((k >> 1) & 3) << 1);
    }
};

// global_load_lds_dwordx4 with a 64-bit SGPR base and a 32-bit lane offset:
// lane l's 16 bytes at base + off land at LDS dst + 16 l (dst wave-uniform).
// Written as asm so that the compiler does not make every later LDS read
// wait for it; the key loop waits with explicit vmcnt counts.  M0 (the LDS
// base read at issue) is saved and restored.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t dst) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(dst), "v"(off), "s"(base) : "memory");
}

// 4 bytes per lane from a 64-bit lane address to LDS dst + 4 l
__device__ __forceinline__ void dma4(const void* src, uint32_t dst) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(dst), "v"(src) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Schedule per 32-key subtile j (buffer j % NBS), NQ steps per part (one
// MFMA each; the compiler moves nothing across steps):
//   part A: S(j+1) = K Q^T, K code pairs read PFK pairs ahead and converted
//           one step before their MFMAs, the online softmax of S(j) between;
//           the last steps read the first V operands of part B;
//   (rare rescale branch; wait for this wave's DMAs of subtile j+2; barrier)
//   part B: O += V^T P(j)^T, V operands read PFV MFMAs ahead, converted one
//           step before use, consecutive MFMAs on different accumulator
//           tiles (operand o: tile o % NDT, key half o / NDT); the DMAs of
//           subtile j + NBS - 1 into the buffer of subtile j - 1, whose last
//           reader was part B of j - 1; the last steps read the first K pairs
//           of subtile j + 2.
// Subtile x is first read at the end of part B of x - 2, after the barrier
// of x - 2, by which every wave has waited for its own DMAs of x.  Subtiles
// are counted from the first of the workgroup's key range.
// One wave per SIMD where the LDS holds one workgroup per CU (head dim 256,
// and fp16 rows of 256 bytes); two at head dim 128 with 8-bit codes.
template <int KV, int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DH == 256 || KV == KV_FP16 ? 1 : 2,
                                                                     DH == 256 || KV == KV_FP16 ? 1 : 2)))
void prefill_dma_kernel(PrefillParams p) {
    using Gm = Geo<DH, KV == KV_FP16 ? 2 : 1>;
    constexpr int NQ = Gm::NQ, NDT = Gm::NDT, NKP = Gm::NKP, NCH = Gm::NCH, CB = Gm::CB;
    constexpr int NDK = Gm::NDK, RPD = Gm::RPD, NM = Gm::NM, NE = Gm::NE;
    constexpr int RB = Gm::RB, KPR = Gm::KPR, PFK = Gm::PFK;
    // V operands in flight: 8 codes, or 8 fp16 values
    using VR = std::conditional_t<KV == KV_FP16, u32x4, u32x2>;
    // DMA instructions per subtile per wave: codes (2 NDK), INT8 scales (1), page ids (1)
    constexpr int ND = 2 * NDK + 1 + (KV == KV_INT8 ? 1 : 0);
    // part A: INT8 scale reads, row maximum, its exchange, exponentials
    constexpr int SO = (KV == KV_INT8) ? (DH == 256 ? 2 : 1) : 0;
    static_assert(SO + NM + 1 + NE <= NQ && PFV <= NQ && PFK <= NKP, "part A schedule");
    // K codes of the NBS buffers, then their V codes; the epilogue reuses it
    __shared__ __attribute__((aligned(1024))) uint8_t s_kv[2][NBS][CB];
    __shared__ __attribute__((aligned(16))) float s_sc[NBS][64];   // INT8: K scales by key, then V scales
    __shared__ __attribute__((aligned(16))) int s_pid[8][64];       // page ids of subtile y at [y & 7][0..1]

    const bool split = p.partition_tokens > 0;
    const int np = split ? p.nparts : 1;
    const int rb = blockIdx.x / np, part = blockIdx.x - rb * np;
    const int kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = p.num_q_heads, Hkv = p.kv.num_kv_heads, G = Hq / Hkv;
    // The page ids of the first NBS - 1 subtiles of the workgroup's range,
    // read before its lengths are known so that the two loads overlap: the
    // range starts at subtile part * P / 32, and ids are clamped to the table
    // row (ids past the context are never used; an id outside the pool is
    // never dereferenced)
    const int jb0 = split ? part * (p.partition_tokens / 32) : 0;
    const int32_t* const bt = p.block_tables + (int64_t)b * p.max_blocks + 2 * jb0;
    const __attribute__((address_space(4))) int32_t* const btc =
        (const __attribute__((address_space(4))) int32_t*)(uintptr_t)bt;
    int pid0[2 * (NBS - 1)];
    {
        const int pcap = max(p.max_blocks - 1 - 2 * jb0, 0);
#pragma unroll
        for (int x = 0; x < 2 * (NBS - 1); ++x) pid0[x] = btc[min(x, pcap)];
    }
    const int qa = p.cu_q_lens[b];
    // lengths beyond the host-stated bounds are clamped so that no page id
    // outside the table is ever read
    const int L = max(0, min(p.context_lens[b], p.max_context_len));
    // a prefill chunk holds at most L tokens; query tokens of a partitioned
    // call are the last n positions even when n > L (the rows before position
    // 0 see no key)
    const int nq = min(max(p.cu_q_lens[b + 1] - qa, 0), p.max_q_len);
    const int n = split ? nq : min(nq, L);
    const int nrows = n * G;
    const int r0 = ROWS * rb;
    if (r0 >= nrows) return;
    const int base = L - n;                          // position of the chunk's first token
    const int rlast = min(r0 + ROWS, nrows) - 1;
    const int kend = base + rlast / G + 1;           // keys [0, kend) are visible to someone
    const int kfull = base + r0 / G + 1;             // keys [0, kfull) are visible to every row
    const int nsub = max(kend, 0) / 32 + ((max(kend, 0) & 31) ? 1 : 0);
    const int nfull = min(max(kfull, 0) / 32, nsub); // subtiles needing no mask

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
    float* const orow = split ? p.o_parts + (rowid * np + part) * DH : p.out + rowid * DH;
    float* const lrow = split ? p.lse_parts + rowid * np + part : p.lse + rowid;

    // this workgroup's subtiles [jb, je)
    const int jb = jb0;
    const int je = split ? min(nsub, jb + p.partition_tokens / 32) : nsub;
    if (jb >= je) {                                  // no key of the partition is visible
        if (rowok) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * a4 + 4 * h32) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (h32 == 0) *lrow = -__builtin_inff();
        }
        return;
    }
    const int nloc = je - jb;
    const int nfloc = min(max(nfull - jb, 0), nloc);
    // the range's page ids are counted from its first page; the loop's ids
    // clamp to the range's last page (prefetches past the range reread it)
    const int plast = min((kend - 1) / BS, 2 * je - 1) - 2 * jb;

    // Q operands.  8-bit codes: MFMA kc of a subtile takes half (kc & 1) of K
    // code pair kc >> 1, whose lane (row, h32) holds d = 32(kc>>1) + 16 h32 +
    // [0,16), so lane (row, h32) of qop[kc] holds d = 32(kc>>1) + 16 h32 +
    // 8(kc&1) + [0,8).  FP16: MFMA kc takes K read kc, whose lane (row, h32)
    // holds d = 16 kc + 8 h32 + [0,8), and so does qop[kc].
    f16x8 qop[NQ];
    {
        const f16* q = static_cast<const f16*>(p.q) + rowid * DH + (KPR == 2 ? 16 : 8) * h32;
#pragma unroll
        for (int kc = 0; kc < NQ; ++kc)
            qop[kc] = *reinterpret_cast<const f16x8*>(q + (KPR == 2 ? 32 * (kc >> 1) + 8 * (kc & 1) : 16 * kc));
    }
    float cscale = p.qk_scale_log2;
    if constexpr (KV == KV_E4M3) cscale *= p.kv.k_scale[kvh];
    float vscale = 1.0f;
    if constexpr (KV == KV_E4M3) vscale = p.kv.v_scale[kvh];
    if constexpr (KV == KV_INT8) vscale = 1.0f / kInt8PFold;
    float m_ref = -__builtin_inff(), l_run = 0.0f;
    // lazy rescaling: the reference maximum moves only when a score passes
    // it by 2^8 in probability.  INT8's P operand carries 64 sigma_v, so there
    // the allowance shrinks per subtile to keep 2^allow * 64 * sigma_max below
    // 64,000 (< 65,504, the largest finite fp16)
    const float grow_raw = 8.0f / cscale, inv_cs = 1.0f / cscale;
    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

    // ---- DMA roles.  DMA h of wave w moves LDS rows 16 h + RPD w + l / NCH
    // of each buffer's K and V, slot l % NCH, from page (16 h + RPD w) / 16 of
    // the subtile: K row rho holds key key_of_row(rho), V row k holds key k.
    uint32_t kof[NDK], vof[NDK];
#pragma unroll
    for (int h = 0; h < NDK; ++h) {
        const int row = 16 * h + RPD * wave + lane / NCH, slot = lane % NCH;
        const int kk = key_of_row(row) & 15;
        kof[h] = (uint32_t)(kk * RB + 16 * (slot ^ Gm::kswz(row)));
        vof[h] = (uint32_t)((row & 15) * RB + 16 * (slot ^ Gm::vswz(row)));
    }
    const int64_t head_off = (int64_t)kvh * BS * RB;
    // the zero page's address, loaded once and kept in scalar registers
    uint64_t zp = reinterpret_cast<uint64_t>(&g_zero_page[0]);
    asm volatile("" : "+s"(zp));
    // page base of (pg, kvh), or the zero page for an id outside the pool;
    // selected with masks (uniform arithmetic, no branch)
    auto page_base = [&](const void* cache, int pg) __attribute__((always_inline)) -> const uint8_t* {
        const uint64_t m = 0ull - (uint64_t)((uint32_t)pg < (uint32_t)p.kv.num_blocks);
        const uint64_t a = reinterpret_cast<uint64_t>(cache) + (uint64_t)((int64_t)pg * Hkv * BS * RB + head_off);
        return reinterpret_cast<const uint8_t*>((a & m) | (zp & ~m));
    };
    // INT8 scales of subtile x: lane l < 32 reads key l's K scale, lane 32 + l
    // key l's V scale (every wave the same, which keeps the DMA counts equal)
    auto scale_src = [&](int pg, int keyin) __attribute__((always_inline)) -> const float* {
        const float* arr = (lane < 32) ? p.kv.k_scale : p.kv.v_scale;
        const bool ok = (uint32_t)pg < (uint32_t)p.kv.num_blocks;
        return ok ? arr + ((int64_t)pg * Hkv + kvh) * BS + keyin : reinterpret_cast<const float*>(zp) + keyin;
    };
    auto issue = [&](int bi, int pg0, int pg1) __attribute__((always_inline)) {
        const uint32_t lk = lds_addr(&s_kv[0][bi][0]), lv = lds_addr(&s_kv[1][bi][0]);
#pragma unroll
        for (int h = 0; h < NDK; ++h) {
            const int first = 16 * h + RPD * wave;   // wave-uniform
            const int pg = (first >> 4) ? pg1 : pg0;
            dma16s(page_base(p.kv.k, pg), kof[h], lk + first * RB);
            dma16s(page_base(p.kv.v, pg), vof[h], lv + first * RB);
        }
        if constexpr (KV == KV_INT8) {
            const int key = lane & 31;
            dma4(scale_src((key >> 4) ? pg1 : pg0, key & 15), lds_addr(&s_sc[bi][0]));
        }
    };
    // The key loop takes its page ids from LDS, where a DMA of every subtile
    // step puts those of a subtile 2 NBS - 1 ahead (lane l: page 2y + (l & 1)):
    // a scalar load in flight would make every LDS wait a wait for it.
    auto issue_ids = [&](int y) __attribute__((always_inline)) {
        dma4(bt + min(2 * y + (lane & 1), plast), lds_addr(&s_pid[y & 7][0]));
    };

    // ---- prologue: the page ids that subtile 0 reads, then the DMA groups
    // the loop would have issued before subtile 0 (codes of subtiles
    // 0 .. NBS-2, page ids of NBS .. 2NBS-2); codes 0 and 1 and the first two
    // groups' page ids complete
    issue_ids(NBS - 1);
#pragma unroll
    for (int x = 0; x < NBS - 1; ++x) {
        issue(x, pid0[2 * x], pid0[2 * x + 1]);
        issue_ids(NBS + x);
    }
    wait_vm<(NBS - 3) * ND>();
    __syncthreads();

    // ---- operand reads.  K read q of buffer bi: lane (r32, h32) reads the
    // 16 bytes of row r32, chunk 2q + h32, at (kb + ka) ^ 32q.  V operand
    // (dt, hf), 8-bit codes: the transposing read at ((vb + va) ^ 32dt) +
    // 16 RB hf.  FP16: two 16-bit transposing reads (ds_read_b64_tr_b16:
    // within each 16 lanes, lane 4p + i receives element i of the four rows
    // that lanes p, p + 4, p + 8, p + 12 address, measured with a probe) at
    // ((vb + va) ^ 64dt) + 16 RB hf and 4 rows further: lane (q, p) of a
    // 16-lane group (q = (l & 15) >> 2, p = l & 3) addresses key 8 h32 + q,
    // dimensions 16 gp + 4p + [0,4) of the tile, so lane l receives keys
    // 8 h32 + [0,4) (then + [4,8)) of dimension l % 32.
    const uint32_t ka = (uint32_t)(r32 * RB + 16 * (h32 ^ Gm::kswz(r32)));
    uint32_t va;
    if constexpr (KV == KV_FP16) {
        // chunk 4dt + 2gp + (p >> 1) of key k at slot c ^ 4(k & 3), k & 3 = q
        const int q4 = (lane & 15) >> 2, p4 = lane & 3, gp = (lane >> 4) & 1;
        va = (uint32_t)((8 * h32 + q4) * RB + 64 * q4 + 32 * gp + 8 * p4);
    } else {
        const int key = 8 * h32 + ((lane & 15) >> 1), gp = (lane >> 4) & 1;
        va = (uint32_t)(key * RB + 16 * (gp ^ Gm::vswz(key)) + 8 * (lane & 1));
    }
    const uint32_t sk0 = lds_addr(&s_kv[0][0][0]), sv0 = lds_addr(&s_kv[1][0][0]);
    auto kread = [&](uint32_t kb, int q) __attribute__((always_inline)) {
        return *(__attribute__((address_space(3))) const u32x4*)(uintptr_t)((kb + ka) ^ (32u * q));
    };
    auto vread = [&](uint32_t vb, int dt, int hf) __attribute__((always_inline)) -> VR {
        if constexpr (KV == KV_FP16) {
            typedef short v4s __attribute__((ext_vector_type(4)));
            const uint32_t a = ((vb + va) ^ (64u * dt)) + 16u * RB * hf;
            const u32x2 r0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(uintptr_t)a));
            const u32x2 r1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(uintptr_t)(a + 4u * RB)));
            return u32x4{r0[0], r0[1], r1[0], r1[1]};
        } else {
            typedef int v2i __attribute__((ext_vector_type(2)));
            const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(uintptr_t)(((vb + va) ^ (32u * dt)) + 16u * RB * hf));
            return u32x2{(uint32_t)r[0], (uint32_t)r[1]};
        }
    };

    // operand `half` of K read w (fp16: the read itself)
    auto kop_of = [&](const u32x4& w, int half) __attribute__((always_inline)) -> f16x8 {
        if constexpr (KPR == 1) return __builtin_bit_cast(f16x8, w);
        else return half ? codes8_to_f16x8<KV>(w[2], w[3]) : codes8_to_f16x8<KV>(w[0], w[1]);
    };
    // ---- S of subtile 0
    f32x16 sc;
    {
        u32x4 raw[NKP];
#pragma unroll
        for (int q = 0; q < NKP; ++q) raw[q] = kread(sk0, q);
#pragma unroll
        for (int kc = 0; kc < NQ; ++kc) sc = mfma32(kop_of(raw[kc / KPR], kc & 1), qop[kc], kc ? sc : f32x16{});
    }
    u32x4 kraw[PFK];                                 // K reads in flight (subtile j + 1)
    VR vraw[PFV];                                    // V operands in flight (subtile j)
    {
        const uint32_t kb1 = sk0 + CB;
#pragma unroll
        for (int q = 0; q < PFK; ++q) kraw[q] = kread(kb1, q);
    }
    int bcur = 0;                                    // buffer of subtile j

    // one subtile j of the range (buffer bcur): the softmax of S(j), in sc,
    // and S(j + 1) into sn
    auto sub = [&](auto mtag, int j, f32x16& sc, f32x16& sn) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mtag)::value;
        constexpr int RM = 16 / NM, RE = 16 / NE;    // scores per max step, per exp step
        const int bn = (bcur + 1 == NBS) ? 0 : bcur + 1, bnn = (bn + 1 == NBS) ? 0 : bn + 1;
        const uint32_t kbn = sk0 + bn * CB;          // K codes of subtile j + 1
        const uint32_t vbc = sv0 + bcur * CB;        // V codes of subtile j
        const int k0 = 32 * (jb + j);                // its first key
        float mloc = -__builtin_inff(), mx = 0.0f, m_new = 0.0f, moff = 0.0f, psum = 0.0f, smax = 0.0f;
        bool grow = false;
        f16x8 pp[2], kop[2];
        f32x4 sks[4], svs[4];
        // page ids of subtile j + NBS - 1, whose codes part B sends for
        const int2 ids = *reinterpret_cast<const int2*>(&s_pid[(j + NBS - 1) & 7][0]);
        // ---------------- part A
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if constexpr (KPR == 2) {
                if ((i & 1) == 0) {
                    // pair i/2 arrived PFK pairs ago: both its operands, then the read PFK pairs ahead
                    const u32x4 w = kraw[(i >> 1) % PFK];
                    kop[0] = kop_of(w, 0);
                    kop[1] = kop_of(w, 1);
                    if ((i >> 1) + PFK < NKP) kraw[(i >> 1) % PFK] = kread(kbn, (i >> 1) + PFK);
                }
            } else {
                // read i arrived PFK reads ago: its operand, then the read PFK ahead
                kop[i & 1] = kop_of(kraw[i % PFK], 0);
                if (i + PFK < NKP) kraw[i % PFK] = kread(kbn, i + PFK);
            }
            sn = mfma32(kop[i & 1], qop[i], i ? sn : f32x16{});
            if (i >= NQ - PFV) vraw[i - (NQ - PFV)] = vread(vbc, (i - (NQ - PFV)) % NDT, (i - (NQ - PFV)) / NDT);
            if constexpr (KV == KV_INT8)
                if (i == 0) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ko = 16 * (u >> 1) + 8 * h32 + 4 * (u & 1);
                        sks[u] = *reinterpret_cast<const f32x4*>(&s_sc[bcur][ko]);
                        svs[u] = *reinterpret_cast<const f32x4*>(&s_sc[bcur][32 + ko]);
                    }
                }
            if (i >= SO && i < SO + NM) {
#pragma unroll
                for (int rr = 0; rr < RM; ++rr) {
                    // element r of this lane's scores is key k0 + 16(r>>3) + 8 h32 + (r&7)
                    const int r = RM * (i - SO) + rr;
                    float v = sc[r];
                    if constexpr (KV == KV_INT8) {
                        v *= sks[r >> 2][r & 3];
                        float s = svs[r >> 2][r & 3];
                        if constexpr (MASKED) s = (k0 + 16 * (r >> 3) + 8 * h32 + (r & 7) < kend) ? s : 0.0f;
                        smax = fmaxf(smax, s);
                    }
                    if constexpr (MASKED) {
                        const int key = k0 + 16 * (r >> 3) + 8 * h32 + (r & 7);
                        v = (key <= rowpos) ? v : -__builtin_inff();
                    }
                    sc[r] = v;
                    mloc = fmaxf(mloc, v);
                }
            }
            if (i == SO + NM) {
                mx = max_halves(mloc);
                float allow = grow_raw;
                if constexpr (KV == KV_INT8)   // log2(1000 / sigma_max), at most 8
                    allow = fminf(8.0f, 9.9657843f - __builtin_amdgcn_logf(max_halves(smax))) * inv_cs;
                grow = mx > m_ref + allow;
                m_new = grow ? mx : m_ref;
                moff = (m_new == -__builtin_inff()) ? 0.0f : -m_new * cscale;
            }
            if (i >= SO + NM + 1 && i < SO + NM + 1 + NE) {
#pragma unroll
                for (int rr = 0; rr < RE; ++rr) {
                    const int r = RE * (i - SO - NM - 1) + rr;
                    float pe = fast_exp2(__builtin_fmaf(sc[r], cscale, moff));
                    psum += pe;
                    if constexpr (KV == KV_INT8) {
                        float vsr = svs[r >> 2][r & 3];
                        if constexpr (MASKED) vsr = (k0 + 16 * (r >> 3) + 8 * h32 + (r & 7) < kend) ? vsr : 0.0f;
                        pe *= vsr * kInt8PFold;
                    }
                    pp[r >> 3][r & 7] = (f16)pe;
                }
            }
            step_fence();
        }
        pin(pp[0]);
        pin(pp[1]);
        pin(psum);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
            const float alpha = (m_ref == -__builtin_inff()) ? 0.0f : fast_exp2((m_ref - m_new) * cscale);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // head dim 128: every accumulator has a VGPR home (about
                    // 186 registers in all), so S needs no copy out of AGPRs
                    // before the softmax; 256: O stays in AGPRs
                    if constexpr (DH == 256) acc[dt][r] = scale_acc(acc[dt][r], alpha);
                    else acc[dt][r] *= alpha;
                }
            asm volatile("s_nop 7" ::: "memory");
        }
        m_ref = m_new;
        l_run += psum;
        // this wave's DMAs of subtile j + 2 are complete; the barrier then
        // publishes them and retires the buffer of subtile j - 1
        wait_vm<(NBS - 4) * ND>();
        subtile_barrier();
        // ---------------- part B
        // masked subtiles zero the V codes of keys past the visible end (the
        // cache holds garbage there, and P = 0 times a NaN code is NaN)
        // (a lane's operand of key half hf holds keys k0 + 16 hf + 8 h32 + [0,8)
        // in order: 4 per dword of codes, 2 per dword of fp16 values)
        constexpr int VW = sizeof(VR) / 4;           // dwords per V operand
        uint32_t vm[2][VW];
        if constexpr (MASKED) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int cnt = min(max(kend - (k0 + 16 * hf + 8 * h32), 0), 8);
                if constexpr (KV == KV_FP16) {
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        vm[hf][x] = cnt >= 2 * x + 2 ? 0xFFFFFFFFu : (cnt == 2 * x + 1 ? 0x0000FFFFu : 0u);
                } else {
                    vm[hf][0] = cnt >= 4 ? 0xFFFFFFFFu : (1u << (8 * cnt)) - 1u;
                    vm[hf][1] = cnt >= 8 ? 0xFFFFFFFFu : (cnt <= 4 ? 0u : (1u << (8 * (cnt - 4))) - 1u);
                }
            }
        }
        f16x8 vop;
        // subtile j + NBS - 1 into the buffer of subtile j - 1, before any
        // new LDS read
        issue((bcur == 0) ? NBS - 1 : bcur - 1, __builtin_amdgcn_readfirstlane(ids.x),
              __builtin_amdgcn_readfirstlane(ids.y));
        issue_ids(j + 2 * NBS - 1);
        step_fence();
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            {
                VR w = vraw[i % PFV];
                if constexpr (MASKED) {
#pragma unroll
                    for (int x = 0; x < VW; ++x) w[x] &= vm[i / NDT][x];
                }
                if constexpr (KV == KV_FP16) vop = __builtin_bit_cast(f16x8, w);
                else vop = codes8_to_f16x8<KV>(w[0], w[1]);
            }
            if (i + PFV < NQ) vraw[i % PFV] = vread(vbc, (i + PFV) % NDT, (i + PFV) / NDT);
            acc[i % NDT] = mfma32(vop, pp[i / NDT], acc[i % NDT]);
            if (i >= NQ - PFK) kraw[i - (NQ - PFK)] = kread(sk0 + bnn * CB, i - (NQ - PFK));   // subtile j + 2
            step_fence();
        }
        bcur = bn;
    };
    // Head dim 128 takes two subtiles per iteration, the score tiles trading
    // roles, so that no copy moves S(j + 1) into place (at 256 the pair
    // raised the register count from 296 to 407)
    f32x16 sb;
    auto run = [&](auto mtag, int j0, int j1) __attribute__((always_inline)) {
        int j = j0;
        if constexpr (DH == 128) {
            for (; j + 1 < j1; j += 2) {
                sub(mtag, j, sc, sb);
                sub(mtag, j + 1, sb, sc);
            }
        }
        for (; j < j1; ++j) {
            sub(mtag, j, sc, sb);
            sc = sb;
        }
    };
    run(std::false_type{}, 0, nfloc);
    run(std::true_type{}, nfloc, nloc);
    // DMAs still in flight write this workgroup's LDS: let them land first
    wait_vm<0>();

    // ---- epilogue: lanes l and l^32 hold halves of the same row's keys; a
    // row with no visible key in the range (partitions only) writes 0, -inf
    const float l = l_run + shfl_xor(l_run, 32);
    const bool empty = !(l > 0.0f);
    const float inv = empty ? 0.0f : vscale / l;
    if (rowok && h32 == 0) *lrow = empty ? -__builtin_inff() : (m_ref * cscale + __builtin_log2f(l)) * kLn2;
    // O leaves through LDS, 64 dimensions at a time: the MFMA layout gives each
    // store instruction 32-byte pieces of 32 rows, the wave's LDS tile (rows
    // of 64 floats + 4 of padding) four whole 256-byte row pieces.  Lane l
    // stores rows 4i + l/16, floats 4(l%16) + [0,4); the row addresses come
    // from the lanes that own the rows (null for rows past the tile).
    __syncthreads();                                 // every wave is past its last LDS read
    constexpr int TS = 68;                           // LDS tile row stride (floats)
    float* const tile = reinterpret_cast<float*>(&s_kv[0][0][0]) + wave * 32 * TS;
    const uint64_t mine = rowok ? reinterpret_cast<uint64_t>(orow) : 0ull;
    float* dst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int src = (4 * i + (lane >> 4)) << 2;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)mine);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(mine >> 32));
        dst[i] = reinterpret_cast<float*>(((uint64_t)hi << 32) | lo);
    }
#pragma unroll
    for (int ps = 0; ps < DH / 64; ++ps) {
#pragma unroll
        for (int dd = 0; dd < 2; ++dd)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int dt = 2 * ps + dd;
                *reinterpret_cast<f32x4*>(tile + r32 * TS + 32 * dd + 8 * a4 + 4 * h32) =
                    f32x4{acc[dt][4 * a4 + 0], acc[dt][4 * a4 + 1], acc[dt][4 * a4 + 2], acc[dt][4 * a4 + 3]} * inv;
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(tile + (4 * i + (lane >> 4)) * TS + 4 * (lane & 15));
            if (dst[i]) *reinterpret_cast<f32x4*>(dst[i] + 64 * ps + 4 * (lane & 15)) = v;
        }
    }
}

template <int DH>
hipError_t launch_dh(const PrefillParams& p, hipStream_t s) {
    const int G = p.num_q_heads / p.kv.num_kv_heads;
    const int64_t tiles = ((int64_t)p.max_q_len * G + ROWS - 1) / ROWS;
    const int64_t np = p.partition_tokens > 0 ? p.nparts : 1;
    const dim3 grid((unsigned)(tiles * np), p.kv.num_kv_heads, p.num_seqs);
    if (grid.x == 0) return hipSuccess;
    const dim3 block(256);
    switch (p.kv.dtype) {
    case KV_FP16:
        if constexpr (DH != 128) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((prefill_dma_kernel<KV_FP16, DH>), grid, block, 0, s, p);
        break;
    case KV_E4M3: hipLaunchKernelGGL((prefill_dma_kernel<KV_E4M3, DH>), grid, block, 0, s, p); break;
    case KV_INT8: hipLaunchKernelGGL((prefill_dma_kernel<KV_INT8, DH>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_dma(const PrefillParams& p, hipStream_t s) {
    if (p.partition_tokens < 0 || p.partition_tokens % 32 != 0 || (p.partition_tokens > 0 && p.nparts < 1))
        return hipErrorInvalidValue;
    switch (p.kv.head_dim) {
    case 128: return launch_dh<128>(p, s);
    case 256: return launch_dh<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace plc
