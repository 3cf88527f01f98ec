// Device helpers shared by the gfx950 kernels of libplc.
//
// Vector types, the KV codecs (E4M3 <-> fp16, INT8 -> fp16), MFMA wrappers and
// wave-level shuffles.  Everything here is CDNA4 (gfx950) specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plc {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum KvType { KV_FP16 = 0, KV_E4M3 = 1, KV_INT8 = 2 };

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// INT8 attention folds each value row's scale sigma_v, times this factor,
// into the fp16 probability operand (p <= 1), and divides the factor out of
// the fp32 result.  The factor keeps typical products away from fp16
// subnormals, and is small enough that no finite fp16 row overflows:
// sigma_v <= 65504 / 127 = 515.8, and 64 * 515.8 = 33,011 < 65504.
constexpr float kInt8PFold = 64.0f;

// ------------------------------------------------------------------ codecs

// Two E4M3FN codes (bytes 2*hi and 2*hi+1 of w) -> two fp16 values.  Exact:
// every finite E4M3FN value is an fp16 value; the hardware converter on
// gfx950 reads OCP E4M3FN.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Four E4M3 codes in a dword -> f16x4 (byte order kept).
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t w) {
    f16x2 a = e4m3x2_to_f16x2<false>(w);
    f16x2 b = e4m3x2_to_f16x2<true>(w);
    return f16x4{a[0], a[1], b[0], b[1]};
}

// Eight codes in two dwords -> one MFMA operand.
__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
    f16x2 a = e4m3x2_to_f16x2<false>(lo);
    f16x2 b = e4m3x2_to_f16x2<true>(lo);
    f16x2 c = e4m3x2_to_f16x2<false>(hi);
    f16x2 d = e4m3x2_to_f16x2<true>(hi);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Two signed int8 codes (bytes 2*hi, 2*hi+1 of w) -> fp16, exact: the byte
// plus 128 becomes the low mantissa byte of 1024 + u, then 1152 is removed.
template <bool HI>
__device__ __forceinline__ f16x2 i8x2_to_f16x2(uint32_t w) {
    uint32_t u = w ^ 0x80808080u;
    constexpr uint32_t sel = HI ? 0x04030402u : 0x04010400u;
    uint32_t bits = __builtin_amdgcn_perm(0x64646464u, u, sel);
    f16x2 x = __builtin_bit_cast(f16x2, bits);
    return x - f16x2{(f16)1152.0f, (f16)1152.0f};
}

__device__ __forceinline__ f16x8 i8x8_to_f16x8(uint32_t lo, uint32_t hi) {
    f16x2 a = i8x2_to_f16x2<false>(lo);
    f16x2 b = i8x2_to_f16x2<true>(lo);
    f16x2 c = i8x2_to_f16x2<false>(hi);
    f16x2 d = i8x2_to_f16x2<true>(hi);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int KV, bool HI>
__device__ __forceinline__ f16x2 codes2_to_f16x2(uint32_t w) {
    if constexpr (KV == KV_E4M3)
        return e4m3x2_to_f16x2<HI>(w);
    else
        return i8x2_to_f16x2<HI>(w);
}

template <int KV>
__device__ __forceinline__ f16x8 codes8_to_f16x8(uint32_t lo, uint32_t hi) {
    if constexpr (KV == KV_E4M3)
        return e4m3x8_to_f16x8(lo, hi);
    else
        return i8x8_to_f16x8(lo, hi);
}

// fp32 -> nearest E4M3FN code, ties to even, saturating at 448, NaN kept.
// Integer rounding on the fp32 bit pattern: normals drop 20 mantissa bits with
// round-half-even; magnitudes below 2^-6 are multiples of 2^-9 after rounding.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;                                  // NaN
    } else if (a >= 0x43E00000u) {                     // >= 448 (and inf)
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {                      // < 2^-6: subnormal grid
        float af = __builtin_bit_cast(float, a);
        code = (uint32_t)__builtin_rintf(af * 512.0f); // 0..8; 8 is 2^-6
    } else {
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);                        // rebias exponent 127 -> 7
    }
    return code | sign;
}

// Quantize one 8-value slice of a 128-value K or V row held by 16 consecutive
// lanes (lane l%16 owns values 8*(l%16)..+7).  E4M3: x / s in IEEE fp32, then
// f32_to_e4m3.  INT8: sigma = max|x| / 127 over the row (a 16-lane reduction,
// so all 16 lanes must call), codes = clamp(rint(x / sigma), -127, 127), an
// all-zero row giving sigma 0 and zero codes.  Returns the 8 codes, low byte
// first; sigma is written for INT8.
template <int KV, int LPR = 16>
__device__ __forceinline__ u32x2 quantize_slice(f16x8 x, float s, float& sigma);

// ------------------------------------------------------------------ MFMA

// D(16x16) += A(16x32) * B(32x16), f16 inputs, fp32 accumulate.
// Lane l holds A row l%16, B column l%16 (8 K-values each, slot group l/16)
// and D rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32).  Lane l holds A row l%32, B column l%32
// (8 K-values, slot group l/32) and D[8*(r/4) + 4*(l/32) + r%4][l%32], r < 16.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ shuffles

__device__ __forceinline__ float shfl_xor(float x, int mask) {
    int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2,
                                                                  __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One lane's eight values of a K or V row held by LPR consecutive lanes (the
// row has 8 * LPR values; INT8 reduces its maximum over those lanes).
template <int KV, int LPR>
__device__ __forceinline__ u32x2 quantize_slice(f16x8 x, float s, float& sigma) {
    uint32_t w[2] = {0, 0};
    if constexpr (KV == KV_E4M3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e >> 2] |= f32_to_e4m3((float)x[e] / s) << (8 * (e & 3));
    } else {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, __builtin_fabsf((float)x[e]));
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, shfl_xor(m, off));
        sigma = m / 127.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = 0.0f;
            if (sigma != 0.0f) {
                q = __builtin_rintf((float)x[e] / sigma);
                q = fminf(fmaxf(q, -127.0f), 127.0f);
            }
            w[e >> 2] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (e & 3));
        }
    }
    return u32x2{w[0], w[1]};
}

template <typename T>
__device__ __forceinline__ T load_nt(const T* p) {
    return __builtin_nontemporal_load(p);
}

// Materialises v in registers at this point.  Arithmetic that produces v
// cannot be sunk past it, and loads that produce v are issued before it (the
// compiler may otherwise sink work into a later branch or past a barrier,
// which orders memory only).
template <typename T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

// ------------------------------------------------------------------ prefill tiles

// Which key MFMA row rho of S^T holds within a 64-key tile: the swap of bits 2
// and 3 makes the eight keys a lane owns for one PV step consecutive.  K is
// stored in LDS in MFMA row order (the map is its own inverse).
__device__ __forceinline__ int key_of_row(int rho) {
    return (rho & 0x33) | ((rho & 0x8) >> 1) | ((rho & 0x4) << 1);
}

// Maximum of x over lanes l and l ^ 32 (the two halves of a score row) with
// the gfx950 cross-half swap: after it, the first operand holds lanes 0-31 of
// x in both halves and the second lanes 32-63 in both.  The nops cover the
// VALU-write-to-swap and swap-to-VALU-read hazards, which the compiler does
// not see inside the asm.
__device__ __forceinline__ float max_halves(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// x *= s on an accumulator held in an AGPR, through one scratch VGPR (the
// compiler would otherwise give the accumulators VGPR homes for the rare
// rescale, which costs Q operands their VGPRs for the whole loop)
__device__ __forceinline__ float scale_acc(float x, float s) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t) : "v"(s));
    return x;
}

// The compiler moves no instruction across a step fence: a key loop written
// as steps of one MFMA and a slice of other work keeps that interleaving.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ void subtile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}


}  // namespace plc
