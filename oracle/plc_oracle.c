/*
 * plc_oracle.c -- plain, slow CPU oracle for paged grouped-query attention
 * over a quantized KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the GPU library; both only read the same seeded inputs.
 *
 * What it computes (sources are the pages this project is built from):
 *  - The cache stores K and V compressed and the model converts them to FP16
 *    for compute (ReVolta README, "Weight and KV formats").  Three storage
 *    types: FP8 E4M3 with calibrated scales ("E4M3 KV"), INT8 with scales
 *    computed per token and head at run time ("INT8 KV"), and FP16.
 *  - Logical tokens live in physical pages found through page IDs
 *    (1Cat-vLLM README, "FlashAttention-V100", Layer 1 "Move KV Cache
 *    Correctly, Wide, and Once").
 *  - Attention keeps fp32 accumulation and causal softmax (Layer 2, "N32
 *    Online Softmax"; "Performance First": FP32 QK/PV).  Split-KV partitions
 *    and prefix / causal-tail pieces are merged from their fp32 partial state
 *    (Layer 2, "Split-KV3" and "Prefix / Causal-Tail Separation").
 *
 * The oracle is the plain definition: dequantize every visible key and value
 * in double, form the scores, take a two-pass softmax, weight the values, and
 * round the result to fp32.  No tiling, no online rescaling, no fused steps.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - "E4M3" is the OCP E4M3FN format: bias 7, no infinities, NaN = S.1111.111,
 *    largest finite 448.  Encoding rounds x/scale (an fp32 division) to the
 *    nearest code, ties to the code with an even last bit, and saturates
 *    finite and infinite magnitudes above 448 to 448; NaN keeps its sign.
 *  - E4M3 scales are one fp32 value per KV head, separately for K and V;
 *    the stored value is decode(code) * scale.
 *  - INT8: sigma = max_d |x_d| / 127 (fp32); code = clamp(rint(x / sigma),
 *    -127, 127) with the division and rounding in fp32 (ties to even);
 *    an all-zero row has sigma = 0 and zero codes.  Value = code * sigma.
 *  - Query row i of a chunk of n new tokens in a sequence whose context is L
 *    tokens (new ones included) sits at position L - n + i and sees keys
 *    0 .. L - n + i.  Query head h reads KV head h / (Hq / Hkv).
 *  - LSE is the natural log of sum_j exp(sm_scale * q . k_j) over the keys
 *    the row sees; a row that sees no key gives o = 0 and lse = -inf.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORC_KV_FP16 0
#define ORC_KV_E4M3 1
#define ORC_KV_INT8 2

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16 value of a bit pattern, from the format's definition. */
double orc_f16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1F;
    int mant = bits & 0x3FF;
    double v;
    if (expo == 0x1F)
        v = mant ? NAN : INFINITY;
    else if (expo == 0)
        v = ldexp((double)mant, -24);                 /* subnormal: m * 2^-24 */
    else
        v = ldexp(1.0 + mant / 1024.0, expo - 15);
    return sign ? -v : v;
}

/* OCP E4M3FN value of a code: sign, 4 exponent bits (bias 7), 3 mantissa bits. */
double orc_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double v;
    if (expo == 0xF && mant == 0x7)
        return NAN;                                   /* the only NaN pattern */
    if (expo == 0)
        v = ldexp((double)mant, -9);                  /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + mant / 8.0, expo - 7);
    return sign ? -v : v;
}

/* Nearest E4M3 code to an fp32 value: exhaustive search over the 127
 * non-negative finite codes, ties to the even code, saturating at 448. */
uint8_t orc_e4m3_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double best_err = a;                              /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(a - orc_e4m3_value((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

/* INT8 symmetric quantization of one row of n fp16 values. */
void orc_int8_encode_row(const uint16_t* x, int n, int8_t* codes, float* sigma_out)
{
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf((float)orc_f16_value(x[i]));
        if (a > m)
            m = a;
    }
    float sigma = m / 127.0f;
    *sigma_out = sigma;
    for (int i = 0; i < n; ++i) {
        if (sigma == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float r = rintf((float)orc_f16_value(x[i]) / sigma);   /* fp32, ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------ */
/* KV append: write new tokens' K/V into their pages                   */
/* ------------------------------------------------------------------ */

/* E4M3 code of the fp16 value with bit pattern x after division by s: the
 * encoder above applied once per distinct fp16 input (2 * Hkv tables of
 * 65,536 entries, filled on first use), so long caches encode quickly. */
typedef struct {
    float scale;
    uint8_t* codes;       /* [65536], NULL until built */
} orc_e4m3_memo;

static uint8_t orc_e4m3_memo_get(orc_e4m3_memo* m, float s, uint16_t x)
{
    if (!m->codes || m->scale != s) {
        if (!m->codes)
            m->codes = (uint8_t*)malloc(65536);
        if (!m->codes)
            abort();
        m->scale = s;
        for (int c = 0; c < 65536; ++c)
            m->codes[c] = orc_e4m3_encode((float)orc_f16_value((uint16_t)c) / s);
    }
    return m->codes[x];
}

/*
 * Token t of the packed new K/V belongs to sequence b with
 * cu_new_lens[b] <= t < cu_new_lens[b+1]; its absolute position is
 * p = start_pos[b] + (t - cu_new_lens[b]); it goes to physical block
 * block_tables[b][p / block_size], slot p % block_size, layout
 * [num_blocks][num_kv_heads][block_size][head_dim].
 * Returns 0, -1 when a target block is outside the pool, -2 without memory.
 */
int orc_kv_append(int32_t kv_dtype,
                  const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* block_tables, int32_t max_blocks,
                  const int32_t* cu_new_lens, const int32_t* start_pos, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  const float* k_scale_head, const float* v_scale_head,
                  void* k_cache, void* v_cache, float* k_scale_tok, float* v_scale_tok)
{
    orc_e4m3_memo* memo = NULL;
    if (kv_dtype == ORC_KV_E4M3) {
        memo = (orc_e4m3_memo*)calloc(2 * (size_t)num_kv_heads, sizeof(orc_e4m3_memo));
        if (!memo)
            return -2;
    }
    int status = 0;
    for (int b = 0; b < num_seqs && status == 0; ++b) {
        for (int t = cu_new_lens[b]; t < cu_new_lens[b + 1]; ++t) {
            int64_t p = (int64_t)start_pos[b] + (t - cu_new_lens[b]);
            if (p / block_size >= max_blocks) {
                status = -1;
                break;
            }
            int32_t blk = block_tables[(int64_t)b * max_blocks + p / block_size];
            if (blk < 0 || blk >= num_blocks) {
                status = -1;
                break;
            }
            int slot = (int)(p % block_size);
            for (int h = 0; h < num_kv_heads; ++h) {
                const uint16_t* srcs[2] = {k_new + ((int64_t)t * num_kv_heads + h) * head_dim,
                                           v_new + ((int64_t)t * num_kv_heads + h) * head_dim};
                void* dsts[2] = {k_cache, v_cache};
                const float* head_scales[2] = {k_scale_head, v_scale_head};
                float* tok_scales[2] = {k_scale_tok, v_scale_tok};
                int64_t row = (((int64_t)blk * num_kv_heads + h) * block_size + slot);
                for (int w = 0; w < 2; ++w) {
                    const uint16_t* x = srcs[w];
                    if (kv_dtype == ORC_KV_FP16) {
                        memcpy((uint16_t*)dsts[w] + row * head_dim, x, sizeof(uint16_t) * head_dim);
                    } else if (kv_dtype == ORC_KV_E4M3) {
                        uint8_t* dst = (uint8_t*)dsts[w] + row * head_dim;
                        float s = head_scales[w][h];
                        for (int d = 0; d < head_dim; ++d)   /* encode(x / s), fp32 division */
                            dst[d] = orc_e4m3_memo_get(&memo[2 * h + w], s, x[d]);
                    } else if (kv_dtype == ORC_KV_INT8) {
                        int8_t* dst = (int8_t*)dsts[w] + row * head_dim;
                        orc_int8_encode_row(x, head_dim, dst, &tok_scales[w][row]);
                    } else {
                        status = -1;
                    }
                }
            }
        }
    }
    if (memo) {
        for (int i = 0; i < 2 * num_kv_heads; ++i)
            free(memo[i].codes);
        free(memo);
    }
    return status;
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint16_t* q;
    int32_t num_q_heads;
    int32_t kv_dtype;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    int32_t num_blocks, block_size, num_kv_heads, head_dim;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* cu_q_lens;
    const int32_t* context_lens;
    int32_t num_seqs;
    double sm_scale;
    const int64_t* rows;
    int64_t n_rows;
    int64_t key_begin, key_end;
    int64_t window;                 /* > 0: keys pos - window + 1 .. pos only */
    float* out;
    float* lse;
    /* decode tables built once per call from the format definitions */
    double e4m3_table[256];
    double* f16_table;
    int status;
} orc_attn_job;

typedef struct {
    orc_attn_job* job;
    int64_t r0, r1;
    int status;
} orc_attn_slice;

/* Dequantized element d of token j (absolute position) of KV head g. */
static double orc_kv_value(const orc_attn_job* J, const void* cache, const float* scale,
                           int32_t blk, int slot, int g, int d)
{
    int64_t row = ((int64_t)blk * J->num_kv_heads + g) * J->block_size + slot;
    int64_t idx = row * J->head_dim + d;
    switch (J->kv_dtype) {
    case ORC_KV_FP16:
        return J->f16_table[((const uint16_t*)cache)[idx]];
    case ORC_KV_E4M3:
        return J->e4m3_table[((const uint8_t*)cache)[idx]] * (double)scale[g];
    default:
        return (double)((const int8_t*)cache)[idx] * (double)scale[row];
    }
}

static int orc_attention_row(const orc_attn_job* J, int64_t r, double* scores, double* q, double* acc)
{
    const int Hq = J->num_q_heads, D = J->head_dim;
    const int64_t t = r / Hq;
    const int h = (int)(r % Hq);
    const int G = Hq / J->num_kv_heads;
    const int g = h / G;
    int b = 0;
    while (b + 1 <= J->num_seqs && J->cu_q_lens[b + 1] <= t)
        ++b;
    if (b >= J->num_seqs)
        return -1;
    const int64_t n = J->cu_q_lens[b + 1] - J->cu_q_lens[b];
    const int64_t L = J->context_lens[b];
    const int64_t pos = L - n + (t - J->cu_q_lens[b]);
    int64_t lo = J->key_begin > 0 ? J->key_begin : 0;
    if (J->window > 0 && pos - J->window + 1 > lo)
        lo = pos - J->window + 1;
    int64_t hi = pos + 1;
    if (J->key_end < hi)
        hi = J->key_end;
    float* o = J->out + r * D;
    if (hi <= lo) {
        for (int d = 0; d < D; ++d)
            o[d] = 0.0f;
        J->lse[r] = -INFINITY;
        return 0;
    }
    for (int d = 0; d < D; ++d)
        q[d] = J->f16_table[J->q[r * D + d]];
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; ++j) {
        if (j / J->block_size >= J->max_blocks)
            return -1;
        int32_t blk = J->block_tables[(int64_t)b * J->max_blocks + j / J->block_size];
        if (blk < 0 || blk >= J->num_blocks)
            return -1;
        int slot = (int)(j % J->block_size);
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += q[d] * orc_kv_value(J, J->k_cache, J->k_scale, blk, slot, g, d);
        s *= J->sm_scale;
        scores[j - lo] = s;
        if (s > m)
            m = s;
    }
    /* pass 2: normalizer and weighted values */
    double l = 0.0;
    for (int d = 0; d < D; ++d)
        acc[d] = 0.0;
    for (int64_t j = lo; j < hi; ++j) {
        int32_t blk = J->block_tables[(int64_t)b * J->max_blocks + j / J->block_size];
        int slot = (int)(j % J->block_size);
        double p = exp(scores[j - lo] - m);
        l += p;
        for (int d = 0; d < D; ++d)
            acc[d] += p * orc_kv_value(J, J->v_cache, J->v_scale, blk, slot, g, d);
    }
    for (int d = 0; d < D; ++d)
        o[d] = (float)(acc[d] / l);
    J->lse[r] = (float)(m + log(l));
    return 0;
}

static int64_t orc_max_context(const orc_attn_job* J)
{
    int64_t m = 1;
    for (int b = 0; b < J->num_seqs; ++b)
        if (J->context_lens[b] > m)
            m = J->context_lens[b];
    return m;
}

static void* orc_attention_worker(void* arg)
{
    orc_attn_slice* S = (orc_attn_slice*)arg;
    const orc_attn_job* J = S->job;
    double* scores = (double*)malloc(sizeof(double) * (size_t)orc_max_context(J));
    double* q = (double*)malloc(sizeof(double) * J->head_dim);
    double* acc = (double*)malloc(sizeof(double) * J->head_dim);
    S->status = (scores && q && acc) ? 0 : -2;
    for (int64_t i = S->r0; i < S->r1 && S->status == 0; ++i) {
        int64_t r = J->rows ? J->rows[i] : i;
        S->status = orc_attention_row(J, r, scores, q, acc);
    }
    free(scores);
    free(q);
    free(acc);
    return NULL;
}

/*
 * Attention for a list of query rows.  Row id r = t * num_q_heads + h, where
 * t indexes the packed new query tokens (q: f16 bits [T][Hq][D]).  out gets
 * fp32 [T][Hq][D] and lse fp32 [T][Hq] at the listed rows only.  Keys are the
 * row's causal range intersected with [key_begin, key_end) (absolute token
 * positions; pass 0 and INT64_MAX for the whole range) and, when window > 0,
 * with the row's sliding window: the query at position pos sees only keys
 * pos - window + 1 .. pos, the most recent window tokens including its own
 * (1Cat-vLLM README, "DFlash2 Long-Context Decay": the draft attends over a
 * sliding window; ReVolta 0.1.2 release notes: the DFlash2 drafter's
 * 2048-token window).  Scales: E4M3 takes
 * [Hkv] per KV head, INT8 takes [num_blocks][Hkv][block_size] per token.
 * rows = NULL means every row 0 .. n_rows-1.  nthreads <= 0 uses all cores.
 * Returns 0, -1 for a table entry outside the pool, -2 when out of memory.
 */
int orc_attention(const uint16_t* q, int32_t num_q_heads, int32_t kv_dtype,
                  const void* k_cache, const void* v_cache,
                  const float* k_scale, const float* v_scale,
                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                  const int32_t* block_tables, int32_t max_blocks,
                  const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_seqs,
                  double sm_scale, const int64_t* rows, int64_t n_rows,
                  int64_t key_begin, int64_t key_end, int64_t window,
                  float* out, float* lse, int32_t nthreads)
{
    orc_attn_job* J = (orc_attn_job*)calloc(1, sizeof(orc_attn_job));
    if (!J)
        return -2;
    J->q = q; J->num_q_heads = num_q_heads; J->kv_dtype = kv_dtype;
    J->k_cache = k_cache; J->v_cache = v_cache; J->k_scale = k_scale; J->v_scale = v_scale;
    J->num_blocks = num_blocks; J->block_size = block_size;
    J->num_kv_heads = num_kv_heads; J->head_dim = head_dim;
    J->block_tables = block_tables; J->max_blocks = max_blocks;
    J->cu_q_lens = cu_q_lens; J->context_lens = context_lens; J->num_seqs = num_seqs;
    J->sm_scale = sm_scale; J->rows = rows; J->n_rows = n_rows;
    J->key_begin = key_begin; J->key_end = key_end; J->window = window;
    J->out = out; J->lse = lse;
    for (int c = 0; c < 256; ++c)
        J->e4m3_table[c] = orc_e4m3_value((uint8_t)c);
    J->f16_table = (double*)malloc(sizeof(double) * 65536);
    if (!J->f16_table) {
        free(J);
        return -2;
    }
    for (int c = 0; c < 65536; ++c)
        J->f16_table[c] = orc_f16_value((uint16_t)c);

    if (nthreads <= 0)
        nthreads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > n_rows)
        nthreads = (int32_t)(n_rows > 0 ? n_rows : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
    orc_attn_slice* sl = (orc_attn_slice*)malloc(sizeof(orc_attn_slice) * nthreads);
    int status = (th && sl) ? 0 : -2;
    if (status == 0) {
        int started = 0;
        for (int i = 0; i < nthreads; ++i) {
            sl[i].job = J;
            sl[i].r0 = n_rows * i / nthreads;
            sl[i].r1 = n_rows * (i + 1) / nthreads;
            sl[i].status = 0;
            if (pthread_create(&th[i], NULL, orc_attention_worker, &sl[i]) != 0) {
                orc_attention_worker(&sl[i]);     /* run inline if no thread */
                th[i] = 0;
            } else {
                ++started;
            }
        }
        for (int i = 0; i < nthreads; ++i) {
            if (th[i])
                pthread_join(th[i], NULL);
            if (sl[i].status != 0)
                status = sl[i].status;
        }
        (void)started;
    }
    free(th);
    free(sl);
    free(J->f16_table);
    free(J);
    return status;
}

/* ------------------------------------------------------------------ */
/* Merge of partial attention states                                   */
/* ------------------------------------------------------------------ */

/*
 * Combine per-part results (o_k, lse_k) of one row into the result over the
 * union of the parts: M = max_k lse_k, w_k = exp(lse_k - M),
 * o = sum_k w_k o_k / sum_k w_k, lse = M + ln(sum_k w_k).  Parts with
 * lse = -inf carry no weight; if every part is empty, o = 0, lse = -inf.
 * Layout: o_parts [rows][nparts][D], lse_parts [rows][nparts].
 */
void orc_lse_merge(const float* o_parts, const float* lse_parts, int64_t rows, int32_t nparts,
                   int32_t head_dim, float* out, float* lse_out)
{
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    for (int64_t r = 0; r < rows; ++r) {
        const float* lp = lse_parts + r * nparts;
        double M = -INFINITY;
        for (int k = 0; k < nparts; ++k)
            if ((double)lp[k] > M)
                M = lp[k];
        float* o = out + r * head_dim;
        if (M == -INFINITY) {
            for (int d = 0; d < head_dim; ++d)
                o[d] = 0.0f;
            lse_out[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int d = 0; d < head_dim; ++d)
            acc[d] = 0.0;
        for (int k = 0; k < nparts; ++k) {
            if (lp[k] == -INFINITY)
                continue;
            double w = exp((double)lp[k] - M);
            wsum += w;
            const float* ok = o_parts + (r * nparts + k) * head_dim;
            for (int d = 0; d < head_dim; ++d)
                acc[d] += w * (double)ok[d];
        }
        for (int d = 0; d < head_dim; ++d)
            o[d] = (float)(acc[d] / wsum);
        lse_out[r] = (float)(M + log(wsum));
    }
    free(acc);
}
