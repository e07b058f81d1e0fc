/*
 * Paged decode attention, fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no source with the HIP kernels.
 *
 * What it computes (plain definition, two-pass softmax, no blocking):
 *   For sequence b and query head h, with g = Hq / Hkv and kv head h / g,
 *   every token t < ctx[b] of the sequence lives in physical block
 *   bt[b][t / T] at slot t % T.  Then
 *       s_t   = scale * sum_d q[b][h][d] * K[p_t][kvh][t % T][d]
 *       out_d = sum_t exp(s_t - max s) * V[p_t][kvh][t % T][d]
 *               / sum_t exp(s_t - max s)
 *   All arithmetic is in double; fp16 inputs are widened exactly.
 *
 * Sources (pages by title):
 *   - "Accelerating LLM Inference Throughput via Asynchronous KV Cache
 *     Prefetching" review, section 3.4 (Algorithm 1: the block table maps a
 *     logical block index to the physical K block that Q*K^T is computed
 *     against) and section 4.1 (logits times V).
 *   - the same review, section 4.2: one block holds T_block = 16 tokens of
 *     d_h = 128 fp16 values per head.
 *   - "How to optimize the memory access latency of an LLM inference
 *     engine?" answer, section 3: page table -> physical page -> blockwise
 *     attention -> reduced output; several query heads share a KV head
 *     under GQA (review, section 4.3 table).
 * The softmax form itself is not printed on the pages; the oracle uses the
 * textbook max-subtracted two-pass softmax, which any online or partitioned
 * softmax equals up to rounding.
 *
 * Layouts (all row-major, element offsets):
 *   q       [B][Hq][D]           fp16 bits
 *   k_cache [NB][Hkv][T][D]      fp16 bits (token-major inside a block)
 *   v_cache [NB][Hkv][T][D]      fp16 bits
 *   bt      [B][MB]              int32 physical block ids
 *   ctx     [B]                  int32 tokens to attend to
 *   out     [B][Hq][D]           double
 * ctx[b] <= 0 gives an all-zero row.  Tokens t >= ctx[b], block-table
 * padding and unused pool blocks are never read.
 *
 * FP8 caches (the PagedAttention answer, section 4, names FP8 KV storage):
 * the same layouts with one OCP E4M3 byte per value; a cached value means
 * decode(byte) * k_scale for K and decode(byte) * v_scale for V, and the
 * attention is the same definition applied to those values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PAO_OK 0
#define PAO_ERR_ARG 1
#define PAO_ERR_BLOCK_ID 2
#define PAO_ERR_CTX 3
#define PAO_ERR_NOMEM 4

/* IEEE binary16 -> double, exact.  1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 is subnormal, 31 is inf/nan. */
double pao_half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* OCP FP8 E4M3 -> double, exact.  1 sign bit, 4 exponent bits (bias 7),
 * 3 fraction bits; exponent 0 is subnormal; no infinities; exponent 15 with
 * fraction 7 (0x7f, 0xff) is NaN, every other exponent-15 code is a normal
 * number (the largest is 448). */
double pao_e4m3_to_double(uint8_t x) {
    const int sign = (x >> 7) & 1;
    const int expo = (x >> 3) & 0xf;
    const int frac = x & 0x7;
    double mag;
    if (expo == 0xf && frac == 0x7) {
        mag = NAN;
    } else if (expo == 0) {
        mag = ldexp((double)frac, -9);
    } else {
        mag = ldexp((double)(8 + frac), expo - 10);
    }
    return sign ? -mag : mag;
}

/* Element idx of a K or V pool: fp16 bits, or E4M3 bytes times their scale. */
typedef struct {
    const void *data;
    int fp8;
    double scale;
} pao_pool;

static double pao_at(pao_pool p, int64_t idx) {
    if (p.fp8) return pao_e4m3_to_double(((const uint8_t *)p.data)[idx]) * p.scale;
    return pao_half_to_double(((const uint16_t *)p.data)[idx]);
}

/* One (b, h) output row.  Returns a PAO_* code. */
static int pao_row(const uint16_t *q, pao_pool k_cache, pao_pool v_cache,
                   const int32_t *bt, const int32_t *ctx, double scale, int b,
                   int h, int Hq, int Hkv, int D, int T, int MB, int64_t NB,
                   double *out_row, double *s /* scratch, >= MB*T */) {
    const int g = Hq / Hkv;
    const int kvh = h / g;
    const int L = ctx[b];
    int d, t;
    for (d = 0; d < D; ++d) out_row[d] = 0.0;
    if (L <= 0) return PAO_OK;
    if ((int64_t)L > (int64_t)MB * T) return PAO_ERR_CTX;

    const uint16_t *qrow = q + ((int64_t)b * Hq + h) * D;

    /* scores */
    double m = -INFINITY;
    for (t = 0; t < L; ++t) {
        const int32_t p = bt[(int64_t)b * MB + t / T];
        if (p < 0 || (int64_t)p >= NB) return PAO_ERR_BLOCK_ID;
        const int64_t krow = (((int64_t)p * Hkv + kvh) * T + t % T) * D;
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += pao_half_to_double(qrow[d]) * pao_at(k_cache, krow + d);
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
    }

    /* weights and normaliser */
    double Z = 0.0;
    for (t = 0; t < L; ++t) {
        s[t] = exp(s[t] - m);
        Z += s[t];
    }

    /* weighted sum of V rows */
    for (t = 0; t < L; ++t) {
        const int32_t p = bt[(int64_t)b * MB + t / T];
        const int64_t vrow = (((int64_t)p * Hkv + kvh) * T + t % T) * D;
        for (d = 0; d < D; ++d) out_row[d] += s[t] * pao_at(v_cache, vrow + d);
    }
    for (d = 0; d < D; ++d) out_row[d] /= Z;
    return PAO_OK;
}

static int pao_check_shape(int B, int Hq, int Hkv, int D, int T, int MB, int64_t NB) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || T <= 0 || MB <= 0 || NB < 0)
        return PAO_ERR_ARG;
    if (Hq % Hkv != 0) return PAO_ERR_ARG;
    return PAO_OK;
}

static int pao_rows(const uint16_t *q, pao_pool k_cache, pao_pool v_cache,
                    const int32_t *bt, const int32_t *ctx, float scale, int B,
                    int Hq, int Hkv, int D, int T, int MB, int64_t NB,
                    const int32_t *rows_b, const int32_t *rows_h, int64_t nrows,
                    double *out, int nthreads) {
    int rc = pao_check_shape(B, Hq, Hkv, D, T, MB, NB);
    if (rc) return rc;
    if (!q || !k_cache.data || !v_cache.data || !bt || !ctx || !rows_b || !rows_h || !out)
        return nrows == 0 ? PAO_OK : PAO_ERR_ARG;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows_b[i] < 0 || rows_b[i] >= B || rows_h[i] < 0 || rows_h[i] >= Hq)
            return PAO_ERR_ARG;

    int err = PAO_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)MB * (size_t)T);
        if (!s) {
#pragma omp critical
            err = PAO_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < nrows; ++i) {
                int r = pao_row(q, k_cache, v_cache, bt, ctx, (double)scale,
                                rows_b[i], rows_h[i], Hq, Hkv, D, T, MB, NB,
                                out + i * D, s);
                if (r) {
#pragma omp critical
                    err = r;
                }
            }
            free(s);
        }
    }
    return err;
}

/* Every (b, h); out is [B][Hq][D]. */
static int pao_all(const uint16_t *q, pao_pool k_cache, pao_pool v_cache,
                   const int32_t *bt, const int32_t *ctx, float scale, int B,
                   int Hq, int Hkv, int D, int T, int MB, int64_t NB, double *out,
                   int nthreads) {
    int rc = pao_check_shape(B, Hq, Hkv, D, T, MB, NB);
    if (rc) return rc;
    const int64_t n = (int64_t)B * Hq;
    int32_t *rb = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    int32_t *rh = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    if (!rb || !rh) {
        free(rb);
        free(rh);
        return PAO_ERR_NOMEM;
    }
    for (int64_t i = 0; i < n; ++i) {
        rb[i] = (int32_t)(i / Hq);
        rh[i] = (int32_t)(i % Hq);
    }
    rc = pao_rows(q, k_cache, v_cache, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB,
                  rb, rh, n, out, nthreads);
    free(rb);
    free(rh);
    return rc;
}

/* fp16 caches. */
int pao_decode_f64(const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *bt,
                   const int32_t *ctx, float scale, int B, int Hq, int Hkv,
                   int D, int T, int MB, int64_t NB, double *out, int nthreads) {
    pao_pool k = {k_cache, 0, 1.0}, v = {v_cache, 0, 1.0};
    return pao_all(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, out, nthreads);
}

/* Rows listed in (rows_b[i], rows_h[i]) for i < nrows; out is [nrows][D]. */
int pao_decode_rows_f64(const uint16_t *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *bt,
                        const int32_t *ctx, float scale, int B, int Hq, int Hkv,
                        int D, int T, int MB, int64_t NB, const int32_t *rows_b,
                        const int32_t *rows_h, int64_t nrows, double *out,
                        int nthreads) {
    pao_pool k = {k_cache, 0, 1.0}, v = {v_cache, 0, 1.0};
    return pao_rows(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, rows_b,
                    rows_h, nrows, out, nthreads);
}

/* E4M3 caches with per-tensor scales (applied in double). */
int pao_decode_fp8_f64(const uint16_t *q, const uint8_t *k_cache,
                       const uint8_t *v_cache, const int32_t *bt,
                       const int32_t *ctx, float scale, float k_scale,
                       float v_scale, int B, int Hq, int Hkv, int D, int T,
                       int MB, int64_t NB, double *out, int nthreads) {
    pao_pool k = {k_cache, 1, (double)k_scale}, v = {v_cache, 1, (double)v_scale};
    return pao_all(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, out, nthreads);
}

int pao_decode_fp8_rows_f64(const uint16_t *q, const uint8_t *k_cache,
                            const uint8_t *v_cache, const int32_t *bt,
                            const int32_t *ctx, float scale, float k_scale,
                            float v_scale, int B, int Hq, int Hkv, int D, int T,
                            int MB, int64_t NB, const int32_t *rows_b,
                            const int32_t *rows_h, int64_t nrows, double *out,
                            int nthreads) {
    pao_pool k = {k_cache, 1, (double)k_scale}, v = {v_cache, 1, (double)v_scale};
    return pao_rows(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, rows_b,
                    rows_h, nrows, out, nthreads);
}

int pao_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
