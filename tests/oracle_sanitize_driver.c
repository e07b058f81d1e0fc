/*
 * Drives the fp64 oracle (oracle/pa_oracle.c) in a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer.  Test infrastructure only.
 *
 *   oracle_sanitize_driver DIR B Hq Hkv D T MB NB scale k_scale v_scale
 *
 * Reads DIR/{q,k,v,k8,v8,bt,ctx}.bin into heap buffers of exactly their
 * sizes (so any read past an array is reported), runs every entry point, and
 * writes DIR/{out16,out8,rows16,rows8}.bin (float64).  Then it runs the
 * error paths (a block id outside the pool, a context longer than the
 * table, query heads not a multiple of KV heads) on copies and prints their
 * status codes, one "name=code" per line.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pao_decode_f64(const uint16_t *, const uint16_t *, const uint16_t *, const int32_t *,
                   const int32_t *, float, int, int, int, int, int, int, int64_t, double *, int);
int pao_decode_rows_f64(const uint16_t *, const uint16_t *, const uint16_t *, const int32_t *,
                        const int32_t *, float, int, int, int, int, int, int, int64_t,
                        const int32_t *, const int32_t *, int64_t, double *, int);
int pao_decode_fp8_f64(const uint16_t *, const uint8_t *, const uint8_t *, const int32_t *,
                       const int32_t *, float, float, float, int, int, int, int, int, int,
                       int64_t, double *, int);
int pao_decode_fp8_rows_f64(const uint16_t *, const uint8_t *, const uint8_t *,
                            const int32_t *, const int32_t *, float, float, float, int, int,
                            int, int, int, int, int64_t, const int32_t *, const int32_t *,
                            int64_t, double *, int);

static void *slurp(const char *dir, const char *name, size_t want) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void *buf = malloc(want ? want : 1);
    if (fread(buf, 1, want, f) != want || fgetc(f) != EOF) {
        fprintf(stderr, "%s: expected %zu bytes\n", path, want);
        exit(2);
    }
    fclose(f);
    return buf;
}

static void spill(const char *dir, const char *name, const double *x, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(x, sizeof(double), n, f) != n) { fprintf(stderr, "write %s\n", path); exit(2); }
    fclose(f);
}

int main(int argc, char **argv) {
    if (argc != 12) { fprintf(stderr, "usage: see the header\n"); return 2; }
    const char *dir = argv[1];
    const int B = atoi(argv[2]), Hq = atoi(argv[3]), Hkv = atoi(argv[4]);
    const int D = atoi(argv[5]), T = atoi(argv[6]), MB = atoi(argv[7]);
    const int64_t NB = atoll(argv[8]);
    const float scale = strtof(argv[9], NULL), ks = strtof(argv[10], NULL),
                vs = strtof(argv[11], NULL);
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)NB * Hkv * T * D;
    const size_t nbt = (size_t)B * MB;
    uint16_t *q = slurp(dir, "q", nq * 2);
    uint16_t *k = slurp(dir, "k", nkv * 2), *v = slurp(dir, "v", nkv * 2);
    uint8_t *k8 = slurp(dir, "k8", nkv), *v8 = slurp(dir, "v8", nkv);
    int32_t *bt = slurp(dir, "bt", nbt * 4), *ctx = slurp(dir, "ctx", (size_t)B * 4);

    double *out = malloc(nq * sizeof(double));
    int rc = pao_decode_f64(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, out, 1);
    if (rc) { fprintf(stderr, "pao_decode_f64: %d\n", rc); return 3; }
    spill(dir, "out16", out, nq);
    rc = pao_decode_fp8_f64(q, k8, v8, bt, ctx, scale, ks, vs, B, Hq, Hkv, D, T, MB, NB, out, 1);
    if (rc) { fprintf(stderr, "pao_decode_fp8_f64: %d\n", rc); return 3; }
    spill(dir, "out8", out, nq);

    /* rows in reverse order, every (b, h) once */
    const int64_t nr = (int64_t)B * Hq;
    int32_t *rb = malloc((size_t)nr * 4), *rh = malloc((size_t)nr * 4);
    for (int64_t i = 0; i < nr; ++i) {
        rb[i] = (int32_t)((nr - 1 - i) / Hq);
        rh[i] = (int32_t)((nr - 1 - i) % Hq);
    }
    rc = pao_decode_rows_f64(q, k, v, bt, ctx, scale, B, Hq, Hkv, D, T, MB, NB, rb, rh, nr,
                             out, 1);
    if (rc) { fprintf(stderr, "pao_decode_rows_f64: %d\n", rc); return 3; }
    spill(dir, "rows16", out, nq);
    rc = pao_decode_fp8_rows_f64(q, k8, v8, bt, ctx, scale, ks, vs, B, Hq, Hkv, D, T, MB, NB,
                                 rb, rh, nr, out, 1);
    if (rc) { fprintf(stderr, "pao_decode_fp8_rows_f64: %d\n", rc); return 3; }
    spill(dir, "rows8", out, nq);

    /* error paths: the first sequence with tokens gets a bad block id, or a
       context longer than its table row */
    int first = -1;
    for (int b = 0; b < B && first < 0; ++b)
        if (ctx[b] > 0) first = b;
    int32_t *bt2 = malloc(nbt * 4), *ctx2 = malloc((size_t)B * 4);
    memcpy(bt2, bt, nbt * 4);
    memcpy(ctx2, ctx, (size_t)B * 4);
    bt2[(size_t)first * MB] = (int32_t)NB;
    printf("block_id_past_pool=%d\n",
           pao_decode_f64(q, k, v, bt2, ctx, scale, B, Hq, Hkv, D, T, MB, NB, out, 1));
    bt2[(size_t)first * MB] = -1;
    printf("block_id_negative=%d\n",
           pao_decode_fp8_f64(q, k8, v8, bt2, ctx, scale, ks, vs, B, Hq, Hkv, D, T, MB, NB,
                              out, 1));
    ctx2[first] = MB * T + 1;
    printf("context_past_table=%d\n",
           pao_decode_f64(q, k, v, bt, ctx2, scale, B, Hq, Hkv, D, T, MB, NB, out, 1));
    printf("heads_not_a_multiple=%d\n",
           pao_decode_f64(q, k, v, bt, ctx, scale, B, Hq, Hq + 1, D, T, MB, NB, out, 1));
    free(q); free(k); free(v); free(k8); free(v8); free(bt); free(ctx);
    free(out); free(rb); free(rh); free(bt2); free(ctx2);
    return 0;
}
