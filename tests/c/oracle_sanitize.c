/* The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built with gcc by tests/test_sanitize_cpu.py together with oracle/oracle.c):
 * segments, the layer with a stored base, with a bf16 base and with an E4M3
 * base, in both storage types, over ragged shapes and ranks 1 .. 64, and the
 * E4M3 decode of every code.  Exits 0 when the checks hold; a sanitizer
 * report aborts the process. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_adapter_numel(int32_t r, int32_t d_in, int32_t d_out);
int64_t oracle_adapter_bytes(int32_t r, int32_t d_in, int32_t d_out, int32_t bytes_per_param);
int32_t oracle_segments(int32_t T, const int32_t *ids, int32_t n_adapters, int32_t *perm, int32_t *seg_indptr,
                        int32_t *seg_adapter);
void oracle_e4m3_decode(const uint8_t *codes, int64_t n, double *out);
int oracle_lora_forward(int32_t T, int32_t d_in, int32_t d_out, int32_t is_bf16, const void *x, int64_t ldx,
                        const int32_t *ids, int32_t n_adapters, const void *pool, const int64_t *a_off,
                        const int64_t *b_off, const int32_t *rank, const float *alpha, const void *y_in,
                        int64_t ldy, const void *W0, int32_t w0_e4m3, double w0_scale, double *v_out, int64_t ldv,
                        double *y_out, int32_t nthreads);

static int failures;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);        \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static uint32_t rng_state = 777u;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}
static float frand(void) { return (float)(rnd() % 2001) / 1000.0f - 1.0f; }

/* fills n elements of a bf16 (uint16 bits, truncated) or fp32 array */
static void fill(void *p, int is_bf16, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        const float f = frand();
        if (is_bf16) {
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
        } else {
            ((float *)p)[i] = f;
        }
    }
}

static void layer_case(int32_t T, int32_t d_in, int32_t d_out, int32_t n, int is_bf16, int base)
{
    const int es = is_bf16 ? 2 : 4;
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T ? T : 1));
    int32_t *rank = malloc(sizeof(int32_t) * (size_t)n);
    float *alpha = malloc(sizeof(float) * (size_t)n);
    int64_t *a_off = malloc(sizeof(int64_t) * (size_t)n), *b_off = malloc(sizeof(int64_t) * (size_t)n);
    int64_t total = 0;
    int32_t max_rank = 1;
    for (int32_t i = 0; i < n; ++i) {
        rank[i] = 1 + (int32_t)(rnd() % 64);
        alpha[i] = (float)(1 + rnd() % 32);
        a_off[i] = total;
        total += (int64_t)rank[i] * d_in;
        b_off[i] = total;
        total += (int64_t)rank[i] * d_out;
        if (rank[i] > max_rank) max_rank = rank[i];
    }
    for (int32_t t = 0; t < T; ++t) ids[t] = (int32_t)(rnd() % (uint32_t)(n + 1)) - 1;
    void *pool = malloc((size_t)(total ? total : 1) * es);
    void *x = malloc((size_t)T * d_in * es + 1);
    void *y_in = malloc((size_t)T * d_out * es + 1);
    void *W0 = malloc((size_t)d_out * d_in * es + 1);
    uint8_t *q = malloc((size_t)d_out * d_in + 1);
    fill(pool, is_bf16, total);
    fill(x, is_bf16, (int64_t)T * d_in);
    fill(y_in, is_bf16, (int64_t)T * d_out);
    fill(W0, is_bf16, (int64_t)d_out * d_in);
    for (int64_t i = 0; i < (int64_t)d_out * d_in; ++i) {
        q[i] = (uint8_t)(rnd() & 0xFF);
        if ((q[i] & 0x7F) == 0x7F) q[i] = 0x38; /* no NaN codes: the sums are checked finite */
    }
    double *v = malloc(sizeof(double) * (size_t)(T ? T : 1) * max_rank);
    double *y = malloc(sizeof(double) * (size_t)(T ? T : 1) * d_out);
    const void *w = base == 1 ? W0 : (base == 2 ? (const void *)q : NULL);
    const int rc = oracle_lora_forward(T, d_in, d_out, is_bf16, x, d_in, ids, n, pool, a_off, b_off, rank, alpha,
                                       base == 0 ? y_in : NULL, d_out, w, base == 2, 0.01, v, max_rank, y, 4);
    CHECK(rc == 0);
    for (int64_t i = 0; i < (int64_t)T * d_out; ++i) CHECK(isfinite(y[i]));
    /* a bad id is rejected */
    if (T > 0) {
        const int32_t keep = ids[0];
        ids[0] = n;
        CHECK(oracle_lora_forward(T, d_in, d_out, is_bf16, x, d_in, ids, n, pool, a_off, b_off, rank, alpha, NULL,
                                  d_out, NULL, 0, 1.0, NULL, 0, y, 1) == -1);
        ids[0] = keep;
    }
    free(ids); free(rank); free(alpha); free(a_off); free(b_off); free(pool);
    free(x); free(y_in); free(W0); free(q); free(v); free(y);
}

int main(void)
{
    CHECK(oracle_adapter_numel(16, 4096, 4096) == 16 * 8192);
    CHECK(oracle_adapter_bytes(8, 4096, 1024, 2) == 8 * 5120 * 2);
    uint8_t codes[256];
    double vals[256];
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    oracle_e4m3_decode(codes, 256, vals);
    CHECK(vals[0x7E] == 448.0 && isnan(vals[0x7F]) && vals[0x01] == ldexp(1.0, -9));
    for (int32_t T = 0; T < 300; T += 37) {
        int32_t ids[300], perm[300], indptr[301], adapter[300];
        for (int32_t t = 0; t < T; ++t) ids[t] = (int32_t)(rnd() % 10) - 1;
        const int32_t S = oracle_segments(T, ids, 9, perm, indptr, adapter);
        CHECK(S >= 0);
        for (int32_t s = 0; s < S; ++s) CHECK(indptr[s] < indptr[s + 1]);
    }
    const int32_t shapes[][4] = {{1, 8, 8, 1}, {7, 24, 40, 3}, {33, 136, 72, 5}, {64, 256, 200, 9}, {0, 16, 16, 2}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int is_bf16 = 0; is_bf16 < 2; ++is_bf16)
            for (int base = 0; base < 3; ++base)
                layer_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], is_bf16, base);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle_sanitize: ok\n");
    return 0;
}
