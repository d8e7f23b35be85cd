/*
 * fp64 CPU oracle for the multi-LoRA batched adapter path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library; the product path never
 * calls it.  It shares no source, header, table or helper with the GPU library
 * and is built with gcc, not hipcc.
 *
 * What it computes is the plain definition, token by token, in the original
 * token order -- no grouping, no sort, no tiling:
 *
 *   "Multi-LoRA Serving in Production: Comparing S-LoRA, Punica, LoRAX, and
 *   vLLM ..." (llms.blog), section "Mathematical Formulation and the Batching
 *   Challenge", layer equation: the output is x W0 plus (alpha/r) (x A) B, with
 *   A of shape d_in x r and B of shape r x d_out.
 *
 *   "Multi-LoRA serving: the single translator with a thousand glossaries"
 *   (blog.lo0.es), section "SGMV: the kernel that holds it all up": every token
 *   t of the batch gets the correction of its own adapter a(t).
 *
 * Storage (row-major): x [T, d_in]; A_i [r_i, d_in]; B_i [d_out, r_i];
 * W0 [d_out, d_in]; y [T, d_out].  In the pages' row-vector notation this is
 * v = x A_i (v_j = sum_k x_k A_i[j,k]) and c = v B_i (c_n = sum_j v_j B_i[n,j]).
 *
 * Precision: every input element is decoded exactly (bf16 bit patterns or
 * fp32) to double; all sums are accumulated in double; the scale alpha/r is
 * formed in double.  Output is double.
 *
 * Quantised base: "Multi-LoRA serving: the single translator with a thousand
 * glossaries" (blog.lo0.es), section "Combined pattern with quantisation and
 * disaggregated serving", serves the adapters in BF16 over an FP8 base.  Here
 * that base is W0 = w0_scale * q, q the matrix of 8-bit E4M3 codes (one fp32
 * scale for the whole matrix, the plainest reading: the pages fix no scale
 * granularity), decoded exactly to double.
 *
 * Planted mistakes: building with -DORACLE_MUTANT=k (k >= 1) compiles one
 * deliberate error so that the pin tests can show they would catch it.  The
 * default build (ORACLE_MUTANT undefined or 0) has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Decode element i of a stored array (is_bf16: uint16 bit patterns; else fp32). */
static double load_elem(const void *base, int is_bf16, int64_t i)
{
    if (is_bf16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }

/*
 * One 8-bit E4M3 code as a double, exactly, from the format's definition in the
 * OCP 8-bit floating point specification (OFP8, revision 1.0), section on the
 * E4M3 encoding: bit 7 is the sign, bits 6..3 the exponent field e (bias 7),
 * bits 2..0 the mantissa field m.  e = 0 encodes the subnormals m/8 * 2^-6
 * (and the two zeros); the pattern with e = 15 and m = 7 is NaN (the format
 * has no infinities); every other code is the normal number (1 + m/8) 2^(e-7),
 * the largest being e = 15, m = 6: 448.
 */
static double e4m3_value(uint8_t c)
{
    const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
#if ORACLE_MUTANT == 14
    (void)0; /* planted: the NaN pattern decoded as a normal number */
#else
    if (e == 15 && m == 7) return NAN;
#endif
    double mag;
#if ORACLE_MUTANT == 12
    mag = ldexp(1.0 + m / 8.0, e - 7); /* planted: subnormals given the implicit one */
#else
    if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
#if ORACLE_MUTANT == 11
        mag = ldexp(1.0 + m / 8.0, e - 8); /* planted: exponent bias 8 */
#else
        mag = ldexp(1.0 + m / 8.0, e - 7);
#endif
#endif
    return sign ? -mag : mag;
}

/* Decodes n E4M3 codes to doubles (see e4m3_value). */
void oracle_e4m3_decode(const uint8_t *codes, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

/*
 * Adapter size: "Multi-LoRA Serving: Many Adapters on One GPU" (gpusmith.com),
 * section "LoRA recap and why adapters are small": a layer with input width k
 * and output width d holds r (k + d) adapter parameters.  Bytes per matrix:
 * "Multi-LoRA serving: the single translator ..." (blog.lo0.es), section "The
 * maths that matters", memory per adapter: (d_in r + r d_out) b.
 */
int64_t oracle_adapter_numel(int32_t r, int32_t d_in, int32_t d_out)
{
#if ORACLE_MUTANT == 9
    return (int64_t)r * d_in + d_out; /* planted: parenthesis dropped */
#else
    return (int64_t)r * ((int64_t)d_in + (int64_t)d_out);
#endif
}

int64_t oracle_adapter_bytes(int32_t r, int32_t d_in, int32_t d_out, int32_t bytes_per_param)
{
    return oracle_adapter_numel(r, d_in, d_out) * bytes_per_param;
}

/*
 * Grouping of the batch's tokens by adapter into contiguous segments, one
 * adapter id per segment ("Multi-LoRA Serving in Production ...", section
 * "Punica and Segmented Gather Matrix-Vector Multiplication (SGMV)").
 *
 * Reading taken where the pages are silent: segments in ascending adapter id;
 * within a segment the original token order; tokens with id < 0 belong to no
 * segment.  Brute force: for each id in turn, scan the whole batch.
 *
 * Outputs: perm[p] = original index of the token at sorted position p
 * (length = tokens with an adapter), seg_indptr[S+1], seg_adapter[S].
 * Returns S, or -1 if an id is >= n_adapters.
 */
int32_t oracle_segments(int32_t T, const int32_t *ids, int32_t n_adapters,
                        int32_t *perm, int32_t *seg_indptr, int32_t *seg_adapter)
{
    for (int32_t t = 0; t < T; ++t)
        if (ids[t] >= n_adapters) return -1;
    int32_t S = 0, p = 0;
    seg_indptr[0] = 0;
    for (int32_t a = 0; a < n_adapters; ++a) {
        int32_t start = p;
#if ORACLE_MUTANT == 8
        for (int32_t t = T - 1; t >= 0; --t) /* planted: reversed order within an id */
#else
        for (int32_t t = 0; t < T; ++t)
#endif
            if (ids[t] == a) perm[p++] = t;
        if (p > start) {
            seg_adapter[S] = a;
            seg_indptr[++S] = p;
        }
    }
    return S;
}

/*
 * The layer output for every token, in fp64.
 *
 *   x       [T, ldx]     activations (bf16 bits or fp32)
 *   ids     [T]          adapter per token, -1 = none
 *   pool    flat         adapter storage; A_i at pool + a_off[i] ([r_i, d_in]),
 *                        B_i at pool + b_off[i] ([d_out, r_i]) (element offsets)
 *   rank    [N], alpha [N]
 *   y_in    [T, ldy]     base output accumulated into; NULL = zero base
 *   W0      [d_out, d_in] when non-NULL the base is x W0 (y_in is then ignored);
 *           stored like x, or, when w0_e4m3 is set, as E4M3 codes (one byte
 *           each) standing for w0_scale * code
 *   v_out   [T, ldv]     optional: the shrink result x A_a(t) (rows of tokens
 *                        without an adapter are left untouched)
 *   y_out   [T, d_out]   result
 *
 * Returns 0, or -1 on a bad id or rank.
 */
int oracle_lora_forward(int32_t T, int32_t d_in, int32_t d_out, int32_t is_bf16,
                        const void *x, int64_t ldx, const int32_t *ids, int32_t n_adapters,
                        const void *pool, const int64_t *a_off, const int64_t *b_off,
                        const int32_t *rank, const float *alpha,
                        const void *y_in, int64_t ldy, const void *W0,
                        int32_t w0_e4m3, double w0_scale, double *v_out, int64_t ldv, double *y_out, int32_t nthreads)
{
    int bad = 0;
    for (int32_t t = 0; t < T; ++t) {
        if (ids[t] >= n_adapters) bad = 1;
        else if (ids[t] >= 0 && rank[ids[t]] < 1) bad = 1;
    }
    if (bad) return -1;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int32_t t = 0; t < T; ++t) {
        double *yrow = y_out + (int64_t)t * d_out;

        /* base term: x W0 (fused) or the stored base output */
        for (int32_t n = 0; n < d_out; ++n) {
            double b = 0.0;
            if (W0 && w0_e4m3) {
                for (int32_t k = 0; k < d_in; ++k) {
#if ORACLE_MUTANT == 13
                    const double w = e4m3_value(((const uint8_t *)W0)[(int64_t)n * d_in + k]); /* planted: scale dropped */
#else
                    const double w = w0_scale * e4m3_value(((const uint8_t *)W0)[(int64_t)n * d_in + k]);
#endif
                    b += load_elem(x, is_bf16, (int64_t)t * ldx + k) * w;
                }
            } else if (W0) {
                for (int32_t k = 0; k < d_in; ++k)
                    b += load_elem(x, is_bf16, (int64_t)t * ldx + k) *
                         load_elem(W0, is_bf16, (int64_t)n * d_in + k);
            } else if (y_in) {
#if ORACLE_MUTANT != 4
                b = load_elem(y_in, is_bf16, (int64_t)t * ldy + n);
#endif /* planted (4): the base output is overwritten instead of accumulated into */
            }
            yrow[n] = b;
        }

#if ORACLE_MUTANT == 7
        int32_t a = ids[t > 0 ? t - 1 : 0]; /* planted: neighbour's adapter */
#else
        int32_t a = ids[t];
#endif
        if (a < 0) continue;
        const int32_t r = rank[a];
#if ORACLE_MUTANT == 2
        const double s = 1.0; /* planted: scale dropped */
#elif ORACLE_MUTANT == 3
        const double s = (double)r / (double)alpha[a]; /* planted: scale inverted */
#else
        const double s = (double)alpha[a] / (double)r;
#endif
        double *v = (double *)malloc(sizeof(double) * (size_t)r);

        /* shrink: v_j = sum_k x[t,k] A_a[j,k] */
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
#if ORACLE_MUTANT == 6
            for (int32_t k = 0; k < d_in - 1; ++k) /* planted: last term dropped */
#else
            for (int32_t k = 0; k < d_in; ++k)
#endif
            {
#if ORACLE_MUTANT == 1
                int64_t ai = a_off[a] + (int64_t)k * r + j; /* planted: A read transposed */
#else
                int64_t ai = a_off[a] + (int64_t)j * d_in + k;
#endif
                acc += load_elem(x, is_bf16, (int64_t)t * ldx + k) * load_elem(pool, is_bf16, ai);
            }
            v[j] = acc;
            if (v_out) v_out[(int64_t)t * ldv + j] = acc;
        }

        /* expand: y[t,n] += s * sum_j v_j B_a[n,j] */
        for (int32_t n = 0; n < d_out; ++n) {
            double acc = 0.0;
            for (int32_t j = 0; j < r; ++j) {
#if ORACLE_MUTANT == 5
                int64_t bi = b_off[a] + (int64_t)j * d_out + n; /* planted: B read transposed */
#else
                int64_t bi = b_off[a] + (int64_t)n * r + j;
#endif
                acc += v[j] * load_elem(pool, is_bf16, bi);
            }
#if ORACLE_MUTANT == 10
            yrow[n] -= s * acc; /* planted: sign flipped */
#else
            yrow[n] += s * acc;
#endif
        }
        free(v);
    }
    return 0;
}
