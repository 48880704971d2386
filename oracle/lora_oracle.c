/*
 * lora_oracle.c -- plain, slow CPU oracle for the batched multi-adapter LoRA
 * update.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU
 * baseline leg of the benchmark call it; the product library never does.  It
 * shares no code, header or table with the HIP path.
 *
 * What it computes, per token t of one linear module (x: [T][d_in],
 * y: [T][d_out], both row-major; idx: int32[T]):
 *
 *   k = idx[t]
 *   if k < 0, k >= n_slots, or rank[k] <= 0     -> y[t,:] is left untouched
 *   else  s   = lora_alpha_k / r_k              (use_rslora = 0)
 *             = lora_alpha_k / sqrt(r_k)        (use_rslora = 1)
 *         h_j = sum_{i < d_in} x[t,i] * At_k[j,i]          j < r_k
 *         y[t,n] <- round( y[t,n] + s * sum_{j < r_k} h_j * B_k[j,n] )
 *
 * Sources on the pages:
 *  - the adapter fields r, lora_alpha, use_rslora and target_modules come from
 *    the example adapter_config.json in "vLLM LoRA Resolver plugins explained"
 *    (blog.gitcode.com), section 3.2 "directory structure requirements";
 *  - the slot limits max_loras / max_lora_rank come from the parameter table
 *    in "Multi-LoRA adapter cache in production" (oh-bug.com), section
 *    "GPU, CPU and disk form the adapter storage hierarchy";
 *  - the shapes A: d_in x r and B: r x d_out per injected linear follow from
 *    that page's size estimate sum (d_in + d_out) * rank * bytes_per_param,
 *    section "adapter capacity cannot be planned by count alone".
 * The pages never write the update itself; the standard LoRA update with the
 * scale above is the plain reading of those fields.  rank[k] <= 0 stands for
 * "slot empty" and for "module not in target_modules": both leave y alone.
 *
 * Precision: inputs are exact (fp32, or bf16 widened exactly); every product
 * and sum is done in double, in ascending index order, with no fused
 * multiply-add (build with -ffp-contract=off); the result is rounded once into
 * the output dtype, round-to-nearest-even.  h stays in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP32 = 1 };

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16 value, ties to even, in one step.
 * bf16 keeps 8 significant bits and binary32's exponent range, so normal
 * values are quantised to 2^(e-8) where v = m * 2^e, 0.5 <= |m| < 1, and
 * values below 2^-126 to the subnormal quantum 2^-133.  v / q and the product
 * back are exact power-of-two scalings; nearbyint() rounds half to even in the
 * default rounding mode.  A result of 2^128 or more is an overflow to inf.
 */
static uint16_t double_to_bf16_rne(double v)
{
    if (isnan(v))
        return (uint16_t)0x7FC0u;            /* quiet NaN */
    float f;
    if (isinf(v) || v == 0.0) {
        f = (float)v;                        /* keeps the sign of zero */
    } else {
        int e;
        frexp(v, &e);
        if (e < -125)
            e = -125;
        double q = ldexp(1.0, e - 8);
        double r = nearbyint(v / q) * q;
        if (fabs(r) >= 0x1p128)
            r = copysign(INFINITY, v);
        if (r == 0.0)
            r = copysign(0.0, v);
        f = (float)r;                        /* exact: r has <= 8 significant bits */
    }
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16)
        return bf16_to_double(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

static void store_elem(void *base, int dtype, int64_t i, double v)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t *)base)[i] = double_to_bf16_rne(v);
    else
        ((float *)base)[i] = (float)v;       /* C conversion: round to nearest even */
}

/* The adapter scale: lora_alpha / r, or lora_alpha / sqrt(r) with rsLoRA. */
double lora_oracle_scale(double lora_alpha, int32_t r, int32_t use_rslora)
{
    if (use_rslora)
        return lora_alpha / sqrt((double)r);
    return lora_alpha / (double)r;
}

/* Bytes of one adapter over the injected linears: sum (d_in + d_out) * r * b. */
int64_t lora_oracle_adapter_bytes(const int32_t *d_in, const int32_t *d_out,
                                  const int32_t *targeted, int32_t n_modules,
                                  int32_t r, int32_t bytes_per_param)
{
    int64_t total = 0;
    for (int32_t m = 0; m < n_modules; ++m)
        if (targeted[m])
            total += ((int64_t)d_in[m] + d_out[m]) * r * bytes_per_param;
    return total;
}

/* Exposed so the tests can pin the rounding against a library routine. */
uint16_t lora_oracle_round_bf16(double v) { return double_to_bf16_rne(v); }

/*
 * Apply one module's LoRA update in place on y.
 *   dtype      ORACLE_BF16 (x, y, At, B are uint16 bf16 bit patterns) or ORACLE_FP32
 *   x          [n_tokens][d_in]
 *   y          [n_tokens][d_out], updated in place
 *   idx        int32[n_tokens], slot per token
 *   rank       int32[n_slots]; <= 0 means nothing to apply for that slot
 *   lora_alpha double[n_slots]; use_rslora int32[n_slots]
 *   At         [n_slots] pointers to rank[k] x d_in row-major (A transposed)
 *   B          [n_slots] pointers to rank[k] x d_out row-major
 *   n_threads  OpenMP threads over tokens (<= 0: library default)
 * Returns the number of tokens that were updated.
 */
int64_t lora_oracle_apply(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                          const void *x, void *y, const int32_t *idx, int32_t n_slots,
                          const int32_t *rank, const double *lora_alpha,
                          const int32_t *use_rslora, const void *const *At,
                          const void *const *B, int32_t n_threads)
{
    int64_t applied = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : applied)
    for (int32_t t = 0; t < n_tokens; ++t) {
        int32_t k = idx[t];
        if (k < 0 || k >= n_slots || rank[k] <= 0)
            continue;
        int32_t r = rank[k];
        double s = lora_oracle_scale(lora_alpha[k], r, use_rslora[k]);
        double *h = (double *)malloc(sizeof(double) * (size_t)r);
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d_in; ++i)
                acc = acc + load_elem(x, dtype, (int64_t)t * d_in + i) *
                                load_elem(At[k], dtype, (int64_t)j * d_in + i);
            h[j] = acc;
        }
        for (int32_t n = 0; n < d_out; ++n) {
            double acc = 0.0;
            for (int32_t j = 0; j < r; ++j)
                acc = acc + h[j] * load_elem(B[k], dtype, (int64_t)j * d_out + n);
            int64_t o = (int64_t)t * d_out + n;
            double yv = load_elem(y, dtype, o);
            store_elem(y, dtype, o, yv + s * acc);
        }
        free(h);
        applied += 1;
    }
    return applied;
}

/*
 * The same update with the two per-adapter output terms an adapter_config can
 * switch on ("vLLM LoRA Resolver plugins explained", section 3.2: the fields
 * "bias" and "use_dora" of the example config, both off there):
 *
 *   y[t,n] <- round( g_k[n] * ( y[t,n] + s * sum_j h_j * B_k[j,n] ) + c_k[n] )
 *
 *   c_k  (bias[k], d_out values of the data dtype, NULL = 0): an output bias the
 *        adapter brings for the module, added as given (a bias trained with the
 *        adapter enters as its difference to the base bias; a bias of lora_B
 *        enters scaled by s);
 *   g_k  (dora[k], d_out doubles, NULL = 1): DoRA's per-output-feature factor
 *        m_n / ||W0 + s B^T A||_n of "DoRA: Weight-Decomposed Low-Rank
 *        Adaptation" (Liu et al., 2024), with y the base product x W0^T without
 *        the base bias; the caller forms it from W0, which the library never
 *        holds.
 * The pages name the two fields and nothing more; this is the plain reading of
 * them written in the order the definition applies (scale the low-rank sum,
 * add it to the base product, apply the magnitude factor, add the bias).
 * Same precision rules as lora_oracle_apply: double, ascending order, no FMA,
 * one rounding.
 */
int64_t lora_oracle_apply_ex(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                             const void *x, void *y, const int32_t *idx, int32_t n_slots,
                             const int32_t *rank, const double *lora_alpha,
                             const int32_t *use_rslora, const void *const *At,
                             const void *const *B, const void *const *bias,
                             const double *const *dora, int32_t n_threads)
{
    int64_t applied = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : applied)
    for (int32_t t = 0; t < n_tokens; ++t) {
        int32_t k = idx[t];
        if (k < 0 || k >= n_slots || rank[k] <= 0)
            continue;
        int32_t r = rank[k];
        double s = lora_oracle_scale(lora_alpha[k], r, use_rslora[k]);
        double *h = (double *)malloc(sizeof(double) * (size_t)r);
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d_in; ++i)
                acc = acc + load_elem(x, dtype, (int64_t)t * d_in + i) *
                                load_elem(At[k], dtype, (int64_t)j * d_in + i);
            h[j] = acc;
        }
        for (int32_t n = 0; n < d_out; ++n) {
            double acc = 0.0;
            for (int32_t j = 0; j < r; ++j)
                acc = acc + h[j] * load_elem(B[k], dtype, (int64_t)j * d_out + n);
            int64_t o = (int64_t)t * d_out + n;
            double v = load_elem(y, dtype, o) + s * acc;
            if (dora && dora[k])
                v = dora[k][n] * v;
            if (bias && bias[k])
                v = v + load_elem(bias[k], dtype, n);
            store_elem(y, dtype, o, v);
        }
        free(h);
        applied += 1;
    }
    return applied;
}

/*
 * Whole modules an adapter saves ("modules_to_save" of the example
 * adapter_config.json in "vLLM LoRA Resolver plugins explained", section 3.2;
 * null in that example).  Such a module is a complete trained copy of the
 * linear: for the adapter's tokens it takes the base module's place, so the
 * output row is the saved module's own product and the base output the caller
 * put in y is discarded:
 *
 *   y[t,n] <- round( sum_{i < d_in} x[t,i] * W_k[n,i]  +  c_k[n] )
 *
 *   W    [n_slots] pointers to d_out x d_in row-major weights (the layout of a
 *        linear layer's weight: row n holds output feature n), NULL when slot k
 *        saves no copy of this module
 *   bias [n_slots] pointers to d_out values, or NULL (no bias); NULL array = none
 * Tokens whose slot is out of range or saves no copy keep their row of y
 * untouched.  The pages name the field and nothing more; this is the plain
 * reading of it.  Same precision rules as lora_oracle_apply: double, ascending
 * index order, no fused multiply-add, one rounding.
 */
int64_t lora_oracle_apply_saved(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                                const void *x, void *y, const int32_t *idx, int32_t n_slots,
                                const void *const *W, const void *const *bias, int32_t n_threads)
{
    int64_t applied = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : applied)
    for (int32_t t = 0; t < n_tokens; ++t) {
        int32_t k = idx[t];
        if (k < 0 || k >= n_slots || W[k] == NULL)
            continue;
        for (int32_t n = 0; n < d_out; ++n) {
            double acc = 0.0;
            for (int32_t i = 0; i < d_in; ++i)
                acc = acc + load_elem(x, dtype, (int64_t)t * d_in + i) *
                                load_elem(W[k], dtype, (int64_t)n * d_in + i);
            if (bias && bias[k])
                acc = acc + load_elem(bias[k], dtype, n);
            store_elem(y, dtype, (int64_t)t * d_out + n, acc);
        }
        applied += 1;
    }
    return applied;
}

int32_t lora_oracle_max_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
