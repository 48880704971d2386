/*
 * oracle_check.c -- drives the CPU oracle (oracle/lora_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Built and run by
 * tests/test_sanitizers.py; not part of the library.
 *
 * Every case is checked against a dense merge written here: the update of a
 * token is x . W with W = s * A . B formed first (A = At transposed), in
 * double, the plain LoRA update the adapter fields r, lora_alpha and
 * use_rslora of the example adapter_config.json ("vLLM LoRA Resolver plugins
 * explained", section 3.2) describe.  The cases cover the edges: no tokens,
 * rank 1, empty slots, negative and too-large slot indices, ragged sizes, fp32
 * and bf16, output bias and DoRA factors; and the saved-module product
 * ("modules_to_save" of the same example config), checked against a plain
 * x . W^T + bias written here.  The exit status is the number of
 * failed checks; the sanitizers abort on the first memory or UB error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { BF16 = 0, FP32 = 1 };

int64_t lora_oracle_apply(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                          const void *x, void *y, const int32_t *idx, int32_t n_slots,
                          const int32_t *rank, const double *lora_alpha,
                          const int32_t *use_rslora, const void *const *At,
                          const void *const *B, int32_t n_threads);
int64_t lora_oracle_apply_ex(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                             const void *x, void *y, const int32_t *idx, int32_t n_slots,
                             const int32_t *rank, const double *lora_alpha,
                             const int32_t *use_rslora, const void *const *At,
                             const void *const *B, const void *const *bias,
                             const double *const *dora, int32_t n_threads);
int64_t lora_oracle_apply_saved(int32_t dtype, int32_t n_tokens, int32_t d_in, int32_t d_out,
                                const void *x, void *y, const int32_t *idx, int32_t n_slots,
                                const void *const *W, const void *const *bias, int32_t n_threads);
double lora_oracle_scale(double lora_alpha, int32_t r, int32_t use_rslora);
int64_t lora_oracle_adapter_bytes(const int32_t *d_in, const int32_t *d_out,
                                  const int32_t *targeted, int32_t n_modules, int32_t r,
                                  int32_t bytes_per_param);
uint16_t lora_oracle_round_bf16(double v);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void)     /* splitmix64, uniform in [-1, 1) */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int failures = 0;

/* One case: n_slots adapters of the given ranks (0 = empty slot), T tokens. */
static void run_case(int dtype, int T, int d_in, int d_out, int n_slots, const int *ranks,
                     const int *idx, int with_terms)
{
    const size_t es = dtype == BF16 ? 2 : 4;
    void *x = malloc((size_t)T * d_in * es + 1), *y = malloc((size_t)T * d_out * es + 1);
    void *y0 = malloc((size_t)T * d_out * es + 1);
    double *xv = malloc(sizeof(double) * ((size_t)T * d_in + 1));
    double *yv = malloc(sizeof(double) * ((size_t)T * d_out + 1));
    const void **At = calloc((size_t)n_slots, sizeof(void *)), **Bp = calloc((size_t)n_slots, sizeof(void *));
    const void **bias = calloc((size_t)n_slots, sizeof(void *));
    const double **dora = calloc((size_t)n_slots, sizeof(double *));
    double **Av = calloc((size_t)n_slots, sizeof(double *)), **Bv = calloc((size_t)n_slots, sizeof(double *));
    double **cv = calloc((size_t)n_slots, sizeof(double *));
    int32_t *rk = calloc((size_t)n_slots, sizeof(int32_t)), *rs = calloc((size_t)n_slots, sizeof(int32_t));
    double *alpha = calloc((size_t)n_slots, sizeof(double));
    /* values on a coarse grid, exact in bf16 and fp32 */
#define PUT(buf, i, v, store)                                                  \
    do {                                                                       \
        double q_ = round((v) * 8.0) / 8.0;                                    \
        if (dtype == BF16)                                                     \
            ((uint16_t *)(buf))[i] = lora_oracle_round_bf16(q_);               \
        else                                                                   \
            ((float *)(buf))[i] = (float)q_;                                   \
        (store) = q_;                                                          \
    } while (0)
    for (int64_t i = 0; i < (int64_t)T * d_in; ++i)
        PUT(x, i, urand(), xv[i]);
    for (int64_t i = 0; i < (int64_t)T * d_out; ++i)
        PUT(y, i, urand(), yv[i]);
    memcpy(y0, y, (size_t)T * d_out * es);
    for (int k = 0; k < n_slots; ++k) {
        rk[k] = ranks[k];
        alpha[k] = 2.0 * ranks[k];
        rs[k] = k & 1;
        if (ranks[k] <= 0)
            continue;
        const int r = ranks[k];
        void *a = malloc((size_t)r * d_in * es), *b = malloc((size_t)r * d_out * es);
        Av[k] = malloc(sizeof(double) * (size_t)r * d_in);
        Bv[k] = malloc(sizeof(double) * (size_t)r * d_out);
        for (int64_t i = 0; i < (int64_t)r * d_in; ++i)
            PUT(a, i, urand(), Av[k][i]);
        for (int64_t i = 0; i < (int64_t)r * d_out; ++i)
            PUT(b, i, urand(), Bv[k][i]);
        At[k] = a;
        Bp[k] = b;
        if (with_terms) {
            void *c = malloc((size_t)d_out * es);
            double *g = malloc(sizeof(double) * (size_t)d_out);
            cv[k] = malloc(sizeof(double) * (size_t)d_out);
            for (int n = 0; n < d_out; ++n) {
                PUT(c, n, urand(), cv[k][n]);
                g[n] = 1.0 + 0.5 * urand();
            }
            bias[k] = c;
            dora[k] = g;
        }
    }
    int64_t applied = with_terms
        ? lora_oracle_apply_ex(dtype, T, d_in, d_out, x, y, idx, n_slots, rk, alpha, rs, At, Bp,
                               bias, dora, 2)
        : lora_oracle_apply(dtype, T, d_in, d_out, x, y, idx, n_slots, rk, alpha, rs, At, Bp, 2);
    int64_t want = 0;
    double worst = 0.0;
    for (int t = 0; t < T; ++t) {
        const int k = idx[t];
        const int on = k >= 0 && k < n_slots && ranks[k] > 0;
        want += on;
        for (int n = 0; n < d_out; ++n) {
            const int64_t o = (int64_t)t * d_out + n;
            double got = dtype == BF16 ? bf16_value(((uint16_t *)y)[o]) : ((float *)y)[o];
            if (!on) {
                if (memcmp((char *)y + o * es, (char *)y0 + o * es, es) != 0)
                    ++failures;
                continue;
            }
            /* dense merge: W[:, n] = s * sum_j A[:, j] B[j, n], then x . W */
            const double s = lora_oracle_scale(alpha[k], ranks[k], rs[k]);
            double acc = 0.0, mag = fabs(yv[o]);
            for (int i = 0; i < d_in; ++i) {
                double w = 0.0;
                for (int j = 0; j < ranks[k]; ++j)
                    w += Av[k][(int64_t)j * d_in + i] * Bv[k][(int64_t)j * d_out + n];
                acc += xv[(int64_t)t * d_in + i] * (s * w);
                mag += fabs(xv[(int64_t)t * d_in + i] * (s * w));
            }
            double ref = yv[o] + acc;
            if (with_terms) {
                ref = dora[k][n] * ref + cv[k][n];
                mag = dora[k][n] * mag + fabs(cv[k][n]);
            }
            /* one rounding into the output type (one unit in the last place
             * allowed, as the merge rounds its double sums in another order),
             * plus double rounding of the sums */
            const double bound = (dtype == BF16 ? ldexp(fabs(ref), -7) : ldexp(fabs(ref), -22)) +
                                 1e-12 * mag + 1e-300;
            const double err = fabs(got - ref) / bound;
            if (err > worst)
                worst = err;
        }
    }
    if (applied != want || worst > 1.0)
        ++failures;
    printf("case dtype=%s T=%d d_in=%d d_out=%d slots=%d terms=%d: applied %lld of %lld, "
           "worst err/bound %.3f\n", dtype == BF16 ? "bf16" : "fp32", T, d_in, d_out, n_slots,
           with_terms, (long long)applied, (long long)want, worst);
    for (int k = 0; k < n_slots; ++k) {
        free((void *)At[k]);
        free((void *)Bp[k]);
        free((void *)bias[k]);
        free((void *)dora[k]);
        free(Av[k]);
        free(Bv[k]);
        free(cv[k]);
    }
    free(At); free(Bp); free(bias); free(dora); free(Av); free(Bv); free(cv);
    free(rk); free(rs); free(alpha); free(x); free(y); free(y0); free(xv); free(yv);
}

/* Saved modules: slots with has_W[k] save a d_out x d_in W (and, for odd k, a
 * bias); the other tokens keep y bit for bit. */
static void run_saved_case(int dtype, int T, int d_in, int d_out, int n_slots, const int *has_W,
                           const int *idx)
{
    const size_t es = dtype == BF16 ? 2 : 4;
    void *x = malloc((size_t)T * d_in * es + 1), *y = malloc((size_t)T * d_out * es + 1);
    void *y0 = malloc((size_t)T * d_out * es + 1);
    double *xv = malloc(sizeof(double) * ((size_t)T * d_in + 1));
    const void **W = calloc((size_t)n_slots, sizeof(void *));
    const void **bias = calloc((size_t)n_slots, sizeof(void *));
    double **Wv = calloc((size_t)n_slots, sizeof(double *)), **cv = calloc((size_t)n_slots, sizeof(double *));
#define PUTS(buf, i, v, dst) do { double v_ = (v); \
        if (dtype == BF16) { float f_ = (float)v_; uint32_t u_; memcpy(&u_, &f_, 4); \
            ((uint16_t *)(buf))[i] = (uint16_t)(u_ >> 16); (dst) = bf16_value(((uint16_t *)(buf))[i]); } \
        else { ((float *)(buf))[i] = (float)v_; (dst) = ((float *)(buf))[i]; } } while (0)
    double scratch;
    for (int64_t i = 0; i < (int64_t)T * d_in; ++i)
        PUTS(x, i, urand(), xv[i]);
    for (int64_t i = 0; i < (int64_t)T * d_out; ++i)
        PUTS(y, i, urand(), scratch);
    memcpy(y0, y, (size_t)T * d_out * es);
    for (int k = 0; k < n_slots; ++k) {
        if (!has_W[k])
            continue;
        void *w = malloc((size_t)d_out * d_in * es);
        Wv[k] = malloc(sizeof(double) * (size_t)d_out * d_in);
        for (int64_t i = 0; i < (int64_t)d_out * d_in; ++i)
            PUTS(w, i, urand(), Wv[k][i]);
        W[k] = w;
        if (k & 1) {
            void *c = malloc((size_t)d_out * es);
            cv[k] = malloc(sizeof(double) * (size_t)d_out);
            for (int n = 0; n < d_out; ++n)
                PUTS(c, n, urand(), cv[k][n]);
            bias[k] = c;
        }
    }
#undef PUTS
    int64_t applied = lora_oracle_apply_saved(dtype, T, d_in, d_out, x, y, idx, n_slots, W, bias, 2);
    int64_t want = 0;
    double worst = 0.0;
    for (int t = 0; t < T; ++t) {
        const int k = idx[t];
        const int on = k >= 0 && k < n_slots && has_W[k];
        want += on;
        for (int n = 0; n < d_out; ++n) {
            const int64_t o = (int64_t)t * d_out + n;
            if (!on) {
                if (memcmp((char *)y + o * es, (char *)y0 + o * es, es) != 0)
                    ++failures;
                continue;
            }
            double ref = cv[k] ? cv[k][n] : 0.0, mag = fabs(ref);
            for (int i = 0; i < d_in; ++i) {
                ref += xv[(int64_t)t * d_in + i] * Wv[k][(int64_t)n * d_in + i];
                mag += fabs(xv[(int64_t)t * d_in + i] * Wv[k][(int64_t)n * d_in + i]);
            }
            double got = dtype == BF16 ? bf16_value(((uint16_t *)y)[o]) : ((float *)y)[o];
            const double bound = (dtype == BF16 ? ldexp(fabs(ref), -8) : ldexp(fabs(ref), -23)) +
                                 1e-12 * mag + 1e-300;
            const double err = fabs(got - ref) / bound;
            if (err > worst)
                worst = err;
        }
    }
    if (applied != want || worst > 1.0)
        ++failures;
    printf("saved case dtype=%s T=%d d_in=%d d_out=%d slots=%d: applied %lld of %lld, "
           "worst err/bound %.3f\n", dtype == BF16 ? "bf16" : "fp32", T, d_in, d_out, n_slots,
           (long long)applied, (long long)want, worst);
    for (int k = 0; k < n_slots; ++k) {
        free((void *)W[k]);
        free((void *)bias[k]);
        free(Wv[k]);
        free(cv[k]);
    }
    free(W); free(bias); free(Wv); free(cv); free(x); free(y); free(y0); free(xv);
}

int main(void)
{
    const int ranks4[4] = {4, 1, 0, 8};
    int idx[37];
    for (int t = 0; t < 37; ++t)
        idx[t] = (t % 7) - 2;            /* -2 .. 4: negatives, empty slot 2, too large 4 */
    for (int dtype = 0; dtype < 2; ++dtype) {
        run_case(dtype, 0, 16, 8, 4, ranks4, idx, 0);         /* no tokens */
        run_case(dtype, 37, 24, 40, 4, ranks4, idx, 0);
        run_case(dtype, 37, 8, 16, 4, ranks4, idx, 1);
        const int r1[1] = {1};
        const int one[3] = {0, 0, -1};
        run_case(dtype, 3, 16, 8, 1, r1, one, 0);             /* rank 1, one slot */
    }
    const int saved4[4] = {1, 1, 0, 1};
    for (int dtype = 0; dtype < 2; ++dtype) {
        run_saved_case(dtype, 0, 16, 8, 4, saved4, idx);      /* no tokens */
        run_saved_case(dtype, 37, 24, 40, 4, saved4, idx);    /* bias on slots 1 and 3 */
    }
    const int32_t din[3] = {5120, 5120, 8192}, dout[3] = {8192, 1024, 5120}, tg[3] = {1, 0, 1};
    if (lora_oracle_adapter_bytes(din, dout, tg, 3, 32, 2) != (int64_t)(13312 + 13312) * 32 * 2)
        ++failures;
    if (lora_oracle_round_bf16(1.0 + ldexp(1.0, -8)) != 0x3f80)   /* a tie rounds to even */
        ++failures;
    printf("failures: %d\n", failures);
    return failures;
}
