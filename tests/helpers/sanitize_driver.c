/*
 * sanitize_driver.c -- drives the C oracle (oracle/lamp_oracle.c,
 * oracle/lamp_mlp_oracle.c) and the C test helpers through every mode and
 * option on small inputs, ordinary and out-of-range values alike, so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (host code only)
 * sees every code path: out-of-bounds accesses, leaks, signed overflow,
 * invalid shifts.  Exit status 0 and no sanitizer report = clean.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by tests/test_sanitize.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_lamp_rows(const float *qh, const float *kh, const float *vh, int S, int D, int causal,
                  int mu, int ps_block, float tau, int mode, int block_k, uint64_t seed,
                  uint64_t head_lin, int row_begin, int row_end, int nthreads, float *ylo,
                  float *yref, double *crit, uint32_t *mask, float *probs, float *out, double *kl,
                  double *kl_lowp, int32_t *count);
int orc_ps_gemm(const float *x, const float *w, int M, int N, int K, int mu, int ps_block,
                int nthreads, float *ylo, float *yref);
int orc_gelu_lamp(const float *ylo, const float *yref, int M, int N, float tau, int nthreads,
                  double *crit, uint32_t *mask, float *ymix, float *out, int32_t *count,
                  double *err, double *err_lowp);
int orc_ln_lamp(const float *ylo, const float *yref, int M, int N, const float *gamma,
                const float *beta, float eps, float tau, int nthreads, uint32_t *mask,
                float *ymix, float *out, int32_t *count, double *err, double *err_lowp,
                double *margin);
double orc_rn_mu(double x, int mu);
typedef double (*rn_fn)(double, int);
int64_t rn_check_range(uint64_t start, uint64_t count, int mu, rn_fn rn, uint32_t *first);
int64_t check_products(uint64_t seed, int64_t n, int mu, int emin, int emax, rn_fn rn,
                       int64_t *traps);
int64_t check_sums_exhaustive(int mu, int emin, int emax, rn_fn rn);
int64_t check_sums_random(uint64_t seed, int64_t n, int mu, int emin, int emax, rn_fn rn);
double emu_exp64_short(double x, int deg);
double max_rel_error(int deg, uint64_t seed, int64_t n, double lo, double hi);

static uint64_t st = 0x9e3779b97f4a7c15ull;
static double unif(void)   /* xorshift64*, [0, 1) */
{
    st ^= st >> 12;
    st ^= st << 25;
    st ^= st >> 27;
    return (double)((st * 0x2545f4914f6cdd1dull) >> 11) * 0x1p-53;
}

/* kind 0: normal; 1: zeros, tiny and huge entries; 2: inf / nan entries */
static void fill(float *x, int n, int kind)
{
    for (int i = 0; i < n; ++i) {
        double u = unif(), g = sqrt(-2.0 * log(unif() + 1e-300)) * cos(6.283185307179586 * u);
        float v = (float)g;
        double c = unif();
        if (kind == 1) {
            if (c < 0.05) v = 0.0f;
            else if (c < 0.10) v *= 0x1p-70f;
            else if (c < 0.15) v *= 0x1p50f;
        } else if (kind == 2) {
            if (c < 0.02) v = INFINITY;
            else if (c < 0.04) v = -INFINITY;
            else if (c < 0.05) v = NAN;
        }
        x[i] = v;
    }
}

static int attention_cases(void)
{
    const int Ss[] = {1, 2, 37, 70};
    const int Ds[] = {4, 12};
    const float taus[] = {0.0f, 1e-2f, INFINITY};
    int bad = 0;
    for (int si = 0; si < 4; ++si)
        for (int di = 0; di < 2; ++di)
            for (int kind = 0; kind < 3; ++kind) {
                const int S = Ss[si], D = Ds[di], W = (S + 31) / 32;
                float *q = malloc(sizeof(float) * S * D), *k = malloc(sizeof(float) * S * D),
                      *v = malloc(sizeof(float) * S * D);
                fill(q, S * D, kind);
                fill(k, S * D, kind);
                fill(v, S * D, kind);
                float *ylo = malloc(sizeof(float) * S * S), *yref = malloc(sizeof(float) * S * S),
                      *probs = malloc(sizeof(float) * S * S), *out = malloc(sizeof(float) * S * D);
                double *crit = malloc(sizeof(double) * S * S), *kl = malloc(sizeof(double) * S),
                       *kll = malloc(sizeof(double) * S);
                uint32_t *mask = malloc(sizeof(uint32_t) * S * W);
                int32_t *count = malloc(sizeof(int32_t) * S);
                for (int causal = 0; causal < 2; ++causal)
                    for (int mode = 0; mode < 3; ++mode)
                        for (int ti = 0; ti < 3; ++ti)
                            for (int mu = 4; mu <= 23; mu += 19)
                                for (int pb = 0; pb <= 4; pb += 4) {
                                    int rc = orc_lamp_rows(q, k, v, S, D, causal, mu, pb, taus[ti],
                                                           mode, 64, 7u, 3u, 0, S, 1, ylo, yref,
                                                           crit, mask, probs, out, kl, kll, count);
                                    bad |= rc != 0;
                                    /* a row range and NULL outputs */
                                    rc = orc_lamp_rows(q, k, v, S, D, causal, mu, pb, taus[ti],
                                                       mode, 16, 7u, 3u, S / 2, S, 1, NULL, NULL,
                                                       NULL, mask, NULL, out, NULL, NULL, NULL);
                                    bad |= rc != 0;
                                }
                /* argument checks */
                bad |= orc_lamp_rows(q, k, v, S, D, 1, 0, 0, 0.1f, 0, 64, 0, 0, 0, S, 1, NULL,
                                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != -1;
                bad |= orc_lamp_rows(q, k, v, S, D, 1, 4, 0, NAN, 0, 64, 0, 0, 0, S, 1, NULL, NULL,
                                     NULL, NULL, NULL, NULL, NULL, NULL, NULL) != -1;
                free(q); free(k); free(v); free(ylo); free(yref); free(probs); free(out);
                free(crit); free(kl); free(kll); free(mask); free(count);
            }
    return bad;
}

static int mlp_cases(void)
{
    int bad = 0;
    for (int kind = 0; kind < 3; ++kind) {
        const int M = 5, N = 37, K = 12, W = (N + 31) / 32;
        float *x = malloc(sizeof(float) * M * K), *w = malloc(sizeof(float) * N * K);
        float *g = malloc(sizeof(float) * N), *b = malloc(sizeof(float) * N);
        fill(x, M * K, kind);
        fill(w, N * K, kind);
        fill(g, N, 0);
        fill(b, N, 0);
        float *ylo = malloc(sizeof(float) * M * N), *yref = malloc(sizeof(float) * M * N),
              *ymix = malloc(sizeof(float) * M * N), *out = malloc(sizeof(float) * M * N);
        double *crit = malloc(sizeof(double) * M * N), *err = malloc(sizeof(double) * M),
               *errl = malloc(sizeof(double) * M), *margin = malloc(sizeof(double) * M);
        uint32_t *mask = malloc(sizeof(uint32_t) * M * W);
        int32_t *count = malloc(sizeof(int32_t) * M);
        for (int mu = 4; mu <= 23; mu += 19)
            for (int pb = 0; pb <= 4; pb += 4) {
                bad |= orc_ps_gemm(x, w, M, N, K, mu, pb, 1, ylo, yref) != 0;
                const float taus[] = {0.0f, 1e-2f, INFINITY};
                for (int ti = 0; ti < 3; ++ti) {
                    bad |= orc_gelu_lamp(ylo, yref, M, N, taus[ti], 1, crit, mask, ymix, out, count,
                                         err, errl) != 0;
                    bad |= orc_gelu_lamp(ylo, yref, M, N, taus[ti], 1, NULL, NULL, NULL, out, NULL,
                                         NULL, NULL) != 0;
                    bad |= orc_ln_lamp(ylo, yref, M, N, g, b, 1e-5f, taus[ti], 1, mask, ymix, out,
                                       count, err, errl, margin) != 0;
                    bad |= orc_ln_lamp(ylo, yref, M, N, g, b, 0.0f, taus[ti], 1, NULL, NULL, out,
                                       NULL, NULL, NULL, NULL) != 0;
                }
            }
        free(x); free(w); free(g); free(b); free(ylo); free(yref); free(ymix); free(out);
        free(crit); free(err); free(errl); free(margin); free(mask); free(count);
    }
    return bad;
}

static int helper_cases(void)
{
    int bad = 0;
    uint32_t first = 0;
    int64_t traps = 0;
    for (int mu = 1; mu <= 23; mu += 11) {
        /* a stretch of bit patterns around the subnormal / normal boundary,
           the largest finite values and the specials */
        bad |= rn_check_range(0x007ff000u, 0x2000u, mu, orc_rn_mu, &first) != 0;
        bad |= rn_check_range(0x7f7ff000u, 0x1800u, mu, orc_rn_mu, &first) != 0;
    }
    (void)check_products(5u, 20000, 4, -30, 30, orc_rn_mu, &traps);
    (void)check_sums_exhaustive(4, -3, 3, orc_rn_mu);
    (void)check_sums_random(6u, 20000, 7, -20, 20, orc_rn_mu);
    /* the shortened exponentials over their range and at the special values
       (the table index and the scale of a clamped or NaN argument) */
    for (int deg = 3; deg <= 4; ++deg) {
        bad |= !(max_rel_error(deg, 11u, 20000, -745.0, 709.0) < 1e-10);
        const double sp[] = {0.0, -0.0, 1e-300, -1e-300, -745.5, 709.9, 1e300, -1e300,
                             INFINITY, -INFINITY, NAN};
        for (unsigned u = 0; u < sizeof sp / sizeof sp[0]; ++u)
            (void)emu_exp64_short(sp[u], deg);
    }
    return bad;
}

int main(void)
{
    int bad = attention_cases();
    bad |= mlp_cases() << 1;
    bad |= helper_cases() << 2;
    printf("sanitize driver: %s (%d)\n", bad ? "FAILED" : "clean", bad);
    return bad ? 1 : 0;
}
