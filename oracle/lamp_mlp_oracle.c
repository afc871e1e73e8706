/*
 * lamp_mlp_oracle.c -- plain, slow CPU oracle for LAMP at the two other
 * closed forms the pages name: an activation function after a matrix
 * product, and layer normalisation after a matrix product.
 *
 * TEST INFRASTRUCTURE ONLY, like lamp_oracle.c (it is compiled into the
 * same oracle library and uses its PS(mu) dot and sequential FP32 dot).
 * Nothing in the product path links, loads or calls it.
 *
 * Source: the LAMP technical summary (gist.science, paper 2601.21623;
 * Korean and Dutch versions), "Theoretical foundation" item 3 (closed forms:
 * an activation function has a diagonal Jacobian, so its sensitive
 * components are read off one by one; for layer normalisation a nearly
 * sparsest selection is found greedily by sorting the input magnitudes) and
 * "Implementation strategy" steps 1-3 (low-precision baseline, look-ahead
 * selection from it, FP32 recompute of the selected components, then f).
 *
 * Readings (the pages state neither rule's formula):
 *  * g is a matrix product y = x W^T (W in the [out, in] layout of a linear
 *    layer) accumulated in PS(mu) along the input dimension, d ascending,
 *    no scale; the uniform FP32 reference is the sequential FP32 dot.
 *  * Activation: GPT-2's GELU, tanh form
 *        GELU(y) = y/2 (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).
 *    A relative error delta in y_j moves the output by GELU'(y_j) y_j delta
 *    and nothing else (diagonal Jacobian), so, in the l1 normwise form the
 *    softmax rule uses, component j is recomputed iff
 *        c_j = |GELU'(y_j) y_j| > tau,
 *    evaluated in double at the low-precision y_j.  The output is
 *    GELU(y^mix) in double, rounded to FP32.
 *  * Layer normalisation: LN(y)_j = gamma_j (y_j - m) / sqrt(v + eps) +
 *    beta_j with the row mean m and population variance v, in double.  Its
 *    Jacobian is diag(gamma) P / sigma with P an orthogonal projection, so
 *    relative input errors delta_j on the components left at low precision
 *    move the normalised output by at most ||y_U||_2 u / sigma; normwise
 *    relative to ||LN|| ~ sqrt(n) the condition is
 *        ||y_U||_2 / (sigma sqrt(n)) <= tau.
 *    The fewest recomputed components that meet it are the largest |y_j|
 *    (magnitudes sorted descending, ties to the lower index): k* = the
 *    smallest k with sum_{i > k} s_i^2 <= tau^2 sigma^2 n, where sigma^2 =
 *    v + eps of the low-precision row (the look-ahead estimate).  The output
 *    is LN of y^mix with its own statistics.
 *  * Accuracy measures (the analogue of the attention KL): per row, the l1
 *    distance to the all-FP32 output for GELU, the l2 distance for LN, for
 *    LAMP and for the all-low-precision baseline.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double orc_ps_dot_blocked(const float *q, const float *k, int D, int mu, int block);
float orc_seq32_dot(const float *q, const float *k, int D);

/* ------------------------------------------------------------------------ */
/* y = x W^T, PS(mu) and FP32 (step 1 and the uniform reference).           */
/* ------------------------------------------------------------------------ */
int orc_ps_gemm(const float *x, const float *w, int M, int N, int K, int mu, int ps_block,
                int nthreads, float *ylo, float *yref)
{
    if (!x || !w || M < 1 || N < 1 || K < 1 || mu < 1 || mu > 23 || ps_block < 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 4)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            const float *xi = x + (size_t)i * K, *wj = w + (size_t)j * K;
            if (ylo)
                ylo[(size_t)i * N + j] = (float)orc_ps_dot_blocked(xi, wj, K, mu, ps_block);
            if (yref)
                yref[(size_t)i * N + j] = orc_seq32_dot(xi, wj, K);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GELU (tanh form) and its derivative, in double.                          */
/* ------------------------------------------------------------------------ */
static const double kGeluA = 0.7978845608028654;   /* sqrt(2/pi) */
static const double kGeluB = 0.044715;

double orc_gelu(double y)
{
    const double u = kGeluA * (y + kGeluB * y * y * y);
    return 0.5 * y * (1.0 + tanh(u));
}

/* d/dy of the above: with t = tanh(u), u' = a (1 + 3 b y^2),
 * GELU' = (1 + t)/2 + y (1 - t^2) u' / 2. */
double orc_gelu_grad(double y)
{
    const double u = kGeluA * (y + kGeluB * y * y * y);
    const double t = tanh(u);
    const double du = kGeluA * (1.0 + 3.0 * kGeluB * y * y);
    return 0.5 * (1.0 + t) + 0.5 * y * (1.0 - t * t) * du;
}

double orc_gelu_criterion(float y)
{
    return fabs(orc_gelu_grad((double)y) * (double)y);
}

/*
 * GELU LAMP over rows of y (M x N): crit, mask bits (bit j%32 of word j/32),
 * y^mix, out = GELU(y^mix) in FP32, count per row, and the l1 distances of
 * the outputs to GELU(y^ref): err (LAMP) and err_lowp (all low precision).
 * Any output may be NULL.
 */
int orc_gelu_lamp(const float *ylo, const float *yref, int M, int N, float tau, int nthreads,
                  double *crit, uint32_t *mask, float *ymix, float *out, int32_t *count,
                  double *err, double *err_lowp)
{
    if (!ylo || !yref || M < 1 || N < 1 || !(tau >= 0.0f))
        return -1;
    const double t = (double)tau;
    const int words = (N + 31) / 32;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        const float *lo = ylo + (size_t)i * N, *rf = yref + (size_t)i * N;
        int32_t cnt = 0;
        double e = 0.0, el = 0.0;
        if (mask)
            memset(mask + (size_t)i * words, 0, sizeof(uint32_t) * (size_t)words);
        for (int j = 0; j < N; ++j) {
            const double c = orc_gelu_criterion(lo[j]);
            const int sel = c > t;
            const float mix = sel ? rf[j] : lo[j];
            const double g_mix = orc_gelu((double)mix);
            const double g_ref = orc_gelu((double)rf[j]);
            const double g_lo = orc_gelu((double)lo[j]);
            if (crit)
                crit[(size_t)i * N + j] = c;
            if (sel) {
                cnt++;
                if (mask)
                    mask[(size_t)i * words + j / 32] |= 1u << (j % 32);
            }
            if (ymix)
                ymix[(size_t)i * N + j] = mix;
            if (out)
                out[(size_t)i * N + j] = (float)g_mix;
            e += fabs(g_mix - g_ref);
            el += fabs(g_lo - g_ref);
        }
        if (count)
            count[i] = cnt;
        if (err)
            err[i] = e;
        if (err_lowp)
            err_lowp[i] = el;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Layer normalisation LAMP.                                                 */
/* ------------------------------------------------------------------------ */
typedef struct {
    float mag;
    int j;
} magkey;

static int magkey_cmp(const void *a, const void *b)
{
    const magkey *x = (const magkey *)a, *y = (const magkey *)b;
    if (x->mag > y->mag) return -1;   /* descending magnitude */
    if (x->mag < y->mag) return 1;
    return (x->j > y->j) - (x->j < y->j);   /* ties: lower index first */
}

/* LN of one row in double (mean, population variance over the n values). */
static void layer_norm(const float *y, int n, const float *gamma, const float *beta, double eps,
                       double *o)
{
    double m = 0.0;
    for (int j = 0; j < n; ++j)
        m += (double)y[j];
    m /= n;
    double v = 0.0;
    for (int j = 0; j < n; ++j)
        v += ((double)y[j] - m) * ((double)y[j] - m);
    v /= n;
    const double r = 1.0 / sqrt(v + eps);
    for (int j = 0; j < n; ++j)
        o[j] = (double)gamma[j] * (((double)y[j] - m) * r) + (double)beta[j];
}

/*
 * LayerNorm LAMP over rows of y (M x N): the greedy selection, mask bits,
 * y^mix, out = LN(y^mix) in FP32, count, the l2 distances of the outputs to
 * LN(y^ref) (err: LAMP, err_lowp: all low precision), and margin = the
 * relative distance |R - T^2| / T^2 of the two comparisons that fix k*
 * (R_{k*} <= T^2 < R_{k*-1}), the smaller of the two (for tie reporting).
 */
int orc_ln_lamp(const float *ylo, const float *yref, int M, int N, const float *gamma,
                const float *beta, float eps, float tau, int nthreads, uint32_t *mask,
                float *ymix, float *out, int32_t *count, double *err, double *err_lowp,
                double *margin)
{
    if (!ylo || !yref || !gamma || !beta || M < 1 || N < 1 || !(tau >= 0.0f) || !(eps >= 0.0f))
        return -1;
    const int words = (N + 31) / 32;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        magkey *keys = (magkey *)malloc(sizeof(magkey) * (size_t)N);
        unsigned char *sel = (unsigned char *)malloc((size_t)N);
        float *mix = (float *)malloc(sizeof(float) * (size_t)N);
        double *o_mix = (double *)malloc(sizeof(double) * (size_t)N);
        double *o_ref = (double *)malloc(sizeof(double) * (size_t)N);
        double *o_lo = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < M; ++i) {
            const float *lo = ylo + (size_t)i * N, *rf = yref + (size_t)i * N;
            /* the look-ahead estimate sigma^2 = v + eps of the low-precision row */
            double m = 0.0;
            for (int j = 0; j < N; ++j)
                m += (double)lo[j];
            m /= N;
            double v = 0.0;
            for (int j = 0; j < N; ++j)
                v += ((double)lo[j] - m) * ((double)lo[j] - m);
            v /= N;
            double T2 = (double)tau * (double)tau * (v + (double)eps) * (double)N;
            if (isnan(T2))   /* tau = +inf with sigma = 0 (or a NaN row): recompute nothing */
                T2 = INFINITY;
            /* magnitudes sorted descending, ties to the lower index */
            for (int j = 0; j < N; ++j) {
                keys[j].mag = fabsf(lo[j]);
                keys[j].j = j;
            }
            qsort(keys, (size_t)N, sizeof(magkey), magkey_cmp);
            /* R_k = sum_{i >= k} s_i^2 (0-based: the components after the top k) */
            int k = N;
            double R = 0.0, R_prev = 0.0;
            for (int kk = N; kk >= 0; --kk) {
                /* R = R_kk */
                if (R <= T2) {
                    k = kk;
                    R_prev = R;
                } else {
                    break;
                }
                if (kk > 0)
                    R += (double)keys[kk - 1].mag * (double)keys[kk - 1].mag;
            }
            /* here R_prev = R_{k} <= T2 and (k > 0) R = R_{k-1} > T2 */
            double mg = INFINITY;
            if (T2 > 0.0 && isfinite(T2)) {
                mg = fabs(R_prev - T2) / T2;
                if (k > 0) {
                    const double m2 = fabs(R - T2) / T2;
                    mg = m2 < mg ? m2 : mg;
                }
            }
            memset(sel, 0, (size_t)N);
            for (int q = 0; q < k; ++q)
                sel[keys[q].j] = 1;
            int32_t cnt = 0;
            if (mask)
                memset(mask + (size_t)i * words, 0, sizeof(uint32_t) * (size_t)words);
            for (int j = 0; j < N; ++j) {
                mix[j] = sel[j] ? rf[j] : lo[j];
                if (sel[j]) {
                    cnt++;
                    if (mask)
                        mask[(size_t)i * words + j / 32] |= 1u << (j % 32);
                }
            }
            layer_norm(mix, N, gamma, beta, (double)eps, o_mix);
            layer_norm(rf, N, gamma, beta, (double)eps, o_ref);
            layer_norm(lo, N, gamma, beta, (double)eps, o_lo);
            double e = 0.0, el = 0.0;
            for (int j = 0; j < N; ++j) {
                e += (o_mix[j] - o_ref[j]) * (o_mix[j] - o_ref[j]);
                el += (o_lo[j] - o_ref[j]) * (o_lo[j] - o_ref[j]);
                if (ymix)
                    ymix[(size_t)i * N + j] = mix[j];
                if (out)
                    out[(size_t)i * N + j] = (float)o_mix[j];
            }
            if (count)
                count[i] = cnt;
            if (err)
                err[i] = sqrt(e);
            if (err_lowp)
                err_lowp[i] = sqrt(el);
            if (margin)
                margin[i] = mg;
        }
        free(keys); free(sel); free(mix); free(o_mix); free(o_ref); free(o_lo);
    }
    return 0;
}
