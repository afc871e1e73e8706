/*
 * lamp_oracle.c -- plain, slow CPU oracle for LAMP attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source with the HIP library.
 *
 * Everything is computed one attention row at a time, in double precision,
 * in the order the method states it.  Source of the method: the LAMP
 * technical summary (gist.science, paper 2601.21623; Korean and Dutch
 * versions), sections "Theoretical foundation" (item 3, softmax closed form)
 * "Implementation strategy" (steps 1-3) and "Experimental results" (PS(mu)
 * format, KL against a uniform FP32 reference, random-selection control,
 * relaxed relative-threshold variant).
 *
 * Readings of points the pages leave open are stated next to the code that
 * takes them (PS rounding semantics, scale, relaxed rule, random control,
 * KL form).  Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_STRICT 0
#define ORC_RELAXED 1
#define ORC_RANDOM 2

/* ------------------------------------------------------------------------ */
/* PS(mu) rounding.                                                          */
/*                                                                           */
/* The pages ("Experimental results") simulate a custom float PS(mu) with    */
/* mu mantissa bits.  Reading: mu stored fraction bits (precision mu+1),     */
/* FP32's exponent range, so the PS(mu) values are exactly the FP32 values   */
/* whose low 23-mu fraction bits are zero (subnormal quantum 2^(-126-mu)).   */
/* Rounding is to nearest, ties to even; a result at or beyond 2^128 after   */
/* rounding overflows to infinity; NaN, infinities and signed zeros pass.    */
/* ------------------------------------------------------------------------ */
double orc_rn_mu(double x, int mu)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    int e;
    frexp(x, &e);            /* |x| in [2^(e-1), 2^e) */
    int b = e - 1;           /* binade exponent of x */
    if (b < -126)
        b = -126;            /* FP32 subnormal range: fixed quantum */
    double ulp = ldexp(1.0, b - mu);
    double r = nearbyint(x / ulp) * ulp;   /* x/ulp is exact: power-of-two scaling */
    if (fabs(r) >= 0x1p128)
        return copysign(INFINITY, x);
    return r;
}

void orc_rn_mu_array(const double *x, double *y, int64_t n, int mu)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_rn_mu(x[i], mu);
}

/* FP32 softmax scale: the FP32 value nearest to 1/sqrt(D).  The pages'
 * y_j is the softmax input; the workloads scale scores by 1/sqrt(D). */
float orc_scale(int D)
{
    return (float)(1.0 / sqrt((double)D));
}

/* PS(mu) dot product, d ascending, accumulator starting at +0:
 *   acc <- RN_mu(acc + RN_mu(q_d * k_d)).
 * The product of two floats is exact in double, so RN_mu(t) is one rounding
 * of the exact product.  acc + RN_mu(t) is a double add followed by RN_mu:
 * both operands have at most 24 significant bits and 53 >= 2*24+2, so the
 * double rounding is innocuous (Figueroa, "When is double rounding
 * innocuous?", 1995); values below 2^-126 are multiples of 2^(-126-mu) and
 * add exactly. */
double orc_ps_dot(const float *q, const float *k, int D, int mu)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d) {
        double t = (double)q[d] * (double)k[d];
        acc = orc_rn_mu(acc + orc_rn_mu(t, mu), mu);
    }
    return acc;
}

/* Blocked ("packed") accumulation order, the order a native low-precision
 * dot-product unit would use (LAMP summary, "Significance": the method as a
 * blueprint for hardware with packed low-precision accumulation; the order
 * itself is a reading, the pages give none).  Every multiply and add is still
 * rounded to PS(mu); only the order changes: the products of each run of
 * `block` consecutive d (the last run may be shorter) are summed from +0 in d
 * order, and each run's sum is then added to the running accumulator, which
 * also starts at +0.  block <= 1 (one product per run) and block >= D (one
 * run) both give the sequential order. */
double orc_ps_dot_blocked(const float *q, const float *k, int D, int mu, int block)
{
    if (block <= 1 || block >= D)
        return orc_ps_dot(q, k, D, mu);
    double acc = 0.0;
    for (int d0 = 0; d0 < D; d0 += block) {
        const int d1 = d0 + block < D ? d0 + block : D;
        double part = 0.0;
        for (int d = d0; d < d1; ++d) {
            double t = (double)q[d] * (double)k[d];
            part = orc_rn_mu(part + orc_rn_mu(t, mu), mu);
        }
        acc = orc_rn_mu(acc + part, mu);
    }
    return acc;
}

/* Uniform FP32 reference: sequential float loop, multiply then add, no
 * fused multiply-add, d ascending (built with -ffp-contract=off). */
float orc_seq32_dot(const float *q, const float *k, int D)
{
    float acc = 0.0f;
    for (int d = 0; d < D; ++d) {
        float p = q[d] * k[d];
        acc = acc + p;
    }
    return acc;
}

/* Scaled scores: one FP32 multiply by the FP32 scale after accumulation. */
static float score_lo(const float *q, const float *k, int D, int mu, int ps_block, float s)
{
    /* exact: PS(mu) values are floats */
    float a = (float)orc_ps_dot_blocked(q, k, D, mu, ps_block);
    float y = a * s;
    return y;
}

static float score_ref(const float *q, const float *k, int D, float s)
{
    float a = orc_seq32_dot(q, k, D);
    float y = a * s;
    return y;
}

/* SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): the state is advanced by the
 * golden-gamma increment, then mixed by two xor-shift-multiply rounds. */
uint64_t orc_splitmix64(uint64_t state)
{
    uint64_t z = state + 0x9e3779b97f4a7c15ULL;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* ------------------------------------------------------------------------ */
/* Look-ahead selection criteria.                                            */
/* ------------------------------------------------------------------------ */

/* Strict rule ("Theoretical foundation", item 3, softmax): recompute y_j iff
 *   2 z_j (1 - z_j) |y_j| > tau,  z = softmax(y^lo) over the valid keys.
 * 1 - z_j is formed without cancellation: for keys at the row maximum it is
 * (sum of the other keys' exponentials) / L, otherwise (L - e_j) / L. */
static void strict_criterion(const float *ylo, int n, double *crit)
{
    float m = ylo[0];
    for (int j = 1; j < n; ++j)
        if (ylo[j] > m)
            m = ylo[j];
    int cnt = 0;
    double A = 0.0;            /* sum of exp(y - m) over keys below the max */
    for (int j = 0; j < n; ++j) {
        if (ylo[j] == m)
            cnt++;
        else
            A += exp((double)ylo[j] - (double)m);
    }
    double L = A + (double)cnt;
    for (int j = 0; j < n; ++j) {
        double e, omz;
        if (ylo[j] == m) {
            e = 1.0;
            omz = (A + (double)(cnt - 1)) / L;
        } else {
            e = exp((double)ylo[j] - (double)m);
            omz = (L - e) / L;
        }
        double z = e / L;
        crit[j] = 2.0 * z * omz * fabs((double)ylo[j]);
    }
}

/* Relaxed relative-threshold rule ("Experimental results", relaxed LAMP):
 * the normalisation constant is dropped.  Reading: z_j is replaced by
 * exp(y_j - m_t), where m_t is the running maximum of y^lo over the valid keys
 * of key blocks 0..floor(j/block_k) (block_k = 64 by default), and the
 * (1 - z_j) factor is bounded by 1:
 *   2 exp(y_j - m_t) |y_j| > tau.
 * Since z_j <= exp(y_j - m_t), every strictly selected key is also selected
 * here. */
static void relaxed_criterion(const float *ylo, int n, int block_k, double *crit)
{
    float mt = -INFINITY;
    for (int b0 = 0; b0 < n; b0 += block_k) {
        int b1 = b0 + block_k < n ? b0 + block_k : n;
        for (int j = b0; j < b1; ++j)
            if (ylo[j] > mt)
                mt = ylo[j];
        for (int j = b0; j < b1; ++j)
            crit[j] = 2.0 * exp((double)ylo[j] - (double)mt) * fabs((double)ylo[j]);
    }
}

typedef struct {
    uint64_t h;
    int j;
} hkey;

static int hkey_cmp(const void *a, const void *b)
{
    const hkey *x = (const hkey *)a, *y = (const hkey *)b;
    if (x->h < y->h) return -1;
    if (x->h > y->h) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

/* Log-sum-exp and its max in double, over n floats. */
static double row_lse(const float *y, int n, double *mout, double *eout)
{
    float m = y[0];
    for (int j = 1; j < n; ++j)
        if (y[j] > m)
            m = y[j];
    double E = 0.0;
    for (int j = 0; j < n; ++j)
        E += exp((double)y[j] - (double)m);
    if (mout) *mout = (double)m;
    if (eout) *eout = E;
    return (double)m + log(E);
}

/* KL(P_ref || P_x) for one row, in the log-sum-exp form:
 *   sum_j p_ref_j (y_ref_j - y_x_j) + lse(y_x) - lse(y_ref). */
static double row_kl(const float *yref, const float *yx, int n)
{
    double mref, Eref;
    double lse_ref = row_lse(yref, n, &mref, &Eref);
    double lse_x = row_lse(yx, n, NULL, NULL);
    double s = 0.0;
    for (int j = 0; j < n; ++j) {
        double p = exp((double)yref[j] - mref) / Eref;
        s += p * ((double)yref[j] - (double)yx[j]);
    }
    return s + lse_x - lse_ref;
}

/* ------------------------------------------------------------------------ */
/* One row of the LAMP attention forward.                                    */
/* Steps ("Implementation strategy"): baseline evaluation at low precision;  */
/* look-ahead selection from the baseline output; recompute of the selected  */
/* components at FP32; then the softmax and P.V ("then f").                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    float *ylo, *yref, *ymix;
    double *crit;
    hkey *keys;
} row_scratch;

static void lamp_row(const float *Qh, const float *Kh, const float *Vh,
                     int S, int D, int causal, int mu, int ps_block, float tau, int mode,
                     int block_k, uint64_t seed, uint64_t head_lin, int i, float s,
                     row_scratch *w,
                     float *o_ylo, float *o_yref, double *o_crit, uint32_t *o_mask,
                     float *o_probs, float *o_out, double *o_kl, double *o_kl_lowp,
                     int32_t *o_count)
{
    const int n = causal ? i + 1 : S;     /* valid keys: j <= i when causal */
    const float *q = Qh + (size_t)i * D;
    const double t = (double)tau;

    /* Step 1: baseline scores at PS(mu); the uniform FP32 reference beside. */
    for (int j = 0; j < n; ++j) {
        w->ylo[j] = score_lo(q, Kh + (size_t)j * D, D, mu, ps_block, s);
        w->yref[j] = score_ref(q, Kh + (size_t)j * D, D, s);
    }

    /* Step 2: look-ahead selection. */
    unsigned char *sel = (unsigned char *)calloc((size_t)n, 1);
    int count = 0;
    if (mode == ORC_RELAXED) {
        relaxed_criterion(w->ylo, n, block_k, w->crit);
        for (int j = 0; j < n; ++j)
            if (w->crit[j] > t) { sel[j] = 1; count++; }
    } else {
        strict_criterion(w->ylo, n, w->crit);
        int kstrict = 0;
        for (int j = 0; j < n; ++j)
            if (w->crit[j] > t) { sel[j] = 1; kstrict++; }
        count = kstrict;
        if (mode == ORC_RANDOM) {
            /* Random control ("Experimental results", selectivity): the same
             * number of components per row as the strict rule, chosen
             * uniformly without replacement as the keys with the smallest
             * SplitMix64 hash of (seed xor linear score index), ties broken
             * by the lower key index. */
            memset(sel, 0, (size_t)n);
            uint64_t rowbase = (head_lin * (uint64_t)S + (uint64_t)i) * (uint64_t)S;
            for (int j = 0; j < n; ++j) {
                w->keys[j].h = orc_splitmix64(seed ^ (rowbase + (uint64_t)j));
                w->keys[j].j = j;
            }
            qsort(w->keys, (size_t)n, sizeof(hkey), hkey_cmp);
            for (int r = 0; r < kstrict; ++r)
                sel[w->keys[r].j] = 1;
        }
    }

    /* Step 3: recompute the selected scores at FP32. */
    for (int j = 0; j < n; ++j)
        w->ymix[j] = sel[j] ? score_ref(q, Kh + (size_t)j * D, D, s) : w->ylo[j];

    /* f: softmax over the valid keys, then P.V, all in double. */
    double M, E;
    row_lse(w->ymix, n, &M, &E);
    if (o_out) {
        double *acc = (double *)calloc((size_t)D, sizeof(double));
        for (int j = 0; j < n; ++j) {
            double p = exp((double)w->ymix[j] - M) / E;
            const float *vj = Vh + (size_t)j * D;
            for (int d = 0; d < D; ++d)
                acc[d] += p * (double)vj[d];
        }
        for (int d = 0; d < D; ++d)
            o_out[d] = (float)acc[d];
        free(acc);
    }
    if (o_probs) {
        for (int j = 0; j < S; ++j)
            o_probs[j] = j < n ? (float)(exp((double)w->ymix[j] - M) / E) : 0.0f;
    }
    if (o_ylo)
        for (int j = 0; j < S; ++j) o_ylo[j] = j < n ? w->ylo[j] : 0.0f;
    if (o_yref)
        for (int j = 0; j < S; ++j) o_yref[j] = j < n ? w->yref[j] : 0.0f;
    if (o_crit)
        for (int j = 0; j < S; ++j) o_crit[j] = j < n ? w->crit[j] : 0.0;
    if (o_mask) {
        int words = (S + 31) / 32;
        for (int wd = 0; wd < words; ++wd) o_mask[wd] = 0u;
        for (int j = 0; j < n; ++j)
            if (sel[j]) o_mask[j >> 5] |= 1u << (j & 31);
    }
    /* Row-wise KL(P_FP32 || P_LAMP) and KL(P_FP32 || P_lowp). */
    if (o_kl) *o_kl = row_kl(w->yref, w->ymix, n);
    if (o_kl_lowp) *o_kl_lowp = row_kl(w->yref, w->ylo, n);
    if (o_count) *o_count = count;
    free(sel);
}

/*
 * Rows [row_begin, row_end) of one attention head.
 *   qh, kh, vh : that head's [S, D] float32 blocks.
 *   head_lin   : linear (b*H + h) index, used only by the random control.
 *   ps_block   : PS(mu) accumulation order: 0 or 1 sequential, else blocked
 *                with runs of ps_block products (orc_ps_dot_blocked).
 * Every output may be NULL; row r is written at offset (r - row_begin):
 *   ylo, yref, probs : [rows, S] float32 (invalid keys written as 0)
 *   crit             : [rows, S] double, the mode's criterion value
 *                      (strict criterion for the random mode)
 *   mask             : [rows, ceil(S/32)] uint32, bit j%32 of word j/32
 *   out              : [rows, D] float32
 *   kl, kl_lowp      : [rows] double
 *   count            : [rows] int32, selected keys per row
 * Returns 0, or -1 on bad arguments.
 */
int orc_lamp_rows(const float *qh, const float *kh, const float *vh,
                  int S, int D, int causal, int mu, int ps_block, float tau, int mode,
                  int block_k, uint64_t seed, uint64_t head_lin, int row_begin, int row_end,
                  int nthreads,
                  float *ylo, float *yref, double *crit, uint32_t *mask,
                  float *probs, float *out, double *kl, double *kl_lowp,
                  int32_t *count)
{
    if (!qh || !kh || !vh || S < 1 || D < 1 || mu < 1 || mu > 23 ||
        row_begin < 0 || row_end > S || row_begin > row_end || block_k < 1 || ps_block < 0 ||
        mode < 0 || mode > 2 || !(tau >= 0.0f))
        return -1;
    const float s = orc_scale(D);
    const int words = (S + 31) / 32;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        row_scratch w;
        w.ylo = (float *)malloc(sizeof(float) * (size_t)S);
        w.yref = (float *)malloc(sizeof(float) * (size_t)S);
        w.ymix = (float *)malloc(sizeof(float) * (size_t)S);
        w.crit = (double *)malloc(sizeof(double) * (size_t)S);
        w.keys = (hkey *)malloc(sizeof(hkey) * (size_t)S);
#pragma omp for schedule(dynamic, 4)
        for (int i = row_begin; i < row_end; ++i) {
            size_t r = (size_t)(i - row_begin);
            lamp_row(qh, kh, vh, S, D, causal, mu, ps_block, tau, mode, block_k, seed, head_lin, i,
                     s, &w,
                     ylo ? ylo + r * S : NULL, yref ? yref + r * S : NULL,
                     crit ? crit + r * S : NULL, mask ? mask + r * words : NULL,
                     probs ? probs + r * S : NULL, out ? out + r * D : NULL,
                     kl ? kl + r : NULL, kl_lowp ? kl_lowp + r : NULL,
                     count ? count + r : NULL);
        }
        free(w.ylo); free(w.yref); free(w.ymix); free(w.crit); free(w.keys);
    }
    return 0;
}

/* Number of threads an OpenMP parallel region uses. */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
