// select.hip -- look-ahead selection (strict rule, random control) with
// stream compaction of the selected keys, and the gather FP32 recompute.
//
// Strict rule: LAMP summary, "Theoretical foundation" item 3 (softmax):
// recompute y_j iff 2 z_j (1 - z_j) |y_j| > tau, z = softmax of the baseline
// scores over the valid keys; "Implementation strategy" step 2 (selection
// from the baseline output) and step 3 (FP32 recompute of the selected
// components only).  Random control: "Experimental results" (the same number
// of components chosen at random).
//
// The criterion is evaluated in double: z_j = e_j / L with e_j = exp(y_j - m)
// and L summed in double; 1 - z_j is (sum of the other keys) / L for keys at
// the row maximum and (L - e_j) / L otherwise, so it never cancels.
#include "lamp_device.h"

namespace lamp {

struct SelectArgs {
    const float *y, *yref;
    int S, causal, W;
    uint64_t n_rows;
    double tau;
    uint32_t *mask, *list, *row_count;
    RowStats *rs;
    double *row_kl, *row_kl_lowp;
    int count_only;
    unsigned long long *n_band;
    int random;       // (count_only, ONE) the random control's selection too
    uint64_t seed;
};

constexpr int kSelChunk = 16;   // keys per lane held in registers (1024 per wave)

// Random control inside the count pass, one wave per row of at most 1024
// keys: the k valid keys with the smallest (SplitMix64(seed ^ linear index),
// j), the same set as random_select_kernel's.  The hashes stay in registers
// (key lane + 64 t in h[t]); a radix select over 8-bit digits, MSB first,
// with a 256-bin histogram per wave in LDS (lane l owns bins 4l .. 4l + 3)
// finds the k-th smallest hash T, stopping at the first digit whose bucket
// is taken whole; then keys with hash < T (or at most the bucket's end) are
// selected, and keys equal to T by increasing j until k.  Mask words for
// every chunk before S and the list segment in key order.
__device__ __forceinline__ void random_pick_row(const SelectArgs &a, uint32_t *hist, uint64_t r,
                                                int n, uint32_t k, int lane)
{
    const int S = a.S;
    const uint64_t base = r * (uint64_t)S;   // linear index of score (b, h, i, 0)
    uint64_t h[kSelChunk];
#pragma unroll
    for (int t = 0; t < kSelChunk; ++t) {
        const int j = lane + 64 * t;
        h[t] = j < n ? splitmix64(a.seed ^ (base + (uint64_t)j)) : ~0ull;
    }
    uint64_t prefix = 0, pmask = 0, ub = 0;
    uint32_t rank = k;
    bool whole = false;
    if (k > 0) {
        for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                hist[4 * lane + q] = 0u;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < kSelChunk; ++t)
                if (64 * t < n && lane + 64 * t < n && (h[t] & pmask) == prefix)
                    atomicAdd(&hist[(uint32_t)(h[t] >> shift) & 255u], 1u);
            __builtin_amdgcn_wave_barrier();
            uint32_t c[4], local = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[4 * lane + q];
                local += c[q];
            }
            uint32_t incl = local;   // inclusive prefix over the lanes
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o, 64);
                if (lane >= o)
                    incl += y;
            }
            // the digit holding the rank: cum < rank <= cum + count (the last
            // digit if the rank exceeds the candidates, which the counts rule
            // out)
            uint32_t cum = incl - local, fdig = 0, fcum = 0, fcnt = 0;
            bool found = false;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t d = 4u * (uint32_t)lane + (uint32_t)q;
                if (!found && ((cum < rank && rank <= cum + c[q]) ||
                               (d == 255u && rank > cum + c[q]))) {
                    found = true;
                    fdig = d;
                    fcum = cum;
                    fcnt = c[q];
                }
                cum += c[q];
            }
            const int src = __builtin_ctzll(ballot(found));
            fdig = (uint32_t)__shfl(fdig, src, 64);
            fcum = (uint32_t)__shfl(fcum, src, 64);
            fcnt = (uint32_t)__shfl(fcnt, src, 64);
            prefix |= (uint64_t)fdig << shift;
            rank -= fcum;
            pmask |= 255ull << shift;
            __builtin_amdgcn_wave_barrier();   // the bins are read before the next clear
            if (rank == fcnt) {   // uniform: the whole bucket is taken
                whole = true;
                ub = prefix | ((1ull << shift) - 1ull);
                break;
            }
        }
    }
    const uint64_t T = prefix;
    const uint64_t seg = row_segment(r, S, a.causal);
    uint32_t eq_before = 0, total = 0;
#pragma unroll
    for (int t = 0; t < kSelChunk; ++t) {
        if (64 * t < S) {   // wave-uniform
            const int j = lane + 64 * t;
            const bool valid = k > 0 && j < n;
            const bool lt = valid && (whole ? h[t] <= ub : h[t] < T);
            const bool eq = valid && !whole && h[t] == T;
            const uint64_t tb = ballot(eq);
            const bool sel = lt || (eq && eq_before + lanes_below(tb) < rank);
            eq_before += (uint32_t)__popcll(tb);
            const uint64_t b = ballot(sel);
            if (a.mask) {
                const int w = 2 * t;
                if (lane == 0 && w < a.W)
                    a.mask[r * (uint64_t)a.W + w] = (uint32_t)b;
                if (lane == 1 && w + 1 < a.W)
                    a.mask[r * (uint64_t)a.W + w + 1] = (uint32_t)(b >> 32);
            }
            if (sel && a.list)
                a.list[seg + total + lanes_below(b)] = (uint32_t)j;
            total += (uint32_t)__popcll(b);
        }
    }
}
constexpr int kSelBatch = 8;    // longer rows: 64-key chunks whose loads issue together

// One wave per row; 4 rows per work-group.  ONE: the whole row fits one
// register chunk (S <= 1024), so scores and exponentials are read and formed
// once; otherwise the row is streamed three times, kSelBatch chunks of 64
// keys at a time with all of a batch's loads issued before its arithmetic
// (range-checked buffer loads: keys past the row read 0 and are skipped).
template <bool ONE>
__global__ __launch_bounds__(kThreads) void strict_select_kernel(SelectArgs a)
{
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    __shared__ uint32_t s_hist[ONE ? 4 : 1][ONE ? 256 : 1];   // per wave (random control)
    exp_table_fill(s_exp);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    // the wave index through readfirstlane: the row and every row quantity
    // (its length, pointers, buffer ranges, loop bounds) are then scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t r = (uint64_t)blockIdx.x * 4 + wave;
    if (r >= a.n_rows)
        return;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const float *y = a.y + r * (uint64_t)S;
    // the reference scores serve only the row KLs: without them (no KL asked
    // for) their loads read an empty range (0) and their sums are skipped
    const bool ref = a.yref != nullptr;
    const float *yr = ref ? a.yref + r * (uint64_t)S : y;
    const __amdgpu_buffer_rsrc_t y_rs = row_rsrc(y, 4u * (uint32_t)n);
    const __amdgpu_buffer_rsrc_t r_rs = row_rsrc(yr, ref ? 4u * (uint32_t)n : 0u);

    float vlo[kSelChunk], vref[kSelChunk];
    double elo[kSelChunk];
    // Row maxima of y^lo and y^ref.
    float m = -INFINITY, mr = -INFINITY;
    if (ONE) {
#pragma unroll
        for (int t = 0; t < kSelChunk; ++t) {
            const int j = lane + 64 * t;
            vlo[t] = j < n ? y[j] : -INFINITY;
            vref[t] = ref && j < n ? yr[j] : -INFINITY;
            m = fmaxf(m, vlo[t]);
            mr = fmaxf(mr, vref[t]);
        }
    } else {
        for (int j0 = 0; j0 < n; j0 += 64 * kSelBatch) {
            float vb[kSelBatch], vrb[kSelBatch];
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u) {
                const uint32_t off = 4u * (uint32_t)(j0 + 64 * u + lane);
                vb[u] = buf_load_f32(y_rs, off);
                vrb[u] = buf_load_f32(r_rs, off);
            }
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u)
                if (j0 + 64 * u + lane < n) {
                    m = fmaxf(m, vb[u]);
                    mr = fmaxf(mr, vrb[u]);
                }
        }
    }
    m = wave_max(m);
    mr = wave_max(mr);

    // A: sum of exp(y^lo - m) below the maximum; cnt: keys at the maximum;
    // Lr, Br: reference sum and sum of e_ref (y^ref - y^lo).  Branch-free,
    // with the exponential of a non-positive argument; an argument that is
    // NaN (a NaN score, or inf - inf) makes the sums it feeds NaN, as a NaN
    // exponential would.
    double A = 0.0, Lr = 0.0, Br = 0.0;
    int cnt = 0;
    bool nan_lo = false, nan_ref = false;
    auto accumulate = [&](float v, float vr, double &e) {
        const bool at = v == m;
        const double dl = (double)v - (double)m, dr = (double)vr - (double)mr;
        const double x = exp64_crit_nonpos(dl, s_exp);
        e = at ? 1.0 : x;
        A += at ? 0.0 : x;
        cnt += at ? 1 : 0;
        nan_lo |= !at && dl != dl;
        if (ref) {   // wave-uniform
            const double er = exp64_sum_nonpos(dr, s_exp);
            Lr += er;
            Br += er * ((double)vr - (double)v);
            nan_ref |= dr != dr;
        }
    };
    if (ONE) {
#pragma unroll
        for (int t = 0; t < kSelChunk; ++t) {
            elo[t] = 0.0;
            if (lane + 64 * t < n)
                accumulate(vlo[t], vref[t], elo[t]);
        }
    } else {
        double e;
        for (int j0 = 0; j0 < n; j0 += 64 * kSelBatch) {
            float vb[kSelBatch], vrb[kSelBatch];
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u) {
                const uint32_t off = 4u * (uint32_t)(j0 + 64 * u + lane);
                vb[u] = buf_load_f32(y_rs, off);
                vrb[u] = buf_load_f32(r_rs, off);
            }
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u)
                if (j0 + 64 * u + lane < n)
                    accumulate(vb[u], vrb[u], e);
        }
    }
    A = wave_sum(A);
    Lr = wave_sum(Lr);
    Br = wave_sum(Br);
    cnt = wave_sum_int(cnt);
    if (ballot(nan_lo) != 0)
        A = __builtin_nan("");
    if (ballot(nan_ref) != 0) {
        Lr = __builtin_nan("");
        Br = __builtin_nan("");
    }
    const double L = A + (double)cnt;
    const double rest_at_max = A + (double)(cnt - 1);
    const double lse_lo = (double)m + log(L);
    const double lse_ref = (double)mr + log(Lr);
    const double kl_lowp = Br / Lr + lse_lo - lse_ref;
    if (lane == 0) {
        RowStats st;
        st.L_lo = L;
        st.L_ref = Lr;
        st.A = Br;
        st.lse_mix = lse_lo;
        st.m_lo = m;
        st.m_ref = mr;
        st.full_pass = 0;
        st.pad = 0;
        a.rs[r] = st;
        if (a.row_kl)
            a.row_kl[r] = kl_lowp;
        if (a.row_kl_lowp)
            a.row_kl_lowp[r] = kl_lowp;
    }

    // Criterion, mask words and compaction into this row's list segment.
    const uint64_t seg = row_segment(r, S, a.causal);
    uint32_t total = 0;
    const int jend = a.count_only ? n : S;
    // c = 2 z (1 - z) |y| with z = e / L and 1 - z = rest / L, rest = L - e
    // (or the sum of the other keys at the maximum): 2 e rest |y| / L^2.
    const double inv_l2 = 1.0 / (L * L);
    uint32_t ties = 0;
    auto decide = [&](int j0, int j, float v, double e) {
        bool sel = false, tie = false;
        if (j < n) {
            const double rest = (v == m) ? rest_at_max : L - e;
            const double c = 2.0 * e * rest * fabs((double)v) * inv_l2;
            sel = c > a.tau;
            tie = near_tie(c, a.tau);
        }
        if (a.n_band)   // near ties are counted only for a summary
            ties += (uint32_t)__popcll(ballot(tie));
        const uint64_t b = ballot(sel);
        if (!a.count_only) {
            if (a.mask) {
                const int w = j0 >> 5;
                if (lane == 0 && w < a.W)
                    a.mask[r * (uint64_t)a.W + w] = (uint32_t)b;
                if (lane == 1 && w + 1 < a.W)
                    a.mask[r * (uint64_t)a.W + w + 1] = (uint32_t)(b >> 32);
            }
            if (sel)
                a.list[seg + total + lanes_below(b)] = (uint32_t)j;
        }
        total += (uint32_t)__popcll(b);
    };
    if (ONE) {
#pragma unroll
        for (int t = 0; t < kSelChunk; ++t)
            if (64 * t < jend)
                decide(64 * t, lane + 64 * t, vlo[t], elo[t]);
    } else {
        for (int j0 = 0; j0 < jend; j0 += 64 * kSelBatch) {
            float vb[kSelBatch];
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u)
                vb[u] = buf_load_f32(y_rs, 4u * (uint32_t)(j0 + 64 * u + lane));
#pragma unroll
            for (int u = 0; u < kSelBatch; ++u) {
                const int jc = j0 + 64 * u;
                if (jc < jend) {   // wave-uniform: every lane takes part in the ballots
                    const int j = jc + lane;
                    double e = 0.0;
                    if (j < n)   // a NaN row already has NaN statistics (no key selected)
                        e = (vb[u] == m) ? 1.0
                                         : exp64_crit_nonpos((double)vb[u] - (double)m, s_exp);
                    decide(jc, j, vb[u], e);
                }
            }
        }
    }
    if (lane == 0)
        a.row_count[r] = total;
    add_ties(a.n_band, ties);
    if constexpr (ONE) {
        if (a.random)
            random_pick_row(a, s_hist[wave], r, n, total, lane);
    }
}

hipError_t launch_strict_select(const Problem &p, const float *ylo, const float *yref,
                                uint32_t *mask, uint32_t *list, uint32_t *row_count,
                                RowStats *rs, double *row_kl, double *row_kl_lowp,
                                int count_only, hipStream_t st, const uint64_t *random_seed)
{
    if (random_seed && (!count_only || p.S > 64 * kSelChunk))
        return hipErrorInvalidValue;
    SelectArgs a;
    a.random = random_seed ? 1 : 0;
    a.seed = random_seed ? *random_seed : 0;
    a.y = ylo;
    a.yref = yref;
    a.S = p.S;
    a.causal = p.causal;
    a.W = (p.S + 31) / 32;
    a.n_rows = p.n_rows;
    a.tau = (double)p.tau;
    a.n_band = p.n_band;
    a.mask = mask;
    a.list = list;
    a.row_count = row_count;
    a.rs = rs;
    a.row_kl = row_kl;
    a.row_kl_lowp = row_kl_lowp;
    a.count_only = count_only;
    const uint64_t grid = (p.n_rows + 3) / 4;
    if (p.S <= 64 * kSelChunk)
        hipLaunchKernelGGL(strict_select_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(strict_select_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Relaxed rule over rows of any length, after score tiles that kept y^lo,
// y^ref and their per-tile partials (the relaxed relative-threshold variant
// of "Experimental results", with m_t the running maximum of y^lo over the
// 64-key blocks up to the key's).  One wave per row and ONE streaming pass:
// block t of the rule is chunk t of 64 keys and also score tile t, whose
// partial carries the block's y^lo maximum, so m_t is known when chunk t
// arrives and each key is decided as the row streams past (one double
// exponential per key, E = exp(y - m_t)).  A selected key's y^mix is its
// y^ref, the sequential FP32 score (the recompute, bit for bit), written in
// place over y^lo.  The softmax sums are taken against shifts known before
// the pass: exp(y - m_lo) = E exp(m_t - m_lo) for the low-precision sum and
// exp(y - M) = E exp(m_t - M), M = max(m_lo, m_ref), for the unselected keys
// of the y^mix sum (one factor per chunk); the selected keys add exp(y^ref -
// M).  The reference sums come from the partials; a selected key's term
// p_ref (y^ref - y^lo) leaves the KL sum.
// ---------------------------------------------------------------------------
struct RelaxedSelectArgs {
    float *y;   // y^lo in, y^mix out
    const float *yref;
    const RefPartial *part;
    int S, causal, tiles, W;
    uint64_t n_rows;
    double tau;
    uint32_t *mask, *row_count;
    RowStats *rs;
    double *row_kl, *row_kl_lowp;
    unsigned long long *n_band;
};

__global__ __launch_bounds__(kThreads) void relaxed_select_kernel(RelaxedSelectArgs a)
{
    __shared__ uint32_t s_qj[4][128];   // per wave: queued selected keys
    __shared__ float s_qv[4][128];      // and their y^lo
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    exp_table_fill(s_exp);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t rr = (uint64_t)blockIdx.x * 4 + wave;
    if (rr >= a.n_rows)
        return;   // no block barrier below: each wave owns its row
    // rows in descending order: long causal rows first, short ones at the end
    const uint64_t r = a.n_rows - 1 - rr;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const int nt = (n + 63) >> 6;   // tiles (= 64-key blocks) holding valid keys
    float *y = a.y + r * (uint64_t)S;
    const float *yr = a.yref + r * (uint64_t)S;
    const RefPartial *pt = a.part + r * (uint64_t)a.tiles;
    const __amdgpu_buffer_rsrc_t y_rs = row_rsrc(y, 4u * (uint32_t)n);

    // Row maxima of y^lo and y^ref; reference sums rescaled to m_ref (zero,
    // and unused, when no KL is asked for: the partials then hold no sums).
    float mlo = -INFINITY, mr = -INFINITY;
    for (int t = lane; t < nt; t += 64) {
        mlo = fmaxf(mlo, pt[t].m_lo);
        mr = fmaxf(mr, pt[t].m);
    }
    mlo = wave_max(mlo);
    mr = wave_max(mr);
    double Lr = 0.0, Br = 0.0;
    for (int t = lane; t < nt; t += 64) {
        const RefPartial p = pt[t];
        const double f = exp64_sum_nonpos((double)p.m - (double)mr, s_exp);
        Lr += p.L * f;
        Br += p.B * f;
    }
    Lr = wave_sum(Lr);
    Br = wave_sum(Br);
    const double M = (double)fmaxf(mlo, mr);

    // l_lo: sum of exp(y^lo - m_lo); l_un / l_sel: the unselected / selected
    // keys' part of the sum of exp(y^mix - M); dA: the selected keys' KL terms.
    // g_lo = exp(m_t - m_lo) and g_mix = exp(m_t - M) change only with m_t.
    float mt = -INFINITY;
    double g_lo = 0.0, g_mix = 0.0;
    double l_lo = 0.0, l_un = 0.0, l_sel = 0.0, dA = 0.0;
    bool has_nan = false;
    uint32_t ties = 0;
    uint32_t total = 0;
    // Selected keys wait in this wave's LDS queue (key, y^lo) and are taken
    // 64 at a time, one per lane: y^ref read, y^mix written, their
    // exponentials formed, so that work costs one lane per selected key.
    uint32_t pend = 0;
    auto take = [&](uint32_t cnt) {   // the first cnt (<= 64) queued keys
        if ((uint32_t)lane < cnt) {
            const uint32_t j = s_qj[wave][lane];
            const float v = s_qv[wave][lane];
            const float h = yr[j];
            y[j] = h;
            l_sel += exp64_sum_nonpos((double)h - M, s_exp);
            dA += exp64_sum_nonpos((double)h - (double)mr, s_exp) * ((double)h - (double)v);
        }
    };
    for (int j0 = 0; j0 < n; j0 += 64 * kSelBatch) {
        float vb[kSelBatch], bm[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u)
            vb[u] = buf_load_f32(y_rs, 4u * (uint32_t)(j0 + 64 * u + lane));
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
            const int c = (j0 >> 6) + u;
            bm[u] = c < nt ? pt[c].m_lo : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
            const int jc = j0 + 64 * u;
            if (jc < n) {   // wave-uniform: every lane takes part in the ballot
                // the block maximum is uniform: a new running maximum is a
                // scalar branch (a NaN block maximum never raises it)
                const float bmu =
                    __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bm[u])));
                if (bmu > mt) {
                    mt = bmu;
                    g_lo = exp64_sum_nonpos((double)mt - (double)mlo, s_exp);
                    g_mix = exp64_sum_nonpos((double)mt - M, s_exp);
                }
                const int j = jc + lane;
                const bool valid = j < n;
                const float v = vb[u];
                // y <= m_t for a valid key; a key past the row gives E = 0
                const double E =
                    exp64_crit_nonpos(valid ? (double)v - (double)mt : -INFINITY, s_exp);
                has_nan |= valid && v != v;
                const double c = 2.0 * E * fabs((double)v);
                const bool sel = valid && c > a.tau;
                if (a.n_band)   // near ties are counted only for a summary
                    ties += (uint32_t)__popcll(ballot(valid && near_tie(c, a.tau)));
                l_lo = fma(E, g_lo, l_lo);
                l_un = sel ? l_un : fma(E, g_mix, l_un);
                const uint64_t b = ballot(sel);
                if (a.mask) {
                    const int w = (jc >> 5) + lane;
                    if (lane < 2 && w < a.W)
                        a.mask[r * (uint64_t)a.W + w] = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
                }
                if (b) {
                    if (sel) {
                        const uint32_t q = pend + lanes_below(b);
                        s_qj[wave][q] = (uint32_t)j;
                        s_qv[wave][q] = v;
                    }
                    const uint32_t nb = (uint32_t)__popcll(b);
                    pend += nb;
                    total += nb;
                    if (pend >= 64) {   // take 64, move the rest (< 64) down
                        __builtin_amdgcn_wave_barrier();
                        take(64);
                        const uint32_t rest = pend - 64;
                        uint32_t qj = 0;
                        float qv = 0.0f;
                        if ((uint32_t)lane < rest) {
                            qj = s_qj[wave][64 + lane];
                            qv = s_qv[wave][64 + lane];
                        }
                        __builtin_amdgcn_wave_barrier();
                        if ((uint32_t)lane < rest) {
                            s_qj[wave][lane] = qj;
                            s_qv[wave][lane] = qv;
                        }
                        __builtin_amdgcn_wave_barrier();
                        pend = rest;
                    }
                }
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    take(pend);
    if (a.mask)   // the mask words past the valid keys
        for (int w = 2 * nt + lane; w < a.W; w += 64)
            a.mask[r * (uint64_t)a.W + w] = 0u;
    l_lo = wave_sum(l_lo);
    l_un = wave_sum(l_un);
    l_sel = wave_sum(l_sel);
    dA = wave_sum(dA);
    if (ballot(has_nan) != 0) {   // a NaN score makes the row's statistics NaN
        l_lo = __builtin_nan("");
        l_un = __builtin_nan("");
    }
    const double Lmix = l_un + l_sel;
    const double lse_ref = (double)mr + log(Lr);
    const double lse_lo = (double)mlo + log(l_lo);
    const double lse_mix = M + log(Lmix);
    // a sum that underflowed (y^mix far below M) is formed again over the row
    // by the finish kernel
    const bool full = !(Lmix >= 1e-280);
    if (lane == 0) {
        RowStats st;
        st.L_lo = l_lo;
        st.L_ref = Lr;
        st.A = Br - dA;
        st.lse_mix = lse_mix;
        st.m_lo = mlo;
        st.m_ref = mr;
        st.full_pass = full ? 1u : 0u;
        st.pad = 0;
        a.rs[r] = st;
        if (a.row_count)
            a.row_count[r] = total;
        if (a.row_kl && !full)
            a.row_kl[r] = (Br - dA) / Lr + lse_mix - lse_ref;
        if (a.row_kl_lowp)
            a.row_kl_lowp[r] = Br / Lr + lse_lo - lse_ref;
    }
    add_ties(a.n_band, ties);
}

hipError_t launch_relaxed_select(const Problem &p, float *y, const float *yref,
                                 const RefPartial *part, uint32_t *mask, uint32_t *row_count,
                                 RowStats *rs, double *row_kl, double *row_kl_lowp,
                                 hipStream_t st)
{
    if (!y || !yref || !part || !rs)
        return hipErrorInvalidValue;
    RelaxedSelectArgs a;
    a.y = y;
    a.yref = yref;
    a.part = part;
    a.S = p.S;
    a.causal = p.causal;
    a.tiles = p.tiles;
    a.W = (p.S + 31) / 32;
    a.n_rows = p.n_rows;
    a.tau = (double)p.tau;
    a.n_band = p.n_band;
    a.mask = mask;
    a.row_count = row_count;
    a.rs = rs;
    a.row_kl = row_kl;
    a.row_kl_lowp = row_kl_lowp;
    const uint64_t grid = (p.n_rows + 3) / 4;
    hipLaunchKernelGGL(relaxed_select_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Random control: per row, the k = row_count[r] valid keys with the smallest
// (SplitMix64(seed ^ linear index), j).  One work-group per row: an 8-pass
// radix select over the 64-bit hashes finds the k-th smallest value T; keys
// with hash < T are selected, and keys equal to T by increasing j until k.
// HPT > 0: each thread keeps its HPT hashes (keys tid + 256 u) in registers,
// so they are formed once (rows of at most 256 HPT keys); HPT = 0 forms them
// again in every pass.  Each pass builds a 256-bin histogram of the current
// digit with LDS atomics and finds the digit holding the rank by a parallel
// exclusive scan of the bins (one bin per thread).
// ---------------------------------------------------------------------------
struct RandomArgs {
    int S, causal, W;
    uint64_t n_rows, seed;
    uint32_t *mask, *list;
    const uint32_t *row_count;
};

// Exclusive prefix sum of one value per thread over a 256-thread block.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t *s_wtot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o)
            inc += y;
    }
    if (lane == 63)
        s_wtot[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w)
        before += s_wtot[w];
    return before + inc - x;
}

template <int HPT>
__global__ __launch_bounds__(kThreads) void random_select_kernel(RandomArgs a)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_wtot[4];
    __shared__ uint64_t s_prefix;
    __shared__ uint32_t s_rank, s_hd;
    __shared__ uint32_t s_eqw[4], s_selw[4];
    __shared__ uint32_t s_eq_before, s_sel_before;
    const uint64_t r = blockIdx.x;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const uint32_t k = a.row_count[r];
    const uint64_t base = r * (uint64_t)S;     // linear index of score (b, h, i, 0)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto hash = [&](int j) { return splitmix64(a.seed ^ (base + (uint64_t)j)); };

    uint64_t hc[HPT > 0 ? HPT : 1];
    if (HPT > 0) {
#pragma unroll
        for (int u = 0; u < (HPT > 0 ? HPT : 1); ++u) {
            const int j = tid + kThreads * u;
            hc[u] = j < n ? hash(j) : ~0ull;
        }
    }

    // Radix select of the k-th smallest hash T (8 digits of 8 bits, MSB first);
    // `rank` ends as the number of keys equal to T that are taken.  A digit
    // whose bucket is taken whole (the rank is its last element; with 64-bit
    // hashes usually after two digits) ends the search: the selection is then
    // every key whose hash lies at or below the bucket's end, `ub`.
    uint64_t prefix = 0, pmask = 0;
    uint32_t rank = k;
    bool whole = false;
    uint64_t ub = 0;
    if (k > 0) {
        for (int shift = 56; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            auto count = [&](uint64_t h) {
                if ((h & pmask) == prefix)
                    atomicAdd(&hist[(uint32_t)(h >> shift) & 255u], 1u);
            };
            if (HPT > 0) {
#pragma unroll
                for (int u = 0; u < (HPT > 0 ? HPT : 1); ++u)
                    if (tid + kThreads * u < n)
                        count(hc[u]);
            } else {
                for (int j = tid; j < n; j += kThreads)
                    count(hash(j));
            }
            __syncthreads();
            const uint32_t hd = hist[tid];
            const uint32_t cum = block_excl_scan(hd, s_wtot);
            // the digit holding the rank: cum < rank <= cum + hist (the last
            // digit if the rank exceeds the candidates, which the counts
            // exclude)
            if ((cum < rank && rank <= cum + hd) || (tid == 255 && rank > cum + hd)) {
                s_prefix = prefix | ((uint64_t)tid << shift);
                s_rank = rank - cum;
                s_hd = hd;
            }
            __syncthreads();
            prefix = s_prefix;
            rank = s_rank;
            pmask |= 255ull << shift;
            if (rank == s_hd) {   // uniform: the whole bucket is taken
                whole = true;
                ub = prefix | ((1ull << shift) - 1ull);
                break;
            }
        }
    }
    const uint64_t T = prefix;

    if (tid == 0) {
        s_eq_before = 0;
        s_sel_before = 0;
    }
    __syncthreads();
    const uint64_t seg = row_segment(r, S, a.causal);
    for (int j0 = 0, u = 0; j0 < S; j0 += kThreads, ++u) {
        const int j = j0 + tid;
        bool lt = false, eq = false;
        if (k > 0 && j < n) {
            uint64_t h;
            if (HPT > 0) {
                h = hc[0];
#pragma unroll
                for (int uu = 1; uu < (HPT > 0 ? HPT : 1); ++uu)
                    h = uu == u ? hc[uu] : h;
            } else {
                h = hash(j);
            }
            lt = whole ? h <= ub : h < T;
            eq = !whole && h == T;
        }
        const uint64_t tb = ballot(eq);
        if (lane == 0)
            s_eqw[wave] = (uint32_t)__popcll(tb);
        __syncthreads();
        uint32_t eq_rank = s_eq_before + lanes_below(tb);
        for (int w = 0; w < wave; ++w)
            eq_rank += s_eqw[w];
        const bool sel = lt || (eq && eq_rank < rank);
        const uint64_t b = ballot(sel);
        const int w32 = (j0 + wave * 64) >> 5;
        if (a.mask && lane < 2 && w32 + lane < a.W)
            a.mask[r * (uint64_t)a.W + w32 + lane] = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
        if (lane == 0)
            s_selw[wave] = (uint32_t)__popcll(b);
        __syncthreads();
        if (a.list && sel) {
            uint32_t pos = s_sel_before + lanes_below(b);
            for (int w = 0; w < wave; ++w)
                pos += s_selw[w];
            if (pos < (uint32_t)n)   // the row's segment holds n entries
                a.list[seg + pos] = (uint32_t)j;
        }
        __syncthreads();
        if (tid == 0) {
            s_eq_before += s_eqw[0] + s_eqw[1] + s_eqw[2] + s_eqw[3];
            s_sel_before += s_selw[0] + s_selw[1] + s_selw[2] + s_selw[3];
        }
        __syncthreads();
    }
}

hipError_t launch_random_select(const Problem &p, uint64_t seed, uint32_t *mask, uint32_t *list,
                                const uint32_t *row_count, hipStream_t st)
{
    RandomArgs a;
    a.S = p.S;
    a.causal = p.causal;
    a.W = (p.S + 31) / 32;
    a.n_rows = p.n_rows;
    a.seed = seed;
    a.mask = mask;
    a.list = list;
    a.row_count = row_count;
    if (p.S <= 4 * kThreads)
        hipLaunchKernelGGL(random_select_kernel<4>, dim3((unsigned)p.n_rows), dim3(kThreads), 0, st, a);
    else if (p.S <= 16 * kThreads)
        hipLaunchKernelGGL(random_select_kernel<16>, dim3((unsigned)p.n_rows), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(random_select_kernel<0>, dim3((unsigned)p.n_rows), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP32 recompute ("Implementation strategy" step 3) of the listed keys: the
// score tiles already formed every score's sequential FP32 dot (multiply then
// add, d ascending, no fused multiply-add) as y^ref, so each thread takes one
// listed key and scatters its y^ref over the baseline score.
// ---------------------------------------------------------------------------
struct RecomputeArgs {
    const float *yref;   // the stored FP32 reference scores, or null (gather dot)
    const float *q, *k;  // [BH, S, D] (the gather dot)
    float s;             // the score scale
    int S, D, causal;
    uint64_t n_rows;
    const uint32_t *list, *row_count;
    float *ymix;
    RowStats *rs;
    double *row_kl;
};

// The softmax statistics of y^mix follow from those of y^lo by correcting the
// changed terms: L_mix = L_lo + sum_sel [exp(y_hi - m_lo) - exp(y_lo - m_lo)]
// and A = A_lo - sum_sel exp(y_hi - m_ref) (y_hi - y_lo) (a recomputed score
// equals its FP32 reference, so its KL term vanishes).  When the correction
// removes most of L_lo (a dominant key moved down) or overflows (a key moved
// far above m_lo) the row is flagged for a full pass in the finish kernel.
//
// One work-group per 64 rows: the rows' list segments are concatenated
// (block-local prefix of the counts) and every thread takes one listed score
// per pass; the per-row corrections are then summed in list order by one
// thread per row, so the result does not depend on scheduling.
constexpr int kRcRows = 64;

// y_hi of row r, key j: the sequential FP32 dot (multiply, then add, d
// ascending) of the query and key rows, scaled.
__device__ __forceinline__ float gather_dot(const RecomputeArgs &a, uint64_t r, uint32_t j)
{
    const uint64_t bh = r / (uint64_t)a.S;
    const float4 *q4 = reinterpret_cast<const float4 *>(a.q + r * (uint64_t)a.D);
    const float4 *k4 = reinterpret_cast<const float4 *>(a.k + (bh * (uint64_t)a.S + j) * a.D);
    float acc = 0.0f;
    for (int d0 = 0; d0 < a.D / 4; d0 += 4) {
        float4 qv[4], kv[4];   // four 16-byte loads of each row in flight
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = d0 + u < a.D / 4;
            qv[u] = in ? q4[d0 + u] : make_float4(0.f, 0.f, 0.f, 0.f);
            kv[u] = in ? k4[d0 + u] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (d0 + u < a.D / 4) {
                float p0 = qv[u].x * kv[u].x;
                acc = acc + p0;
                float p1 = qv[u].y * kv[u].y;
                acc = acc + p1;
                float p2 = qv[u].z * kv[u].z;
                acc = acc + p2;
                float p3 = qv[u].w * kv[u].w;
                acc = acc + p3;
            }
        }
    }
    return acc * a.s;
}

__global__ __launch_bounds__(kThreads) void recompute_kernel(RecomputeArgs a)
{
    __shared__ uint32_t s_off[kRcRows + 1];
    __shared__ float s_mlo[kRcRows], s_mref[kRcRows];
    __shared__ double s_dl[kThreads], s_da[kThreads];
    __shared__ double s_exp[64];   // 2^(k/64) for exp64 (synchronised below)
    exp_table_fill(s_exp);
    const int tid = threadIdx.x;
    const uint64_t r0 = (uint64_t)blockIdx.x * kRcRows;
    RowStats st{};
    uint32_t cnt = 0;
    if (tid < kRcRows) {
        const uint64_t r = r0 + tid;
        if (r < a.n_rows) {
            const int i = (int)(r % (uint64_t)a.S);
            const uint32_t n = a.causal ? (uint32_t)i + 1u : (uint32_t)a.S;
            cnt = min(a.row_count[r], n);
            st = a.rs[r];
        }
        s_off[tid + 1] = cnt;
        s_mlo[tid] = st.m_lo;
        s_mref[tid] = st.m_ref;
    }
    __syncthreads();
    if (tid == 0) {
        s_off[0] = 0;
        for (int t = 1; t <= kRcRows; ++t)
            s_off[t] += s_off[t - 1];
    }
    __syncthreads();
    const uint32_t total = s_off[kRcRows];
    if (total == 0)
        return;
    double dL = 0.0, dA = 0.0;
    for (uint32_t base = 0; base < total; base += kThreads) {
        const uint32_t e = base + tid;
        double cl = 0.0, ca = 0.0;
        if (e < total) {
            int lo = 0, hi = kRcRows;   // row lr with s_off[lr] <= e < s_off[lr + 1]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_off[mid] <= e)
                    lo = mid;
                else
                    hi = mid;
            }
            const int lr = lo;
            const uint64_t r = r0 + lr;
            const uint32_t j = a.list[row_segment(r, a.S, a.causal) + (e - s_off[lr])];
            if (j < (uint32_t)a.S) {
                // the stored FP32 reference score (the sequential FP32 dot the
                // recompute forms, the same bits), or that dot formed here
                // from the gathered query and key rows
                const float yhi = a.yref ? a.yref[r * (uint64_t)a.S + j]
                                         : gather_dot(a, r, j);
                float *slot = a.ymix + r * (uint64_t)a.S + j;
                const float ylo = *slot;
                *slot = yhi;
                const double ml = (double)s_mlo[lr], mr = (double)s_mref[lr];
                cl = exp64_crit((double)yhi - ml, s_exp) - exp64_crit((double)ylo - ml, s_exp);
                if (a.row_kl)
                    ca = exp64_sum((double)yhi - mr, s_exp) * ((double)yhi - (double)ylo);
            }
        }
        s_dl[tid] = cl;
        s_da[tid] = ca;
        __syncthreads();
        if (tid < kRcRows) {
            const uint32_t b = max(s_off[tid], base), en = min(s_off[tid + 1], base + kThreads);
            for (uint32_t x = b; x < en; ++x) {
                dL += s_dl[x - base];
                dA += s_da[x - base];
            }
        }
        __syncthreads();
    }
    if (tid < kRcRows && cnt > 0) {
        const uint64_t r = r0 + tid;
        const double Lmix = st.L_lo + dL;
        const double Amix = st.A - dA;
        const double lse_ref = (double)st.m_ref + log(st.L_ref);
        RowStats o = st;
        o.A = Amix;
        if (Lmix >= 0.25 * st.L_lo && isfinite(Lmix)) {
            o.lse_mix = (double)st.m_lo + log(Lmix);
            if (a.row_kl)
                a.row_kl[r] = Amix / st.L_ref + o.lse_mix - lse_ref;
        } else {
            o.full_pass = 1;
        }
        a.rs[r] = o;
    }
}

hipError_t launch_recompute(const Problem &p, const uint32_t *list, const uint32_t *row_count,
                            const float *yref, float *ymix, RowStats *rs, double *row_kl,
                            hipStream_t st)
{
    if (!yref && row_kl)   // the KL's reference statistics come with y^ref
        return hipErrorInvalidValue;
    RecomputeArgs a;
    a.yref = yref;
    a.q = p.q;
    a.k = p.k;
    a.s = p.pc.s;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.n_rows = p.n_rows;
    a.list = list;
    a.row_count = row_count;
    a.ymix = ymix;
    a.rs = rs;
    a.row_kl = row_kl;
    const uint64_t grid = (p.n_rows + kRcRows - 1) / kRcRows;
    hipLaunchKernelGGL(recompute_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lamp
