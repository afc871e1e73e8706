// relaxed.hip -- relaxed relative-threshold LAMP in one fused pass.
//
// The LAMP summary's "Experimental results" introduce a relaxed variant that
// drops the normalisation constant so that the selection fits one-pass
// (online-softmax) attention kernels; the strict rule needs the whole row
// ("Significance and claims", limitations).  Reading used here: key j is
// recomputed iff
//     2 exp(y^lo_j - m_t) |y^lo_j| > tau,
// where m_t is the running maximum of the PS(mu) scores over the valid keys of
// 64-key blocks 0..floor(j/64).  Every strictly selected key is selected here
// too, since z_j <= exp(y_j - m_t) and 1 - z_j <= 1.
//
// One work-group owns 64 query rows of one head and walks the key tiles of
// 64 keys in order.  Per tile: PS(mu) and FP32 scores (the same micro-tile as
// the strict score kernel), block max, running max m_t, selection, mask bits,
// y^mix = selected ? y^ref : y^lo (the FP32 recompute of a selected score is
// bit-identical to its FP32 reference score, which this pass already holds),
// online softmax of y^mix with P.V on MFMA, and online statistics of y^ref for
// the row KL(P_FP32 || P_LAMP).
#include "lamp_device.h"

namespace lamp {

typedef double doublex4 __attribute__((ext_vector_type(4)));

struct RelaxedArgs {
    const float *q, *k, *v;
    int S, D, Dv, causal, tiles, BH, W;
    double tau;
    PsConst pc;
    const uint8_t *unsafe_q, *unsafe_k;
    float *out;
    uint32_t *mask, *row_count;
    double *row_kl, *row_kl_lowp;
    float *ymix_raw, *yref_out, *row_m;
    double *row_l;
    unsigned long long *exact_tiles;
};

// Max / sum over the 16 lanes that share a row (lane groups of 16).
__device__ __forceinline__ float group16_max(float v)
{
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double group16_sum(double v)
{
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint32_t group16_sum_u(uint32_t v)
{
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

struct RelaxedSmem {
    union {
        TileSmem tile;
        float p[kTile][kTile];   // P tile of the online softmax, [row][key]
    } u;
    float v[kTile * 128];        // V tile, [key][col], up to 128 columns at a time
};

template <int PATH>
__device__ __forceinline__ void relaxed_tile_scores(RelaxedSmem &sm, const RelaxedArgs &a,
                                                    const float *Qh, const float *Kh, int row0,
                                                    int col0, float lo[4][4], float ref[4][4])
{
    TileAcc acc;
    score_tile<PATH>(sm.u.tile, acc, Qh, Kh, row0, col0, a.S, a.D, a.pc);
    tile_scores<PATH>(acc, a.pc, lo, ref);
}

// FAST_KERNEL: the work-group's query block and every key block it visits
// allow the FP32 fast path; the other instance takes the remaining query
// blocks (exact double path per tile where needed, plain FP32 at mu = 23).
template <int NB, bool FAST_KERNEL>
__global__ __launch_bounds__(kThreads) void relaxed_kernel(RelaxedArgs a)
{
    __shared__ RelaxedSmem sm;
    const int S = a.S, D = a.D, Dv = a.Dv;
    // heaviest query blocks first (causal work grows with the block index)
    const int qb = a.tiles - 1 - (int)(blockIdx.x / a.BH);
    const int bh = (int)(blockIdx.x % a.BH);
    const int row0 = qb * kTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tx = tid & 15, ty = tid >> 4;
    const size_t head = (size_t)bh * S * D;
    const float *Qh = a.q + head, *Kh = a.k + head, *Vh = a.v + head;
    const bool qsafe = !a.unsafe_q[bh * a.tiles + qb];
    const bool want_lowp = a.row_kl_lowp != nullptr;
    const int t_end = a.causal ? qb : a.tiles - 1;
    {
        bool all_fast = a.pc.mu <= 10 && qsafe;
        for (int t = 0; t <= t_end && all_fast; ++t)
            all_fast = !a.unsafe_k[bh * a.tiles + t];
        if (all_fast != FAST_KERNEL)
            return;
    }

    // Row state for rows ty*4 + r (replicated over the 16 lanes of the row).
    float m_t[4], m_mix[4], m_ref[4], m_lo[4];
    double l_mix[4], l_ref[4], kl_a[4], l_lo[4], kl_b[4];
    uint32_t cnt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_t[r] = m_mix[r] = m_ref[r] = m_lo[r] = -INFINITY;
        l_mix[r] = l_ref[r] = kl_a[r] = l_lo[r] = kl_b[r] = 0.0;
        cnt[r] = 0;
    }
    const int nb = Dv / 16;   // <= NB column blocks of 16
    // P.V accumulators (FP64 MFMA: FP32 accumulation over long rows drifts
    // beyond the 1e-6 bar)
    doublex4 acc[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q)
        acc[q] = doublex4{0.0, 0.0, 0.0, 0.0};

    for (int t = 0; t <= t_end; ++t) {
        const int col0 = t * kTile;
        float lo[4][4], ref[4][4];
        const int path = FAST_KERNEL ? PATH_FAST
                         : a.pc.mu == 23 ? PATH_FP32
                         : (a.pc.mu <= 10 && qsafe && !a.unsafe_k[bh * a.tiles + t]) ? PATH_FAST
                                                                                       : PATH_EXACT;
        if (FAST_KERNEL || path == PATH_FAST) {
            relaxed_tile_scores<PATH_FAST>(sm, a, Qh, Kh, row0, col0, lo, ref);
        } else if (path == PATH_EXACT) {
            if (tid == 0 && a.exact_tiles)
                atomicAdd(a.exact_tiles, 1ull);
            relaxed_tile_scores<PATH_EXACT>(sm, a, Qh, Kh, row0, col0, lo, ref);
        } else {
            relaxed_tile_scores<PATH_FP32>(sm, a, Qh, Kh, row0, col0, lo, ref);
        }

        float pmix[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + ty * 4 + r;
            bool valid[4];
            float bmax = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = col0 + tx + 16 * c;
                valid[c] = i < S && j < S && (!a.causal || j <= i);
                if (valid[c])
                    bmax = fmaxf(bmax, lo[r][c]);
            }
            bmax = group16_max(bmax);
            m_t[r] = fmaxf(m_t[r], bmax);

            // selection and y^mix
            float mix[4];
            bool sel[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                sel[c] = false;
                if (valid[c]) {
                    const double crit = 2.0 * exp((double)lo[r][c] - (double)m_t[r]) *
                                        fabs((double)lo[r][c]);
                    sel[c] = crit > a.tau;
                }
                mix[c] = sel[c] ? ref[r][c] : lo[r][c];
            }
            // mask bits: ballot per key offset c, 16 bits per row group
            const int gsh = (lane >> 4) * 16;
            uint32_t bits[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bits[c] = (uint32_t)(__ballot(sel[c]) >> gsh) & 0xffffu;
            if (i < S) {
                const uint32_t w0 = bits[0] | (bits[1] << 16), w1 = bits[2] | (bits[3] << 16);
                cnt[r] += tx == 0 ? (uint32_t)(__popc(w0) + __popc(w1)) : 0u;
                if (a.mask && tx == 0) {
                    const uint64_t mrow = ((uint64_t)bh * S + i) * (uint64_t)a.W;
                    if (2 * t < a.W)
                        a.mask[mrow + 2 * t] = w0;
                    if (2 * t + 1 < a.W)
                        a.mask[mrow + 2 * t + 1] = w1;
                }
                const uint64_t yrow = ((uint64_t)bh * S + i) * (uint64_t)S;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (!valid[c])
                        continue;
                    const int j = col0 + tx + 16 * c;
                    if (a.ymix_raw)
                        a.ymix_raw[yrow + j] = mix[c];
                    if (a.yref_out)
                        a.yref_out[yrow + j] = ref[r][c];
                }
            }

            // online softmax of y^mix
            float bm = -INFINITY, br = -INFINITY, bl = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (valid[c]) {
                    bm = fmaxf(bm, mix[c]);
                    br = fmaxf(br, ref[r][c]);
                    bl = fmaxf(bl, lo[r][c]);
                }
            bm = group16_max(bm);
            br = group16_max(br);
            const float mm_new = fmaxf(m_mix[r], bm);
            const float mr_new = fmaxf(m_ref[r], br);
            const double alpha = (m_mix[r] == -INFINITY) ? 0.0 : exp((double)m_mix[r] - (double)mm_new);
            const double beta = (m_ref[r] == -INFINITY) ? 0.0 : exp((double)m_ref[r] - (double)mr_new);
            double sl = 0.0, sr = 0.0, sa = 0.0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pmix[r][c] = 0.0f;
                if (valid[c]) {
                    const double pe = exp((double)mix[c] - (double)mm_new);
                    pmix[r][c] = (float)pe;
                    sl += pe;
                    const double er = exp((double)ref[r][c] - (double)mr_new);
                    sr += er;
                    sa += er * ((double)ref[r][c] - (double)mix[c]);
                }
            }
            l_mix[r] = l_mix[r] * alpha + sl;
            l_ref[r] = l_ref[r] * beta + sr;
            kl_a[r] = kl_a[r] * beta + sa;
            m_mix[r] = (i < S) ? mm_new : m_mix[r];
            m_ref[r] = (i < S) ? mr_new : m_ref[r];
            // rescale this row's P.V accumulators (MFMA rows 4*(lane/16)+r)
#pragma unroll
            for (int q = 0; q < NB; ++q)
                acc[q][r] *= alpha;

            if (want_lowp) {
                bl = group16_max(bl);
                const float ml_new = fmaxf(m_lo[r], bl);
                const double gam = (m_lo[r] == -INFINITY) ? 0.0 : exp((double)m_lo[r] - (double)ml_new);
                const double betal = beta;
                double sll = 0.0, sb = 0.0;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (valid[c]) {
                        sll += exp((double)lo[r][c] - (double)ml_new);
                        sb += exp((double)ref[r][c] - (double)mr_new) *
                              ((double)ref[r][c] - (double)lo[r][c]);
                    }
                l_lo[r] = l_lo[r] * gam + sll;
                kl_b[r] = kl_b[r] * betal + sb;
                m_lo[r] = (i < S) ? ml_new : m_lo[r];
            }
        }

        // P.V: P tile to LDS (aliases the score staging), V tile to LDS, MFMA.
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                sm.u.p[ty * 4 + r][tx + 16 * c] = pmix[r][c];
        for (int h = 0; h < Dv; h += 128) {
            const int Dc = min(128, Dv - h);
            const int n4 = kTile * Dc / 4;
            if (h > 0)
                __syncthreads();
            for (int e = tid; e < n4; e += kThreads) {
                const int key = e / (Dc / 4), col = h + (e % (Dc / 4)) * 4;
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (col0 + key < S && col < D)
                    x = *reinterpret_cast<const float4 *>(Vh + (size_t)(col0 + key) * D + col);
                *reinterpret_cast<float4 *>(sm.v + key * Dc + (col - h)) = x;
            }
            __syncthreads();
#pragma unroll 4
            for (int kk = 0; kk < kTile / 4; ++kk) {
                const float av = sm.u.p[wave * 16 + mfma64_row(lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    if (q < nb && q * 16 >= h && q * 16 < h + Dc) {
                        const float bv = sm.v[(kk * 4 + (lane >> 4)) * Dc + q * 16 - h + (lane & 15)];
                        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av, (double)bv,
                                                                      acc[q], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
    }

    // Finalise rows: combine the 16 lanes' partial sums.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = row0 + ty * 4 + r;
        const double lm = group16_sum(l_mix[r]);
        const double lr = group16_sum(l_ref[r]);
        const double ka = group16_sum(kl_a[r]);
        const uint32_t ct = group16_sum_u(cnt[r]);
        double ll = 0.0, kb = 0.0;
        if (want_lowp) {
            ll = group16_sum(l_lo[r]);
            kb = group16_sum(kl_b[r]);
        }
        if (i >= S)
            continue;
        const uint64_t row = (uint64_t)bh * S + i;
        if (a.mask)   // words of key tiles past the causal limit hold no selection
            for (int w = 2 * (t_end + 1) + tx; w < a.W; w += 16)
                a.mask[row * (uint64_t)a.W + w] = 0u;
        if (tx == 0) {
            if (a.row_kl)
                a.row_kl[row] = ka / lr + ((double)m_mix[r] + log(lm)) - ((double)m_ref[r] + log(lr));
            if (want_lowp)
                a.row_kl_lowp[row] = kb / lr + ((double)m_lo[r] + log(ll)) - ((double)m_ref[r] + log(lr));
            if (a.row_count)
                a.row_count[row] = ct;
            if (a.row_m)
                a.row_m[row] = m_mix[r];
            if (a.row_l)
                a.row_l[row] = lm;
        }
        // out rows of this lane's MFMA accumulators are 4*(lane/16)+r = ty*4+r
        const double inv = 1.0 / lm;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            if (q >= nb)
                continue;
            const int col = q * 16 + (lane & 15);
            if (col < D)
                a.out[row * (uint64_t)D + col] = (float)(acc[q][r] * inv);
        }
    }
}

hipError_t launch_relaxed(const Problem &p, const uint8_t *unsafe, float *out, uint32_t *mask,
                          uint32_t *row_count, double *row_kl, double *row_kl_lowp,
                          float *ymix_raw, float *yref_out, float *row_m, double *row_l,
                          unsigned long long *exact_tiles, bool fast, hipStream_t st)
{
    if (p.D > 128)
        return hipErrorInvalidValue;   // the fused kernel keeps <= 8 MFMA column blocks
    RelaxedArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.S = p.S;
    a.D = p.D;
    a.Dv = (p.D + 15) / 16 * 16;
    a.causal = p.causal;
    a.tiles = p.tiles;
    a.BH = p.BH;
    a.W = (p.S + 31) / 32;
    a.tau = (double)p.tau;
    a.pc = p.pc;
    a.unsafe_q = unsafe;
    a.unsafe_k = unsafe + (size_t)p.BH * p.tiles;
    a.out = out;
    a.mask = mask;
    a.row_count = row_count;
    a.row_kl = row_kl;
    a.row_kl_lowp = row_kl_lowp;
    a.ymix_raw = ymix_raw;
    a.yref_out = yref_out;
    a.row_m = row_m;
    a.row_l = row_l;
    a.exact_tiles = exact_tiles;
    const uint64_t grid = (uint64_t)p.BH * p.tiles;
    if (fast) {
        if (p.mu > 10)
            return hipSuccess;
        if (a.Dv <= 64)
            hipLaunchKernelGGL((relaxed_kernel<4, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((relaxed_kernel<8, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    if (a.Dv <= 64)
        hipLaunchKernelGGL((relaxed_kernel<4, false>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((relaxed_kernel<8, false>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// probs of the relaxed path from its raw y^mix and final row statistics.
__global__ __launch_bounds__(kThreads) void normalise_kernel(const float *ymix, const float *row_m,
                                                             const double *row_l, float *probs,
                                                             int S, int causal)
{
    const uint64_t r = blockIdx.x;
    const int i = (int)(r % (uint64_t)S);
    const int n = causal ? i + 1 : S;
    const float m = row_m[r];
    const double inv = 1.0 / row_l[r];
    const float *y = ymix + r * (uint64_t)S;
    float *pr = probs + r * (uint64_t)S;
    for (int j = threadIdx.x; j < S; j += kThreads)
        pr[j] = j < n ? (float)(exp((double)y[j] - (double)m) * inv) : 0.0f;
}

hipError_t launch_normalise(const Problem &p, const float *ymix, const float *row_m,
                            const double *row_l, float *probs, hipStream_t st)
{
    hipLaunchKernelGGL(normalise_kernel, dim3((unsigned)p.n_rows), dim3(kThreads), 0, st, ymix,
                       row_m, row_l, probs, p.S, p.causal);
    return hipGetLastError();
}

}  // namespace lamp
