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
    double *row_kl_lowp;
    int count_only;
};

// One wave per row; 4 rows per work-group.
__global__ __launch_bounds__(kThreads) void strict_select_kernel(SelectArgs a)
{
    const int lane = threadIdx.x & 63;
    const uint64_t r = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.n_rows)
        return;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const float *y = a.y + r * (uint64_t)S;
    const bool want_lowp = a.row_kl_lowp != nullptr && a.yref != nullptr;
    const float *yr = want_lowp ? a.yref + r * (uint64_t)S : nullptr;

    // Row maximum (and the reference row's, for KL(P_ref || P_lowp)).
    float m = -INFINITY, mr = -INFINITY;
    for (int j = lane; j < n; j += 64) {
        m = fmaxf(m, y[j]);
        if (want_lowp)
            mr = fmaxf(mr, yr[j]);
    }
    m = wave_max(m);
    if (want_lowp)
        mr = wave_max(mr);

    // A = sum of exp(y - m) below the maximum; cnt = keys at the maximum.
    double A = 0.0, Lr = 0.0, Br = 0.0;
    int cnt = 0;
    for (int j = lane; j < n; j += 64) {
        const float v = y[j];
        if (v == m)
            cnt++;
        else
            A += exp((double)v - (double)m);
        if (want_lowp) {
            const double er = exp((double)yr[j] - (double)mr);
            Lr += er;
            Br += er * ((double)yr[j] - (double)v);
        }
    }
    A = wave_sum(A);
    cnt = wave_sum_int(cnt);
    const double L = A + (double)cnt;
    const double rest_at_max = A + (double)(cnt - 1);
    if (want_lowp) {
        Lr = wave_sum(Lr);
        Br = wave_sum(Br);
        if (lane == 0)
            a.row_kl_lowp[r] = Br / Lr + ((double)m + log(L)) - ((double)mr + log(Lr));
    }

    // Criterion, mask words and compaction into this row's list segment.
    const uint64_t seg = row_segment(r, S, a.causal);
    uint32_t total = 0;
    const int jend = a.count_only ? n : S;
    for (int j0 = 0; j0 < jend; j0 += 64) {
        const int j = j0 + lane;
        bool sel = false;
        if (j < n) {
            const float v = y[j];
            double e, omz;
            if (v == m) {
                e = 1.0;
                omz = rest_at_max / L;
            } else {
                e = exp((double)v - (double)m);
                omz = (L - e) / L;
            }
            const double c = 2.0 * (e / L) * omz * fabs((double)v);
            sel = c > a.tau;
        }
        const uint64_t b = __ballot(sel);
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
    }
    if (lane == 0)
        a.row_count[r] = total;
}

hipError_t launch_strict_select(const Problem &p, const float *ylo, const float *yref,
                                uint32_t *mask, uint32_t *list, uint32_t *row_count,
                                double *row_kl_lowp, int count_only, hipStream_t st)
{
    SelectArgs a;
    a.y = ylo;
    a.yref = yref;
    a.S = p.S;
    a.causal = p.causal;
    a.W = (p.S + 31) / 32;
    a.n_rows = p.n_rows;
    a.tau = (double)p.tau;
    a.mask = mask;
    a.list = list;
    a.row_count = row_count;
    a.row_kl_lowp = row_kl_lowp;
    a.count_only = count_only;
    const uint64_t grid = (p.n_rows + 3) / 4;
    hipLaunchKernelGGL(strict_select_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Random control: per row, the k = row_count[r] valid keys with the smallest
// (SplitMix64(seed ^ linear index), j).  One work-group per row: an 8-pass
// radix select over the 64-bit hashes finds the k-th smallest value T; keys
// with hash < T are selected, and keys equal to T by increasing j until k.
// ---------------------------------------------------------------------------
struct RandomArgs {
    int S, causal, W;
    uint64_t n_rows, seed;
    uint32_t *mask, *list;
    const uint32_t *row_count;
};

__global__ __launch_bounds__(kThreads) void random_select_kernel(RandomArgs a)
{
    __shared__ uint32_t hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ uint32_t s_rank;
    __shared__ uint32_t s_eqw[4], s_selw[4];
    __shared__ uint32_t s_eq_before, s_sel_before;
    const uint64_t r = blockIdx.x;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const uint32_t k = a.row_count[r];
    const uint64_t base = r * (uint64_t)S;     // linear index of score (b, h, i, 0)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Radix select of the k-th smallest hash T (8 digits of 8 bits, MSB first);
    // `rank` ends as the number of keys equal to T that are taken.
    uint64_t prefix = 0, pmask = 0;
    uint32_t rank = k;
    if (k > 0) {
        for (int shift = 56; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            for (int j = tid; j < n; j += kThreads) {
                const uint64_t h = splitmix64(a.seed ^ (base + (uint64_t)j));
                if ((h & pmask) == prefix)
                    atomicAdd(&hist[(uint32_t)(h >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t cum = 0;
                int d = 0;
                for (; d < 255; ++d) {
                    if (cum + hist[d] >= rank)
                        break;
                    cum += hist[d];
                }
                s_prefix = prefix | ((uint64_t)d << shift);
                s_rank = rank - cum;
            }
            __syncthreads();
            prefix = s_prefix;
            rank = s_rank;
            pmask |= 255ull << shift;
        }
    }
    const uint64_t T = prefix;

    if (tid == 0) {
        s_eq_before = 0;
        s_sel_before = 0;
    }
    __syncthreads();
    const uint64_t seg = row_segment(r, S, a.causal);
    for (int j0 = 0; j0 < S; j0 += kThreads) {
        const int j = j0 + tid;
        bool lt = false, eq = false;
        if (k > 0 && j < n) {
            const uint64_t h = splitmix64(a.seed ^ (base + (uint64_t)j));
            lt = h < T;
            eq = h == T;
        }
        const uint64_t tb = __ballot(eq);
        if (lane == 0)
            s_eqw[wave] = (uint32_t)__popcll(tb);
        __syncthreads();
        uint32_t eq_rank = s_eq_before + lanes_below(tb);
        for (int w = 0; w < wave; ++w)
            eq_rank += s_eqw[w];
        const bool sel = lt || (eq && eq_rank < rank);
        const uint64_t b = __ballot(sel);
        const int w32 = (j0 + wave * 64) >> 5;
        if (a.mask && lane == 0 && w32 < a.W)
            a.mask[r * (uint64_t)a.W + w32] = (uint32_t)b;
        if (a.mask && lane == 1 && w32 + 1 < a.W)
            a.mask[r * (uint64_t)a.W + w32 + 1] = (uint32_t)(b >> 32);
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
    hipLaunchKernelGGL(random_select_kernel, dim3((unsigned)p.n_rows), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gather FP32 recompute ("Implementation strategy" step 3): one wave per row;
// each lane takes one listed key, forms the sequential FP32 dot of q_i and
// k_j (multiply then add, d ascending, no fused multiply-add), scales it and
// scatters it over the baseline score.
// ---------------------------------------------------------------------------
struct RecomputeArgs {
    const float *q, *k;
    int S, D, causal;
    uint64_t n_rows;
    float s;
    const uint32_t *list, *row_count;
    float *ymix;
};

__global__ __launch_bounds__(kThreads) void recompute_kernel(RecomputeArgs a)
{
    const int lane = threadIdx.x & 63;
    const uint64_t r = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.n_rows)
        return;
    const int i = (int)(r % (uint64_t)a.S);
    const uint32_t n = a.causal ? (uint32_t)i + 1u : (uint32_t)a.S;
    const uint32_t cnt = min(a.row_count[r], n);
    if (cnt == 0)
        return;
    const uint64_t bh = r / (uint64_t)a.S;
    const float *qi = a.q + r * (uint64_t)a.D;
    const float *Kh = a.k + bh * (uint64_t)a.S * a.D;
    const uint64_t seg = row_segment(r, a.S, a.causal);
    for (uint32_t e = lane; e < cnt; e += 64) {
        const uint32_t j = a.list[seg + e];
        if (j >= (uint32_t)a.S)
            continue;
        const float4 *kj = reinterpret_cast<const float4 *>(Kh + (size_t)j * a.D);
        const float4 *q4 = reinterpret_cast<const float4 *>(qi);
        float acc = 0.0f;
        for (int d4 = 0; d4 < a.D / 4; ++d4) {
            const float4 x = q4[d4], y = kj[d4];
            float p0 = x.x * y.x;
            acc = acc + p0;
            float p1 = x.y * y.y;
            acc = acc + p1;
            float p2 = x.z * y.z;
            acc = acc + p2;
            float p3 = x.w * y.w;
            acc = acc + p3;
        }
        a.ymix[r * (uint64_t)a.S + j] = acc * a.s;
    }
}

hipError_t launch_recompute(const Problem &p, const uint32_t *list, const uint32_t *row_count,
                            float *ymix, hipStream_t st)
{
    RecomputeArgs a;
    a.q = p.q;
    a.k = p.k;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.n_rows = p.n_rows;
    a.s = p.pc.s;
    a.list = list;
    a.row_count = row_count;
    a.ymix = ymix;
    const uint64_t grid = (p.n_rows + 3) / 4;
    hipLaunchKernelGGL(recompute_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lamp
