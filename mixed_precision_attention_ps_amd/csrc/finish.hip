// finish.hip -- final softmax over the mixed scores, P.V on MFMA (FP64
// accumulation), row-wise
// KL(P_FP32 || P_LAMP), and the row reductions into the summary.
//
// "Implementation strategy" step 3 of the LAMP summary ends with "then apply
// f": here f is the attention softmax followed by P.V.  The KL against the
// uniform FP32 reference is the accuracy measure of "Experimental results",
// taken per attention row in the log-sum-exp form
//   KL_i = sum_j p_ref_j (y_ref_j - y_mix_j) + lse(y_mix) - lse(y_ref).
#include "lamp_device.h"

namespace lamp {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kFinRows = 64;   // query rows per work-group (16 per wave)

struct FinishArgs {
    const float *ymix, *v;
    const RowStats *rs;
    float *probs, *out;
    double *row_kl;
    int S, D, causal, blocks_per_head;
};

// probs_j = exp(y^mix_j - lse_mix) on the valid keys (0 elsewhere), and
// out = P.V.  P.V runs on the FP32 MFMA (v_mfma_f32_16x16x4f32) into a
// partial sum that is flushed into a double accumulator every 16 keys: one
// partial carries at most 4 FP32 roundings (relative 2.4e-7 of its
// sum_j p_j |v_jd|), so the total stays inside the 1e-6 bar, whereas FP32
// accumulation over hundreds of keys drifts by ~10 ulp of a dominant term.
// Each KS-key step: thread (row tid/4, keys KS/4 * (tid%4)..) forms KS/4
// probabilities; the P and V tiles go to double-buffered LDS (one barrier per
// step) while the next step's scores and V rows are already being loaded;
// wave w multiplies rows 16w..16w+15 of P by V.  DV = 16 NB is the padded
// head dimension (compile-time, so every MFMA and LDS index is static).
// PIN: `ymix` already holds the probabilities (P.V only: no lse, no probs
// write).
template <int NB, int KS, bool PIN>
__global__ __launch_bounds__(kThreads) void finish_kernel(FinishArgs a)
{
    constexpr int kFinKeys = KS;          // keys per step
    constexpr int kFinPP = KS + 4;        // P tile row pitch (2-way LDS reads)
    constexpr int KPT = KS / 4;           // keys per thread per step
    constexpr int DV = 16 * NB;
    constexpr int VP = DV + 16;                  // V tile row pitch (2-way LDS reads)
    constexpr int NV4 = kFinKeys * DV / 4;             // float4 in a V tile
    constexpr int V4 = (NV4 + kThreads - 1) / kThreads;   // per thread per step
    __shared__ float sP[2][kFinRows][kFinPP];
    __shared__ float sV[2][kFinKeys][VP];
    __shared__ double s_lse[kFinRows];
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    if (!PIN) {
        exp_table_fill(s_exp);
        __syncthreads();
    }

    const int S = a.S, D = a.D;
    // heaviest row blocks first (causal work grows with the block index), so
    // the light ones fill the tail of the launch
    const int BH = (int)(gridDim.x / a.blocks_per_head);
    const int bh = (int)(blockIdx.x % BH);
    const int row0 = (a.blocks_per_head - 1 - (int)(blockIdx.x / BH)) * kFinRows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // lse of each row; rows flagged by the recompute get a pass over the row.
    for (int rr = 0; rr < (PIN ? 0 : kFinRows / 4); ++rr) {
        const int lr = wave * (kFinRows / 4) + rr;
        const int i = row0 + lr;
        double lse = 0.0;
        if (i < S) {
            const uint64_t r = (uint64_t)bh * S + i;
            const RowStats st = a.rs[r];
            lse = st.lse_mix;
            if (st.full_pass) {
                const int n = a.causal ? i + 1 : S;
                const float *ym = a.ymix + r * (uint64_t)S;
                float mm = -INFINITY;
                for (int j = lane; j < n; j += 64)
                    mm = fmaxf(mm, ym[j]);
                mm = wave_max(mm);
                double l = 0.0;
                for (int j = lane; j < n; j += 64)
                    l += exp64((double)ym[j] - (double)mm, s_exp);
                l = wave_sum(l);
                lse = (double)mm + log(l);
                if (lane == 0 && a.row_kl)
                    a.row_kl[r] = st.A / st.L_ref + lse - ((double)st.m_ref + log(st.L_ref));
            }
        }
        if (lane == 0)
            s_lse[lr] = lse;
    }
    __syncthreads();

    const int prow = tid >> 2, kseg = (tid & 3) * KPT;
    const int ip = row0 + prow;
    const bool prow_ok = ip < S;
    const int np = prow_ok ? (a.causal ? ip + 1 : S) : 0;
    const uint64_t rp = (uint64_t)bh * S + (prow_ok ? ip : 0);
    const float *ymp = a.ymix + rp * (uint64_t)S;
    float *prp = (!PIN && a.probs) ? a.probs + rp * (uint64_t)S : nullptr;
    const double lse_p = PIN ? 0.0 : s_lse[prow];
    const bool vec = (S & 3) == 0;
    const int nkeys = a.causal ? min(S, row0 + kFinRows) : S;   // keys the block attends
    const int nsteps = (nkeys + kFinKeys - 1) / kFinKeys;
    const float *Vh = a.v + (size_t)bh * S * D;

    auto load_scores = [&](int j0, float (&y)[KPT]) {
        const int jb = j0 + kseg;
        if (vec) {
#pragma unroll
            for (int e = 0; e < KPT; e += 4) {
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (jb + e < np)   // a float4 never crosses S (S % 4 == 0)
                    x = *reinterpret_cast<const float4 *>(ymp + jb + e);
                y[e] = x.x;
                y[e + 1] = x.y;
                y[e + 2] = x.z;
                y[e + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                y[e] = (jb + e < np) ? ymp[jb + e] : 0.0f;
        }
    };
    auto load_v = [&](int j0, float4 (&vv)[V4]) {
#pragma unroll
        for (int u = 0; u < V4; ++u) {
            const int e = tid + u * kThreads;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < NV4 && j0 + key < S && col < D)
                x = *reinterpret_cast<const float4 *>(Vh + (size_t)(j0 + key) * D + col);
            vv[u] = x;
        }
    };

    double acc[NB][4];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[q][v] = 0.0;
    float ycur[KPT], ynext[KPT];
    float4 vcur[V4], vnext[V4];
    if (nsteps > 0) {
        load_scores(0, ycur);
        load_v(0, vcur);
    }
    for (int s = 0; s < nsteps; ++s) {
        const int j0 = s * kFinKeys;
        const int buf = s & 1;
        if (s + 1 < nsteps) {
            load_scores(j0 + kFinKeys, ynext);
            load_v(j0 + kFinKeys, vnext);
        }
        float pv[KPT];
        const int jb = j0 + kseg;
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            pv[e] = (jb + e < np) ? (PIN ? ycur[e] : exp_f32((double)ycur[e] - lse_p)) : 0.0f;
        if (prp && prow_ok) {
            if (vec) {
#pragma unroll
                for (int e = 0; e < KPT; e += 4)
                    if (jb + e < S)
                        *reinterpret_cast<float4 *>(prp + jb + e) =
                            make_float4(pv[e], pv[e + 1], pv[e + 2], pv[e + 3]);
            } else {
                for (int e = 0; e < KPT; ++e)
                    if (jb + e < S)
                        prp[jb + e] = pv[e];
            }
        }
#pragma unroll
        for (int e = 0; e < KPT; e += 4)
            *reinterpret_cast<float4 *>(&sP[buf][prow][kseg + e]) =
                make_float4(pv[e], pv[e + 1], pv[e + 2], pv[e + 3]);
#pragma unroll
        for (int u = 0; u < V4; ++u) {
            const int e = tid + u * kThreads;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            if (e < NV4)
                *reinterpret_cast<float4 *>(&sV[buf][key][col]) = vcur[u];
        }
        __syncthreads();
#pragma unroll
        for (int k16 = 0; k16 < kFinKeys / 16; ++k16) {
            floatx4 part[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q)
                part[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int kk = k16 * 4 + k4;
                const float av = sP[buf][wave * 16 + (lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    const float bv = sV[buf][kk * 4 + (lane >> 4)][q * 16 + (lane & 15)];
                    part[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, part[q], 0, 0, 0);
                }
            }
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[q][v] += (double)part[q][v];
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            ycur[e] = ynext[e];
#pragma unroll
        for (int u = 0; u < V4; ++u)
            vcur[u] = vnext[u];
    }

    // Keys past the causal limit of every row in the block: probabilities 0.
    // Wave w clears rows 16w..16w+15, each row's tail in contiguous 1 KB
    // stores (64 lanes x 16 bytes).
    if (!PIN && a.probs) {
        const int z0 = nsteps * kFinKeys;
        for (int rr = 0; rr < kFinRows / 4; ++rr) {
            const int iz = row0 + wave * (kFinRows / 4) + rr;
            if (iz >= S)
                break;
            float *pz = a.probs + ((uint64_t)bh * S + iz) * (uint64_t)S;
            if (vec) {
                for (int j = z0 + lane * 4; j < S; j += 256)
                    *reinterpret_cast<float4 *>(pz + j) = make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                for (int j = z0 + lane; j < S; j += 64)
                    pz[j] = 0.0f;
            }
        }
    }

    // Lane holds rows 16*wave + 4*(lane/16) + v of column 16q + lane%16.
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int col = q * 16 + (lane & 15);
        if (col >= D)
            continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = row0 + wave * 16 + 4 * (lane >> 4) + v;
            if (i < S)
                a.out[((size_t)bh * S + i) * D + col] = (float)acc[q][v];
        }
    }
}

template <bool PIN>
static hipError_t launch_finish_kernel(const FinishArgs &a, const Problem &p, hipStream_t st)
{
    const dim3 grid((unsigned)((uint64_t)p.BH * a.blocks_per_head)), block(kThreads);
    switch ((p.D + 15) / 16) {
    case 1: hipLaunchKernelGGL((finish_kernel<1, 32, PIN>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((finish_kernel<2, 32, PIN>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((finish_kernel<3, 32, PIN>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((finish_kernel<4, 32, PIN>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((finish_kernel<5, 32, PIN>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((finish_kernel<6, 32, PIN>), grid, block, 0, st, a); break;
    case 7: hipLaunchKernelGGL((finish_kernel<7, 32, PIN>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((finish_kernel<8, 32, PIN>), grid, block, 0, st, a); break;
    case 9: case 10: case 11: case 12:
        hipLaunchKernelGGL((finish_kernel<12, 16, PIN>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((finish_kernel<16, 16, PIN>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_finish(const Problem &p, const float *ymix, const RowStats *rs, float *probs,
                         float *out, double *row_kl, hipStream_t st)
{
    FinishArgs a;
    a.ymix = ymix;
    a.v = p.v;
    a.rs = rs;
    a.probs = probs;
    a.out = out;
    a.row_kl = row_kl;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.blocks_per_head = (p.S + kFinRows - 1) / kFinRows;
    return launch_finish_kernel<false>(a, p, st);
}

hipError_t launch_pv(const Problem &p, const float *probs, float *out, hipStream_t st)
{
    FinishArgs a;
    a.ymix = probs;
    a.v = p.v;
    a.rs = nullptr;
    a.probs = nullptr;
    a.out = out;
    a.row_kl = nullptr;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.blocks_per_head = (p.S + kFinRows - 1) / kFinRows;
    return launch_finish_kernel<true>(a, p, st);
}

// ---------------------------------------------------------------------------
// Row reductions into the device summary (one work-group, fixed order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void stats_kernel(const double *row_kl, const double *row_kl_lowp,
                                                     const uint32_t *row_count, uint64_t n_rows,
                                                     DevStats *ds)
{
    __shared__ double s_sum[1024], s_max[1024], s_low[1024];
    __shared__ unsigned long long s_cnt[1024];
    const int tid = threadIdx.x;
    double sum = 0.0, mx = -INFINITY, low = 0.0;
    unsigned long long cnt = 0;
    for (uint64_t r = tid; r < n_rows; r += 1024) {
        if (row_kl) {
            sum += row_kl[r];
            mx = fmax(mx, row_kl[r]);
        }
        if (row_kl_lowp)
            low += row_kl_lowp[r];
        if (row_count)
            cnt += row_count[r];
    }
    s_sum[tid] = sum;
    s_max[tid] = mx;
    s_low[tid] = low;
    s_cnt[tid] = cnt;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (tid < o) {
            s_sum[tid] += s_sum[tid + o];
            s_max[tid] = fmax(s_max[tid], s_max[tid + o]);
            s_low[tid] += s_low[tid + o];
            s_cnt[tid] += s_cnt[tid + o];
        }
        __syncthreads();
    }
    if (tid == 0) {
        ds->kl_sum = s_sum[0];
        ds->kl_max = row_kl ? s_max[0] : 0.0;
        ds->kl_lowp_sum = s_low[0];
        ds->n_selected = s_cnt[0];
    }
}

hipError_t launch_stats(const Problem &p, const double *row_kl, const double *row_kl_lowp,
                        const uint32_t *row_count, DevStats *ds, hipStream_t st)
{
    hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(1024), 0, st, row_kl, row_kl_lowp, row_count,
                       p.n_rows, ds);
    return hipGetLastError();
}

// Zero fill with plain vector stores (no memset nodes in captured graphs).
__global__ void zero_kernel(uint32_t *p, size_t n)
{
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x)
        p[e] = 0u;
}

hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t st)
{
    const size_t n = bytes / 4;
    const size_t blocks = (n + kThreads - 1) / kThreads;
    const unsigned grid = (unsigned)(blocks < 65536 ? (blocks ? blocks : 1) : 65536);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(kThreads), 0, st, (uint32_t *)ptr, n);
    return hipGetLastError();
}

}  // namespace lamp

// ---------------------------------------------------------------------------
// Diagnostic: the device exponentials on caller data (accuracy tests).
// ---------------------------------------------------------------------------
namespace lamp {
__global__ void exp_probe_kernel(const double *x, double *y64, float *y32, int n)
{
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    exp_table_fill(s_exp);
    __syncthreads();
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) {
        y64[e] = exp64(x[e], s_exp);
        y32[e] = exp_f32(x[e]);
    }
}
}  // namespace lamp

extern "C" int lamp_diag_exp(const double *x, double *y64, float *y32, int n, void *stream)
{
    if (!x || !y64 || !y32 || n < 0)
        return -1;
    if (n == 0)
        return 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(lamp::exp_probe_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       (hipStream_t)stream, x, y64, y32, n);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
