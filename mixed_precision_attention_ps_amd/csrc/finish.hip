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

typedef double doublex4 __attribute__((ext_vector_type(4)));

constexpr int kFinRows = 16;   // query rows per work-group (one MFMA row block)
constexpr int kFinKeys = 64;   // keys per P.V step

struct FinishArgs {
    const float *ymix, *yref, *v;
    float *probs, *out;
    double *row_kl;
    int S, D, Dv, causal, blocks_per_head;
};

__global__ __launch_bounds__(kThreads) void finish_kernel(FinishArgs a)
{
    extern __shared__ float smem[];
    float(*sP)[kFinKeys] = reinterpret_cast<float(*)[kFinKeys]>(smem);   // [16][64]
    float *sV = smem + kFinRows * kFinKeys;                                // [64][<=128]
    __shared__ float s_m[kFinRows];
    __shared__ double s_invl[kFinRows];

    const int S = a.S, D = a.D, Dv = a.Dv;
    const int bh = blockIdx.x / a.blocks_per_head;
    const int row0 = (blockIdx.x % a.blocks_per_head) * kFinRows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Phase 1: per-row statistics of y^mix and y^ref, and the row KL.
    for (int rr = 0; rr < 4; ++rr) {
        const int lr = wave * 4 + rr;
        const int i = row0 + lr;
        if (i >= S) {
            if (lane == 0) {
                s_m[lr] = 0.0f;
                s_invl[lr] = 0.0;
            }
            continue;
        }
        const int n = a.causal ? i + 1 : S;
        const uint64_t r = (uint64_t)bh * S + i;
        const float *ym = a.ymix + r * (uint64_t)S;
        const float *yr = a.yref + r * (uint64_t)S;
        float mm = -INFINITY, mr = -INFINITY;
        for (int j = lane; j < n; j += 64) {
            mm = fmaxf(mm, ym[j]);
            mr = fmaxf(mr, yr[j]);
        }
        mm = wave_max(mm);
        mr = wave_max(mr);
        double lm = 0.0, lref = 0.0, aref = 0.0;
        for (int j = lane; j < n; j += 64) {
            const float xm = ym[j], xr = yr[j];
            lm += exp((double)xm - (double)mm);
            const double er = exp((double)xr - (double)mr);
            lref += er;
            aref += er * ((double)xr - (double)xm);
        }
        lm = wave_sum(lm);
        lref = wave_sum(lref);
        aref = wave_sum(aref);
        if (lane == 0) {
            if (a.row_kl)
                a.row_kl[r] = aref / lref + ((double)mm + log(lm)) - ((double)mr + log(lref));
            s_m[lr] = mm;
            s_invl[lr] = 1.0 / lm;
        }
    }
    __syncthreads();

    // Phase 2: probabilities (written if requested) and P.V on MFMA.
    const int prow = tid >> 4, pk = tid & 15;
    const int ip = row0 + prow;
    const int np = ip < S ? (a.causal ? ip + 1 : S) : 0;
    const uint64_t rp = (uint64_t)bh * S + (ip < S ? ip : 0);
    const float *ymp = a.ymix + rp * (uint64_t)S;
    const float mp = s_m[prow];
    const double invl = s_invl[prow];
    const int nkeys = a.causal ? min(S, row0 + kFinRows) : S;   // keys this block attends
    const int nb = Dv / 16;                                      // 16-wide column blocks
    // P.V accumulates in double on the FP64 MFMA: FP32 accumulation over
    // hundreds of keys drifts by ~10 ulp of a dominant term, beyond 1e-6.
    doublex4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc[q] = doublex4{0.0, 0.0, 0.0, 0.0};
    const size_t vhead = (size_t)bh * S * D;

    for (int j0 = 0; j0 < S; j0 += kFinKeys) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int jj = pk + 16 * c;
            const int j = j0 + jj;
            float pv = 0.0f;
            if (j < np)
                pv = (float)(exp((double)ymp[j] - (double)mp) * invl);
            if (a.probs && ip < S && j < S)
                a.probs[rp * (uint64_t)S + j] = pv;
            sP[prow][jj] = pv;
        }
        if (j0 < nkeys) {
            // V tile in column chunks of at most 128 (LDS: 64 x 128 floats).
            for (int h = 0; h < Dv; h += 128) {
                const int Dc = min(128, Dv - h);
                const int n4 = kFinKeys * Dc / 4;
                __syncthreads();
                for (int e = tid; e < n4; e += kThreads) {
                    const int key = e / (Dc / 4), col = h + (e % (Dc / 4)) * 4;
                    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (j0 + key < S && col < D)
                        x = *reinterpret_cast<const float4 *>(a.v + vhead + (size_t)(j0 + key) * D + col);
                    *reinterpret_cast<float4 *>(sV + key * Dc + (col - h)) = x;
                }
                __syncthreads();
#pragma unroll 4
                for (int kk = 0; kk < kFinKeys / 4; ++kk) {
                    const float av = sP[mfma64_row(lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int cb = wave + 4 * q;
                        if (cb * 16 >= h && cb * 16 < h + Dc) {
                            const float bv = sV[(kk * 4 + (lane >> 4)) * Dc + cb * 16 - h + (lane & 15)];
                            acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av, (double)bv,
                                                                          acc[q], 0, 0, 0);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // MFMA 16x16 result layout: lane holds rows 4*(lane/16)+v, column lane%16.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cb = wave + 4 * q;
        if (cb >= nb)
            continue;
        const int col = cb * 16 + (lane & 15);
        if (col >= D)
            continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = row0 + 4 * (lane >> 4) + v;
            if (i < S)
                a.out[((size_t)bh * S + i) * D + col] = (float)acc[q][v];
        }
    }
}

hipError_t launch_finish(const Problem &p, const float *ymix, const float *yref, float *probs,
                         float *out, double *row_kl, hipStream_t st)
{
    FinishArgs a;
    a.ymix = ymix;
    a.yref = yref;
    a.v = p.v;
    a.probs = probs;
    a.out = out;
    a.row_kl = row_kl;
    a.S = p.S;
    a.D = p.D;
    a.Dv = (p.D + 15) / 16 * 16;
    a.causal = p.causal;
    a.blocks_per_head = (p.S + kFinRows - 1) / kFinRows;
    const size_t shmem = sizeof(float) * (kFinRows * kFinKeys + kFinKeys * min(a.Dv, 128));
    const uint64_t grid = (uint64_t)p.BH * a.blocks_per_head;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)grid), dim3(kThreads), shmem, st, a);
    return hipGetLastError();
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
