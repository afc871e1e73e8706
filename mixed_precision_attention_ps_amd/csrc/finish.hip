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
    int tail_done;   // the zeros past the block's last key are already written
};

// probs_j = exp(y^mix_j - lse_mix) on the valid keys (0 elsewhere), and
// out = P.V.  P.V runs on the FP32 MFMA (v_mfma_f32_16x16x4f32) into a
// partial sum that is flushed into a double accumulator every 16 keys: one
// partial carries at most 4 FP32 roundings (relative 2.4e-7 of its
// sum_j p_j |v_jd|), so the total stays inside the 1e-6 bar, whereas FP32
// accumulation over hundreds of keys drifts by ~10 ulp of a dominant term.
// Each KS-key step: thread (row tid / (4 WS), keys KPT (tid % (4 WS)) ..)
// forms KPT = KS / (4 WS) probabilities; the P and V tiles go to
// double-buffered LDS (one barrier per
// step) while the next step's scores and V rows are already being loaded;
// wave w multiplies rows 16(w%4)..16(w%4)+15 of P by V.  DV = 16 NB is the
// padded head dimension (compile-time, so every MFMA and LDS index is
// static).  WS: the work-group has 4 WS waves, wave w taking the column
// blocks NB/WS * (w/4) .. of its rows (WS = 2 at D = 96 and 128: each wave
// then holds half the P.V accumulators, and twice the waves fit on a SIMD).
template <int NB, int KS, int WS>
__global__ __launch_bounds__(kThreads * WS) void finish_kernel(FinishArgs a)
{
    constexpr int NT = kThreads * WS;      // threads per work-group
    constexpr int NBW = NB / WS;           // MFMA column blocks per wave
    static_assert(NB % WS == 0, "column split");
    constexpr int kFinKeys = KS;          // keys per step
    constexpr int kFinPP = KS + 4;        // P tile row pitch (2-way LDS reads)
    constexpr int TPR = NT / kFinRows;    // threads per P row
    constexpr int KPT = KS / TPR;         // keys per thread per step
    static_assert(KPT % 4 == 0, "float4 P stores");
    constexpr int DV = 16 * NB;
    constexpr int VP = DV + 16;                  // V tile row pitch (2-way LDS reads)
    constexpr int NV4 = kFinKeys * DV / 4;             // float4 in a V tile
    constexpr int V4 = (NV4 + NT - 1) / NT;            // per thread per step
    __shared__ float sP[2][kFinRows][kFinPP];
    __shared__ float sV[2][kFinKeys][VP];
    __shared__ double s_lse[kFinRows];
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    __shared__ int s_vbad;         // a causal diagonal step met a non-finite V value
    exp_table_fill(s_exp);
    if (threadIdx.x == 0)
        s_vbad = 0;
    __syncthreads();

    const int S = a.S, D = a.D;
    // heaviest row blocks first (causal work grows with the block index), so
    // the light ones fill the tail of the launch
    const int BH = (int)(gridDim.x / a.blocks_per_head);
    const int bh = (int)(blockIdx.x % BH);
    const int row0 = (a.blocks_per_head - 1 - (int)(blockIdx.x / BH)) * kFinRows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // row group and first column block (compile-time 0 for WS = 1)
    const int rw = WS == 1 ? wave : (wave & 3), cb0 = WS == 1 ? 0 : (wave >> 2) * NBW;
    constexpr int kRowsPerWave = kFinRows / (4 * WS);

    // lse of each row; rows flagged by the recompute get a pass over the row.
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int lr = wave * kRowsPerWave + rr;
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

    const int prow = tid / TPR, kseg = (tid % TPR) * KPT;
    const int ip = row0 + prow;
    const bool prow_ok = ip < S;
    const int np = prow_ok ? (a.causal ? ip + 1 : S) : 0;
    const uint64_t rp = (uint64_t)bh * S + (prow_ok ? ip : 0);
    const float *ymp = a.ymix + rp * (uint64_t)S;
    float *prp = a.probs ? a.probs + rp * (uint64_t)S : nullptr;
    const double lse_p = s_lse[prow];
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
            const int e = tid + u * NT;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < NV4 && j0 + key < S && col < D)
                x = *reinterpret_cast<const float4 *>(Vh + (size_t)(j0 + key) * D + col);
            vv[u] = x;
        }
    };

    double acc[NBW][4];
#pragma unroll
    for (int q = 0; q < NBW; ++q)
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
        // issue priority: the step's probabilities and staging (exponentials,
        // stores: what the barrier waits on) at 2, its MFMA steps at 0, so
        // that a work-group's barrier is reached sooner on a SIMD shared with
        // others' MFMA work (S = 4096 layer: 1.88 -> 1.82 ms)
        __builtin_amdgcn_s_setprio(2);
        float pv[KPT];
        const int jb = j0 + kseg;
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            pv[e] = (jb + e < np) ? exp_f32((double)ycur[e] - lse_p) : 0.0f;
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
        // Causal steps that reach the block's own rows hold keys past some
        // rows' limits, whose probability 0 would turn a non-finite V value
        // into NaN (0 * inf) in the product: such values are staged as 0 and
        // added back below for the rows that see their key.
        const bool diag = a.causal && j0 + kFinKeys > row0;
#pragma unroll
        for (int u = 0; u < V4; ++u) {
            const int e = tid + u * NT;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            if (e < NV4) {
                float4 x = vcur[u];
                if (diag && !(finite4(x))) {
                    x = finite_or_zero(x);
                    s_vbad = 1;
                }
                *reinterpret_cast<float4 *>(&sV[buf][key][col]) = x;
            }
        }
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int k16 = 0; k16 < kFinKeys / 16; ++k16) {
            floatx4 part[NBW];
#pragma unroll
            for (int q = 0; q < NBW; ++q)
                part[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int kk = k16 * 4 + k4;
                const float av = sP[buf][rw * 16 + (lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const float bv = sV[buf][kk * 4 + (lane >> 4)][(cb0 + q) * 16 + (lane & 15)];
                    part[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, part[q], 0, 0, 0);
                }
            }
#pragma unroll
            for (int q = 0; q < NBW; ++q)
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
    if (a.probs && !a.tail_done) {
        const int z0 = nsteps * kFinKeys;
        for (int rr = 0; rr < kRowsPerWave; ++rr) {
            const int iz = row0 + wave * kRowsPerWave + rr;
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

    // Non-finite V values staged as 0 on the diagonal steps: each one at a
    // key the row sees adds its infinity or NaN (what any positive
    // probability times it gives), keys past the row add nothing.
    if (s_vbad) {
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int col = (cb0 + q) * 16 + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = row0 + rw * 16 + 4 * (lane >> 4) + v;
                if (col < D && i < S)
                    for (int j = row0; j <= i; ++j) {
                        const float x = Vh[(size_t)j * D + col];
                        if (!isfinite(x))
                            acc[q][v] += (double)x;
                    }
            }
        }
    }

    // Lane holds rows 16 (wave % 4) + 4 (lane / 16) + v of column
    // 16 (cb0 + q) + lane % 16.
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int col = (cb0 + q) * 16 + (lane & 15);
        if (col >= D)
            continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = row0 + rw * 16 + 4 * (lane >> 4) + v;
            if (i < S)
                a.out[((size_t)bh * S + i) * D + col] = (float)acc[q][v];
        }
    }
}

static hipError_t launch_finish_kernel(const FinishArgs &a, const Problem &p, hipStream_t st)
{
    const dim3 grid((unsigned)((uint64_t)p.BH * a.blocks_per_head)), block(kThreads);
    const dim3 block2(2 * kThreads);
    switch ((p.D + 15) / 16) {
    case 1: hipLaunchKernelGGL((finish_kernel<1, 32, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((finish_kernel<2, 32, 1>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((finish_kernel<3, 32, 1>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((finish_kernel<4, 32, 1>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((finish_kernel<5, 32, 1>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((finish_kernel<6, 32, 2>), grid, block2, 0, st, a); break;
    case 7: hipLaunchKernelGGL((finish_kernel<7, 32, 1>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((finish_kernel<8, 32, 2>), grid, block2, 0, st, a); break;
    case 9: case 10: case 11: case 12:
        hipLaunchKernelGGL((finish_kernel<12, 16, 1>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((finish_kernel<16, 16, 1>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_finish(const Problem &p, const float *ymix, const RowStats *rs, float *probs,
                         float *out, double *row_kl, hipStream_t st, bool tail_done)
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
    // (the tail starts at the block's last row + 1 rounded up to a key step,
    // which is the next 64-key block: the score tiles' mirrored zero tiles)
    a.tail_done = tail_done && p.causal && kFinRows == kTile ? 1 : 0;
    return launch_finish_kernel(a, p, st);
}


// ---------------------------------------------------------------------------
// Row reductions into the device summary, in a fixed order: work-group b
// reduces rows [b c, (b + 1) c) (c = ceil(n_rows / work-groups)) into its
// partial; the last work-group to finish (a completion count in the zeroed
// summary) combines the partials in work-group order.
// ---------------------------------------------------------------------------
constexpr int kStatsThreads = 512;

struct StatsAcc {
    double sum, max, low;
    unsigned long long cnt;
};

__device__ __forceinline__ void stats_combine(StatsAcc &a, const StatsAcc &b)
{
    a.sum += b.sum;
    a.max = fmax(a.max, b.max);
    a.low += b.low;
    a.cnt += b.cnt;
}

// Tree over the work-group's threads (fixed order); thread 0 gets the total.
__device__ StatsAcc stats_block_reduce(StatsAcc v, StatsAcc *sh)
{
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int o = kStatsThreads / 2; o > 0; o >>= 1) {
        if (tid < o) {
            StatsAcc a = sh[tid];
            stats_combine(a, sh[tid + o]);
            sh[tid] = a;
        }
        __syncthreads();
    }
    return sh[0];
}

__global__ __launch_bounds__(kStatsThreads) void stats_kernel(const double *row_kl,
                                                              const double *row_kl_lowp,
                                                              const uint32_t *row_count,
                                                              uint64_t n_rows, DevStats *ds)
{
    __shared__ StatsAcc sh[kStatsThreads];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const uint64_t per = (n_rows + gridDim.x - 1) / gridDim.x;
    const uint64_t r0 = per * blockIdx.x;
    const uint64_t r1 = min(n_rows, r0 + per);
    StatsAcc v{0.0, -INFINITY, 0.0, 0ull};
    for (uint64_t r = r0 + tid; r < r1; r += kStatsThreads) {
        if (row_kl) {
            const double x = row_kl[r];
            v.sum += x;
            v.max = fmax(v.max, x);
        }
        if (row_kl_lowp)
            v.low += row_kl_lowp[r];
        if (row_count)
            v.cnt += row_count[r];
    }
    const StatsAcc b = stats_block_reduce(v, sh);
    if (tid == 0) {
        StatsPart &pt = ds->part[blockIdx.x];
        pt.sum = b.sum;
        pt.max = b.max;
        pt.low = b.low;
        pt.cnt = b.cnt;
        __threadfence();   // the partial is visible before the count says so
        s_last = atomicAdd(&ds->blocks_done, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    // the other work-groups' partials, read past this CU's cache
    StatsAcc t{0.0, -INFINITY, 0.0, 0ull};
    if (tid < (int)gridDim.x) {
        const volatile StatsPart &pt = ds->part[tid];
        t.sum = pt.sum;
        t.max = pt.max;
        t.low = pt.low;
        t.cnt = pt.cnt;
    }
    const StatsAcc total = stats_block_reduce(t, sh);
    if (tid == 0) {
        ds->kl_sum = total.sum;
        ds->kl_max = row_kl ? total.max : 0.0;
        ds->kl_lowp_sum = total.low;
        ds->n_selected = total.cnt;
    }
}

hipError_t launch_stats(const Problem &p, const double *row_kl, const double *row_kl_lowp,
                        const uint32_t *row_count, DevStats *ds, hipStream_t st)
{
    static_assert(kStatsBlocks <= kStatsThreads, "one partial per thread in the last step");
    // about 1024 rows per work-group at least
    const uint64_t want = (p.n_rows + 1023) / 1024;
    const unsigned grid = (unsigned)(want < 1 ? 1 : (want < kStatsBlocks ? want : kStatsBlocks));
    hipLaunchKernelGGL(stats_kernel, dim3(grid), dim3(kStatsThreads), 0, st, row_kl, row_kl_lowp,
                       row_count, p.n_rows, ds);
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
