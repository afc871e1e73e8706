// mlp.hip -- LAMP at the pages' two other closed forms, after a matrix
// product y = x W^T accumulated in PS(mu): an activation function (GELU) and
// layer normalisation.
//
// LAMP summary, "Theoretical foundation" item 3 (an activation function's
// Jacobian is diagonal, so its sensitive components are read off one by one;
// for layer normalisation a nearly sparsest selection follows greedily from
// the input magnitudes sorted) and "Implementation strategy" steps 1-3.  The
// formulas are readings (the pages give neither):
//   * GELU, tanh form; recompute y_j iff |GELU'(y_j) y_j| > tau (the l1
//     change of the output per unit relative change of y_j, as in the softmax
//     rule), evaluated in double at the low-precision y_j.
//   * LayerNorm; recompute the largest |y_j| (ties to the lower index) until
//     the rest has ||y_U||_2 <= tau sigma sqrt(n), sigma^2 = var + eps of the
//     low-precision row.
//
// Kernels:
//   * gemm_scan_kernel: per 64-row block of x or W, whether every value lies
//     in the fast path's operand range (many work-groups per block).
//   * ps_gemm_kernel<FAST, EPI>: one work-group per 64x64 tile of y, the
//     score-tile machinery of the attention path with x as the query rows and
//     W as the keys (K = the head dimension), no scale.  EPI_STORE writes
//     y^lo and y^ref; EPI_GELU applies the GELU rule in the epilogue (the
//     tile's FP32 reference is the recompute, bit for bit), writes GELU(y^mix),
//     the mask words, per-(row, tile) l1 error partials and, when asked for,
//     y^mix and y^ref.
//   * ln_lamp_kernel: one work-group per row: statistics of y^lo, a bitonic
//     sort of (magnitude, index) keys in LDS, the suffix sums of squares over
//     the sorted order, the recompute count k*, then LN(y^mix), the mask, the
//     count and the l2 errors.
//   * row_reduce_kernel: the GELU error partials per row.
//   * ps_gemm_narrow_kernel: the fast path on 32 x 32 tiles, for products
//     whose 64 x 64 tiles would load the CUs unevenly.
#include "lamp_device.h"

namespace lamp {

// ---------------------------------------------------------------------------
// Operand range scan of one matrix: flags[b] != 0 when 64-row block b holds a
// value outside {0} U [2^-40, 2^40] (or a non-finite one).  A 64-row block is
// one contiguous span of 64 K floats; grid.y splits it into kScanSpan-float
// pieces so that the scan of a long-K operand still fills the GPU.  The flags
// are cleared before the launch; a work-group that finds an unsafe value
// sets its block's flag (a rare event: one atomic per such work-group).
// ---------------------------------------------------------------------------
constexpr int kScanSpan = 16384;                        // floats per work-group
constexpr int kScanV4 = kScanSpan / (4 * kThreads);     // float4 loads per thread

__device__ __forceinline__ bool mlp_safe(float x)
{
    const uint32_t m = __float_as_uint(x) & 0x7fffffffu;
    return m == 0u || (m - 0x2b800000u) <= (0x53800000u - 0x2b800000u);
}

__global__ __launch_bounds__(kThreads) void gemm_scan_kernel(const float *a, int rows, int K,
                                                             uint32_t *flags)
{
    const int b = blockIdx.x;
    const int r0 = b * kTile, r1 = min(rows, r0 + kTile);
    const size_t n4 = (size_t)(r1 - r0) * K / 4;   // K % 4 == 0
    const float4 *p = reinterpret_cast<const float4 *>(a + (size_t)r0 * K);
    const size_t e0 = (size_t)blockIdx.y * (kScanSpan / 4);
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kScanV4; ++u) {
        const size_t e = e0 + (size_t)u * kThreads + threadIdx.x;
        if (e < n4) {
            const float4 v = p[e];
            ok = ok && mlp_safe(v.x) && mlp_safe(v.y) && mlp_safe(v.z) && mlp_safe(v.w);
        }
    }
    const int any_bad = __syncthreads_or(ok ? 0 : 1);
    if (any_bad && threadIdx.x == 0)
        atomicOr(&flags[b], 1u);
}

// ---------------------------------------------------------------------------
// GELU (tanh form) in double through the logistic function, which has no
// cancellation anywhere: with u = sqrt(2/pi) (y + 0.044715 y^3) and
// s = 1 / (1 + exp(-2u)) (so that (1 + tanh u) / 2 = s),
//   GELU(y)  = y s,
//   GELU'(y) = s + 2 y s (1 - s) u',  u' = sqrt(2/pi) (1 + 3 * 0.044715 y^2).
// ---------------------------------------------------------------------------
struct Gelu {
    double g, dg;
};

__device__ __forceinline__ Gelu gelu64(double y, const double *s_exp)
{
    const double a = 0.7978845608028654, b = 0.044715;
    const double u = a * (y + b * y * y * y);
    const double e = exp64(-2.0 * u, s_exp);   // +inf for very negative u
    const double s = 1.0 / (1.0 + e);          // 0 when e is +inf
    const double one_minus_s = e < 1e300 ? e * s : 1.0;
    const double du = a * (1.0 + 3.0 * b * y * y);
    Gelu r;
    r.g = y * s;
    r.dg = s + 2.0 * y * s * one_minus_s * du;
    return r;
}

enum { EPI_STORE = 0, EPI_GELU = 1 };

struct GemmArgs {
    const float *x, *w;          // x [M, K], w [N, K]
    int M, N, K, tiles_n, W;
    PsConst pc;                  // s = 1
    const uint32_t *unsafe_x, *unsafe_w;
    float *ylo, *yref;           // [M, N] or null
    float *out;                  // [M, N] (GELU)
    uint32_t *mask;              // [M, W] or null (GELU)
    double *err_part, *errl_part;   // [M, W]: per (row, 32-column block) (GELU)
    double tau;
    unsigned long long *exact_tiles;
    long long n_tiles;
    unsigned long long *n_band;   // near ties of the GELU criterion
};

template <int PATH, int EPI, int P>
__device__ __forceinline__ void gemm_tile(TileSmem &sm, const double *s_exp, const GemmArgs &a,
                                          int ti, int tj)
{
    TileAcc acc;
    score_tile<PATH, P, true>(sm, acc, a.x, a.w, ti * kTile, tj * kTile, a.M, a.N, a.K, a.pc);
    float lo[4][4], ref[4][4];
    tile_scores<PATH, P>(acc, a.pc, lo, ref);
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4, lane = tid & 63;
    uint32_t ties = 0;   // this thread's near ties of the GELU criterion
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = ti * kTile + ty * 4 + r;
        bool valid[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            valid[c] = i < a.M && tj * kTile + tx + 16 * c < a.N;
        const size_t rowoff = (size_t)(i < a.M ? i : 0) * a.N;
        if (EPI == EPI_STORE && (a.ylo || a.yref)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = tj * kTile + tx + 16 * c;
                if (!valid[c])
                    continue;
                if (a.ylo)
                    a.ylo[rowoff + j] = lo[r][c];
                if (a.yref)
                    a.yref[rowoff + j] = ref[r][c];
            }
        }
        if (EPI == EPI_GELU) {
            double el0 = 0.0, em0 = 0.0, el1 = 0.0, em1 = 0.0;
            bool sel[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = tj * kTile + tx + 16 * c;
                const Gelu gl = gelu64((double)lo[r][c], s_exp);
                const double crit = fabs(gl.dg * (double)lo[r][c]);
                sel[c] = valid[c] && crit > a.tau;
                ties += (valid[c] && near_tie(crit, a.tau)) ? 1u : 0u;
                const Gelu gr = gelu64((double)ref[r][c], s_exp);
                const double gm = sel[c] ? gr.g : gl.g;
                if (valid[c]) {
                    a.out[rowoff + j] = (float)gm;
                    if (a.ylo)   // y^mix
                        a.ylo[rowoff + j] = sel[c] ? ref[r][c] : lo[r][c];
                    if (a.yref)
                        a.yref[rowoff + j] = ref[r][c];
                    const double dm = fabs(gm - gr.g), dl = fabs(gl.g - gr.g);
                    em0 += c < 2 ? dm : 0.0;
                    el0 += c < 2 ? dl : 0.0;
                    em1 += c < 2 ? 0.0 : dm;
                    el1 += c < 2 ? 0.0 : dl;
                }
            }
            // mask words: key tx + 16 c of this row group is bit (tx + 16 c) % 32
            // of word 2 tj + c / 2; lanes 16 (lane / 16) .. + 15 hold the row
            const int gsh = lane & 48;
            uint32_t bits[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bits[c] = (uint32_t)(ballot(sel[c]) >> gsh) & 0xffffu;
            // partials per 32-column block: keys tx, tx + 16 | tx + 32, tx + 48
            em0 = group16_sum(em0);
            el0 = group16_sum(el0);
            em1 = group16_sum(em1);
            el1 = group16_sum(el1);
            if (i < a.M && tx == 0) {
                if (a.mask) {
                    const uint32_t w0 = bits[0] | (bits[1] << 16), w1 = bits[2] | (bits[3] << 16);
                    if (2 * tj < a.W)
                        a.mask[(size_t)i * a.W + 2 * tj] = w0;
                    if (2 * tj + 1 < a.W)
                        a.mask[(size_t)i * a.W + 2 * tj + 1] = w1;
                }
                if (2 * tj < a.W) {
                    a.err_part[(size_t)i * a.W + 2 * tj] = em0;
                    a.errl_part[(size_t)i * a.W + 2 * tj] = el0;
                }
                if (2 * tj + 1 < a.W) {
                    a.err_part[(size_t)i * a.W + 2 * tj + 1] = em1;
                    a.errl_part[(size_t)i * a.W + 2 * tj + 1] = el1;
                }
            }
        }
    }
    if (EPI == EPI_GELU)
        add_ties(a.n_band, (uint32_t)wave_sum_int((int)ties));
}

// FAST: the tiles whose operands allow the FP32 fast path (one work-group per
// tile); otherwise a bounded grid striding over the other tiles (exact double
// path, or plain FP32 at mu = 23), exiting at once when there are none.
// P: the run width of the blocked PS(mu) order (run_width(a.pc.blk)).
template <bool FAST, int EPI, int P>
__global__ __launch_bounds__(kThreads) void ps_gemm_kernel(GemmArgs a)
{
    __shared__ TileSmem sm;
    __shared__ double s_exp[64];
    exp_table_fill(s_exp);
    __syncthreads();
    auto path_of = [&](long long g, int &ti, int &tj) {
        ti = (int)(g / a.tiles_n);
        tj = (int)(g % a.tiles_n);
        if (a.pc.mu == 23)
            return (int)PATH_FP32;
        if (a.pc.mu <= 10 && !a.unsafe_x[ti] && !a.unsafe_w[tj])
            return (int)PATH_FAST;
        return (int)PATH_EXACT;
    };
    if (!FAST) {
        bool need = false;
        for (long long g = blockIdx.x + (long long)threadIdx.x * gridDim.x; g < a.n_tiles;
             g += (long long)blockDim.x * gridDim.x) {
            int ti, tj;
            need |= path_of(g, ti, tj) != PATH_FAST;
        }
        if (!__syncthreads_or(need ? 1 : 0))
            return;
    }
    for (long long g = blockIdx.x; g < a.n_tiles; g += FAST ? a.n_tiles : gridDim.x) {
        int ti, tj;
        const int path = path_of(g, ti, tj);
        if (FAST) {
            if (path == PATH_FAST)
                gemm_tile<PATH_FAST, EPI, P>(sm, s_exp, a, ti, tj);
        } else if (path == PATH_EXACT) {
            if (threadIdx.x == 0 && a.exact_tiles)
                atomicAdd(a.exact_tiles, 1ull);
            gemm_tile<PATH_EXACT, EPI, P>(sm, s_exp, a, ti, tj);
        } else if (path == PATH_FP32) {
            gemm_tile<PATH_FP32, EPI, P>(sm, s_exp, a, ti, tj);
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow fast-path tiles: 32 x 32 outputs per work-group, 2 x 2 per thread.
//
// A product with few 64 x 64 tiles (the layer-norm shape: 1024 x 1600, 400
// tiles, 1600 waves for 1024 SIMDs) leaves the SIMDs that hold two waves to
// set the time.  A dot cannot be split over K without changing the
// sequential PS(mu) sums, so the finer grain comes from fewer outputs per
// thread: four times the waves, each a quarter of the work.  Same PS(mu)
// multiply-add and the same blocked order as the wide tile; the LDS holds
// [d][row] and [d][slot] slices of 32 rows, key j in slot (j % 16) * 2 + j / 16
// so that a thread reads its two keys as one 8-byte load.  Fast path only:
// a 32 x 32 tile takes the fast path exactly when the 64 x 64 tile holding it
// does (the operand flags are per 64-row block), and those 64 x 64 tiles are
// the generic kernel's.
// ---------------------------------------------------------------------------
constexpr int kNarrow = 32;

struct alignas(16) NarrowSmem {
    float q[kDChunk][kNarrow];
    float qs[kDChunk][kNarrow];
    float k[kDChunk][kNarrow];
};

__device__ __forceinline__ int narrow_slot(int j) { return (j & 15) * 2 + (j >> 4); }

template <int P>
__device__ __forceinline__ void narrow_flush(float (&lo)[2][2], float (&blk)[2][2],
                                             const PsConst &pc)
{
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            lo[r][c] = ps_round_split(lo[r][c] + blk[r][c], pc.split);
            blk[r][c] = 0.0f;
        }
}

template <int EPI, int P>
__global__ __launch_bounds__(kThreads) void ps_gemm_narrow_kernel(GemmArgs a)
{
    __shared__ NarrowSmem sm;
    __shared__ double s_exp[64];
    const int tiles_n32 = (a.N + kNarrow - 1) / kNarrow;
    const int ti = (int)(blockIdx.x / tiles_n32), tj = (int)(blockIdx.x % tiles_n32);
    if (a.unsafe_x[ti >> 1] || a.unsafe_w[tj >> 1])
        return;   // the generic kernel's 64 x 64 tile
    if (EPI == EPI_GELU)
        exp_table_fill(s_exp);
    constexpr bool BLOCKED = P != 0;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4, lane = tid & 63;
    const int row0 = ti * kNarrow, col0 = tj * kNarrow, K = a.K;
    const PsConst pc = a.pc;
    float lo[2][2], ref[2][2], blk[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            lo[r][c] = ref[r][c] = blk[r][c] = 0.0f;
    // one float4 of x and of W per thread and slice: row tid / 8, d (tid % 8) * 4
    const int lrow = tid >> 3, ld = (tid & 7) * 4;
    const float *xb = a.x + (size_t)row0 * K, *wb = a.w + (size_t)col0 * K;
    const int xrows = a.M - row0, wrows = a.N - col0;
    float4 xv = load_slice(xb, lrow, xrows, K, ld);
    float4 wv = load_slice(wb, lrow, wrows, K, ld);
    const int run = P == kDChunk ? pc.blk : K;
    for (int r0 = 0; r0 < K; r0 += run) {
        const int r1 = min(K, r0 + run);
        for (int d0 = r0; d0 < r1; d0 += kDChunk) {
            __syncthreads();
            {
                const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
                const float wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.q[ld + e][lrow] = xa[e];
                    sm.qs[ld + e][lrow] = xa[e] * pc.qscale;
                    sm.k[ld + e][narrow_slot(lrow)] = wa[e];
                }
            }
            __syncthreads();
            progress_priority(d0, K);
            if (d0 + kDChunk < K) {
                xv = load_slice(xb, lrow, xrows, K, d0 + kDChunk + ld);
                wv = load_slice(wb, lrow, wrows, K, d0 + kDChunk + ld);
            }
#pragma unroll
            for (int dd = 0; dd < kDChunk; ++dd) {
                const float2 qv = *reinterpret_cast<const float2 *>(&sm.q[dd][ty * 2]);
                const float2 sv = *reinterpret_cast<const float2 *>(&sm.qs[dd][ty * 2]);
                const float2 kv = *reinterpret_cast<const float2 *>(&sm.k[dd][tx * 2]);
                const float qa[2] = {qv.x, qv.y}, sa[2] = {sv.x, sv.y}, ka[2] = {kv.x, kv.y};
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        ps_mac_fast(qa[r], sa[r], ka[c], BLOCKED ? blk[r][c] : lo[r][c],
                                    ref[r][c], pc.split);
                if (BLOCKED && P < kDChunk && dd % (P ? P : 1) == (P ? P : 1) - 1)
                    narrow_flush<P>(lo, blk, pc);
            }
        }
        if (BLOCKED)
            narrow_flush<P>(lo, blk, pc);
    }

    uint32_t ties = 0;   // this thread's near ties of the GELU criterion
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = row0 + ty * 2 + r;
        const size_t rowoff = (size_t)(i < a.M ? i : 0) * a.N;
        float ylo[2], yref[2];
        bool valid[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            ylo[c] = lo[r][c] * pc.out_scale;
            yref[c] = ref[r][c] * pc.s;
            valid[c] = i < a.M && col0 + tx + 16 * c < a.N;
        }
        if (EPI == EPI_STORE) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (!valid[c])
                    continue;
                const int j = col0 + tx + 16 * c;
                if (a.ylo)
                    a.ylo[rowoff + j] = ylo[c];
                if (a.yref)
                    a.yref[rowoff + j] = yref[c];
            }
        } else {
            double em = 0.0, el = 0.0;
            bool sel[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = col0 + tx + 16 * c;
                const Gelu gl = gelu64((double)ylo[c], s_exp);
                const double crit = fabs(gl.dg * (double)ylo[c]);
                sel[c] = valid[c] && crit > a.tau;
                ties += (valid[c] && near_tie(crit, a.tau)) ? 1u : 0u;
                const Gelu gr = gelu64((double)yref[c], s_exp);
                const double gm = sel[c] ? gr.g : gl.g;
                if (valid[c]) {
                    a.out[rowoff + j] = (float)gm;
                    if (a.ylo)   // y^mix
                        a.ylo[rowoff + j] = sel[c] ? yref[c] : ylo[c];
                    if (a.yref)
                        a.yref[rowoff + j] = yref[c];
                    em += fabs(gm - gr.g);
                    el += fabs(gl.g - gr.g);
                }
            }
            // key tx + 16 c is bit tx + 16 c of word tj; lanes 16 (lane / 16)
            // .. + 15 hold row pair ty
            const int gsh = lane & 48;
            const uint32_t b0 = (uint32_t)(ballot(sel[0]) >> gsh) & 0xffffu;
            const uint32_t b1 = (uint32_t)(ballot(sel[1]) >> gsh) & 0xffffu;
            em = group16_sum(em);
            el = group16_sum(el);
            if (i < a.M && tx == 0) {
                if (a.mask)
                    a.mask[(size_t)i * a.W + tj] = b0 | (b1 << 16);
                a.err_part[(size_t)i * a.W + tj] = em;
                a.errl_part[(size_t)i * a.W + tj] = el;
            }
        }
    }
    if (EPI == EPI_GELU)
        add_ties(a.n_band, (uint32_t)wave_sum_int((int)ties));
}

// Per-row sums of the GELU error partials (one per 32-column block): one wave
// per row, lane-strided partial sums and a wave reduction.
__global__ __launch_bounds__(kThreads) void row_reduce_kernel(const double *ep, const double *elp,
                                                              int M, int nb, double *err,
                                                              double *errl)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (i >= M)
        return;   // no barrier below: each wave owns its row
    double e = 0.0, el = 0.0;
    for (int t = lane; t < nb; t += 64) {
        e += ep[(size_t)i * nb + t];
        el += elp[(size_t)i * nb + t];
    }
    e = wave_sum(e);
    el = wave_sum(el);
    if (lane == 0) {
        if (err)
            err[i] = e;
        if (errl)
            errl[i] = el;
    }
}

// ---------------------------------------------------------------------------
// Layer normalisation LAMP, one work-group per row (N <= kLnMaxN).
// ---------------------------------------------------------------------------
constexpr int kLnMaxN = 8192;
constexpr int kLnPerThread = kLnMaxN / kThreads;   // 32

struct LnArgs {
    const float *ylo, *yref;     // [M, N]
    const float *gamma, *beta;   // [N]
    int M, N, W, P;              // P: N rounded up to a power of two (the sort width)
    double eps, tau;
    float *out;                  // [M, N]
    float *ymix;                 // [M, N] or null
    uint32_t *mask;              // [M, W] or null
    uint32_t *row_count;         // [M] or null
    double *err, *errl;          // [M] or null
};

// Block sum of a double over the 256 threads (every thread gets the result).
__device__ __forceinline__ double block_sum_d(double x, double *s_red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x = wave_sum(x);
    __syncthreads();   // s_red may still be read by the previous call
    if (lane == 0)
        s_red[wave] = x;
    __syncthreads();
    return (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

__global__ __launch_bounds__(kThreads) void ln_lamp_kernel(LnArgs a)
{
    extern __shared__ uint64_t s_key[];   // P sort keys, then selection flags
    __shared__ double s_red[4];
    __shared__ uint32_t s_cnt[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = blockIdx.x;
    const int N = a.N;
    const float *lo = a.ylo + (size_t)i * N, *rf = a.yref + (size_t)i * N;

    // statistics of the low-precision row (the look-ahead estimate of sigma)
    double s1 = 0.0;
    for (int j = tid; j < N; j += kThreads)
        s1 += (double)lo[j];
    const double m_lo = block_sum_d(s1, s_red) / N;
    double s2 = 0.0;
    for (int j = tid; j < N; j += kThreads) {
        const double d = (double)lo[j] - m_lo;
        s2 += d * d;
    }
    const double v_lo = block_sum_d(s2, s_red) / N;
    double T2 = a.tau * a.tau * (v_lo + a.eps) * (double)N;
    if (isnan(T2))   // tau = +inf with sigma = 0 (or a NaN row): recompute nothing
        T2 = INFINITY;

    // sort keys: descending magnitude, ties to the lower index, as one
    // ascending 64-bit order: (~|y| bits) << 32 | j; padding keys sort last
    for (int p = tid; p < a.P; p += kThreads) {
        uint64_t key = ~0ull;
        if (p < N) {
            const uint32_t mag = __float_as_uint(lo[p]) & 0x7fffffffu;
            key = ((uint64_t)(~mag) << 32) | (uint32_t)p;
        }
        s_key[p] = key;
    }
    __syncthreads();
    for (int size = 2; size <= a.P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = tid; p < a.P / 2; p += kThreads) {
                // element pair (lo_idx, hi_idx) of this compare step
                const int lo_idx = 2 * p - (p & (stride - 1));
                const int hi_idx = lo_idx + stride;
                const bool up = (lo_idx & size) == 0;
                const uint64_t x = s_key[lo_idx], y = s_key[hi_idx];
                if ((x > y) == up) {
                    s_key[lo_idx] = y;
                    s_key[hi_idx] = x;
                }
            }
            __syncthreads();
        }
    }

    // suffix sums of squares over the sorted order: thread tid owns sorted
    // positions [tid * c, tid * c + c); R_k > T^2 exactly for k < k*, so k*
    // is the number of positions with R_k > T^2
    const int c = (N + kThreads - 1) / kThreads;
    const int q0 = tid * c;
    double mine = 0.0;
    float mg[kLnPerThread];
#pragma unroll
    for (int u = 0; u < kLnPerThread; ++u) {
        mg[u] = 0.0f;
        if (u < c && q0 + u < N) {
            mg[u] = __uint_as_float(~(uint32_t)(s_key[q0 + u] >> 32));
            mine += (double)mg[u] * (double)mg[u];
        }
    }
    // exclusive suffix of the thread totals (threads above tid)
    __shared__ double s_tot[kThreads];
    s_tot[tid] = mine;
    __syncthreads();
    double above = 0.0;
    for (int t = tid + 1; t < kThreads; ++t)
        above += s_tot[t];
    // R_k = above + (my squares from k on), summed upwards from my last
    // position: every partial sum is of nonnegative terms (no cancellation)
    uint32_t nbig = 0;   // positions k in my range with R_k > T^2
    double suf = 0.0;
#pragma unroll
    for (int u = kLnPerThread - 1; u >= 0; --u) {
        if (u < c && q0 + u < N) {
            suf += (double)mg[u] * (double)mg[u];
            nbig += above + suf > T2 ? 1u : 0u;
        }
    }
    nbig = (uint32_t)wave_sum_int((int)nbig);
    __syncthreads();
    if (lane == 0)
        s_cnt[wave] = nbig;
    __syncthreads();
    const int kstar = (int)(s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3]);

    // selection flags (reuse the key array as a byte map after a barrier)
    int selj[kLnPerThread];
#pragma unroll
    for (int u = 0; u < kLnPerThread; ++u)
        selj[u] = (u < c && q0 + u < kstar) ? (int)(uint32_t)s_key[q0 + u] : -1;
    __syncthreads();
    uint8_t *s_sel = reinterpret_cast<uint8_t *>(s_key);
    for (int j = tid; j < N; j += kThreads)
        s_sel[j] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kLnPerThread; ++u)
        if (selj[u] >= 0)
            s_sel[selj[u]] = 1;
    __syncthreads();

    // y^mix and the three layer norms (mix, ref, lo) in double
    double sm = 0.0, sr = 0.0;
    for (int j = tid; j < N; j += kThreads) {
        sm += (double)(s_sel[j] ? rf[j] : lo[j]);
        sr += (double)rf[j];
    }
    const double m_mix = block_sum_d(sm, s_red) / N;
    const double m_ref = block_sum_d(sr, s_red) / N;
    double vm = 0.0, vr = 0.0;
    for (int j = tid; j < N; j += kThreads) {
        const double dm = (double)(s_sel[j] ? rf[j] : lo[j]) - m_mix;
        const double dr = (double)rf[j] - m_ref;
        vm += dm * dm;
        vr += dr * dr;
    }
    const double r_mix = 1.0 / sqrt(block_sum_d(vm, s_red) / N + a.eps);
    const double r_ref = 1.0 / sqrt(block_sum_d(vr, s_red) / N + a.eps);
    const double r_lo = 1.0 / sqrt(v_lo + a.eps);
    double em = 0.0, el = 0.0;
    for (int j = tid; j < N; j += kThreads) {
        const bool s = s_sel[j] != 0;
        const float ym = s ? rf[j] : lo[j];
        const double g = (double)a.gamma[j], b = (double)a.beta[j];
        const double o_mix = g * (((double)ym - m_mix) * r_mix) + b;
        const double o_ref = g * (((double)rf[j] - m_ref) * r_ref) + b;
        const double o_lo = g * (((double)lo[j] - m_lo) * r_lo) + b;
        a.out[(size_t)i * N + j] = (float)o_mix;
        if (a.ymix)
            a.ymix[(size_t)i * N + j] = ym;
        em += (o_mix - o_ref) * (o_mix - o_ref);
        el += (o_lo - o_ref) * (o_lo - o_ref);
    }
    em = block_sum_d(em, s_red);
    el = block_sum_d(el, s_red);
    if (a.mask) {
        for (int w = tid; w < a.W; w += kThreads) {
            uint32_t word = 0;
            for (int b = 0; b < 32; ++b) {
                const int j = 32 * w + b;
                if (j < N && s_sel[j])
                    word |= 1u << b;
            }
            a.mask[(size_t)i * a.W + w] = word;
        }
    }
    if (tid == 0) {
        if (a.row_count)
            a.row_count[i] = (uint32_t)kstar;
        if (a.err)
            a.err[i] = sqrt(em);
        if (a.errl)
            a.errl[i] = sqrt(el);
    }
}

// Fraction of the last round of work-groups over the 256 CUs that is full:
// n work-groups of equal work take ceil(n / 256) rounds.
static double cu_balance(long long n)
{
    const double rounds = (double)((n + 255) / 256);
    return (double)n / (256.0 * rounds);
}

// The narrow tiles for products of fewer than 1024 wide tiles that they
// spread over the CUs clearly more evenly (measured on MI355X with the
// progress priority: 25-800 tiles gain 8-160 %, except multiples of 256;
// from 1024 tiles on the wide tiles run 2-9 % faster).
static bool use_narrow_tiles(long long tiles64, long long tiles32)
{
    return tiles64 < 1024 && cu_balance(tiles32) > cu_balance(tiles64) + 0.05;
}

// ---------------------------------------------------------------------------
static PsConst gemm_ps_const(int mu, int block, int K)
{
    PsConst c = make_ps_const(mu, 1);   // s = 1/sqrt(1) = 1: no scale
    set_ps_block(c, block, K);
    return c;
}

hipError_t launch_mlp(const MlpProblem &p, const MlpBuffers &b, hipStream_t st,
                      void **stage_events)
{
    auto rec = [&](int e) {
        return stage_events ? hipEventRecord((hipEvent_t)stage_events[e], st) : hipSuccess;
    };
    const int tiles_m = (p.M + kTile - 1) / kTile, tiles_n = (p.N + kTile - 1) / kTile;
    hipError_t e;
    if ((e = rec(2 * 0)) != hipSuccess)   // scan stage
        return e;
    if ((e = launch_zero(b.unsafe, sizeof(uint32_t) * (size_t)(tiles_m + tiles_n), st)) !=
        hipSuccess)
        return e;
    const unsigned spans = (unsigned)(((size_t)kTile * p.K + kScanSpan - 1) / kScanSpan);
    hipLaunchKernelGGL(gemm_scan_kernel, dim3(tiles_m, spans), dim3(kThreads), 0, st, p.x, p.M,
                       p.K, b.unsafe);
    hipLaunchKernelGGL(gemm_scan_kernel, dim3(tiles_n, spans), dim3(kThreads), 0, st, p.w, p.N,
                       p.K, b.unsafe + tiles_m);
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 0 + 1)) != hipSuccess)
        return e;
    GemmArgs a;
    a.x = p.x;
    a.w = p.w;
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.tiles_n = tiles_n;
    a.W = (p.N + 31) / 32;
    a.pc = gemm_ps_const(p.mu, p.ps_block, p.K);
    a.unsafe_x = b.unsafe;
    a.unsafe_w = b.unsafe + tiles_m;
    a.ylo = b.ylo;
    a.yref = b.yref;
    a.out = b.out;
    a.mask = b.mask;
    a.err_part = b.err_part;
    a.errl_part = b.errl_part;
    a.tau = (double)p.tau;
    a.n_band = p.n_band;
    a.exact_tiles = b.exact_tiles;
    a.n_tiles = (long long)tiles_m * tiles_n;
    if (a.n_tiles > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const dim3 block(kThreads);
    const unsigned gfast = (unsigned)a.n_tiles;
    const unsigned ggen = (unsigned)(a.n_tiles < 2048 ? a.n_tiles : 2048);
    const bool gelu = p.op == MLP_GELU;
    if ((e = rec(2 * 6)) != hipSuccess)   // exact stage
        return e;
#define LAMP_GEMM_LAUNCH1(FASTK, EPIK, grid)                                                    \
    do {                                                                                        \
        switch (run_width(a.pc.blk)) {                                                          \
        case 0: hipLaunchKernelGGL((ps_gemm_kernel<FASTK, EPIK, 0>), grid, block, 0, st, a); break;  \
        case 4: hipLaunchKernelGGL((ps_gemm_kernel<FASTK, EPIK, 4>), grid, block, 0, st, a); break;  \
        case 8: hipLaunchKernelGGL((ps_gemm_kernel<FASTK, EPIK, 8>), grid, block, 0, st, a); break;  \
        case 16: hipLaunchKernelGGL((ps_gemm_kernel<FASTK, EPIK, 16>), grid, block, 0, st, a); break; \
        default: hipLaunchKernelGGL((ps_gemm_kernel<FASTK, EPIK, 32>), grid, block, 0, st, a); break; \
        }                                                                                       \
    } while (0)
#define LAMP_GEMM_LAUNCH(FASTK, grid)                                                           \
    do {                                                                                        \
        if (gelu)                                                                               \
            LAMP_GEMM_LAUNCH1(FASTK, EPI_GELU, grid);                                           \
        else                                                                                    \
            LAMP_GEMM_LAUNCH1(FASTK, EPI_STORE, grid);                                          \
    } while (0)
    LAMP_GEMM_LAUNCH(false, dim3(ggen));
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 6 + 1)) != hipSuccess ||
        (e = rec(2 * 1)) != hipSuccess)
        return e;
    if (p.mu <= 10) {
        const long long n32 = (long long)((p.M + kNarrow - 1) / kNarrow) *
                              ((p.N + kNarrow - 1) / kNarrow);
        if (use_narrow_tiles(a.n_tiles, n32)) {
            if (n32 > 0x7fffffffLL)
                return hipErrorInvalidValue;
            const dim3 g32((unsigned)n32);
#define LAMP_NARROW_LAUNCH(EPIK)                                                                  \
    do {                                                                                          \
        switch (run_width(a.pc.blk)) {                                                            \
        case 0: hipLaunchKernelGGL((ps_gemm_narrow_kernel<EPIK, 0>), g32, block, 0, st, a); break;   \
        case 4: hipLaunchKernelGGL((ps_gemm_narrow_kernel<EPIK, 4>), g32, block, 0, st, a); break;   \
        case 8: hipLaunchKernelGGL((ps_gemm_narrow_kernel<EPIK, 8>), g32, block, 0, st, a); break;   \
        case 16: hipLaunchKernelGGL((ps_gemm_narrow_kernel<EPIK, 16>), g32, block, 0, st, a); break; \
        default: hipLaunchKernelGGL((ps_gemm_narrow_kernel<EPIK, 32>), g32, block, 0, st, a); break; \
        }                                                                                         \
    } while (0)
            if (gelu)
                LAMP_NARROW_LAUNCH(EPI_GELU);
            else
                LAMP_NARROW_LAUNCH(EPI_STORE);
#undef LAMP_NARROW_LAUNCH
        } else {
            LAMP_GEMM_LAUNCH(true, dim3(gfast));
        }
    }
#undef LAMP_GEMM_LAUNCH
#undef LAMP_GEMM_LAUNCH1
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 1 + 1)) != hipSuccess ||
        (e = rec(2 * 4)) != hipSuccess)
        return e;
    if (gelu) {
        hipLaunchKernelGGL(row_reduce_kernel, dim3((p.M + 3) / 4), block, 0, st, b.err_part,
                           b.errl_part, p.M, a.W, b.err, b.errl);
    } else if (p.op == MLP_LAYERNORM) {
        LnArgs l;
        l.ylo = b.ylo;
        l.yref = b.yref;
        l.gamma = p.gamma;
        l.beta = p.beta;
        l.M = p.M;
        l.N = p.N;
        l.W = (p.N + 31) / 32;
        int P = 1;
        while (P < p.N)
            P <<= 1;
        l.P = P;
        l.eps = (double)p.eps;
        l.tau = (double)p.tau;
        l.out = b.out;
        l.ymix = b.ymix;
        l.mask = b.mask;
        l.row_count = b.row_count;
        l.err = b.err;
        l.errl = b.errl;
        hipLaunchKernelGGL(ln_lamp_kernel, dim3(p.M), block, sizeof(uint64_t) * (size_t)P, st, l);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return rec(2 * 4 + 1);
}

// Row counts of the GELU rule from its mask words.
__global__ __launch_bounds__(kThreads) void mask_count_kernel(const uint32_t *mask, int M, int W,
                                                              uint32_t *count)
{
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= M)
        return;
    uint32_t c = 0;
    for (int w = 0; w < W; ++w)
        c += (uint32_t)__popc(mask[(size_t)i * W + w]);
    count[i] = c;
}

hipError_t launch_mask_count(const uint32_t *mask, int M, int N, uint32_t *count, hipStream_t st)
{
    hipLaunchKernelGGL(mask_count_kernel, dim3((M + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       st, mask, M, (N + 31) / 32, count);
    return hipGetLastError();
}

}  // namespace lamp
