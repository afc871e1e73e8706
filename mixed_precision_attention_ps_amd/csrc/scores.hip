// scores.hip -- operand range scan and the PS(mu) / FP32 score tile kernel.
//
// Step 1 of LAMP ("Implementation strategy": baseline evaluation at low
// precision), with the uniform FP32 reference scores of "Experimental
// results" computed in the same pass from the same FP32 products.
#include "lamp_device.h"

namespace lamp {

PsConst make_ps_const(int mu, int D)
{
    PsConst c;
    c.mu = mu;
    c.sh = (uint32_t)(23 - mu);
    c.split = (float)((1u << c.sh) + 1u);
    c.qscale = ldexpf(1.0f, mu - 23);
    c.s = (float)(1.0 / sqrt((double)D));
    c.out_scale = ldexpf(c.s, 23 - mu);
    c.blk = 0;
    return c;
}

void set_ps_block(PsConst &c, int block, int len)
{
    c.blk = (block <= 1 || block >= len) ? 0 : block;
}

// Unsafe operand (1): not zero and not a finite magnitude in [2^-40, 2^40].
__device__ __forceinline__ uint32_t operand_unsafe(float x)
{
    const uint32_t a = __float_as_uint(x) & 0x7fffffffu;
    const uint32_t lo = 0x2b800000u;   // 2^-40
    const uint32_t hi = 0x53800000u;   // 2^40
    return (uint32_t)(a != 0u) & (uint32_t)((a - lo) > (hi - lo));
}

// One work-group per 64-row block of Q or K: flag = block holds an unsafe
// value.  The flags are or-ed without a branch, so a thread's loads are all in
// flight at once.
__global__ __launch_bounds__(kThreads) void operand_scan_kernel(const float *__restrict__ q,
                                                                const float *__restrict__ k,
                                                                int BH, int S, int D, int tiles,
                                                                uint8_t *__restrict__ unsafe)
{
    const int blk = blockIdx.x;                  // [0, 2 * BH * tiles)
    const int which = blk / (BH * tiles);
    const int rem = blk % (BH * tiles);
    const int bh = rem / tiles, t = rem % tiles;
    const float4 *base = reinterpret_cast<const float4 *>(
        (which == 0 ? q : k) + ((size_t)bh * S + (size_t)t * kTile) * D);
    const int rows = min(kTile, S - t * kTile);
    const int n4 = rows * D / 4;
    uint32_t bad = 0;
#pragma unroll 4
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const float4 v = base[e];
        bad |= operand_unsafe(v.x) | operand_unsafe(v.y) | operand_unsafe(v.z) |
               operand_unsafe(v.w);
    }
    const int any_bad = __syncthreads_or((int)bad);
    if (threadIdx.x == 0)
        unsafe[blk] = any_bad ? 1 : 0;
}

hipError_t launch_operand_scan(const Problem &p, uint8_t *unsafe, hipStream_t st)
{
    const int grid = 2 * p.BH * p.tiles;
    hipLaunchKernelGGL(operand_scan_kernel, dim3(grid), dim3(kThreads), 0, st, p.q, p.k, p.BH,
                       p.S, p.D, p.tiles, unsafe);
    return hipGetLastError();
}

// Tile (ti, tj) of tile index t within a head: the lower triangle (tj <= ti)
// in row order when causal (causal == 2: the strict lower triangle, tj < ti,
// the diagonal tiles being the launch's last work-groups), the full square
// otherwise.
__device__ __forceinline__ void tile_coords(int t, int tiles, int causal, int &ti, int &tj)
{
    if (causal == 2) {
        // row a >= 1 holds tiles a (a - 1) / 2 .. a (a + 1) / 2 - 1
        int a = (int)((sqrtf(8.0f * (float)t + 1.0f) + 1.0f) * 0.5f);
        while (a * (a - 1) / 2 > t) --a;
        while ((a + 1) * a / 2 <= t) ++a;
        ti = a;
        tj = t - a * (a - 1) / 2;
    } else if (causal) {
        int a = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
        while ((a + 1) * (a + 2) / 2 <= t) ++a;
        while (a * (a + 1) / 2 > t) --a;
        ti = a;
        tj = t - a * (a + 1) / 2;
    } else {
        ti = t / tiles;
        tj = t % tiles;
    }
}

struct ScoreArgs {
    const float *q, *k;
    int S, D, causal, tiles, tiles_per_head;
    PsConst pc;
    const uint8_t *unsafe_q, *unsafe_k;
    float *ylo, *yref;
    float *pzero;        // causal: zero the mirrored upper tile (may be null)
    RefPartial *part;
    int ref_sums;        // part: L and B too (else only the maxima; L = B = 0)
    int lo_max;          // part: m_lo too (else -inf)
    unsigned long long *exact_tiles;
    long long n_tiles;   // BH x tiles per head
    int BH;
    int tile_set;        // causal: 2 = off-diagonal tiles in the tile loop (the
                         // diagonal ones from diag_from on), else 1
    long long diag_from; // fast kernel, >= 0: work-groups from here on take the
                         // diagonal tiles (diag_tile), after the others
};


template <int PATH, int P, int NC = 4>
__device__ __forceinline__ void score_tile_store(TileSmem &sm, const double *s_exp,
                                                 const ScoreArgs &a, int bh, int ti, int tj)
{
    const size_t head = (size_t)bh * a.S * a.D;
    TileAcc acc;
    score_tile<PATH, P, false, NC>(sm, acc, a.q + head, a.k + head, ti * kTile, tj * kTile, a.S,
                                   a.S, a.D, a.pc);
    float lo[4][4], ref[4][4];
    tile_scores<PATH, P>(acc, a.pc, lo, ref);
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = ti * kTile + ty * 4 + r;
        if (i >= a.S)
            continue;
        const size_t rowoff = ((size_t)bh * a.S + i) * a.S;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = tj * kTile + tx + 16 * c;
            if (j >= a.S || (a.causal && j > i))
                continue;
            if (a.ylo)
                a.ylo[rowoff + j] = lo[r][c];
            if (a.yref)
                a.yref[rowoff + j] = ref[r][c];
        }
    }
    if (a.part) {
        // this tile's maxima of its reference and PS(mu) scores and, when a
        // KL is asked for, the softmax sums of its reference scores, per row:
        // every key is evaluated (no divergent branch) and the keys outside
        // the row are masked out of the sums.  The fast path's scores are
        // finite (its operands are bounded), so its exponential needs no NaN
        // handling; the other paths keep NaN in the sums.
        float m[4], mlo[4];
        bool valid[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * kTile + ty * 4 + r;
            m[r] = -INFINITY;
            mlo[r] = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = tj * kTile + tx + 16 * c;
                valid[r][c] = i < a.S && j < a.S && (!a.causal || j <= i);
                m[r] = fmaxf(m[r], valid[r][c] ? ref[r][c] : -INFINITY);
            }
            m[r] = group16_max(m[r]);
        }
        if (a.lo_max) {   // uniform over the launch
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    mlo[r] = fmaxf(mlo[r], valid[r][c] ? lo[r][c] : -INFINITY);
                mlo[r] = group16_max(mlo[r]);
            }
        }
        double L[4], B[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            L[r] = 0.0;
            B[r] = 0.0;
        }
        if (a.ref_sums) {   // uniform over the launch
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const double x = (double)ref[r][c] - (double)m[r];
                    const double e = PATH == PATH_FAST ? exp64_sum_nonpos(x, s_exp) : exp64_sum(x, s_exp);
                    // y_ref - y_lo in FP32: exact when the two are within a factor
                    // of two (Sterbenz), else within half an ulp of the difference
                    const double dy = (double)(ref[r][c] - lo[r][c]);
                    L[r] += valid[r][c] ? e : 0.0;
                    B[r] = valid[r][c] ? fma(e, dy, B[r]) : B[r];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                L[r] = group16_sum(L[r]);
                B[r] = group16_sum(B[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * kTile + ty * 4 + r;
            if (tx == 0 && i < a.S) {
                RefPartial rp;
                rp.L = L[r];
                rp.B = B[r];
                rp.m = m[r];
                rp.m_lo = mlo[r];
                a.part[((size_t)bh * a.S + i) * a.tiles + tj] = rp;
            }
        }
    }
}

#ifndef LAMP_SCORES_XCD
#define LAMP_SCORES_XCD 1
#endif
// Tile index g -> (head, tile of the head).  Work-groups go to the GPU's
// eight XCDs in turn (g mod 8), each XCD with its own L2: when the heads
// split evenly over the XCDs, XCD x takes heads x, x + 8, ..., each head's
// tiles one after another, so that a head's Q and K rows are fetched into
// one L2 only.  Otherwise heads in order.
__device__ __forceinline__ void head_tile_of(long long g, int BH, int tiles_per_head, int &bh,
                                             long long &t)
{
    constexpr int kXcd = 8;
    if (LAMP_SCORES_XCD && BH % kXcd == 0) {
        const long long l = g / kXcd;
        bh = (int)(l / tiles_per_head) * kXcd + (int)(g % kXcd);
        t = l % tiles_per_head;
    } else {
        bh = (int)(g / tiles_per_head);
        t = g % tiles_per_head;
    }
}

// Causal diagonal tile g (head-major over the heads' tiles, the score
// kernel's XCD order) when it is on the fast path, by one work-group (s_exp
// filled and synchronised).  Wave w holds the tile's rows 16 w .. 16 w + 15,
// which see keys up to 16 w + 15 only: it multiplies the key groups c <= w
// (keys tx + 16 c) and leaves the rest, all above the diagonal, at +0
// (masked in the epilogue).  The waves take their own copy of the tile loop
// (wave-uniform); every copy passes the same barriers of the shared operand
// staging.  The other paths' diagonal tiles stay with the generic kernel.
// Sequential order only: with the blocked orders' run sums the copies need
// 109 registers (four waves per SIMD), and their diagonal tiles stay in the
// plain tile loop.
template <int P>
__device__ __forceinline__ void diag_tile(TileSmem &sm, const double *s_exp, const ScoreArgs &a,
                                          long long g)
{
    int bh;
    long long t;
    head_tile_of(g, a.BH, a.tiles, bh, t);
    const int ti = (int)t;
    if (a.pc.mu > 10 || a.unsafe_q[bh * a.tiles + ti] || a.unsafe_k[bh * a.tiles + ti])
        return;
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: score_tile_store<PATH_FAST, P, 1>(sm, s_exp, a, bh, ti, ti); break;
    case 1: score_tile_store<PATH_FAST, P, 2>(sm, s_exp, a, bh, ti, ti); break;
    case 2: score_tile_store<PATH_FAST, P, 3>(sm, s_exp, a, bh, ti, ti); break;
    default: score_tile_store<PATH_FAST, P, 4>(sm, s_exp, a, bh, ti, ti); break;
    }
}

// Two kernels share the tile grid: the fast kernel takes the tiles whose
// operands allow the FP32 fast path (and returns on the others); the generic
// kernel takes every other tile (exact double path, or plain FP32 at mu = 23).
// Keeping the exact path out of the fast kernel keeps its register budget,
// and so its occupancy, to what the fast path needs.  The fast kernel has one
// work-group per tile; the generic one a bounded grid that strides over the
// tiles (it usually finds none to do, and then costs a few microseconds).
// P: the run width of the blocked PS(mu) order (run_width(a.pc.blk)).
template <bool FAST_KERNEL, int P>
__global__ __launch_bounds__(kThreads) void ps_scores_kernel(ScoreArgs a)
{
    __shared__ TileSmem sm;
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    auto tile_path = [&](long long g, int &bh, int &ti, int &tj) {
        long long t;
        head_tile_of(g, a.BH, a.tiles_per_head, bh, t);
        tile_coords((int)t, a.tiles, a.causal ? (FAST_KERNEL ? a.tile_set : 1) : 0, ti, tj);
        if (a.pc.mu == 23)
            return (int)PATH_FP32;
        if (a.pc.mu <= 10 && !a.unsafe_q[bh * a.tiles + ti] && !a.unsafe_k[bh * a.tiles + tj])
            return (int)PATH_FAST;
        return (int)PATH_EXACT;
    };
    if (!FAST_KERNEL) {
        // the threads look at this work-group's tiles in parallel; without a
        // tile for the generic paths the work-group is done
        bool need = false;
        for (long long g = blockIdx.x + (long long)threadIdx.x * gridDim.x; g < a.n_tiles;
             g += (long long)blockDim.x * gridDim.x) {
            int bh, ti, tj;
            need |= tile_path(g, bh, ti, tj) != PATH_FAST;
        }
        if (!__syncthreads_or(need ? 1 : 0))
            return;
    }
    exp_table_fill(s_exp);
    __syncthreads();
    // sequential order: the diagonal tiles are the grid's last work-groups
    // (they fill the tail of the launch)
    if constexpr (FAST_KERNEL && P == 0) {
        if (a.diag_from >= 0 && (long long)blockIdx.x >= a.diag_from) {
            diag_tile<P>(sm, s_exp, a, (long long)blockIdx.x - a.diag_from);
            return;
        }
    }
    // the mirrored zero tiles: every tile's work-group in the fast kernel,
    // or in the generic one when no fast kernel runs (mu > 10)
    const bool zero_fill = a.pzero && a.causal && (FAST_KERNEL || a.pc.mu > 10);
    for (long long g = blockIdx.x; g < a.n_tiles; g += FAST_KERNEL ? a.n_tiles : gridDim.x) {
        int bh, ti, tj;
        const int path = tile_path(g, bh, ti, tj);
        if (zero_fill && tj < ti)   // rows of block tj (whole), keys of block ti
            zero_block(a.pzero, a.S, bh, tj * kTile, kTile, ti * kTile,
                       min(a.S, (ti + 1) * kTile), kThreads);
        if (FAST_KERNEL) {
            if (path == PATH_FAST)
                score_tile_store<PATH_FAST, P>(sm, s_exp, a, bh, ti, tj);
        } else if (path == PATH_EXACT) {
            if (threadIdx.x == 0 && a.exact_tiles)
                atomicAdd(a.exact_tiles, 1ull);
            score_tile_store<PATH_EXACT, P>(sm, s_exp, a, bh, ti, tj);
        } else if (path == PATH_FP32) {
            score_tile_store<PATH_FP32, P>(sm, s_exp, a, bh, ti, tj);
        }
    }
}


constexpr long long kGenericGrid = 2048;   // work-groups of the generic kernel
constexpr long long kGenericGridBeside = 512;   // ... when the fast kernel runs too

hipError_t launch_ps_scores(const Problem &p, const uint8_t *unsafe, float *ylo, float *yref,
                            RefPartial *part, unsigned long long *exact_tiles, bool fast,
                            hipStream_t st, float *pzero)
{
    ScoreArgs a;
    a.q = p.q;
    a.k = p.k;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.tiles = p.tiles;
    a.tiles_per_head = p.causal ? p.tiles * (p.tiles + 1) / 2 : p.tiles * p.tiles;
    a.pc = p.pc;
    a.unsafe_q = unsafe;
    a.unsafe_k = unsafe + (size_t)p.BH * p.tiles;
    a.ylo = ylo;
    a.yref = yref;
    a.pzero = pzero;
    a.part = part;
    a.ref_sums = p.ref_sums ? 1 : 0;
    a.lo_max = p.lo_max ? 1 : 0;
    a.exact_tiles = exact_tiles;
    const long long grid = (long long)p.BH * a.tiles_per_head;
    if (grid > 0x7fffffffLL)
        return hipErrorInvalidValue;
    a.n_tiles = grid;
    a.BH = p.BH;
    a.tile_set = 1;
    a.diag_from = -1;
    if (grid == 0)
        return hipSuccess;
#define LAMP_SCORES_LAUNCH(FASTK, G)                                                           \
    do {                                                                                       \
        switch (run_width(p.pc.blk)) {                                                         \
        case 0: hipLaunchKernelGGL((ps_scores_kernel<FASTK, 0>), G, dim3(kThreads), 0, st, a); break;  \
        case 4: hipLaunchKernelGGL((ps_scores_kernel<FASTK, 4>), G, dim3(kThreads), 0, st, a); break;  \
        case 8: hipLaunchKernelGGL((ps_scores_kernel<FASTK, 8>), G, dim3(kThreads), 0, st, a); break;  \
        case 16: hipLaunchKernelGGL((ps_scores_kernel<FASTK, 16>), G, dim3(kThreads), 0, st, a); break; \
        default: hipLaunchKernelGGL((ps_scores_kernel<FASTK, 32>), G, dim3(kThreads), 0, st, a); break; \
        }                                                                                      \
    } while (0)
    if (fast) {
        if (p.mu <= 10 && p.causal && p.tiles > 1 && run_width(p.pc.blk) == 0) {
            // one launch: the off-diagonal tiles, then the diagonal ones
            ScoreArgs o = a;
            o.tile_set = 2;
            o.tiles_per_head = p.tiles * (p.tiles - 1) / 2;
            o.n_tiles = (long long)p.BH * o.tiles_per_head;
            o.diag_from = o.n_tiles;
            const long long nd = (long long)p.BH * p.tiles;
            if (o.n_tiles + nd > 0x7fffffffLL)
                return hipErrorInvalidValue;
            hipLaunchKernelGGL((ps_scores_kernel<true, 0>), dim3((unsigned)(o.n_tiles + nd)),
                               dim3(kThreads), 0, st, o);
        } else if (p.mu <= 10) {
            LAMP_SCORES_LAUNCH(true, dim3((unsigned)grid));
        }
    } else {
        // beside the fast kernel the generic one usually finds no tile: a
        // smaller grid, whose threads still cover every tile in one look
        const long long cap = p.mu <= 10 ? kGenericGridBeside : kGenericGrid;
        const long long g = grid < cap ? grid : cap;
        LAMP_SCORES_LAUNCH(false, dim3((unsigned)g));
    }
#undef LAMP_SCORES_LAUNCH
    return hipGetLastError();
}

}  // namespace lamp
