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
#include <type_traits>

#include "lamp_device.h"

namespace lamp {

typedef float floatx4 __attribute__((ext_vector_type(4)));

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
    float *pzero;   // causal: the block's probability zero tails (may be null)
    double *row_l;
    unsigned long long *exact_tiles;
    unsigned long long *n_band;
};

// Online state of one query row: maxima of y^lo (m_t), y^mix and y^ref, and
// the sums relative to them.  Each row is owned by the 16 lanes of one wave
// that hold it, so its LDS copy needs no barrier.
struct RowState {
    float m_t, m_mix, m_ref;
    uint32_t cnt;
    double l_mix, l_ref, kl_a, l_lo, kl_b;
};

template <int DV>
struct RelaxedSmem {
    union {
        TileSmem tile;                 // PS(mu) operand staging
        float p[kTile][kTile + 4];     // P tile of the online softmax, [row][key]
    } u;
    float v[kTile][DV + 16];           // V tile, [key][col] (padded rows: 2-way LDS reads)
    RowState row[kTile];
};

template <int PATH, int P>
__device__ __forceinline__ void relaxed_tile_scores(TileSmem &sm, const RelaxedArgs &a,
                                                    const float *Qh, const float *Kh, int row0,
                                                    int col0, float lo[4][4], float ref[4][4])
{
    TileAcc acc;
    score_tile<PATH, P>(sm, acc, Qh, Kh, row0, col0, a.S, a.S, a.D, a.pc);
    tile_scores<PATH, P>(acc, a.pc, lo, ref);
}

// exp of a difference of row maxima (-inf when a maximum is still unset).
__device__ __forceinline__ double exp_delta(float from, float to, const double *s_exp)
{
    return from == -INFINITY ? 0.0 : exp64_sum((double)from - (double)to, s_exp);
}

// Per-score exponentials (double): E = exp(y^lo - m_t) serves the criterion
// (exp64_crit) and, scaled by exp(m_t - m_mix), the softmax term of an
// unselected score; e_ref = exp(y^ref - m_ref) serves the reference sums and,
// scaled by exp(m_ref - m_mix), the softmax term of a selected score (whose
// y^mix is y^ref) (exp64_sum, as the row factors).  Two double exps per
// score; the row factors are per tile.
// P: the run width of the blocked PS(mu) order (run_width(a.pc.blk)).
// Occupancy: at D <= 64 three waves per SIMD (168 registers, a few spilled;
// 5 % faster than two without spills), at D <= 128 two.
template <int NB, bool FAST_KERNEL, int P>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(FAST_KERNEL ? (NB == 4 ? 3 : 2) : 1)))
void relaxed_kernel(RelaxedArgs a)
{
    constexpr int DV = 16 * NB;
    constexpr int NV4 = kTile * DV / 4;                   // float4 in a V tile
    constexpr int V4 = (NV4 + kThreads - 1) / kThreads;   // per thread
    __shared__ RelaxedSmem<DV> sm;
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    __shared__ int s_vbad;         // the diagonal V tile holds a non-finite value
    exp_table_fill(s_exp);
    if (threadIdx.x == 0)
        s_vbad = 0;
    __syncthreads();
    const int S = a.S, D = a.D;
    // heaviest query blocks first (causal work grows with the block index);
    // (batches of heads per XCD, as the row kernel takes them, made this
    // kernel slower: 1.94 -> 2.21 ms on the GPT-2-XL layer)
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
    // the zero tails of this block's probability rows (keys of the blocks
    // past it), written here, beside the ALU-bound tile work, rather than
    // by the memory-bound probabilities pass
    if (a.pzero && a.causal)
        zero_block(a.pzero, S, bh, row0, min(kTile, S - row0), row0 + kTile, S, kThreads);

    if (tx == 0)
        for (int r = 0; r < 4; ++r) {
            RowState z;
            z.m_t = z.m_mix = z.m_ref = -INFINITY;
            z.cnt = 0;
            z.l_mix = z.l_ref = z.kl_a = z.l_lo = z.kl_b = 0.0;
            sm.row[ty * 4 + r] = z;
        }
    // P.V accumulators in double: the FP32 MFMA partial of every 16 keys is
    // flushed into them (at most 4 FP32 roundings per partial, 2.4e-7 of its
    // magnitude; FP32 accumulation over a long row drifts beyond 1e-6)
    double acc[NB][4];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[q][v] = 0.0;

    // Output rows of this block: a uniform base (scalar registers) and a
    // 32-bit offset per lane, formed in the loop.  Per-row output addresses
    // are loop invariants that the compiler hoists out of the key loop; twelve
    // of them spilled and came back from scratch, each reload a full memory
    // wait in the epilogue.
    const uint64_t blk_row = (uint64_t)bh * S + row0;
    uint32_t *const mask_blk = a.mask ? a.mask + blk_row * (uint64_t)a.W : nullptr;
    float *const ymix_blk = a.ymix_raw ? a.ymix_raw + blk_row * (uint64_t)S : nullptr;
    float *const yref_blk = a.yref_out ? a.yref_out + blk_row * (uint64_t)S : nullptr;
    // the wave's near ties of the criterion: counted from ballots of the
    // band test (a scalar count, no vector register kept across the loop)
    uint32_t ties = 0;
    const bool count_ties = a.n_band != nullptr && a.tau < INFINITY;
    const double tie_band = 0x1p-16 * a.tau;
    // Issue priority: the tile's multiply-adds at 0, its softmax epilogue
    // (LDS row state, reductions, exponentials: dependent chains) at 2, so
    // that a wave in its epilogue issues ahead of the other work-groups' MAC
    // loops on the SIMD (GPT-2-XL layer 1.70 -> 1.65 ms).
    for (int t = 0; t <= t_end; ++t) {
        __builtin_amdgcn_s_setprio(0);
        const int col0 = t * kTile;
        float lo[4][4], ref[4][4];
        const int path = FAST_KERNEL ? PATH_FAST
                         : a.pc.mu == 23 ? PATH_FP32
                         : (a.pc.mu <= 10 && qsafe && !a.unsafe_k[bh * a.tiles + t]) ? PATH_FAST
                                                                                       : PATH_EXACT;
        if (FAST_KERNEL || path == PATH_FAST) {
            relaxed_tile_scores<PATH_FAST, P>(sm.u.tile, a, Qh, Kh, row0, col0, lo, ref);
        } else if (path == PATH_EXACT) {
            if (tid == 0 && a.exact_tiles)
                atomicAdd(a.exact_tiles, 1ull);
            relaxed_tile_scores<PATH_EXACT, P>(sm.u.tile, a, Qh, Kh, row0, col0, lo, ref);
        } else {
            relaxed_tile_scores<PATH_FP32, P>(sm.u.tile, a, Qh, Kh, row0, col0, lo, ref);
        }

        __builtin_amdgcn_s_setprio(2);
        float pmix[4][4];
        const int gsh = (lane >> 4) * 16;
        // one query row at a time, with a compile-time row index so that the
        // score and state arrays stay in registers
        auto row_step = [&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int i = row0 + ty * 4 + r;
            bool valid[4];
            float bl = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = col0 + tx + 16 * c;
                valid[c] = i < S && j < S && (!a.causal || j <= i);
                if (valid[c])
                    bl = fmaxf(bl, lo[r][c]);
            }
            bl = group16_max(bl);
            RowState &rs = sm.row[ty * 4 + r];
            const float m_t = rs.m_t, m_mix = rs.m_mix, m_ref = rs.m_ref;
            const float mt_new = fmaxf(m_t, bl);

            // selection and y^mix
            double E[4];
            float mix[4];
            bool sel[4];
            float bm = -INFINITY, br = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                E[c] = valid[c] ? exp64_crit((double)lo[r][c] - (double)mt_new, s_exp) : 0.0;
                const double crit = 2.0 * E[c] * fabs((double)lo[r][c]);
                sel[c] = valid[c] && crit > a.tau;
                if (count_ties)
                    ties += (uint32_t)__popcll(ballot(valid[c] && fabs(crit - a.tau) <= tie_band));
                mix[c] = sel[c] ? ref[r][c] : lo[r][c];
                if (valid[c]) {
                    bm = fmaxf(bm, mix[c]);
                    br = fmaxf(br, ref[r][c]);
                }
            }
            // mask bits: ballot per key offset c, 16 bits per row group
            uint32_t bits[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bits[c] = (uint32_t)(ballot(sel[c]) >> gsh) & 0xffffu;
            const uint32_t w0 = bits[0] | (bits[1] << 16), w1 = bits[2] | (bits[3] << 16);
            if (i < S) {
                // row within the block, opaque to the compiler so that its
                // offsets are formed here (one multiply) rather than hoisted
                uint32_t lr = (uint32_t)(ty * 4 + r);
                asm volatile("" : "+v"(lr));
                if (mask_blk && tx == 0) {
                    const uint32_t mo = lr * (uint32_t)a.W;
                    if (2 * t < a.W)
                        mask_blk[mo + 2 * t] = w0;
                    if (2 * t + 1 < a.W)
                        mask_blk[mo + 2 * t + 1] = w1;
                }
                if (ymix_blk || yref_blk) {
                    const uint32_t yo = lr * (uint32_t)S;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (!valid[c])
                            continue;
                        const uint32_t j = (uint32_t)(col0 + tx + 16 * c);
                        if (ymix_blk)
                            ymix_blk[yo + j] = mix[c];
                        if (yref_blk)
                            yref_blk[yo + j] = ref[r][c];
                    }
                }
            }

            // online softmax of y^mix and reference statistics
            bm = group16_max(bm);
            br = group16_max(br);
            const float mm_new = fmaxf(m_mix, bm);
            const float mr_new = fmaxf(m_ref, br);
            const double alpha = exp_delta(m_mix, mm_new, s_exp);
            // row factors; a factor that would overflow (maxima more than
            // ~700 apart) falls back to a direct exp per score
            const double f_lo = exp64_sum((double)mt_new - (double)mm_new, s_exp);
            const double f_ref = exp64_sum((double)mr_new - (double)mm_new, s_exp);
            const bool direct = !(f_lo < 1e300 && f_ref < 1e300);
            double sl = 0.0, sr = 0.0, sa = 0.0, sll = 0.0, sb = 0.0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pmix[r][c] = 0.0f;
                if (valid[c]) {
                    const double er = exp64_sum((double)ref[r][c] - (double)mr_new, s_exp);
                    double pe;
                    if (!direct)
                        pe = sel[c] ? er * f_ref : E[c] * f_lo;
                    else
                        pe = exp64_sum((double)mix[c] - (double)mm_new, s_exp);
                    pmix[r][c] = (float)pe;
                    sl += pe;
                    sr += er;
                    sa += er * ((double)ref[r][c] - (double)mix[c]);
                    sll += E[c];
                    sb += er * ((double)ref[r][c] - (double)lo[r][c]);
                }
            }
            sl = group16_sum(sl);
            sr = group16_sum(sr);
            sa = group16_sum(sa);
            if (want_lowp) {
                sll = group16_sum(sll);
                sb = group16_sum(sb);
            }
            if (i < S && tx == 0) {
                const double beta = exp_delta(m_ref, mr_new, s_exp);
                rs.l_mix = rs.l_mix * alpha + sl;
                rs.l_ref = rs.l_ref * beta + sr;
                rs.kl_a = rs.kl_a * beta + sa;
                if (want_lowp) {
                    rs.l_lo = rs.l_lo * exp_delta(m_t, mt_new, s_exp) + sll;
                    rs.kl_b = rs.kl_b * beta + sb;
                }
                rs.m_t = mt_new;
                rs.m_mix = mm_new;
                rs.m_ref = mr_new;
                rs.cnt += (uint32_t)(__popc(w0) + __popc(w1));
            }
            // rescale this row's P.V accumulators (MFMA rows 4*(lane/16)+r)
#pragma unroll
            for (int q = 0; q < NB; ++q)
                acc[q][r] *= (i < S) ? alpha : 0.0;
        };
        row_step(std::integral_constant<int, 0>{});
        row_step(std::integral_constant<int, 1>{});
        row_step(std::integral_constant<int, 2>{});
        row_step(std::integral_constant<int, 3>{});

        // V tile: loaded after the softmax epilogue (its registers would
        // otherwise stay live across it and spill), just before the P.V stage
        float4 vreg[V4];
#pragma unroll
        for (int u = 0; u < V4; ++u) {
            const int e = tid + u * kThreads;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < NV4 && col0 + key < S && col < D)
                x = *reinterpret_cast<const float4 *>(Vh + (size_t)(col0 + key) * D + col);
            vreg[u] = x;
        }

        // P.V: P tile (aliases the score staging) and V tile to LDS, MFMA.
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                sm.u.p[ty * 4 + r][tx + 16 * c] = pmix[r][c];
        // The causal diagonal tile holds keys past some rows' limits, whose
        // probability 0 would turn a non-finite V value into NaN (0 * inf) in
        // the product: such values are staged as 0 and added back at the end
        // for the rows that see their key.
        const bool diag = a.causal && t == qb;
#pragma unroll
        for (int u = 0; u < V4; ++u) {
            const int e = tid + u * kThreads;
            const int key = e / (DV / 4), col = (e % (DV / 4)) * 4;
            if (e < NV4) {
                float4 x = vreg[u];
                if (diag && !finite4(x)) {
                    x = finite_or_zero(x);
                    s_vbad = 1;
                }
                *reinterpret_cast<float4 *>(&sm.v[key][col]) = x;
            }
        }
        __syncthreads();
#pragma unroll
        for (int k16 = 0; k16 < kTile / 16; ++k16) {
            floatx4 part[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q)
                part[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int kk = k16 * 4 + k4;
                const float av = sm.u.p[wave * 16 + (lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    const float bv = sm.v[kk * 4 + (lane >> 4)][q * 16 + (lane & 15)];
                    part[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, part[q], 0, 0, 0);
                }
            }
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[q][v] += (double)part[q][v];
        }
    }

    // Finalise rows.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = row0 + ty * 4 + r;
        if (i >= S)
            continue;
        const RowState rs = sm.row[ty * 4 + r];
        const uint64_t row = (uint64_t)bh * S + i;
        if (a.mask)   // words of key tiles past the causal limit hold no selection
            for (int w = 2 * (t_end + 1) + tx; w < a.W; w += 16)
                a.mask[row * (uint64_t)a.W + w] = 0u;
        if (tx == 0) {
            const double lse_ref = (double)rs.m_ref + log(rs.l_ref);
            if (a.row_kl)
                a.row_kl[row] = rs.kl_a / rs.l_ref + ((double)rs.m_mix + log(rs.l_mix)) - lse_ref;
            if (want_lowp)
                a.row_kl_lowp[row] = rs.kl_b / rs.l_ref + ((double)rs.m_t + log(rs.l_lo)) - lse_ref;
            if (a.row_count)
                a.row_count[row] = rs.cnt;
            if (a.row_m)
                a.row_m[row] = rs.m_mix;
            if (a.row_l)
                a.row_l[row] = rs.l_mix;
        }
        // out rows of this lane's MFMA accumulators are 4*(lane/16)+r = ty*4+r
        const double inv = 1.0 / rs.l_mix;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int col = q * 16 + (lane & 15);
            if (col < D) {
                double o = acc[q][r];
                // non-finite V values of the diagonal tile, staged as 0: each
                // one at a key the row sees adds its infinity or NaN (what any
                // positive probability times it gives)
                if (s_vbad)
                    for (int j = row0; j <= i; ++j) {
                        const float x = Vh[(size_t)j * D + col];
                        if (!isfinite(x))
                            o += (double)x;
                    }
                a.out[row * (uint64_t)D + col] = (float)(o * inv);
            }
        }
    }
    add_ties(a.n_band, ties);
}

hipError_t launch_relaxed(const Problem &p, const uint8_t *unsafe, float *out, uint32_t *mask,
                          uint32_t *row_count, double *row_kl, double *row_kl_lowp,
                          float *ymix_raw, float *yref_out, float *row_m, double *row_l,
                          unsigned long long *exact_tiles, bool fast, hipStream_t st,
                          float *pzero)
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
    a.n_band = p.n_band;
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
    a.pzero = pzero;
    a.exact_tiles = exact_tiles;
    const uint64_t grid = (uint64_t)p.BH * p.tiles;
    const dim3 g((unsigned)grid), b(kThreads);
    if (fast && p.mu > 10)
        return hipSuccess;
#define LAMP_RELAXED_LAUNCH(NB, P)                                                         \
    do {                                                                                   \
        if (fast)                                                                          \
            hipLaunchKernelGGL((relaxed_kernel<NB, true, P>), g, b, 0, st, a);             \
        else                                                                               \
            hipLaunchKernelGGL((relaxed_kernel<NB, false, P>), g, b, 0, st, a);            \
    } while (0)
#define LAMP_RELAXED_LAUNCH_P(NB)                                                          \
    do {                                                                                   \
        switch (run_width(p.pc.blk)) {                                                     \
        case 0: LAMP_RELAXED_LAUNCH(NB, 0); break;                                         \
        case 4: LAMP_RELAXED_LAUNCH(NB, 4); break;                                         \
        case 8: LAMP_RELAXED_LAUNCH(NB, 8); break;                                         \
        case 16: LAMP_RELAXED_LAUNCH(NB, 16); break;                                       \
        default: LAMP_RELAXED_LAUNCH(NB, 32); break;                                       \
        }                                                                                  \
    } while (0)
    if (a.Dv <= 64)
        LAMP_RELAXED_LAUNCH_P(4);
    else
        LAMP_RELAXED_LAUNCH_P(8);
#undef LAMP_RELAXED_LAUNCH_P
#undef LAMP_RELAXED_LAUNCH
    return hipGetLastError();
}

// probs of the relaxed path from its raw y^mix and final row statistics:
// one wave per row, 16-byte loads and stores when rows are 16-byte aligned.
__global__ __launch_bounds__(kThreads) void normalise_kernel(const float *ymix, const float *row_m,
                                                             const double *row_l, float *probs,
                                                             int S, int causal, uint64_t n_rows,
                                                             int tail_done)
{
    const int lane = threadIdx.x & 63;
    // wave index through readfirstlane: the row's quantities are scalar
    const uint64_t r = (uint64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= n_rows)
        return;
    const int i = (int)(r % (uint64_t)S);
    const int n = causal ? i + 1 : S;
    // tail_done: the keys past the row's 64-key block hold zeros already
    const int jend = tail_done && causal ? min(S, (i / kTile + 1) * kTile) : S;
    const double shift = (double)row_m[r] + log(row_l[r]);
    const float *y = ymix + r * (uint64_t)S;
    float *pr = probs + r * (uint64_t)S;
    if ((S & 3) == 0) {
        for (int j = lane * 4; j < jend; j += 256) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < n)
                x = *reinterpret_cast<const float4 *>(y + j);
            float4 o;
            o.x = j < n ? exp_f32((double)x.x - shift) : 0.0f;
            o.y = j + 1 < n ? exp_f32((double)x.y - shift) : 0.0f;
            o.z = j + 2 < n ? exp_f32((double)x.z - shift) : 0.0f;
            o.w = j + 3 < n ? exp_f32((double)x.w - shift) : 0.0f;
            *reinterpret_cast<float4 *>(pr + j) = o;
        }
    } else {
        for (int j = lane; j < jend; j += 64)
            pr[j] = j < n ? exp_f32((double)y[j] - shift) : 0.0f;
    }
}

hipError_t launch_normalise(const Problem &p, const float *ymix, const float *row_m,
                            const double *row_l, float *probs, hipStream_t st, bool tail_done)
{
    const uint64_t grid = (p.n_rows + 3) / 4;
    hipLaunchKernelGGL(normalise_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, ymix, row_m,
                       row_l, probs, p.S, p.causal, p.n_rows, tail_done ? 1 : 0);
    return hipGetLastError();
}

}  // namespace lamp
