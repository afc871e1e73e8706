// decode.hip -- relaxed LAMP for decode shapes: a few new queries per head
// against a long key/value cache.
//
// LAMP summary, "Experimental results" (the relaxed relative-threshold rule,
// which drops the softmax normalisation so that selection needs no look-ahead
// over the row) and "Implementation strategy" steps 1-3, at the shape of
// autoregressive inference (the summary's closing remarks on deployment): Nq
// query rows per (batch, head), each the last Nq positions of a sequence of S
// keys.  Query t of a causal problem sees keys 0 .. S - Nq + t.
//
// The work is split along the keys (flash-decoding style), so that the whole
// GPU streams the cache once:
//   1. decode_scores_kernel, one work-group per (head, 256-key chunk): every
//      thread owns one key, loads its K row once and forms the PS(mu) and the
//      sequential FP32 score of that key against all Nq queries (queries
//      broadcast from LDS); y^lo, y^ref and the maximum of y^lo over each
//      64-key block go to HBM (4 + 4 bytes per score, next to 4 D / Nq bytes of
//      K).  The FP32 fast path is taken optimistically; a chunk that meets an
//      operand outside {0} U [2^-40, 2^40] (or any mu > 10) is redone on the
//      exact double path.
//   2. decode_softmax_kernel, one wave per (head, 64-key block), without
//      barriers: for each query, the running maximum m_t of the relaxed rule
//      (the prefix maximum of the block maxima up to the key's block), the rule
//      2 exp(y^lo - m_t) |y^lo| > tau, the mask words, y^mix, the block's
//      softmax partial sums (of y^mix, y^ref and y^lo, each against the
//      block's own maximum) and its P.V partial, with each V row read once for
//      all queries.
//   3. decode_combine_kernel, one work-group per (head, query): the block partials
//      rescaled to the global maxima: out, the row's log-sum-exp, the row KL
//      (FP32 reference vs LAMP, and vs all-low-precision) and the count.
//   4. decode_probs_kernel (only when probabilities are asked for).
#include "lamp_device.h"

namespace lamp {

constexpr int kDecChunk = 256;   // keys per work-group (one per thread)

struct DecodeArgs {
    const float *q, *k, *v;   // q [BH, nq, D]; k, v [BH, S, D]
    int S, D, nq, causal, n_chunks, n_blk, BH;
    double tau;
    PsConst pc;
    float *ylo, *yref;        // [BH, nq, S]
    float *bmax;              // [BH, nq, n_blk]: max of valid y^lo per 64-key block
    uint32_t *mask;           // [BH, nq, W] or null
    int W;
    uint8_t *unsafe;          // [BH, n_chunks]: chunk left to the exact kernel
    DecPartial *part;         // [BH, n_blk, nq]
    float *acc;               // [BH, n_blk, nq, D]
    unsigned long long *exact_chunks;
    unsigned long long *n_band;
};

// Keys 0 .. last_key(t) are valid for query t.
__device__ __forceinline__ int dec_last_key(const DecodeArgs &a, int t)
{
    return a.causal ? a.S - a.nq + t : a.S - 1;
}

// Zero, or a finite magnitude in [2^-40, 2^40] (the fast path's premise).
__device__ __forceinline__ bool dec_safe(float x)
{
    const uint32_t m = __float_as_uint(x) & 0x7fffffffu;
    return m == 0u || (m - 0x2b800000u) <= (0x53800000u - 0x2b800000u);
}

// ---------------------------------------------------------------------------
// 1. Scores.
//
// Fast kernel (mu <= 10): the chunk's K rows are staged through LDS in
// 32-wide head-dimension slices, loaded with coalesced 16-byte loads (a key's
// 128-byte slice segment by 8 neighbouring lanes) and stored transposed
// ([d][key], padded), so that thread = key reads its values conflict-free;
// the next slice is loaded while the current one is used.  Every loaded
// value and every query is checked against the fast path's operand range; a
// chunk that fails is flagged and left to the exact kernel, which strides
// over the flagged chunks (all chunks when mu > 10) and forms PS(mu) in
// double from each key's row.
// ---------------------------------------------------------------------------
// head-dimension entries of K per LDS pass: 32 (a full 128-byte line per key
// and load) for few queries, where the pass is bound by the cache stream; 16
// (half the LDS, more work-groups per CU) for many, where it is bound by ALU
template <int NQ>
constexpr int dec_slice() { return NQ <= 4 ? 32 : 16; }

template <int NQ>
__device__ __forceinline__ void dec_store_scores(const DecodeArgs &a, int bh, int chunk,
                                                 const float (&lo)[NQ], const float (&ref)[NQ])
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int j = chunk * kDecChunk + tid;
    const int blk = (chunk * kDecChunk) / 64 + (tid >> 6);
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        if (t >= a.nq)
            break;
        const bool valid = j <= dec_last_key(a, t);
        const size_t row = (size_t)bh * a.nq + t;
        if (valid) {
            a.ylo[row * a.S + j] = lo[t];
            a.yref[row * a.S + j] = ref[t] * a.pc.s;
        }
        const float bm = wave_max(valid ? lo[t] : -INFINITY);
        if (lane == 0 && blk < a.n_blk)
            a.bmax[row * a.n_blk + blk] = bm;
    }
}

// The queries and the queries times 2^(mu-23) into LDS (s_q[t * D/4 + d4],
// s_qs likewise), with the operand-range check of every value.
__device__ __forceinline__ void dec_stage_queries(const DecodeArgs &a, int bh, float4 *s_q,
                                                  float4 *s_qs, bool &safe)
{
    const int D4 = a.D / 4;
    const float4 *qb = reinterpret_cast<const float4 *>(a.q + (size_t)bh * a.nq * a.D);
    for (int e = threadIdx.x; e < a.nq * D4; e += kThreads) {
        const float4 x = qb[e];
        s_q[e] = x;
        s_qs[e] = make_float4(x.x * a.pc.qscale, x.y * a.pc.qscale, x.z * a.pc.qscale,
                              x.w * a.pc.qscale);
        safe = safe && dec_safe(x.x) && dec_safe(x.y) && dec_safe(x.z) && dec_safe(x.w);
    }
}

// Dynamic LDS of the score kernels: the two query arrays, nq * D / 4 float4
// each.
extern __shared__ float4 dec_dyn_lds[];

// BLOCKED: the blocked PS(mu) accumulation order (a.pc.blk >= 4, a power of
// two, so runs end only after the last of a group of 4 positions).
template <int NQ, bool BLOCKED>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(DecodeArgs a)
{
    constexpr int kDecSlice = dec_slice<NQ>();
    __shared__ float s_k[kDecSlice][kDecChunk + 1];   // K slice, [d][key]
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = a.D, S = a.S, D4 = D / 4;
    float4 *s_q = dec_dyn_lds, *s_qs = dec_dyn_lds + a.nq * D4;
    const PsConst pc = a.pc;
    bool safe = true;
    dec_stage_queries(a, bh, s_q, s_qs, safe);

    const int key0 = chunk * kDecChunk;
    constexpr int kV4 = kDecSlice * kDecChunk / 4 / kThreads;   // float4 per thread per slice
    auto load_slice = [&](int d0, float4 (&r)[kV4]) {
#pragma unroll
        for (int u = 0; u < kV4; ++u) {
            const int f = tid + kThreads * u;
            const int kk = f / (kDecSlice / 4), d = d0 + 4 * (f % (kDecSlice / 4));
            const int key = key0 + kk;
            r[u] = (key < S && d < D)
                       ? *reinterpret_cast<const float4 *>(a.k + ((size_t)bh * S + key) * D + d)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    float4 kr[kV4];
    load_slice(0, kr);
    float lo[NQ], ref[NQ], run[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        lo[t] = 0.0f;
        ref[t] = 0.0f;
        run[t] = 0.0f;
    }
    for (int d0 = 0; d0 < D; d0 += kDecSlice) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kV4; ++u) {
            const int f = tid + kThreads * u;
            const int kk = f / (kDecSlice / 4), dd = 4 * (f % (kDecSlice / 4));
            s_k[dd][kk] = kr[u].x;
            s_k[dd + 1][kk] = kr[u].y;
            s_k[dd + 2][kk] = kr[u].z;
            s_k[dd + 3][kk] = kr[u].w;
            safe = safe && dec_safe(kr[u].x) && dec_safe(kr[u].y) && dec_safe(kr[u].z) &&
                   dec_safe(kr[u].w);
        }
        __syncthreads();
        if (d0 + kDecSlice < D)
            load_slice(d0 + kDecSlice, kr);
        const int dn = min(kDecSlice, D - d0);   // a multiple of 4
        for (int dd = 0; dd < dn; dd += 4) {
            const float ka[4] = {s_k[dd][tid], s_k[dd + 1][tid], s_k[dd + 2][tid],
                                 s_k[dd + 3][tid]};
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                if (t < a.nq) {
                    const int qi = t * D4 + (d0 + dd) / 4;
                    const float4 qv = s_q[qi], sv = s_qs[qi];
                    const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
                    const float sa[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ps_mac_fast(qa[e], sa[e], ka[e], BLOCKED ? run[t] : lo[t], ref[t],
                                    pc.split);
                }
            }
            if (BLOCKED && ((d0 + dd + 4) & (pc.blk - 1)) == 0) {   // a run ends here
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    lo[t] = ps_round_split(lo[t] + run[t], pc.split);
                    run[t] = 0.0f;
                }
            }
        }
    }
    if (BLOCKED)   // the last run
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            lo[t] = ps_round_split(lo[t] + run[t], pc.split);
    const bool ok = __syncthreads_and(safe ? 1 : 0);
    if (tid == 0)
        a.unsafe[(size_t)bh * a.n_chunks + chunk] = ok ? 0 : 1;
    if (!ok)
        return;   // the exact kernel takes this chunk
#pragma unroll
    for (int t = 0; t < NQ; ++t)
        lo[t] = lo[t] * pc.out_scale;
    dec_store_scores<NQ>(a, bh, chunk, lo, ref);
}

// Exact path: PS(mu) in double (mu > 10, or a chunk the fast kernel flagged);
// plain FP32 at mu = 23.  A bounded grid strides over the chunks; each
// work-group first checks its chunks' flags in parallel and exits when none
// is its.
template <int NQ>
__global__ __launch_bounds__(kThreads) void decode_scores_exact_kernel(DecodeArgs a)
{
    const long long total = (long long)a.BH * a.n_chunks;
    const bool all = a.pc.mu > 10;
    if (!all) {
        bool need = false;
        for (long long g = blockIdx.x + (long long)threadIdx.x * gridDim.x; g < total;
             g += (long long)blockDim.x * gridDim.x)
            need |= a.unsafe[g] != 0;
        if (!__syncthreads_or(need ? 1 : 0))
            return;
    }
    const int tid = threadIdx.x, D = a.D, D4 = D / 4;
    float4 *s_q = dec_dyn_lds, *s_qs = dec_dyn_lds + a.nq * D4;
    const PsConst pc = a.pc;
    for (long long g = blockIdx.x; g < total; g += gridDim.x) {
        if (!all && !a.unsafe[g])
            continue;   // uniform over the work-group
        const int bh = (int)(g / a.n_chunks), chunk = (int)(g % a.n_chunks);
        bool unused = true;
        __syncthreads();   // the previous chunk's readers of s_q are done
        dec_stage_queries(a, bh, s_q, s_qs, unused);
        __syncthreads();
        if (tid == 0 && a.exact_chunks)
            atomicAdd(a.exact_chunks, 1ull);
        const int j = chunk * kDecChunk + tid;
        const int jr = j < a.S ? j : a.S - 1;   // rows past S re-read the last row
        const float4 *k4 = reinterpret_cast<const float4 *>(a.k + ((size_t)bh * a.S + jr) * D);
        // blocked order (pc.blk > 0): run sums rund (PS(mu)) / runf (mu = 23)
        // added into lod / lof where a run ends
        const bool blocked = pc.blk != 0;
        double lod[NQ], rund[NQ];
        float lo[NQ], ref[NQ], lof[NQ], runf[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            lod[t] = rund[t] = 0.0;
            ref[t] = lof[t] = runf[t] = 0.0f;
        }
        for (int d4 = 0; d4 < D4; ++d4) {
            const float4 kv = k4[d4];
            const float ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                if (t < a.nq) {
                    const float4 qv = s_q[t * D4 + d4];
                    const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (pc.mu < 23) {
                            const double pr = (double)qa[e] * (double)ka[e];
                            double &acc = blocked ? rund[t] : lod[t];
                            acc = ps_rn64(acc + ps_rn64(pr, pc.mu), pc.mu);
                        }
                        const float p = qa[e] * ka[e];
                        if (blocked)
                            runf[t] = runf[t] + p;
                        ref[t] = ref[t] + p;
                    }
                }
            }
            if (blocked && (((d4 + 1) * 4) & (pc.blk - 1)) == 0) {
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    lod[t] = ps_rn64(lod[t] + rund[t], pc.mu);
                    lof[t] = lof[t] + runf[t];
                    rund[t] = 0.0;
                    runf[t] = 0.0f;
                }
            }
        }
        if (blocked)   // the last run
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                lod[t] = ps_rn64(lod[t] + rund[t], pc.mu);
                lof[t] = lof[t] + runf[t];
            }
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            lo[t] = pc.mu < 23 ? (float)lod[t] * pc.s : (blocked ? lof[t] : ref[t]) * pc.s;
        dec_store_scores<NQ>(a, bh, chunk, lo, ref);
    }
}

// ---------------------------------------------------------------------------
// 2. Relaxed selection, softmax partials and P.V partial per 64-key block.
//
// Every wave owns one 64-key block (lane = key) and works alone: no barrier.
// For each query it forms the rule's running maximum (the prefix maximum of
// the block maxima), the rule, the mask words and y^mix (in place over y^lo),
// and the block's partial sums; then the block's P.V partial with lane = head
// dimension, the block's probabilities broadcast from LDS, each V row read
// once for all queries (FP32 over 8 keys at a time, flushed into double, the
// block total stored in FP32: at most 5.4e-7 of sum p|v| in all).
// ---------------------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(kThreads) void decode_softmax_kernel(DecodeArgs a)
{
    __shared__ float s_p[4][NQ][64];   // per wave: exp(y^mix - block max), per query
    __shared__ double s_exp[64];       // 2^(k/64) for exp64
    exp_table_fill(s_exp);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh = blockIdx.y;
    const int blk = blockIdx.x * 4 + wave;   // this wave's 64-key block
    if (blk >= a.n_blk)
        return;   // no barrier below
    const int nq = a.nq, S = a.S, D = a.D;
    const int j = blk * 64 + lane;
    uint32_t ties = 0;   // near ties of the criterion (wave-uniform)

    for (int t = 0; t < nq; ++t) {
        const size_t row = (size_t)bh * nq + t;
        const int last = dec_last_key(a, t);
        const bool valid = j <= last;
        const float *bm = a.bmax + row * a.n_blk;
        float mt = -INFINITY;
        for (int b = lane; b <= blk; b += 64)
            mt = fmaxf(mt, bm[b]);
        mt = wave_max(mt);

        float ylo = 0.0f, yref = 0.0f;
        if (valid) {
            ylo = a.ylo[row * S + j];
            yref = a.yref[row * S + j];
        }
        const double E = valid ? exp64_crit((double)ylo - (double)mt, s_exp) : 0.0;
        const double crit = 2.0 * E * fabs((double)ylo);
        const bool sel = valid && crit > a.tau;
        if (a.n_band)   // near ties are counted only for a summary
            ties += (uint32_t)__popcll(ballot(valid && near_tie(crit, a.tau)));
        const float ymix = sel ? yref : ylo;
        const uint64_t b = ballot(sel);
        if (a.mask) {
            const int w = blk * 2 + lane;
            if (lane < 2 && w < a.W)
                a.mask[row * a.W + w] = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
        }
        if (sel)
            a.ylo[row * S + j] = ymix;   // y^lo becomes y^mix in place
        const float M_mix = wave_max(valid ? ymix : -INFINITY);
        const float M_ref = wave_max(valid ? yref : -INFINITY);
        const float M_lo = wave_max(valid ? ylo : -INFINITY);
        const double em = valid ? exp64_sum_nonpos((double)ymix - (double)M_mix, s_exp) : 0.0;
        const double er = valid ? exp64_sum_nonpos((double)yref - (double)M_ref, s_exp) : 0.0;
        const double el = valid ? exp64_sum_nonpos((double)ylo - (double)M_lo, s_exp) : 0.0;
        s_p[wave][t][lane] = (float)em;
        const double l_mix = wave_sum(em);
        const double l_ref = wave_sum(er);
        const double sa = wave_sum(er * ((double)yref - (double)ymix));
        const double l_lo = wave_sum(el);
        const double sb = wave_sum(er * ((double)yref - (double)ylo));
        if (lane == 0) {
            DecPartial pt;
            pt.m_mix = M_mix;
            pt.m_ref = M_ref;
            pt.m_lo = M_lo;
            pt.cnt = (uint32_t)__popcll(b);
            pt.l_mix = l_mix;
            pt.l_ref = l_ref;
            pt.a = sa;
            pt.l_lo = l_lo;
            pt.b = sb;
            a.part[((size_t)bh * a.n_blk + blk) * nq + t] = pt;
        }
    }
    add_ties(a.n_band, ties);
    __builtin_amdgcn_wave_barrier();

    // P.V partial of this block
    const int nk = min(64, S - blk * 64);
    const float *Vb = a.v + ((size_t)bh * S + (size_t)blk * 64) * D;
    // a block with keys past some query's limit, or past S (the first
    // query's limit is the smallest)
    const bool edge = blk * 64 + 63 > dec_last_key(a, 0);
    for (int d0 = 0; d0 < D; d0 += 64) {
        const int d = d0 + lane;
        double accd[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            accd[t] = 0.0;
        // 32 V rows in flight per lane, consumed 8 keys per FP32 partial
        for (int k0 = 0; k0 < nk; k0 += 32) {
            // rows past the block's keys re-read its last row (their
            // probabilities are 0) and lanes past D re-read column D - 1
            // (not stored), so the loads need no guard
            float vv[32];
#pragma unroll
            for (int u = 0; u < 32; ++u)
                vv[u] = Vb[(size_t)min(k0 + u, nk - 1) * D + min(d, D - 1)];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int kg = k0 + 8 * g;
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    if (t < nq) {
                        const float4 p0 = *reinterpret_cast<const float4 *>(&s_p[wave][t][kg]);
                        const float4 p1 =
                            *reinterpret_cast<const float4 *>(&s_p[wave][t][kg + 4]);
                        const float pa[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                        float f = 0.0f;
                        if (edge) {
                            // keys past this query's limit (or past S) carry
                            // probability 0: their V value is left out, so a
                            // non-finite one cannot turn 0 * inf into NaN
                            const int lim = dec_last_key(a, t) - blk * 64;
#pragma unroll
                            for (int u = 0; u < 8; ++u)
                                f = __builtin_fmaf(pa[u], kg + u <= lim ? vv[8 * g + u] : 0.0f,
                                                   f);
                        } else {
#pragma unroll
                            for (int u = 0; u < 8; ++u)
                                f = __builtin_fmaf(pa[u], vv[8 * g + u], f);
                        }
                        accd[t] += (double)f;
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            if (t < nq && d < D)
                a.acc[(((size_t)bh * a.n_blk + blk) * nq + t) * D + d] = (float)accd[t];
    }
}

// ---------------------------------------------------------------------------
// 3. Combine the block partials.
// ---------------------------------------------------------------------------
struct CombineArgs {
    const DecPartial *part;
    const float *acc;
    int nq, D, n_blk, n_rows;
    float *out;
    double *row_lse;   // [BH, nq]: log-sum-exp of y^mix
    double *row_kl, *row_kl_lowp;
    uint32_t *row_count;
};

constexpr int kCombineSeg = 1024;   // block factors staged in LDS at a time

// One work-group per (head, query) row.  The statistics: every thread takes
// blocks c = tid (mod 256).  The output: thread (d = lane, part = wave) sums
// the blocks c = part (mod 4), eight at a time (independent loads in flight).
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(CombineArgs a)
{
    __shared__ double s_exp[64];
    __shared__ float s_m[3][4];
    __shared__ double s_s[5][4];
    __shared__ uint32_t s_c[4];
    __shared__ double s_o[4][64];
    __shared__ float s_f[kCombineSeg];   // exp(m_mix of block - M) per block
    exp_table_fill(s_exp);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;   // (bh, t) row
    const int bh = r / a.nq, t = r % a.nq;
    auto P = [&](int c) -> const DecPartial & {
        return a.part[((size_t)bh * a.n_blk + c) * a.nq + t];
    };
    float Mm = -INFINITY, Mr = -INFINITY, Ml = -INFINITY;
    for (int c = tid; c < a.n_blk; c += kThreads) {
        Mm = fmaxf(Mm, P(c).m_mix);
        Mr = fmaxf(Mr, P(c).m_ref);
        Ml = fmaxf(Ml, P(c).m_lo);
    }
    Mm = wave_max(Mm);
    Mr = wave_max(Mr);
    Ml = wave_max(Ml);
    if (lane == 0) {
        s_m[0][wave] = Mm;
        s_m[1][wave] = Mr;
        s_m[2][wave] = Ml;
    }
    __syncthreads();
    Mm = fmaxf(fmaxf(s_m[0][0], s_m[0][1]), fmaxf(s_m[0][2], s_m[0][3]));
    Mr = fmaxf(fmaxf(s_m[1][0], s_m[1][1]), fmaxf(s_m[1][2], s_m[1][3]));
    Ml = fmaxf(fmaxf(s_m[2][0], s_m[2][1]), fmaxf(s_m[2][2], s_m[2][3]));
    double sum[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    uint32_t cnt = 0;
    for (int c = tid; c < a.n_blk; c += kThreads) {
        const DecPartial &p = P(c);
        if (p.m_mix == -INFINITY)
            continue;   // no valid key in this block
        const double fm = exp64_sum_nonpos((double)p.m_mix - (double)Mm, s_exp);
        const double fr = exp64_sum_nonpos((double)p.m_ref - (double)Mr, s_exp);
        const double fl = exp64_sum_nonpos((double)p.m_lo - (double)Ml, s_exp);
        sum[0] += p.l_mix * fm;
        sum[1] += p.l_ref * fr;
        sum[2] += p.a * fr;
        sum[3] += p.l_lo * fl;
        sum[4] += p.b * fr;
        cnt += p.cnt;
    }
#pragma unroll
    for (int e = 0; e < 5; ++e) {
        sum[e] = wave_sum(sum[e]);
        if (lane == 0)
            s_s[e][wave] = sum[e];
    }
    cnt = (uint32_t)wave_sum_int((int)cnt);
    if (lane == 0)
        s_c[wave] = cnt;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 5; ++e)
        sum[e] = (s_s[e][0] + s_s[e][1]) + (s_s[e][2] + s_s[e][3]);
    cnt = s_c[0] + s_c[1] + s_c[2] + s_c[3];
    const double Lm = sum[0], Lr = sum[1], A = sum[2], Ll = sum[3], B = sum[4];

    // out = sum_c exp(M_c - M) acc_c / L_mix; the block factors go through
    // LDS in segments of kCombineSeg blocks
    const double inv = 1.0 / Lm;
    for (int d0 = 0; d0 < a.D; d0 += 64) {
        const int d = d0 + lane;
        double o = 0.0;
        for (int c0 = 0; c0 < a.n_blk; c0 += kCombineSeg) {
            const int nc = min(kCombineSeg, a.n_blk - c0);
            __syncthreads();   // the previous segment's readers are done
            for (int c = tid; c < nc; c += kThreads) {
                const float m = P(c0 + c).m_mix;
                s_f[c] = m == -INFINITY ? 0.0f
                                        : (float)exp64_sum_nonpos((double)m - (double)Mm, s_exp);
            }
            __syncthreads();
            if (d < a.D) {
                const float *ac = a.acc + (((size_t)bh * a.n_blk + c0) * a.nq + t) * a.D + d;
                const size_t stride = (size_t)a.nq * a.D;
                for (int cb = wave * 8; cb < nc; cb += 32) {
                    float x[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        x[u] = cb + u < nc ? ac[(size_t)(cb + u) * stride] : 0.0f;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (cb + u < nc)
                            o += (double)s_f[cb + u] * (double)x[u];
                }
            }
        }
        s_o[wave][lane] = o;
        __syncthreads();
        if (wave == 0 && d < a.D)
            a.out[(size_t)r * a.D + d] =
                (float)(((s_o[0][lane] + s_o[1][lane]) + (s_o[2][lane] + s_o[3][lane])) * inv);
        __syncthreads();
    }
    if (wave == 0) {
        const double lg = log(lane == 0 ? Lm : (lane == 1 ? Lr : Ll));
        const double lse_mix = (double)Mm + lane_read(lg, 0);
        const double lse_ref = (double)Mr + lane_read(lg, 1);
        const double lse_lo = (double)Ml + lane_read(lg, 2);
        if (lane == 0) {
            if (a.row_lse)
                a.row_lse[r] = lse_mix;
            if (a.row_count)
                a.row_count[r] = cnt;
            if (a.row_kl)
                a.row_kl[r] = A / Lr + lse_mix - lse_ref;
            if (a.row_kl_lowp)
                a.row_kl_lowp[r] = B / Lr + lse_lo - lse_ref;
        }
    }
}

// ---------------------------------------------------------------------------
// 4. Probabilities: p = exp(y^mix - lse_mix) on valid keys, 0 elsewhere.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void decode_probs_kernel(const float *ymix,
                                                                const double *row_lse,
                                                                float *probs, int S, int nq,
                                                                int causal)
{
    // work-group (x, r): keys 1024 x .. 1024 x + 1023 of row r, 4 per thread
    const int r = blockIdx.y;
    const int t = r % nq;
    const int last = causal ? S - nq + t : S - 1;
    const double lse = row_lse[r];
    const float *y = ymix + (size_t)r * S;
    float *pr = probs + (size_t)r * S;
    const int j0 = blockIdx.x * 4 * kThreads + threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = j0 + e * kThreads;
        if (j < S)
            pr[j] = j <= last ? exp_f32((double)y[j] - lse) : 0.0f;
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_decode(const DecodeProblem &p, const DecodeBuffers &b, hipStream_t st,
                         void **stage_events)
{
    auto rec = [&](int e) {
        return stage_events ? hipEventRecord((hipEvent_t)stage_events[e], st) : hipSuccess;
    };
    DecodeArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.S = p.S;
    a.D = p.D;
    a.nq = p.nq;
    a.causal = p.causal;
    a.n_chunks = (p.S + kDecChunk - 1) / kDecChunk;
    a.n_blk = (p.S + 63) / 64;
    a.tau = (double)p.tau;
    a.n_band = p.n_band;
    a.pc = make_ps_const(p.mu, p.D);
    set_ps_block(a.pc, p.ps_block, p.D);
    a.ylo = b.ylo;
    a.yref = b.yref;
    a.bmax = b.bmax;
    a.mask = b.mask;
    a.W = (p.S + 31) / 32;
    a.part = b.part;
    a.acc = b.acc;
    a.exact_chunks = b.exact_chunks;
    a.unsafe = b.unsafe;
    a.BH = p.BH;
    if (a.n_chunks > 65535 * 32 || p.BH > 65535)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.n_chunks, (unsigned)p.BH), block(kThreads);
    hipError_t e;
    if ((e = rec(2 * 1)) != hipSuccess)   // scores stage
        return e;
    const size_t qlds = 2 * sizeof(float4) * (size_t)p.nq * (p.D / 4);
#define LAMP_DEC_LAUNCH(K, BLK)                                                        \
    do {                                                                               \
        if (p.nq <= 1) hipLaunchKernelGGL((K<1, BLK>), grid, block, qlds, st, a);      \
        else if (p.nq <= 2) hipLaunchKernelGGL((K<2, BLK>), grid, block, qlds, st, a); \
        else if (p.nq <= 4) hipLaunchKernelGGL((K<4, BLK>), grid, block, qlds, st, a); \
        else if (p.nq <= 8) hipLaunchKernelGGL((K<8, BLK>), grid, block, qlds, st, a); \
        else hipLaunchKernelGGL((K<16, BLK>), grid, block, qlds, st, a);               \
    } while (0)
    if (p.mu <= 10) {
        if (a.pc.blk != 0)
            LAMP_DEC_LAUNCH(decode_scores_kernel, true);
        else
            LAMP_DEC_LAUNCH(decode_scores_kernel, false);
    }
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 1 + 1)) != hipSuccess ||
        (e = rec(2 * 6)) != hipSuccess)   // exact stage
        return e;
    {
        const long long total = (long long)p.BH * a.n_chunks;
        const dim3 ge((unsigned)(total < 2048 ? total : 2048));
#define LAMP_DEC_LAUNCH_E(K)                                                    \
    do {                                                                        \
        if (p.nq <= 1) hipLaunchKernelGGL((K<1>), ge, block, qlds, st, a);      \
        else if (p.nq <= 2) hipLaunchKernelGGL((K<2>), ge, block, qlds, st, a); \
        else if (p.nq <= 4) hipLaunchKernelGGL((K<4>), ge, block, qlds, st, a); \
        else if (p.nq <= 8) hipLaunchKernelGGL((K<8>), ge, block, qlds, st, a); \
        else hipLaunchKernelGGL((K<16>), ge, block, qlds, st, a);               \
    } while (0)
        LAMP_DEC_LAUNCH_E(decode_scores_exact_kernel);
#undef LAMP_DEC_LAUNCH_E
    }
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 6 + 1)) != hipSuccess ||
        (e = rec(2 * 2)) != hipSuccess)
        return e;
    const dim3 grid2((unsigned)((a.n_blk + 3) / 4), (unsigned)p.BH);
#define LAMP_DEC_LAUNCH2(K)                                                     \
    do {                                                                        \
        if (p.nq <= 1) hipLaunchKernelGGL((K<1>), grid2, block, 0, st, a);      \
        else if (p.nq <= 2) hipLaunchKernelGGL((K<2>), grid2, block, 0, st, a); \
        else if (p.nq <= 4) hipLaunchKernelGGL((K<4>), grid2, block, 0, st, a); \
        else if (p.nq <= 8) hipLaunchKernelGGL((K<8>), grid2, block, 0, st, a); \
        else hipLaunchKernelGGL((K<16>), grid2, block, 0, st, a);               \
    } while (0)
    LAMP_DEC_LAUNCH2(decode_softmax_kernel);
#undef LAMP_DEC_LAUNCH2
#undef LAMP_DEC_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 2 + 1)) != hipSuccess ||
        (e = rec(2 * 4)) != hipSuccess)
        return e;
    CombineArgs c;
    c.part = b.part;
    c.acc = b.acc;
    c.nq = p.nq;
    c.D = p.D;
    c.n_blk = a.n_blk;
    c.n_rows = p.BH * p.nq;
    c.out = b.out;
    c.row_lse = b.row_lse;
    c.row_kl = b.row_kl;
    c.row_kl_lowp = b.row_kl_lowp;
    c.row_count = b.row_count;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)c.n_rows), block, 0, st, c);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (b.probs) {
        const dim3 gp((unsigned)((p.S + 4 * kThreads - 1) / (4 * kThreads)),
                      (unsigned)(p.BH * p.nq));
        hipLaunchKernelGGL(decode_probs_kernel, gp, block, 0, st, b.ylo, b.row_lse, b.probs, p.S,
                           p.nq, p.causal);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return rec(2 * 4 + 1);
}

}  // namespace lamp
