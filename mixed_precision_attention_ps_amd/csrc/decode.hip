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
//   2. decode_softmax_kernel, one work-group per (head, 256-key chunk): for
//      each query, the running maximum m_t of the relaxed rule (the prefix
//      maximum of the block maxima up to the key's 64-key block), the rule
//      2 exp(y^lo - m_t) |y^lo| > tau, the mask words, y^mix, the chunk's
//      softmax partial sums (of y^mix, y^ref and y^lo, each against the
//      chunk's own maximum) and its P.V partial, with each V row read once for
//      all queries.
//   3. decode_combine_kernel, one wave per (head, query): the chunk partials
//      rescaled to the global maxima: out, the row's log-sum-exp, the row KL
//      (FP32 reference vs LAMP, and vs all-low-precision) and the count.
//   4. decode_probs_kernel (only when probabilities are asked for).
#include "lamp_device.h"

namespace lamp {

constexpr int kDecChunk = 256;   // keys per work-group (one per thread)

struct DecodeArgs {
    const float *q, *k, *v;   // q [BH, nq, D]; k, v [BH, S, D]
    int S, D, nq, causal, n_chunks, n_blk;
    double tau;
    PsConst pc;
    float *ylo, *yref;        // [BH, nq, S]
    float *bmax;              // [BH, nq, n_blk]: max of valid y^lo per 64-key block
    uint32_t *mask;           // [BH, nq, W] or null
    int W;
    DecPartial *part;         // [BH, n_chunks, nq]
    double *acc;              // [BH, n_chunks, nq, D]
    unsigned long long *exact_chunks;
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
// ---------------------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(DecodeArgs a)
{
    __shared__ float4 s_q[NQ][64];    // the queries (D <= 256)
    __shared__ float4 s_qs[NQ][64];   // the queries times 2^(mu-23)
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = a.D, D4 = D / 4, nq = a.nq;
    const PsConst pc = a.pc;
    bool safe = true;
    for (int e = tid; e < nq * D4; e += kThreads) {
        const int t = e / D4, d4 = e % D4;
        const float4 x = reinterpret_cast<const float4 *>(a.q + ((size_t)bh * nq + t) * D)[d4];
        s_q[t][d4] = x;
        s_qs[t][d4] = make_float4(x.x * pc.qscale, x.y * pc.qscale, x.z * pc.qscale,
                                  x.w * pc.qscale);
        safe = safe && dec_safe(x.x) && dec_safe(x.y) && dec_safe(x.z) && dec_safe(x.w);
    }
    __syncthreads();

    const int j = chunk * kDecChunk + tid;
    const int jr = j < a.S ? j : a.S - 1;   // rows past S re-read the last row
    const float4 *k4 = reinterpret_cast<const float4 *>(a.k + ((size_t)bh * a.S + jr) * D);
    float lo[NQ], ref[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        lo[t] = 0.0f;
        ref[t] = 0.0f;
    }
    const bool fast = pc.mu <= 10;
    if (fast) {
        // FP32 fast path, 64 head-dimension entries of the key row at a time
        for (int d0 = 0; d0 < D4; d0 += 16) {
            float4 kr[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                kr[u] = d0 + u < D4 ? k4[d0 + u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < 16; ++u)
                safe = safe && dec_safe(kr[u].x) && dec_safe(kr[u].y) && dec_safe(kr[u].z) &&
                       dec_safe(kr[u].w);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (d0 + u >= D4)
                    break;
                const float ka[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    if (t < nq) {
                        const float4 qv = s_q[t][d0 + u], sv = s_qs[t][d0 + u];
                        const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
                        const float sa[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            ps_mac_fast(qa[e], sa[e], ka[e], lo[t], ref[t], pc.sh, pc.half_m1,
                                        pc.keep);
                    }
                }
            }
        }
    }
    // The exact path (mu > 10, or an operand outside the fast path's range
    // anywhere in this chunk or the queries): PS(mu) in double.
    const bool exact = !__syncthreads_and((fast && safe) ? 1 : 0);
    if (exact) {
        if (tid == 0 && a.exact_chunks)
            atomicAdd(a.exact_chunks, 1ull);
        double lod[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            lod[t] = 0.0;
            ref[t] = 0.0f;
        }
        for (int d4 = 0; d4 < D4; ++d4) {
            const float4 kv = k4[d4];
            const float ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                if (t < nq) {
                    const float4 qv = s_q[t][d4];
                    const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (pc.mu < 23) {
                            const double pr = (double)qa[e] * (double)ka[e];
                            lod[t] = ps_rn64(lod[t] + ps_rn64(pr, pc.mu), pc.mu);
                        }
                        const float p = qa[e] * ka[e];
                        ref[t] = ref[t] + p;
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            lo[t] = pc.mu < 23 ? (float)lod[t] * pc.s : ref[t] * pc.s;
    } else {
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            lo[t] = lo[t] * pc.out_scale;
    }

    const int lane = tid & 63;
    const int blk = (chunk * kDecChunk) / 64 + (tid >> 6);
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        if (t >= nq)
            break;
        const bool valid = j <= dec_last_key(a, t);
        const float yr = ref[t] * pc.s;
        const size_t row = (size_t)bh * nq + t;
        if (valid) {
            a.ylo[row * a.S + j] = lo[t];
            a.yref[row * a.S + j] = yr;
        }
        const float bm = wave_max(valid ? lo[t] : -INFINITY);
        if (lane == 0 && blk < a.n_blk)
            a.bmax[row * a.n_blk + blk] = bm;
    }
}

// ---------------------------------------------------------------------------
// 2. Relaxed selection, chunk softmax partials and P.V partial.
// ---------------------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(kThreads) void decode_softmax_kernel(DecodeArgs a)
{
    __shared__ float s_p[NQ][kDecChunk];   // exp(y^mix - chunk max), per query
    __shared__ float s_red[4][8];
    __shared__ double s_redd[4][8];
    __shared__ double s_acc[4][64];
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    exp_table_fill(s_exp);
    __syncthreads();
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = a.nq, S = a.S, D = a.D;
    const int j = chunk * kDecChunk + tid;
    const int blk0 = (chunk * kDecChunk) / 64;
    const int myblk = blk0 + wave;

    auto block_max = [&](float x) {
        x = wave_max(x);
        if (lane == 0)
            s_red[wave][0] = x;
        __syncthreads();
        x = fmaxf(fmaxf(s_red[0][0], s_red[1][0]), fmaxf(s_red[2][0], s_red[3][0]));
        __syncthreads();
        return x;
    };
    // five double sums at once over the work-group
    auto block_sum5 = [&](double (&x)[5]) {
#pragma unroll
        for (int e = 0; e < 5; ++e) {
            x[e] = wave_sum(x[e]);
            if (lane == 0)
                s_redd[wave][e] = x[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 5; ++e)
            x[e] = (s_redd[0][e] + s_redd[1][e]) + (s_redd[2][e] + s_redd[3][e]);
        __syncthreads();
    };

    for (int t = 0; t < nq; ++t) {
        const size_t row = (size_t)bh * nq + t;
        const int last = dec_last_key(a, t);
        const bool valid = j <= last;
        const float *bm = a.bmax + row * a.n_blk;
        // running maximum of the relaxed rule: prefix maximum of the block
        // maxima up to this key's block
        float carry = -INFINITY;
        for (int b = tid; b < blk0; b += kThreads)
            carry = fmaxf(carry, bm[b]);
        carry = block_max(carry);
        float mt = carry;
        for (int b = blk0; b <= myblk && b < a.n_blk; ++b)
            mt = fmaxf(mt, bm[b]);

        float ylo = 0.0f, yref = 0.0f;
        if (valid) {
            ylo = a.ylo[row * S + j];
            yref = a.yref[row * S + j];
        }
        const double E = valid ? exp64((double)ylo - (double)mt, s_exp) : 0.0;
        const bool sel = valid && 2.0 * E * fabs((double)ylo) > a.tau;
        const float ymix = sel ? yref : ylo;
        const uint64_t b = __ballot(sel);
        if (a.mask) {
            const int w = (chunk * kDecChunk + wave * 64) / 32 + lane;
            if (lane < 2 && w < a.W)
                a.mask[row * a.W + w] = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
        }
        if (sel)
            a.ylo[row * S + j] = ymix;   // y^lo becomes y^mix in place
        const float M_mix = block_max(valid ? ymix : -INFINITY);
        const float M_ref = block_max(valid ? yref : -INFINITY);
        const float M_lo = block_max(valid ? ylo : -INFINITY);
        const double em = valid ? exp64((double)ymix - (double)M_mix, s_exp) : 0.0;
        const double er = valid ? exp64((double)yref - (double)M_ref, s_exp) : 0.0;
        const double el = valid ? exp64((double)ylo - (double)M_lo, s_exp) : 0.0;
        s_p[t][tid] = (float)em;
        double sums[5] = {em, er, er * ((double)yref - (double)ymix), el,
                          er * ((double)yref - (double)ylo)};
        block_sum5(sums);
        if (lane == 0)
            s_red[wave][1] = __uint_as_float((uint32_t)__popcll(b));
        __syncthreads();
        if (tid == 0) {
            DecPartial pt;
            pt.m_mix = M_mix;
            pt.m_ref = M_ref;
            pt.m_lo = M_lo;
            pt.cnt = __float_as_uint(s_red[0][1]) + __float_as_uint(s_red[1][1]) +
                     __float_as_uint(s_red[2][1]) + __float_as_uint(s_red[3][1]);
            pt.l_mix = sums[0];
            pt.l_ref = sums[1];
            pt.a = sums[2];
            pt.l_lo = sums[3];
            pt.b = sums[4];
            a.part[((size_t)bh * a.n_chunks + chunk) * nq + t] = pt;
        }
        __syncthreads();
    }

    // P.V partial: thread (d = lane (+64 per pass), key group = wave) sums its
    // 64 keys in FP32 over 8 keys at a time, flushed into double.
    const int kb = chunk * kDecChunk + wave * 64;
    const int nk = max(0, min(64, S - kb));
    const float *Vh = a.v + (size_t)bh * S * D;
    for (int d0 = 0; d0 < D; d0 += 64) {
        const int d = d0 + lane;
        double accd[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t)
            accd[t] = 0.0;
        for (int k0 = 0; k0 < nk; k0 += 8) {
            float accf[NQ];
#pragma unroll
            for (int t = 0; t < NQ; ++t)
                accf[t] = 0.0f;
            const int k1 = min(nk, k0 + 8);
            for (int kk = k0; kk < k1; ++kk) {
                const float vv = d < D ? Vh[(size_t)(kb + kk) * D + d] : 0.0f;
#pragma unroll
                for (int t = 0; t < NQ; ++t)
                    if (t < nq)
                        accf[t] = __builtin_fmaf(s_p[t][wave * 64 + kk], vv, accf[t]);
            }
#pragma unroll
            for (int t = 0; t < NQ; ++t)
                accd[t] += (double)accf[t];
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            if (t >= nq)
                break;
            s_acc[wave][lane] = accd[t];
            __syncthreads();
            if (wave == 0 && d < D)
                a.acc[(((size_t)bh * a.n_chunks + chunk) * nq + t) * D + d] =
                    (s_acc[0][lane] + s_acc[1][lane]) + (s_acc[2][lane] + s_acc[3][lane]);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// 3. Combine the chunk partials: one wave per (head, query).
// ---------------------------------------------------------------------------
struct CombineArgs {
    const DecPartial *part;
    const double *acc;
    int nq, D, n_chunks, n_rows;
    float *out;
    double *row_lse;   // [BH, nq]: log-sum-exp of y^mix
    double *row_kl, *row_kl_lowp;
    uint32_t *row_count;
};

__global__ __launch_bounds__(kThreads) void decode_combine_kernel(CombineArgs a)
{
    __shared__ double s_exp[64];
    exp_table_fill(s_exp);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x * 4 + wave;   // (bh, t) row
    if (r >= a.n_rows)
        return;
    const int bh = r / a.nq, t = r % a.nq;
    auto P = [&](int c) -> const DecPartial & {
        return a.part[((size_t)bh * a.n_chunks + c) * a.nq + t];
    };
    float Mm = -INFINITY, Mr = -INFINITY, Ml = -INFINITY;
    for (int c = lane; c < a.n_chunks; c += 64) {
        Mm = fmaxf(Mm, P(c).m_mix);
        Mr = fmaxf(Mr, P(c).m_ref);
        Ml = fmaxf(Ml, P(c).m_lo);
    }
    Mm = wave_max(Mm);
    Mr = wave_max(Mr);
    Ml = wave_max(Ml);
    double Lm = 0.0, Lr = 0.0, A = 0.0, Ll = 0.0, B = 0.0;
    uint32_t cnt = 0;
    for (int c = lane; c < a.n_chunks; c += 64) {
        const DecPartial &p = P(c);
        if (p.m_mix == -INFINITY)
            continue;   // no valid key in this chunk
        const double fm = exp64_nonpos((double)p.m_mix - (double)Mm, s_exp);
        const double fr = exp64_nonpos((double)p.m_ref - (double)Mr, s_exp);
        const double fl = exp64_nonpos((double)p.m_lo - (double)Ml, s_exp);
        Lm += p.l_mix * fm;
        Lr += p.l_ref * fr;
        A += p.a * fr;
        Ll += p.l_lo * fl;
        B += p.b * fr;
        cnt += p.cnt;
    }
    Lm = wave_sum(Lm);
    Lr = wave_sum(Lr);
    A = wave_sum(A);
    Ll = wave_sum(Ll);
    B = wave_sum(B);
    cnt = (uint32_t)wave_sum_int((int)cnt);
    // out = sum_c exp(M_c - M) acc_c / L_mix
    const double inv = 1.0 / Lm;
    for (int d = lane; d < a.D; d += 64) {
        double o = 0.0;
        for (int c = 0; c < a.n_chunks; ++c) {
            const DecPartial &p = P(c);
            if (p.m_mix == -INFINITY)
                continue;
            const double fm = exp64_nonpos((double)p.m_mix - (double)Mm, s_exp);
            o += fm * a.acc[(((size_t)bh * a.n_chunks + c) * a.nq + t) * a.D + d];
        }
        a.out[(size_t)r * a.D + d] = (float)(o * inv);
    }
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

// ---------------------------------------------------------------------------
// 4. Probabilities: p = exp(y^mix - lse_mix) on valid keys, 0 elsewhere.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void decode_probs_kernel(const float *ymix,
                                                                const double *row_lse,
                                                                float *probs, int S, int nq,
                                                                int causal)
{
    const int r = blockIdx.y;   // (bh, t) row
    const int t = r % nq;
    const int last = causal ? S - nq + t : S - 1;
    const double lse = row_lse[r];
    for (int j = blockIdx.x * kThreads + threadIdx.x; j < S; j += gridDim.x * kThreads)
        probs[(size_t)r * S + j] =
            j <= last ? exp_f32((double)ymix[(size_t)r * S + j] - lse) : 0.0f;
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
    a.pc = make_ps_const(p.mu, p.D);
    a.ylo = b.ylo;
    a.yref = b.yref;
    a.bmax = b.bmax;
    a.mask = b.mask;
    a.W = (p.S + 31) / 32;
    a.part = b.part;
    a.acc = b.acc;
    a.exact_chunks = b.exact_chunks;
    if (a.n_chunks > 65535 * 32 || p.BH > 65535)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.n_chunks, (unsigned)p.BH), block(kThreads);
    hipError_t e;
    if ((e = rec(2 * 1)) != hipSuccess)   // scores stage
        return e;
#define LAMP_DEC_LAUNCH(K)                                                     \
    do {                                                                       \
        if (p.nq <= 1) hipLaunchKernelGGL((K<1>), grid, block, 0, st, a);      \
        else if (p.nq <= 2) hipLaunchKernelGGL((K<2>), grid, block, 0, st, a); \
        else if (p.nq <= 4) hipLaunchKernelGGL((K<4>), grid, block, 0, st, a); \
        else if (p.nq <= 8) hipLaunchKernelGGL((K<8>), grid, block, 0, st, a); \
        else hipLaunchKernelGGL((K<16>), grid, block, 0, st, a);               \
    } while (0)
    LAMP_DEC_LAUNCH(decode_scores_kernel);
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 1 + 1)) != hipSuccess ||
        (e = rec(2 * 2)) != hipSuccess)
        return e;
    LAMP_DEC_LAUNCH(decode_softmax_kernel);
#undef LAMP_DEC_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess || (e = rec(2 * 2 + 1)) != hipSuccess ||
        (e = rec(2 * 4)) != hipSuccess)
        return e;
    CombineArgs c;
    c.part = b.part;
    c.acc = b.acc;
    c.nq = p.nq;
    c.D = p.D;
    c.n_chunks = a.n_chunks;
    c.n_rows = p.BH * p.nq;
    c.out = b.out;
    c.row_lse = b.row_lse;
    c.row_kl = b.row_kl;
    c.row_kl_lowp = b.row_kl_lowp;
    c.row_count = b.row_count;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((c.n_rows + 3) / 4)), block, 0, st,
                       c);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (b.probs) {
        const unsigned gx = (unsigned)min(a.n_chunks, 64);
        hipLaunchKernelGGL(decode_probs_kernel, dim3(gx, (unsigned)(p.BH * p.nq)), block, 0, st,
                           b.ylo, b.row_lse, b.probs, p.S, p.nq, p.causal);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return rec(2 * 4 + 1);
}

}  // namespace lamp
