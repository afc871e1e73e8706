// rows.hip -- fused row pass for rows of at most 1024 keys.
//
// LAMP summary, "Implementation strategy": step 2 (look-ahead selection from
// the baseline output, with the softmax rule of "Theoretical foundation" item
// 3: recompute y_j iff 2 z_j (1 - z_j) |y_j| > tau; or the relaxed
// relative-threshold rule of "Experimental results", read as 2 exp(y_j - m_t)
// |y_j| > tau with m_t the running maximum over the 64-key blocks up to j's)
// and step 3 (recompute the selected components at FP32, then apply f), for
// one attention row per wave:
//   * the row's PS(mu) scores stay in registers (16 per lane);
//   * its softmax statistics are formed in double (own exp);
//   * the criterion gives the mask words (ballots) and a compacted list of the
//     selected keys in LDS (ballot + lane prefix);
//   * the selected scores are recomputed by a gather FP32 dot (sequential,
//     multiply then add), one lane per listed key; each one's exp(y_hi - m)
//     goes into its list slot and its y_hi into y^mix (when asked for);
//   * the row's log-sum-exp is corrected for the changed terms (or recomputed
//     over the row when the correction would cancel or overflow);
//   * probabilities are written as full rows (zeros past the valid keys);
//   * the row KLs against the FP32 reference use the reference statistics the
//     score kernel left per 64-key tile.
#include "lamp_device.h"

namespace lamp {

constexpr int kRowChunk = 16;   // keys per lane: rows of at most 1024 keys

struct RowsArgs {
    const float *q, *k, *ylo, *yref;
    const RefPartial *part;
    int S, D, causal, tiles, W;
    uint64_t n_rows;
    double tau;
    float s;
    uint32_t *mask, *row_count;
    float *pbuf, *ymix_out;
    double *row_kl, *row_kl_lowp;
    unsigned long long *n_band;
};

// D4 = D / 4 when the head dimension is a compile-time constant (all loads of
// a recomputed dot issue back to back), 0 for a runtime D.
//
// Register discipline: the loops over a lane's 16 keys are unrolled (the row
// lives in registers) and guarded only by wave-uniform conditions (the chunk
// holds valid keys); per-key validity is a select, never a branch, and the
// per-chunk selection is kept as one bit per lane rather than as 16 wave
// masks (a chunk's mask is re-formed by a ballot when needed).  Scalar
// registers then hold no per-chunk state.
//
// Probabilities: p_j = exp(y_j - lse_mix) = e_j / L_mix for every key whose
// score did not change (e_j = exp(y_j - m), kept in FP32 after the criterion),
// and e_hi / L_mix for a recomputed key (e_hi = exp(y_hi - m) formed in the
// recompute loop and kept, rounded to FP32, in the LDS list).  Only a row
// that takes the full pass (the correction would cancel or overflow)
// evaluates exp(y - lse_mix) per key; it forms its recomputed scores a second
// time, since the list then holds e_hi.
//
// The kernel is bound by VALU issue (about 1,400 wave instructions per row of
// 1,024 keys): one double exponential per valid key, none in the probability
// loop.
//
// RELAXED: the selection uses exp(y_j - m_t) = e_j exp(m - m_t), with the
// block maxima of y^lo taken from the score tiles' per-tile partials (lane t
// holds block t's; a prefix maximum across lanes gives m_t); keys where that
// product would lose precision (e_j below 1e-300, or a row whose factor
// overflows) take exp(y_j - m_t) directly.  Everything after the selection is
// the strict pass's.
template <int D4, bool RELAXED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void strict_rows_kernel(RowsArgs a)
{
    // per wave: the selected keys (compacted, in key order), and per listed
    // key e_hi = exp(y_hi - m) in FP32 (full-pass rows: y_hi)
    __shared__ uint16_t s_key[4][64 * kRowChunk];
    __shared__ float s_val[4][64 * kRowChunk];
    __shared__ float4 s_q[4][64];                    // the wave's query row (D <= 256)
    __shared__ double s_exp[64];                     // 2^(k/64) for exp64
    exp_table_fill(s_exp);
    __syncthreads();
    // the wave index is uniform: readfirstlane tells the compiler so, which
    // makes the row, its length and every chunk guard scalar
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // rows in descending order: the launch ends on the short rows at the top
    // of the first head (causal work grows with the row index)
    const uint64_t rr = (uint64_t)blockIdx.x * 4 + wave;
    if (rr >= a.n_rows)
        return;   // no block barrier below: each wave owns its row
    const uint64_t r = a.n_rows - 1 - rr;
    const int S = a.S;
    const int i = (int)(r % (uint64_t)S);
    const int n = a.causal ? i + 1 : S;
    const int nch = (n + 63) >> 6;   // chunks of 64 keys holding valid keys
    const float *y = a.ylo + r * (uint64_t)S;
    // the row's valid scores and its probabilities, as buffer ranges: loads
    // past the valid keys read 0 and stores past the row are dropped, with
    // no branch (a guarded load would wait for its data before the next one)
    const __amdgpu_buffer_rsrc_t y_rs = row_rsrc(y, 4u * (uint32_t)n);
    const __amdgpu_buffer_rsrc_t p_rs = row_rsrc(a.pbuf + r * (uint64_t)S, 4u * (uint32_t)S);

    // The row and its maximum (all 16 loads issued back to back).  This
    // lane's per-tile partial of the score kernel (tile = lane) is read here
    // by the relaxed pass (its selection needs the block maxima), after the
    // selection by the strict one.
    float v[kRowChunk];
#pragma unroll
    for (int t = 0; t < kRowChunk; ++t)
        v[t] = buf_load_f32(y_rs, 4u * (uint32_t)(lane + 64 * t));
    RefPartial early{0.0, 0.0, -INFINITY, -INFINITY};
    if constexpr (RELAXED)
        if (lane < nch)   // nch = the tiles that hold valid keys
            early = a.part[r * (uint64_t)a.tiles + lane];
    // Key lane + 64 t is valid iff 64 t < n - lane.  Each loop below forms
    // n - lane from its own opaque copy of n, so the chunk compares are
    // formed where they are used instead of being kept, 16 mask pairs at a
    // time, in scalar registers across the loops (which spilled them).
    auto fresh = [&]() {
        int x = n;
        asm volatile("" : "+s"(x));
        return x - lane;
    };
    float m = -INFINITY;
    {
        const int rem = fresh();
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            v[t] = 64 * t < rem ? v[t] : -INFINITY;
            m = fmaxf(m, v[t]);
        }
    }
    m = wave_max(m);

    // e_j = exp(y_j - m); A = sum below the maximum; cnt = keys at it.  The
    // keys past n hold -inf and give e = 0.  A NaN score gives e = 0 here and
    // makes the whole row NaN below (through A).
    double e[kRowChunk];
    double A = 0.0;
    int cnt = 0;
    bool has_nan = false;
    const int rem_e = fresh();
#pragma unroll
    for (int t = 0; t < kRowChunk; ++t) {
        e[t] = 0.0;
        if (t < nch) {
            const bool at = 64 * t < rem_e && v[t] == m;
            const double x = exp64_nonpos((double)v[t] - (double)m, s_exp);
            e[t] = at ? 1.0 : x;
            A += at ? 0.0 : x;
            cnt += __popcll(__ballot(at));
            has_nan |= v[t] != v[t];
        }
    }
    A = wave_sum(A);
    const bool row_nan = __ballot(has_nan) != 0;
    if (row_nan)
        A = __builtin_nan("");
    const double L = A + (double)cnt;
    const double rest_at_max = A + (double)(cnt - 1);

    // Relaxed rule: m_t of chunk t (= 64-key block t) on lane t, the prefix
    // maximum of the block maxima; f_t = exp(m - m_t) >= 1.
    float mt = -INFINITY;
    double ft = 1.0;
    bool direct_row = false;
    if constexpr (RELAXED) {
        mt = early.m_lo;
#pragma unroll
        for (int off = 1; off < kRowChunk; off <<= 1) {
            const float o = __shfl_up(mt, off, 64);
            if (lane >= off)
                mt = fmaxf(mt, o);
        }
        ft = lane < nch ? exp64((double)m - (double)mt, s_exp) : 1.0;
        direct_row = __ballot(lane < nch && !(ft < 1e300)) != 0;
    }

    // Strict criterion 2 z (1 - z) |y| > tau with z = e / L and 1 - z =
    // rest / L, evaluated as e rest |y| > tau L^2 / 2; relaxed criterion
    // 2 exp(y - m_t) |y| > tau.  Mask words and compaction.  e in FP32 is
    // kept for the probabilities (p = e / L_mix).
    const double tau_l2 = a.tau * (L * L) * 0.5;
    uint32_t selbits = 0;
    uint32_t total = 0;
    uint32_t ties = 0;
    float ef[kRowChunk];
    const int rem_c = fresh();
#pragma unroll
    for (int t = 0; t < kRowChunk; ++t) {
        const int j0 = 64 * t;
        ef[t] = 0.0f;
        if (t < nch) {   // chunks past the valid keys: zero mask words below
            const int j = j0 + lane;
            const bool valid = j0 < rem_c;
            bool sel;
            if constexpr (RELAXED) {
                ef[t] = (float)e[t];
                double E = e[t] * lane_read(ft, t);
                const bool dir = valid && (direct_row || e[t] < 1e-300);
                if (__ballot(dir) != 0) {
                    const float mtt = lane_read(mt, t);
                    if (dir)
                        E = exp64((double)v[t] - (double)mtt, s_exp);
                }
                const double crit = 2.0 * E * fabs((double)v[t]);
                sel = valid && crit > a.tau;
                ties += (uint32_t)__popcll(__ballot(valid && near_tie(crit, a.tau)));
            } else {
                const bool at = valid && v[t] == m;
                ef[t] = (float)e[t];
                const double rest = at ? rest_at_max : L - e[t];
                const double crit = e[t] * rest * fabs((double)v[t]);
                sel = valid && crit > tau_l2;
                ties += (uint32_t)__popcll(__ballot(valid && near_tie(crit, tau_l2)));
            }
            const uint64_t b = __ballot(sel);
            if (a.mask) {
                const int w = (j0 >> 5) + lane;
                if (lane < 2 && w < a.W)
                    a.mask[r * (uint64_t)a.W + w] = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
            }
            if (sel)
                s_key[wave][total + lanes_below(b)] = (uint16_t)j;
            selbits |= (sel ? 1u : 0u) << t;
            total += (uint32_t)__popcll(b);
        }
    }
    if (a.mask)   // the mask words of the chunks past the valid keys
        for (int w = 2 * nch + lane; w < a.W; w += 64)
            a.mask[r * (uint64_t)a.W + w] = 0u;
    add_ties(a.n_band, ties);

    // Reference statistics from the score kernel's per-tile partials.
    const bool kl = a.part != nullptr && (a.row_kl || a.row_kl_lowp);
    double Lr = 1.0, Br = 0.0;
    float mr = 0.0f;
    if (kl) {
        const int nt = a.causal ? (i / kTile) + 1 : a.tiles;
        RefPartial mine{0.0, 0.0, -INFINITY, 0.0f};
        if constexpr (RELAXED)
            mine = early;
        else if (lane < nt)
            mine = a.part[r * (uint64_t)a.tiles + lane];
        mr = wave_max(mine.m);
        const double f = lane < nt ? exp64_nonpos((double)mine.m - (double)mr, s_exp) : 0.0;
        Lr = wave_sum(mine.L * f);
        Br = wave_sum(mine.B * f);
    }

    // FP32 recompute of the selected keys (one lane per key): read from the
    // reference scores when the score tiles kept them (the same sequential
    // FP32 dot, so the same bits), else a gather dot with the query row read
    // from LDS and each key row in batches of up to 4 x 16 bytes issued back
    // to back.
    const uint64_t bh = r / (uint64_t)S;
    const float *yr = a.yref ? a.yref + r * (uint64_t)S : nullptr;
    if (!yr) {
        const float4 *qg = reinterpret_cast<const float4 *>(a.q + r * (uint64_t)a.D);
        if (lane < a.D / 4)
            s_q[wave][lane] = qg[lane];
    }
    const float4 *q4 = s_q[wave];
    // y_hi of key j: sequential FP32 dot (multiply, then add, d ascending)
    auto dot_hi = [&](uint32_t j) {
        const float4 *k4 = reinterpret_cast<const float4 *>(a.k + (bh * (uint64_t)S + j) * a.D);
        float acc = 0.0f;
        auto mac4 = [&acc](float4 x, float4 z) {
            float p0 = x.x * z.x;
            acc = acc + p0;
            float p1 = x.y * z.y;
            acc = acc + p1;
            float p2 = x.z * z.z;
            acc = acc + p2;
            float p3 = x.w * z.w;
            acc = acc + p3;
        };
        if constexpr (D4 > 0) {
            // opaque zero offset: keeps the query-row LDS reads inside the
            // loop instead of 4*D4 registers hoisted out of it
            uint32_t qoff = 0;
            asm volatile("" : "+v"(qoff));
            constexpr int kB = 4;   // D4 is a multiple of 4
#pragma unroll
            for (int b0 = 0; b0 < D4; b0 += kB) {
                float4 kr[kB];
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    kr[u] = k4[b0 + u];
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    mac4(q4[qoff + b0 + u], kr[u]);
            }
        } else {
            for (int d4 = 0; d4 < a.D / 4; ++d4)
                mac4(q4[d4], k4[d4]);
        }
        return acc * a.s;
    };
    double dL = 0.0, dA = 0.0;
    for (uint32_t ei = lane; ei < total; ei += 64) {
        const uint32_t j = s_key[wave][ei];
        const float yl = y[j];
        const float yhi = yr ? yr[j] : dot_hi(j);
        const double ehi = exp64((double)yhi - (double)m, s_exp);
        s_val[wave][ei] = (float)ehi;
        if (a.ymix_out)   // y^mix is y^lo in place: only recomputed keys change
            a.ymix_out[r * (uint64_t)S + j] = yhi;
        dL += ehi - exp64_nonpos((double)yl - (double)m, s_exp);
        if (kl)
            dA += exp64((double)yhi - (double)mr, s_exp) * ((double)yhi - (double)yl);
    }
    dL = wave_sum(dL);
    dA = wave_sum(dA);
    __builtin_amdgcn_wave_barrier();

    // Slot in the compacted list of this lane's key in chunk t (meaningful
    // when the key is selected), given the chunk's selection mask b and the
    // number of keys selected in the chunks before it.
    auto slot = [&](uint64_t b, uint32_t before) {
        return min(before + lanes_below(b), (uint32_t)(64 * kRowChunk - 1));
    };
    // y^mix in registers: y^lo read again (the probabilities, which may share
    // its buffer, are not written yet) and the recomputed scores scattered
    // over it.
    auto load_ymix = [&]() {
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t)
            v[t] = buf_load_f32(y_rs, 4u * (uint32_t)(lane + 64 * t));
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t)
            v[t] = lane + 64 * t < n ? v[t] : -INFINITY;
        uint32_t before = 0;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            if (t < nch) {
                const bool sel = (selbits >> t) & 1u;
                const uint64_t b = __ballot(sel);
                if (b) {
                    const float h = s_val[wave][slot(b, before)];
                    v[t] = sel ? h : v[t];
                    before += (uint32_t)__popcll(b);
                }
            }
        }
    };

    const double Lmix = L + dL;
    const bool corrected = Lmix >= 0.25 * L && isfinite(Lmix);
    // log-sum-exp of y^mix = mix_base + log(mix_l)
    double mix_base = (double)m, mix_l = Lmix;
    // 1 / L_mix (lane 0) and 1 / L_ref (lane 1) by one division
    const double rcp = 1.0 / (lane == 0 ? Lmix : Lr);
    if (corrected) {
        // p = e / L_mix, in FP32: e and 1 / L_mix rounded to FP32 and their
        // product, at most 3 roundings (1.8e-7 of p)
        const float inv = (float)lane_read(rcp, 0);
        uint32_t before = 0;
        const int rem_p = fresh();
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            const int j = lane + 64 * t;
            if (64 * t < S) {
                float pv = 0.0f;
                if (t < nch) {
                    const bool sel = (selbits >> t) & 1u;
                    const uint64_t b = __ballot(sel);
                    float ev = ef[t];
                    if (b) {
                        const float eh = s_val[wave][slot(b, before)];
                        ev = sel ? eh : ev;
                        before += (uint32_t)__popcll(b);
                    }
                    pv = 64 * t < rem_p ? ev * inv : 0.0f;
                }
                buf_store_f32(p_rs, 4u * (uint32_t)j, pv);
            }
        }
    } else {
        // Full pass over y^mix: the list's scores formed again
        for (uint32_t ei = lane; ei < total; ei += 64)
            s_val[wave][ei] = yr ? yr[s_key[wave][ei]] : dot_hi(s_key[wave][ei]);
        __builtin_amdgcn_wave_barrier();
        load_ymix();
        float mm = -INFINITY;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t)
            mm = fmaxf(mm, v[t]);
        mm = wave_max(mm);
        double l = 0.0;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            if (t < nch) {
                const double x = exp64_nonpos((double)v[t] - (double)mm, s_exp);
                l += lane + 64 * t < n ? x : 0.0;
            }
        }
        mix_base = (double)mm;
        mix_l = row_nan ? __builtin_nan("") : wave_sum(l);
        const double lse_mix = mix_base + log(mix_l);
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            const int j = lane + 64 * t;
            if (64 * t < S) {
                float pv = 0.0f;
                if (t < nch) {
                    const float x = exp_f32((double)v[t] - lse_mix);
                    pv = j < n ? x : 0.0f;
                }
                buf_store_f32(p_rs, 4u * (uint32_t)j, pv);
            }
        }
    }
    // KL(P_ref || P) = sum p_ref (y_ref - y) + lse(y) - lse(y_ref): the three
    // logarithms log L_lo, log L_ref, log L_mix in one evaluation (lanes 0-2)
    double kl_lo = 0.0, kl_mix = 0.0;
    if (kl) {
        const double lg = log(lane == 0 ? L : (lane == 1 ? Lr : mix_l));
        const double lse_lo = (double)m + lane_read(lg, 0);
        const double lse_ref = (double)mr + lane_read(lg, 1);
        const double lse_mix = mix_base + lane_read(lg, 2);
        const double inv_lr = lane_read(rcp, 1);
        kl_lo = Br * inv_lr + lse_lo - lse_ref;
        kl_mix = (Br - dA) * inv_lr + lse_mix - lse_ref;
    }
    if (lane == 0) {
        if (a.row_count)
            a.row_count[r] = total;
        if (kl) {
            if (a.row_kl_lowp)
                a.row_kl_lowp[r] = kl_lo;
            if (a.row_kl)
                a.row_kl[r] = kl_mix;
        }
    }
}

// y^mix, when asked for, is formed in place over y^lo (ymix_out == ylo); the
// probabilities may share y^lo's buffer only when y^mix is not asked for.
hipError_t launch_strict_rows(const Problem &p, const float *ylo, const float *yref,
                              const RefPartial *part, uint32_t *mask, uint32_t *row_count,
                              float *pbuf, float *ymix_out, double *row_kl, double *row_kl_lowp,
                              bool relaxed, hipStream_t st)
{
    if (p.S > 64 * kRowChunk || (ymix_out && (ymix_out != ylo || pbuf == ylo)) ||
        (relaxed && !part))
        return hipErrorInvalidValue;
    RowsArgs a;
    a.q = p.q;
    a.k = p.k;
    a.ylo = ylo;
    a.yref = yref;
    a.part = part;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.tiles = p.tiles;
    a.W = (p.S + 31) / 32;
    a.n_rows = p.n_rows;
    a.tau = (double)p.tau;
    a.s = p.pc.s;
    a.mask = mask;
    a.row_count = row_count;
    a.pbuf = pbuf;
    a.ymix_out = ymix_out;
    a.row_kl = row_kl;
    a.row_kl_lowp = row_kl_lowp;
    a.n_band = p.n_band;
    const uint64_t grid = (p.n_rows + 3) / 4;
#define LAMP_ROWS_LAUNCH(RLX)                                                                 \
    do {                                                                                      \
        if (p.D == 64)                                                                        \
            hipLaunchKernelGGL((strict_rows_kernel<16, RLX>), dim3((unsigned)grid),           \
                               dim3(kThreads), 0, st, a);                                     \
        else if (p.D == 128)                                                                  \
            hipLaunchKernelGGL((strict_rows_kernel<32, RLX>), dim3((unsigned)grid),           \
                               dim3(kThreads), 0, st, a);                                     \
        else                                                                                  \
            hipLaunchKernelGGL((strict_rows_kernel<0, RLX>), dim3((unsigned)grid),            \
                               dim3(kThreads), 0, st, a);                                     \
    } while (0)
    if (relaxed)
        LAMP_ROWS_LAUNCH(true);
    else
        LAMP_ROWS_LAUNCH(false);
#undef LAMP_ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace lamp
