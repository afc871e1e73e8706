// rows.hip -- fused row pass and P.V for rows of at most 1024 keys.
//
// LAMP summary, "Implementation strategy": step 2 (look-ahead selection from
// the baseline output, with the softmax rule of "Theoretical foundation" item
// 3: recompute y_j iff 2 z_j (1 - z_j) |y_j| > tau; or the relaxed
// relative-threshold rule of "Experimental results", read as 2 exp(y_j - m_t)
// |y_j| > tau with m_t the running maximum over the 64-key blocks up to j's)
// and step 3 (recompute the selected components at FP32, then apply f: the
// softmax and P.V).
//
// One work-group owns 16 consecutive query rows of one head:
//   * phase A, one row per wave at a time (4 rows per wave):
//       - the row's PS(mu) scores stay in registers (16 per lane);
//       - its softmax statistics are formed in double (own exp);
//       - the criterion gives the mask words (ballots) and a compacted list
//         of the selected keys in LDS (ballot + lane prefix);
//       - the selected scores' FP32 values are read from the stored
//         reference scores, or formed by a gather FP32 dot (sequential,
//         multiply then add), one lane per listed key;
//       - the row's log-sum-exp is corrected for the changed terms (or
//         recomputed over the row when the correction would cancel or
//         overflow);
//       - probabilities are written as full rows (zeros past the valid keys);
//       - the row's softmax sums go to LDS, from which the work-group
//         forms the 16 rows' KLs (16 lanes per row) once phase A is done;
//   * phase B, the whole work-group: out = P.V for its 16 rows on the FP32
//     MFMA, the probabilities read back from the rows phase A just wrote,
//     the keys split over the four waves.  The MFMA work of one
//     work-group overlaps the VALU-bound phase A of the others on the CU.
#include "lamp_device.h"

namespace lamp {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowChunk = 16;   // keys per lane: rows of at most 1024 keys
constexpr int kGroupRows = 16;  // query rows per work-group (4 per wave)

struct RowsArgs {
    const float *q, *k, *v, *ylo, *yref;
    const RefPartial *part;
    int S, D, causal, tiles, W, BH, groups;
    double tau;
    float s;
    uint32_t *mask, *row_count;
    float *pbuf, *ymix_out, *out;
    double *row_kl, *row_kl_lowp;   // null: not asked for
    int kl;                         // a row KL is asked for (needs part)
    int tail_done;                  // zeros past the valid blocks already written
    unsigned long long *n_band;
};

// LDS: phase A's per-wave selection lists and query rows, then phase B's
// reduction of the four waves' P.V tiles (DV: V's columns padded to 64 NBW;
// QN: float4 per query row, D / 4 for a compile-time D, else the maximum).
template <int DV, int QN>
union RowsSmem {
    struct {
        uint16_t key[4][64 * kRowChunk];   // selected keys, compacted, key order
        float val[4][64 * kRowChunk];      // per listed key exp(y_hi - m) (FP32)
        float4 q[4][QN];                   // the wave's query row (gather dot)
    } a;
    struct {
        float red[4][kGroupRows][DV + 4];   // the four waves' P.V tiles (FP32)
    } r;
};

// Phase A for row r (wave-uniform).  D4 = D / 4 when the head dimension is
// a compile-time constant (the gather dot's loads issue back to back), 0 for
// a runtime D.
//
// Register discipline: the loops over a lane's 16 keys are unrolled (the row
// lives in registers) and guarded only by wave-uniform conditions (the chunk
// holds valid keys); per-key validity is a select, never a branch, and the
// per-chunk selection is kept as one bit per lane rather than as 16 wave
// masks (a chunk's mask is re-formed by a ballot when needed).
//
// Probabilities: p_j = exp(y_j - lse_mix) = e_j / L_mix for every key whose
// score did not change (e_j = exp(y_j - m), kept in FP32 after the
// criterion), and e_hi / L_mix for a recomputed key (e_hi = exp(y_hi - m)
// formed in the recompute loop and kept, rounded to FP32, in the LDS list).
// Only a row that takes the full pass (the correction would cancel or
// overflow) evaluates exp(y - lse_mix) per key.
//
// RELAXED: the selection uses exp(y_j - m_t) = e_j exp(m - m_t), with the
// block maxima of y^lo taken from the score tiles' per-tile partials (lane t
// holds block t's; a prefix maximum across lanes gives m_t); keys where that
// product would lose precision (e_j below 1e-300, or a row whose factor
// overflows) take exp(y_j - m_t) directly.  Everything after the selection
// is the strict pass's.
template <int D4, bool RELAXED, int DV, int QN, typename Args>
__device__ __forceinline__ void row_pass(Args &a, RowsSmem<DV, QN> &sm, const double *s_exp,
                                         int wave, int lane_in, uint64_t r, uint32_t &ties,
                                         RowKL *rk_slot)
{
    // the lane index through an opaque copy: everything derived from it is
    // formed inside the pass, not hoisted out of the caller's row loop and
    // kept (spilled) across rows
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    uint16_t *s_key = sm.a.key[wave];
    float *s_val = sm.a.val[wave];
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

    float v[kRowChunk];
    {
        const uint32_t lo = 4u * (uint32_t)lane;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t)
            v[t] = buf_load_f32(y_rs, lo + 256u * t);
    }
    // This lane's per-tile partial of the score kernel (tile = lane; nch =
    // the tiles that hold valid keys): the relaxed rule's block maximum of
    // y^lo, and for the KL the tile maximum of y^ref.
    const bool kl = a.kl != 0;
    float blk_max = -INFINITY, ref_max = -INFINITY;
    if ((RELAXED || kl) && lane < nch) {
        const RefPartial q = a.part[r * (uint64_t)a.tiles + lane];
        blk_max = q.m_lo;
        ref_max = q.m;
    }
    // Key lane + 64 t is valid iff 64 t < n - lane.  Each loop below forms
    // n - lane from its own opaque copy of n, so the chunk compares are
    // formed where they are used instead of being kept, 16 mask pairs at a
    // time, in scalar registers across the loops.
    auto fresh = [&]() {
        int x = n;
        asm volatile("" : "+s"(x));
        return x - lane;
    };
    // this lane's byte offset in a row, through an opaque copy per loop: each
    // loop's 16 buffer accesses then take it plus an immediate offset (256 t)
    // instead of 16 offsets formed once and kept across the loops
    auto lane_off = [&]() {
        uint32_t o = 4u * (uint32_t)lane;
        asm volatile("" : "+v"(o));
        return o;
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
    {
        const int rem = fresh();
        const double md = (double)m;
        // (the exponential of 0 is exactly 1: a key at the maximum needs no
        // select for e, only for the sum below it)
        // (ballots of plain compares, masked by the valid lanes afterwards,
        // stay scalar lane masks)
        uint64_t nan_lanes = 0;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            e[t] = 0.0;
            if (t < nch) {
                const uint64_t vmask = ballot(64 * t < rem);
                const bool at = 64 * t < rem && v[t] == m;
                const double x = exp64_crit_nonpos((double)v[t] - md, s_exp);
                e[t] = x;
                A += at ? 0.0 : x;
                cnt += __popcll(ballot(v[t] == m) & vmask);
                nan_lanes |= ballot(v[t] != v[t]);
            }
        }
        has_nan = nan_lanes != 0;
    }
    A = wave_sum(A);
    const bool row_nan = has_nan;
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
        mt = blk_max;
#pragma unroll
        for (int off = 1; off < kRowChunk; off <<= 1) {
            const float o = __shfl_up(mt, off, 64);
            if (lane >= off)
                mt = fmaxf(mt, o);
        }
        ft = lane < nch ? exp64_crit((double)m - (double)mt, s_exp) : 1.0;
        direct_row = ballot(lane < nch && !(ft < 1e300)) != 0;
    }

    // Strict criterion 2 z (1 - z) |y| > tau with z = e / L and 1 - z =
    // rest / L, evaluated as e rest |y| > tau L^2 / 2; relaxed criterion
    // 2 exp(y - m_t) |y| > tau.  Compaction of the selected keys; chunk t's
    // two mask words collect in lanes 2t and 2t + 1 (one store per row).
    // e in FP32 is kept for the probabilities (p = e / L_mix); sel_e sums the
    // selected keys' e (their terms leave L when they are recomputed).  The
    // near ties lie in (rhs (1 - 2^-16), rhs (1 + 2^-16)], rhs the
    // threshold the criterion is compared with.
    const double tau_l2 = a.tau * (L * L) * 0.5;
    const double rhs = RELAXED ? a.tau : tau_l2;
    const double tie_lo = rhs * (1.0 - 0x1p-16), tie_hi = rhs * (1.0 + 0x1p-16);
    // (only when a summary is asked for; near_tie's finite threshold)
    const bool count_ties = a.n_band != nullptr && rhs < INFINITY;
    uint32_t selbits = 0;
    uint32_t total = 0;
    uint32_t mword = 0;
    double sel_e = 0.0;
    float ef[kRowChunk];
    {
        const int rem = fresh();
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            ef[t] = 0.0f;
            if (t < nch) {   // chunks past the valid keys: zero mask words below
                const bool valid = 64 * t < rem;
                double crit;
                ef[t] = (float)e[t];
                if constexpr (RELAXED) {
                    double E = e[t] * lane_read(ft, t);
                    const bool dir = valid && (direct_row || e[t] < 1e-300);
                    if (ballot(dir) != 0) {
                        const float mtt = lane_read(mt, t);
                        if (dir)
                            E = exp64_crit((double)v[t] - (double)mtt, s_exp);
                    }
                    crit = 2.0 * E * fabs((double)v[t]);
                } else {
                    const bool at = valid && v[t] == m;
                    const double rest = at ? rest_at_max : L - e[t];
                    crit = e[t] * rest * fabs((double)v[t]);
                }
                const uint64_t vmask = ballot(valid);
                const uint64_t b = ballot(crit > rhs) & vmask;
                if (count_ties)
                    ties += (uint32_t)__popcll(ballot(crit > tie_lo) & ~ballot(crit > tie_hi) &
                                               vmask);
                mword = lane == 2 * t ? (uint32_t)b
                                      : (lane == 2 * t + 1 ? (uint32_t)(b >> 32) : mword);
                const bool sel = valid && crit > rhs;
                if (sel)
                    s_key[total + lanes_below(b)] = (uint16_t)(64 * t + lane);
                sel_e += sel ? e[t] : 0.0;
                selbits |= (sel ? 1u : 0u) << t;
                total += (uint32_t)__popcll(b);
            }
        }
    }
    if (a.mask)   // every word of the row: chunk t's in lanes 2t, 2t + 1, zeros past the valid keys
        for (int w = lane; w < a.W; w += 64)
            a.mask[r * (uint64_t)a.W + w] = w < 2 * nch ? mword : 0u;

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
            sm.a.q[wave][lane] = qg[lane];
        __builtin_amdgcn_wave_barrier();
    }
    const float4 *q4 = sm.a.q[wave];
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
    // dL: the change of L (the selected keys' exp(y_hi - m) in, their e
    // out); dA: sum of exp(y_hi - m_ref) (y_hi - y_lo) over the selected keys
    // (the KL's correction; m_ref = the row maximum of y^ref, so every term
    // is at most |y_hi - y_lo|)
    const double mr = kl ? (double)wave_max(ref_max) : 0.0;
    double dL = -sel_e, dA = 0.0;
    for (uint32_t ei = lane; ei < total; ei += 64) {
        const uint32_t j = s_key[ei];
        // y^lo of the key, read before y^mix may overwrite it in place
        const float yl = kl ? y[j] : 0.0f;
        const float yhi = yr ? yr[j] : dot_hi(j);
        const double ehi = exp64_sum((double)yhi - (double)m, s_exp);
        s_val[ei] = (float)ehi;
        if (a.ymix_out)   // y^mix is y^lo in place: only recomputed keys change
            a.ymix_out[r * (uint64_t)S + j] = yhi;
        dL += ehi;
        if (kl)
            dA += exp64_sum((double)yhi - mr, s_exp) * ((double)yhi - (double)yl);
    }
    dL = wave_sum(dL);
    if (kl)
        dA = wave_sum(dA);
    __builtin_amdgcn_wave_barrier();

    // Slot in the compacted list of this lane's key in chunk t (meaningful
    // when the key is selected), given the chunk's selection mask b and the
    // number of keys selected in the chunks before it.
    auto slot = [&](uint64_t b, uint32_t before) {
        return min(before + lanes_below(b), (uint32_t)(64 * kRowChunk - 1));
    };

    // The row's probabilities past its valid chunks are 0: 16-byte stores
    // over keys 64 nch .. S - 1 (4-byte ones when S is not a multiple of 4)
    auto zero_tail = [&]() {
        if (a.tail_done)
            return;
        float *pr = a.pbuf + r * (uint64_t)S;
        if ((S & 3) == 0) {
            for (int j = 64 * nch + 4 * lane; j < S; j += 256)
                *reinterpret_cast<float4 *>(pr + j) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            for (int j = 64 * nch + lane; j < S; j += 64)
                pr[j] = 0.0f;
        }
    };

    const double Lmix = L + dL;
    const bool corrected = Lmix >= 0.25 * L && isfinite(Lmix);
    // log-sum-exp of y^mix = mix_base + log(mix_l)
    double mix_base = (double)m, mix_l = Lmix;
    if (corrected) {
        // p = e / L_mix, in FP32: e and 1 / L_mix rounded to FP32 and their
        // product, at most 3 roundings (1.8e-7 of p)
        const float inv = (float)(1.0 / Lmix);
        uint32_t before = 0;
        const int rem = fresh();
        const uint32_t lo = lane_off();
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            if (t < nch) {
                const bool sel = (selbits >> t) & 1u;
                const uint64_t b = ballot(sel);
                float ev = ef[t];
                if (b) {
                    const float eh = s_val[slot(b, before)];
                    ev = sel ? eh : ev;
                    before += (uint32_t)__popcll(b);
                }
                buf_store_f32(p_rs, lo + 256u * t, 64 * t < rem ? ev * inv : 0.0f);
            }
        }
        zero_tail();
    } else {
        // Full pass over y^mix: the list's scores formed again, y^lo read
        // again (the probabilities, which may share its buffer, are not
        // written yet) and the recomputed scores scattered over it
        for (uint32_t ei = lane; ei < total; ei += 64)
            s_val[ei] = yr ? yr[s_key[ei]] : dot_hi(s_key[ei]);
        __builtin_amdgcn_wave_barrier();
        {
            const uint32_t lo = lane_off();
#pragma unroll
            for (int t = 0; t < kRowChunk; ++t)
                v[t] = buf_load_f32(y_rs, lo + 256u * t);
        }
        {
            const int rem = fresh();
#pragma unroll
            for (int t = 0; t < kRowChunk; ++t)
                v[t] = 64 * t < rem ? v[t] : -INFINITY;
        }
        {
            uint32_t before = 0;
#pragma unroll
            for (int t = 0; t < kRowChunk; ++t) {
                if (t < nch) {
                    const bool sel = (selbits >> t) & 1u;
                    const uint64_t b = ballot(sel);
                    if (b) {
                        const float h = s_val[slot(b, before)];
                        v[t] = sel ? h : v[t];
                        before += (uint32_t)__popcll(b);
                    }
                }
            }
        }
        float mm = -INFINITY;
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t)
            mm = fmaxf(mm, v[t]);
        mm = wave_max(mm);
        double l = 0.0;
        {
            const int rem = fresh();
#pragma unroll
            for (int t = 0; t < kRowChunk; ++t) {
                if (t < nch) {
                    const double x = exp64_nonpos((double)v[t] - (double)mm, s_exp);
                    l += 64 * t < rem ? x : 0.0;
                }
            }
        }
        mix_base = (double)mm;
        mix_l = row_nan ? __builtin_nan("") : wave_sum(l);
        const double lse_mix = mix_base + log(mix_l);
        const int rem = fresh();
        const uint32_t lo = lane_off();
#pragma unroll
        for (int t = 0; t < kRowChunk; ++t) {
            if (t < nch) {
                const float x = exp_f32((double)v[t] - lse_mix);
                buf_store_f32(p_rs, lo + 256u * t, 64 * t < rem ? x : 0.0f);
            }
        }
        zero_tail();
    }
    if (lane == 0) {
        if (a.row_count)
            a.row_count[r] = total;
        if (kl) {
            RowKL rk;
            rk.L = L;
            rk.mix_l = mix_l;
            rk.dA = dA;
            rk.m = m;
            rk.mix_base = (float)mix_base;
            *rk_slot = rk;
        }
    }
}

// Phase B: out rows i0 .. i0 + 15 of head bh = P.V over the keys they see,
// on the FP32 MFMA (v_mfma_f32_16x16x4f32), split over the keys: wave w
// takes the 16-key steps w, w + 4, ..., with no barrier in the loop, and the
// four partial tiles are summed through LDS at the end.
//
// Operands straight from memory, in the MFMA's lane layout: lane (g = l / 16,
// c = l % 16) loads the probabilities of row i0 + c at keys k0 + 4g .. + 3
// (one float4: MFMA m of the step takes component m, i.e. key k0 + 4g + m)
// and the V rows k0 + 4g + m at columns CPL c .. CPL c + CPL - 1 (float4
// loads); MFMA column block cb multiplies by column CPL c + cb, so its output
// lane (g, c) holds out[i0 + 4g + q][CPL c + cb].  The loads are
// range-checked buffer loads, with no branch or exec mask: the probabilities
// over the group's rows (rows past S read 0, keys past S are set to 0), V
// over the head (keys past S read 0; a column past D only feeds an output
// column that is not stored).  The probabilities are read back from the rows
// phase A just wrote (L2).  (A second step's loads kept in flight would need
// 20 more registers than the 96 of five waves per SIMD; the other waves on
// the SIMD hide the loads' latency instead.)
//
// The FP32 partial of every 16 keys (4 MFMAs) is flushed into a double
// accumulator: one partial carries at most 4 FP32 roundings (2.4e-7 of its
// sum_j p_j |v_jd|); the four waves' sums are rounded to FP32 once more for
// the reduction (6e-8 each), inside the 1e-6 bar.
//
// Causal steps that reach the group's own rows hold keys past some rows'
// limits, whose probability 0 would turn a non-finite V value into NaN
// (0 * inf) in the product: such values are taken as 0 and added back at the
// end for the rows that see their key.
template <int DV, int QN>
__device__ __forceinline__ void group_pv(const RowsArgs &a, RowsSmem<DV, QN> &sm, int bh, int i0)
{
    constexpr int CPL = DV / 16;   // V columns per lane = MFMA column blocks
    constexpr int F4 = CPL / 4;    // float4 per lane per key row
    const int S = a.S, D = a.D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int nk = a.causal ? min(S, i0 + kGroupRows) : S;   // keys the group sees
    const int nsteps = (nk + 15) / 16;
    const int nrows = min(kGroupRows, S - i0);
    const __amdgpu_buffer_rsrc_t p_rs =
        row_rsrc(a.pbuf + ((uint64_t)bh * S + i0) * (uint64_t)S, 4u * (uint32_t)(nrows * S));
    const __amdgpu_buffer_rsrc_t v_rs = row_rsrc(a.v + (size_t)bh * S * D, 4u * (uint32_t)(S * D));
    const bool vec = (S & 3) == 0;
    const uint32_t p_off = 4u * (uint32_t)(c * S);
    auto comp = [](const float4 &x, int e) {
        return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
    };

    double acc[CPL][4];
#pragma unroll
    for (int cb = 0; cb < CPL; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc[cb][q] = 0.0;
    bool vbad = false;
    for (int s = wave; s < nsteps; s += 4) {
        const int k0 = 16 * s;
        const int j = k0 + 4 * g;
        float4 p;
        if (vec) {   // S % 4 == 0: a float4 lies wholly inside or past the row
            p = buf_load_f32x4(p_rs, p_off + 4u * (uint32_t)j);
        } else {
            p.x = buf_load_f32(p_rs, p_off + 4u * (uint32_t)j);
            p.y = buf_load_f32(p_rs, p_off + 4u * (uint32_t)(j + 1));
            p.z = buf_load_f32(p_rs, p_off + 4u * (uint32_t)(j + 2));
            p.w = buf_load_f32(p_rs, p_off + 4u * (uint32_t)(j + 3));
        }
        float4 v[4][F4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int f = 0; f < F4; ++f)
                v[m][f] = buf_load_f32x4(v_rs, 4u * (uint32_t)((j + m) * D + CPL * c + 4 * f));
        // keys past S read the next row's probabilities: taken as 0
        p.x = j < S ? p.x : 0.f;
        p.y = j + 1 < S ? p.y : 0.f;
        p.z = j + 2 < S ? p.z : 0.f;
        p.w = j + 3 < S ? p.w : 0.f;
        if (a.causal && k0 + 16 > i0) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int f = 0; f < F4; ++f)
                    if (j + m >= i0 && CPL * c + 4 * f < D && !finite4(v[m][f])) {
                        v[m][f] = finite_or_zero(v[m][f]);
                        vbad = true;
                    }
        }
        floatx4 part[CPL];
#pragma unroll
        for (int cb = 0; cb < CPL; ++cb)
            part[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float av = comp(p, m);
#pragma unroll
            for (int cb = 0; cb < CPL; ++cb)
                part[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, comp(v[m][cb / 4], cb % 4),
                                                                 part[cb], 0, 0, 0);
        }
#pragma unroll
        for (int cb = 0; cb < CPL; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[cb][q] += (double)part[cb][q];
    }

    // Sum of the four waves' tiles: lane (g, c) of wave w puts its rows
    // 4g + q, columns CPL c + cb into red[w]; then thread t sums the four for
    // row t / 16, columns CPL (t % 16) ...  (The or-reduction is not a fence
    // for this wave's LDS writes: it comes first, and a plain barrier orders
    // the tile writes before their reads.)
    const bool any_bad = __syncthreads_or(vbad ? 1 : 0) != 0;
    float(*red)[kGroupRows][DV + 4] = sm.r.red;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int cb = 0; cb < CPL; ++cb)
            red[wave][4 * g + q][CPL * c + cb] = (float)acc[cb][q];
    __syncthreads();
    const int orow = tid >> 4, oc = (tid & 15) * CPL;
    const int i = i0 + orow;
    if (i < S) {
        const float *Vh = a.v + (size_t)bh * S * D;
        float o[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int col = oc + e;
            double x = (double)red[0][orow][col] + (double)red[1][orow][col] +
                       (double)red[2][orow][col] + (double)red[3][orow][col];
            // non-finite V values taken as 0 on the diagonal steps: each one
            // at a key the row sees adds its infinity or NaN (what any positive
            // probability times it gives)
            if (any_bad && col < D)
                for (int j = i0; j <= i; ++j) {
                    const float v = Vh[(size_t)j * D + col];
                    if (!isfinite(v))
                        x += (double)v;
                }
            o[e] = (float)x;
        }
        float *orow_p = a.out + ((size_t)bh * S + i) * D;
#pragma unroll
        for (int f = 0; f < F4; ++f)
            if (oc + 4 * f < D)
                *reinterpret_cast<float4 *>(orow_p + oc + 4 * f) =
                    make_float4(o[4 * f], o[4 * f + 1], o[4 * f + 2], o[4 * f + 3]);
    }
}

// The group's row KLs from the rows' softmax sums (phase A) and the score
// tiles' per-tile reference statistics:
//   KL(P_ref || P_x) = sum_j p_ref_j (y^ref_j - y^x_j) + lse(y^x) - lse(y^ref)
// with sum_j p_ref_j (y^ref_j - y^lo_j) = B / L_ref from the partials; for
// y^mix the selected keys' terms leave B (their y^mix is y^ref): dA / L_ref.
// 16 lanes per row (lane = 64-key tile, rows of at most 1024 keys): a row's
// partials are one contiguous read, reduced by DPP within the 16 lanes; wave
// w takes rows 4w .. 4w + 3 of the group.
__device__ __forceinline__ void group_kl(const RowsArgs &a, const RowKL *s_rk, const double *s_exp,
                                         int bh, int i0)
{
    const int tid = threadIdx.x, t = tid & 15, lr = tid >> 4;
    const int i = min(i0 + lr, a.S - 1);   // every lane takes part in the DPP sums
    const uint64_t r = (uint64_t)bh * a.S + i;
    const int nt = a.causal ? (i / kTile) + 1 : a.tiles;
    RefPartial q{0.0, 0.0, -INFINITY, 0.0f};
    if (t < nt)
        q = a.part[r * (uint64_t)a.tiles + t];
    const float mr = group16_max(q.m);
    const double f = t < nt ? exp64_sum_nonpos((double)q.m - (double)mr, s_exp) : 0.0;
    const double Lr = group16_sum(q.L * f);
    const double Br = group16_sum(q.B * f);
    if (t != 0 || i0 + lr >= a.S)
        return;
    const RowKL k = s_rk[lr];
    const double lse_ref = (double)mr + log(Lr);
    const double inv_lr = 1.0 / Lr;
    if (a.row_kl_lowp)
        a.row_kl_lowp[r] = Br * inv_lr + ((double)k.m + log(k.L)) - lse_ref;
    if (a.row_kl)
        a.row_kl[r] = (Br - k.dA) * inv_lr + ((double)k.mix_base + log(k.mix_l)) - lse_ref;
}

// 16 rows per work-group, heaviest (causal) groups first so that the light
// ones fill the tail of the launch.  Five waves per SIMD at DV = 64 (96
// VGPRs; 29 KB of LDS per work-group); wider V tiles take more LDS.
template <int D4, bool RELAXED, int DV>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DV == 64 ? 5 : (DV == 128 ? 3 : 2)))) void rows_pv_kernel(RowsArgs a)
{
    constexpr int QN = D4 > 0 ? D4 : 64;
    __shared__ RowsSmem<DV, QN> sm;
    __shared__ double s_exp[64];   // 2^(k/64) for exp64
    __shared__ RowKL s_rk[kGroupRows];   // the rows' softmax sums for the KLs
    exp_table_fill(s_exp);
    __syncthreads();
    // the wave index is uniform: readfirstlane tells the compiler so, which
    // makes the row, its length and every chunk guard scalar
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // batches of five heads per XCD: a batch's V stays in L2 between the
    // groups of a head (all of an XCD's heads in turn cycle more V through
    // it than it holds)
    int bh, g;
    xcd_head_batches(blockIdx.x, a.BH, a.groups, 5, bh, g);
    const int i0 = g * kGroupRows;
    uint32_t ties = 0;
    // The arguments through an opaque pointer to the kernel-argument segment,
    // loaded (scalar loads) where each row pass uses them rather than held
    // in scalar registers across the row loop.
    typedef __attribute__((address_space(4))) const RowsArgs KArgs;
    KArgs *kargs = (KArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    // Issue priority: phase A (each row a chain of memory round trips and
    // reductions) above phase B (MFMA steps) of the other work-groups on the
    // SIMD: the row kernel 0.555 -> 0.542 ms on the GPT-2-XL layer.
    __builtin_amdgcn_s_setprio(2);
    // rows i0 + wave + 4 k: neighbouring lengths, so the waves stay even
#pragma unroll 1
    for (int k = 0; k < kGroupRows / 4; ++k) {
        const int i = i0 + wave + 4 * k;
        KArgs *ak = kargs;
        asm volatile("" : "+s"(ak));
        if (i < a.S)
            row_pass<D4, RELAXED, DV, QN>(*ak, sm, s_exp, wave, lane, (uint64_t)bh * a.S + i, ties,
                                      &s_rk[wave + 4 * k]);
        __builtin_amdgcn_wave_barrier();
    }
    add_ties(a.n_band, ties);
    __syncthreads();   // the group's probabilities are written; LDS is free
    if (a.kl)
        group_kl(a, s_rk, s_exp, bh, i0);
    __builtin_amdgcn_s_setprio(0);   // phase B
    group_pv<DV, QN>(a, sm, bh, i0);
}

// y^mix, when asked for, is formed in place over y^lo (ymix_out == ylo); the
// probabilities may share y^lo's buffer only when y^mix is not asked for.
hipError_t launch_rows_pv(const Problem &p, const float *ylo, const float *yref,
                          const RefPartial *part, uint32_t *mask, uint32_t *row_count,
                          float *pbuf, float *ymix_out, float *out, double *row_kl,
                          double *row_kl_lowp, bool relaxed, hipStream_t st, bool tail_done)
{
    const bool kl = row_kl || row_kl_lowp;
    if (p.S > 64 * kRowChunk || (ymix_out && (ymix_out != ylo || pbuf == ylo)) ||
        (relaxed && !part) || (kl && !part) || !pbuf || !out)
        return hipErrorInvalidValue;
    RowsArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.ylo = ylo;
    a.yref = yref;
    a.part = part;
    a.S = p.S;
    a.D = p.D;
    a.causal = p.causal;
    a.tiles = p.tiles;
    a.W = (p.S + 31) / 32;
    a.BH = p.BH;
    a.groups = (p.S + kGroupRows - 1) / kGroupRows;
    a.tau = (double)p.tau;
    a.s = p.pc.s;
    a.mask = mask;
    a.row_count = row_count;
    a.pbuf = pbuf;
    a.ymix_out = ymix_out;
    a.out = out;
    a.row_kl = row_kl;
    a.row_kl_lowp = row_kl_lowp;
    a.kl = kl ? 1 : 0;
    a.tail_done = tail_done ? 1 : 0;
    a.n_band = p.n_band;
    const uint64_t grid = (uint64_t)p.BH * a.groups;
    if (grid > 0x7fffffffULL)
        return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(kThreads);
    const int nbw = ((p.D + 15) / 16 + 3) / 4;   // MFMA column blocks per wave
#define LAMP_ROWS_LAUNCH(RLX)                                                                 \
    do {                                                                                      \
        if (p.D == 64)                                                                        \
            hipLaunchKernelGGL((rows_pv_kernel<16, RLX, 64>), g, b, 0, st, a);                \
        else if (p.D == 128)                                                                  \
            hipLaunchKernelGGL((rows_pv_kernel<32, RLX, 128>), g, b, 0, st, a);               \
        else if (nbw == 1)                                                                    \
            hipLaunchKernelGGL((rows_pv_kernel<0, RLX, 64>), g, b, 0, st, a);                 \
        else if (nbw == 2)                                                                    \
            hipLaunchKernelGGL((rows_pv_kernel<0, RLX, 128>), g, b, 0, st, a);                \
        else if (nbw == 3)                                                                    \
            hipLaunchKernelGGL((rows_pv_kernel<0, RLX, 192>), g, b, 0, st, a);                \
        else                                                                                  \
            hipLaunchKernelGGL((rows_pv_kernel<0, RLX, 256>), g, b, 0, st, a);                \
    } while (0)
    if (relaxed)
        LAMP_ROWS_LAUNCH(true);
    else
        LAMP_ROWS_LAUNCH(false);
#undef LAMP_ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace lamp
