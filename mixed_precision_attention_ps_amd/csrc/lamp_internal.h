// lamp_internal.h -- launch-level interface between the C ABI (lamp_api.cpp)
// and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lamp {

constexpr int kTile = 64;        // query rows and keys per score tile
constexpr int kDChunk = 32;      // head-dimension slice staged in LDS at a time (multiple of 16)
constexpr int kThreads = 256;    // threads per work-group (4 wave64)

// Per-launch constants of the PS(mu) arithmetic.
struct PsConst {
    int mu;
    uint32_t sh;        // 23 - mu: fraction bits dropped
    float split;        // 2^sh + 1: Veltkamp splitting constant (rounding of a sum)
    float qscale;       // 2^(mu-23): scaled operand of the product fma
    float out_scale;    // s * 2^(23-mu): scale of the scaled-domain accumulator
    float s;            // FP32 value nearest to 1/sqrt(D)
    int blk;            // accumulation order: 0 sequential, else runs of blk
                        // (a power of two, 4 <= blk < dot length) products
};

PsConst make_ps_const(int mu, int D);
// Sets the accumulation order: runs of `block` products for a dot of `len`
// terms; block <= 1 or >= len is the sequential order (blk = 0).
void set_ps_block(PsConst &c, int block, int len);

struct Problem {
    const float *q, *k, *v;
    int BH, S, D, causal, mu;
    float tau;
    PsConst pc;
    int tiles;            // ceil(S / 64)
    uint64_t n_rows;      // BH * S
    uint64_t head_valid;  // valid pairs per head
    bool lo_max = true;   // per-tile partials carry m_lo (the relaxed rule's block
                          // maxima; else -inf)
    bool ref_sums = true; // per-tile partials carry the reference sums L, B
                          // (false: only the maxima, when no KL is asked for)
    unsigned long long *n_band = nullptr;   // near-tie count of the criterion
};

// Operand range scan: unsafe[bh * tiles + t] = 1 when a 64-row block of Q
// (first BH*tiles entries) or K (next BH*tiles entries) holds a value outside
// {0} U [2^-40, 2^40] (including inf / nan).
hipError_t launch_operand_scan(const Problem &p, uint8_t *unsafe, hipStream_t st);

// Softmax statistics of the FP32 reference scores of one row over one 64-key
// tile: m = max y^ref, L = sum exp(y^ref - m), B = sum exp(y^ref - m)(y^ref - y^lo),
// and m_lo = max y^lo over the tile's valid keys (the block maximum of the
// relaxed rule).
struct RefPartial {
    double L, B;
    float m;
    float m_lo;
};

// PS(mu) and FP32 scores of every valid pair into dense [BH, S, S] buffers
// (either may be null), and optionally the per-row, per-tile RefPartial
// [BH*S, tiles].  fast = true: the tiles on the FP32 fast path (launches
// nothing if mu > 10); fast = false: every other tile.  pzero (causal only,
// may be null): a [BH, S, S] buffer whose entries above the causal diagonal
// tiles (rows of 64-key block a, keys of blocks b > a) are set to 0, each by
// the work-group of the mirrored tile (b, a): the probabilities' zero tails,
// written beside the ALU-bound score work instead of by the row pass.
hipError_t launch_ps_scores(const Problem &p, const uint8_t *unsafe, float *ylo, float *yref,
                            RefPartial *part, unsigned long long *exact_tiles, bool fast,
                            hipStream_t st, float *pzero = nullptr);

// Softmax sums of one row after the fused row pass, for the row KLs: L =
// sum exp(y^lo - m), the log-sum-exp of y^mix = mix_base + log(mix_l), and
// dA = sum over the recomputed keys of exp(y^ref - m_ref) (y^ref - y^lo),
// m_ref the row maximum of y^ref.
struct RowKL {
    double L, mix_l, dA;
    float m, mix_base;
};

// Fused row pass and P.V (S <= 1024), 16 rows per work-group: row softmax
// statistics, the strict criterion (relaxed = false) or the relaxed one
// (relaxed = true: needs part, for the 64-key block maxima), mask words,
// compaction of the selected keys, their FP32 recompute, the corrected
// softmax, probabilities into pbuf (full rows, zeros past the valid keys;
// tail_done: the zeros past a row's last valid 64-key block are not
// written, because the score tiles wrote them through pzero or because pbuf
// is scratch whose tails nothing reads),
// y^mix (optional), counts, the row KLs (row_kl / row_kl_lowp, optional; need
// part), then out = P.V.  ylo may alias pbuf or ymix_out (rows are read
// before written).  yref: the FP32 reference scores [BH, S, S] when the
// score tiles kept them (the selected scores' FP32 values are then read from
// it, bit for bit what the gather FP32 dot gives), or null (the dot is
// formed).
hipError_t launch_rows_pv(const Problem &p, const float *ylo, const float *yref,
                          const RefPartial *part, uint32_t *mask, uint32_t *row_count,
                          float *pbuf, float *ymix_out, float *out, double *row_kl,
                          double *row_kl_lowp, bool relaxed, hipStream_t st,
                          bool tail_done = false);

// Per-row statistics of the strict / random path (double sums, float maxima).
struct RowStats {
    double L_lo;      // sum_j exp(y^lo_j - m_lo)
    double L_ref;     // sum_j exp(y^ref_j - m_ref)
    double A;         // sum_j exp(y^ref_j - m_ref) (y^ref_j - y^mix_j); before the
                      // recompute (y^mix = y^lo) this is the low-precision term
    double lse_mix;   // log-sum-exp of y^mix over the valid keys
    float m_lo, m_ref;
    uint32_t full_pass;   // 1: lse_mix must be recomputed from the whole row
    uint32_t pad;
};

// Strict row softmax + selection.  count_only: row statistics and row_count
// only (random mode); otherwise also mask words (if non-null) and the per-row
// compacted index segments in `list`.  Writes RowStats with lse_mix = lse(y^lo),
// row_kl (if non-null) and row_kl_lowp (if non-null) = KL(P_ref || P_lowp);
// the recompute kernel updates the rows that have selections.  yref may be
// null when neither KL is asked for (the reference sums are then skipped).
// random_seed (count_only, rows of at most 1024 keys): the random control's
// selection too, in the same pass (the row_count keys with the smallest
// hashes, as launch_random_select takes them): mask words and list.
hipError_t launch_strict_select(const Problem &p, const float *ylo, const float *yref,
                                uint32_t *mask, uint32_t *list, uint32_t *row_count,
                                RowStats *rs, double *row_kl, double *row_kl_lowp,
                                int count_only, hipStream_t st,
                                const uint64_t *random_seed = nullptr);

// Relaxed rule over rows of any length after score tiles that kept y^lo (in
// y, replaced in place by y^mix), y^ref and the per-tile partials: mask words
// (if non-null), row_count (if non-null), RowStats with lse_mix of y^mix (the
// finish kernel takes it from there), row_kl and row_kl_lowp (if non-null).
hipError_t launch_relaxed_select(const Problem &p, float *y, const float *yref,
                                 const RefPartial *part, uint32_t *mask, uint32_t *row_count,
                                 RowStats *rs, double *row_kl, double *row_kl_lowp,
                                 hipStream_t st);

// Random control: per row, row_count[r] keys with the smallest hashes.
hipError_t launch_random_select(const Problem &p, uint64_t seed, uint32_t *mask, uint32_t *list,
                                const uint32_t *row_count, hipStream_t st);

// FP32 recompute of the listed scores, scattered into ymix, with the rows'
// softmax and KL statistics updated for the changed scores.  yref: the
// stored FP32 reference scores (a listed key's recompute is its y^ref, the
// same sequential dot), or null when no row KL is asked for: the dot is then
// formed from the gathered query and key rows.
hipError_t launch_recompute(const Problem &p, const uint32_t *list, const uint32_t *row_count,
                            const float *yref, float *ymix, RowStats *rs, double *row_kl,
                            hipStream_t st);

// Final softmax (probs may alias ymix), P.V on MFMA; rows flagged full_pass
// get lse_mix (and row_kl) from a pass over the row here.
// tail_done (causal): the zeros past each row block's last key (the next
// 64-key block on) are already in probs, from the score tiles' pzero.
hipError_t launch_finish(const Problem &p, const float *ymix, const RowStats *rs, float *probs,
                         float *out, double *row_kl, hipStream_t st, bool tail_done = false);

// Relaxed fused one-pass kernel.  ymix_raw: if non-null, y^mix of valid
// entries is written there (for the probs pass / inspection); row_m / row_l:
// per-row final max and sum of the online softmax (for the probs pass).
// fast = true: query blocks whose every visited tile is on the FP32 fast
// path; fast = false: the other query blocks.  pzero (causal, may be null):
// each query block's work-group also writes the zeros of its rows past its
// own 64-key block into this [BH, S, S] buffer (the probabilities).
hipError_t launch_relaxed(const Problem &p, const uint8_t *unsafe, float *out, uint32_t *mask,
                          uint32_t *row_count, double *row_kl, double *row_kl_lowp,
                          float *ymix_raw, float *yref_out, float *row_m, double *row_l,
                          unsigned long long *exact_tiles, bool fast, hipStream_t st,
                          float *pzero = nullptr);

// probs[r][j] = exp(ymix[r][j] - row_m[r]) / row_l[r] on valid keys, 0 elsewhere
// (tail_done, causal: 0 only up to the end of the row's 64-key block; the
// rest was written by the fused kernel through pzero).
hipError_t launch_normalise(const Problem &p, const float *ymix, const float *row_m,
                            const double *row_l, float *probs, hipStream_t st,
                            bool tail_done = false);

// Decode shapes (relaxed rule): nq query rows per head against S keys.
struct DecodeProblem {
    const float *q, *k, *v;   // q [BH, nq, D]; k, v [BH, S, D]
    int BH, S, D, nq, causal, mu;
    float tau;
    int ps_block;             // accumulation order (0 sequential)
    unsigned long long *n_band = nullptr;   // near-tie count of the criterion
};

// Softmax partial sums of one (head, 64-key block, query): maxima of y^mix,
// y^ref and y^lo over the block's valid keys (-inf when it has none), and the
// sums against them: l_mix = sum exp(y^mix - m_mix), l_ref = sum exp(y^ref -
// m_ref), a = sum exp(y^ref - m_ref)(y^ref - y^mix), l_lo = sum exp(y^lo -
// m_lo), b = sum exp(y^ref - m_ref)(y^ref - y^lo); cnt = selected keys.
struct DecPartial {
    float m_mix, m_ref, m_lo;
    uint32_t cnt;
    double l_mix, l_ref, a, l_lo, b;
};

struct DecodeBuffers {
    float *ylo, *yref;          // [BH, nq, S]; ylo ends as y^mix
    float *bmax;                // [BH, nq, ceil(S/64)]
    uint8_t *unsafe;            // [BH, ceil(S/256)]: chunks for the exact path
    uint32_t *mask;             // [BH, nq, ceil(S/32)] or null
    DecPartial *part;           // [BH, ceil(S/64), nq]
    float *acc;                 // [BH, ceil(S/64), nq, D]: P.V partials
    float *out;                 // [BH, nq, D]
    double *row_lse;            // [BH, nq]
    double *row_kl, *row_kl_lowp;   // [BH, nq] or null
    uint32_t *row_count;        // [BH, nq] or null
    float *probs;               // [BH, nq, S] or null
    unsigned long long *exact_chunks;
};

// The decode kernels in order; stage events (2 per stage, as in the main
// entry point) are recorded around the fast score pass, the exact score pass,
// the selection / softmax pass and the combine (+ probabilities) pass when
// given.
hipError_t launch_decode(const DecodeProblem &p, const DecodeBuffers &b, hipStream_t st,
                         void **stage_events);

// Matrix product y = x W^T in PS(mu) followed by an activation (GELU) or a
// layer normalisation, with the LAMP rule of that closed form.
enum { MLP_GEMM = 0, MLP_GELU = 1, MLP_LAYERNORM = 2 };

struct MlpProblem {
    const float *x, *w;           // x [M, K], w [N, K]
    const float *gamma, *beta;    // [N] (layer normalisation)
    int M, N, K, mu, op;
    float tau, eps;
    int ps_block;                 // accumulation order (0 sequential)
    unsigned long long *n_band = nullptr;   // near-tie count of the GELU criterion
};

struct MlpBuffers {
    uint32_t *unsafe;             // [ceil(M/64) + ceil(N/64)] operand range flags
    float *ylo, *yref;            // [M, N]: y^lo (GELU: y^mix) and y^ref, or null
    float *ymix;                  // [M, N] or null (layer normalisation)
    float *out;                   // [M, N]
    uint32_t *mask;               // [M, ceil(N/32)] or null
    double *err_part, *errl_part; // [M, ceil(N/64)] (GELU)
    double *err, *errl;           // [M] or null
    uint32_t *row_count;          // [M] or null (layer normalisation)
    unsigned long long *exact_tiles;
};

// The operand scans, the product (fast tiles and the others), then the GELU
// row reduction or the layer-normalisation row pass; stage events as in the
// attention path (scan, exact, scores, finish).
hipError_t launch_mlp(const MlpProblem &p, const MlpBuffers &b, hipStream_t st,
                      void **stage_events);

// Per-row popcount of mask words (the GELU counts).
hipError_t launch_mask_count(const uint32_t *mask, int M, int N, uint32_t *count, hipStream_t st);

// Device-side summary.
// stats_kernel's work-groups: each reduces a fixed slice of the rows
constexpr int kStatsBlocks = 128;

struct StatsPart {
    double sum, max, low;
    unsigned long long cnt;
};

struct DevStats {
    unsigned long long n_selected;
    unsigned long long n_exact_tiles;
    double kl_sum, kl_max, kl_lowp_sum;
    unsigned long long n_tie_band;   // criterion values within 2^-16 tau of tau
    // stats_kernel's per-work-group partials and the count of work-groups
    // that have written theirs (zeroed with the rest of the summary)
    unsigned int blocks_done, pad;
    StatsPart part[kStatsBlocks];
};

hipError_t launch_stats(const Problem &p, const double *row_kl, const double *row_kl_lowp,
                        const uint32_t *row_count, DevStats *ds, hipStream_t st);

// Zero `bytes` (a multiple of 4) with a fill kernel.
hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t st);

// Start offset of row r's segment in the compacted index list: the number of
// valid pairs in all earlier rows.
__host__ __device__ inline uint64_t row_segment(uint64_t r, int S, int causal)
{
    uint64_t bh = r / (uint64_t)S, i = r % (uint64_t)S;
    if (causal)
        return bh * ((uint64_t)S * (S + 1) / 2) + i * (i + 1) / 2;
    return r * (uint64_t)S;
}

}  // namespace lamp
