/*
 * lamp.h -- C ABI of the LAMP attention forward library for MI355X (gfx950).
 *
 * Look-Ahead Mixed-Precision (LAMP) attention, as described in the LAMP
 * technical summary (gist.science, paper 2601.21623):
 *   1. baseline K.Q scores y^lo with emulated low-precision accumulation
 *      PS(mu) ("Experimental results": custom float with mu mantissa bits);
 *   2. look-ahead selection from the baseline softmax z ("Theoretical
 *      foundation" item 3): strict rule 2 z_j (1 - z_j) |y_j| > tau, or the
 *      relaxed relative-threshold rule that drops the normalisation constant
 *      (one pass, online softmax), or a random control with the strict count;
 *   3. FP32 recompute of the selected scores only ("Implementation strategy"
 *      step 3), then softmax, P.V and a row-wise KL(P_FP32 || P_LAMP).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; float32,
 *     contiguous, row-major.  Q, K, V, out: [B, H, S, D] (d fastest).
 *     Score-shaped buffers: [B, H, S, S] (key fastest).  The library never
 *     allocates or frees caller memory and never keeps a caller pointer past
 *     the call.
 *   - Query row i may attend key j ("valid") iff j <= i when causal = 1,
 *     always when causal = 0.
 *   - PS(mu): mu stored fraction bits (precision mu + 1), FP32 exponent range
 *     with subnormals, round to nearest even after every multiply and every
 *     add, d ascending from +0.  Operands stay FP32.  mu = 23 is FP32.
 *   - Scores are scaled once after accumulation, in FP32, by s = the FP32
 *     value nearest to 1/sqrt(D).
 *   - Work is enqueued on the given stream (NULL = the default stream);
 *     outputs are valid once the stream is synchronised.  A non-NULL host
 *     `stats` makes the call wait for its own work.
 *   - Errors: every argument check runs before any HIP call.  No C++
 *     exception crosses this boundary.  The thread-local text of the last
 *     error is available from lamp_last_error().  Launches are checked with
 *     hipGetLastError, so a call that passes its argument checks first clears
 *     the calling thread's pending HIP error state.
 */
#ifndef LAMP_H
#define LAMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Selection modes. */
enum {
    LAMP_STRICT = 0,  /* 2 z_j (1 - z_j) |y^lo_j| > tau over the full row      */
    LAMP_RELAXED = 1, /* 2 exp(y^lo_j - m_t) |y^lo_j| > tau, m_t = running max
                         of y^lo over 64-key blocks 0..floor(j/64); one pass   */
    LAMP_RANDOM = 2   /* per row, as many keys as LAMP_STRICT selects at tau,
                         the ones with the smallest SplitMix64(seed xor
                         (((b*H + h)*S + i)*S + j)), ties by lower j           */
};

/* Return codes. */
enum {
    LAMP_OK = 0,
    LAMP_ERR_INVALID_ARG = -1, /* NULL required pointer, size < 1, mu not in
                                  [1, 23], tau NaN or negative, causal not 0/1,
                                  unknown mode, undersized workspace          */
    LAMP_ERR_UNSUPPORTED = -2, /* D % 4 != 0, D > 256, or sizes that overflow */
    LAMP_ERR_HIP = -3,         /* a HIP runtime call failed                    */
    LAMP_ERR_NO_MEMORY = -4    /* the library-managed workspace could not grow */
};

/* Host-side summary, filled after the call's own work has finished. */
typedef struct {
    uint64_t n_rows;        /* B*H*S                                          */
    uint64_t n_valid;       /* valid (query, key) pairs                       */
    uint64_t n_selected;    /* scores recomputed in FP32                      */
    uint64_t n_exact_tiles; /* 64x64 score tiles that left the FP32 fast path
                               for the exact double-precision PS path (inputs
                               outside [2^-40, 2^40], non-finite, or mu > 10) */
    double kl_sum;          /* sum over rows of KL(P_FP32 || P_LAMP)          */
    double kl_max;          /* max over rows of the same                      */
    double kl_lowp_sum;     /* sum over rows of KL(P_FP32 || P_lowp), the
                               all-low-precision baseline                     */
    uint64_t n_tie_band;    /* valid keys whose selection criterion c lies
                               within a relative 2^-16 of tau, |c - tau| <=
                               2^-16 tau: the near-ties that a single-
                               precision evaluation of c could not decide and
                               the library decides in double precision (the
                               strict rule's ">" of "Theoretical foundation"
                               item 3; the relaxed rule's and the GELU
                               rule's likewise).  LAMP_RANDOM: those of the
                               strict rule that fixes the per-row counts.
                               Always 0 for the layer norm (no per-key
                               criterion)                                     */
    int32_t impl;           /* the implementation that ran (LAMP_IMPL_*)     */
    int32_t reserved;       /* 0                                              */
} lamp_stats;

/* Implementations a call can run (lamp_stats.impl, lamp_last_impl()). */
enum {
    LAMP_IMPL_NONE = 0,
    LAMP_IMPL_STRICT_ROWS = 1,     /* strict, rows of <= 1024 keys: score tiles,
                                      one wave per row (statistics, selection,
                                      recompute, probabilities), P.V          */
    LAMP_IMPL_STRICT_STREAM = 2,   /* strict, longer rows: score tiles, row
                                      selection, list recompute, finish       */
    LAMP_IMPL_RANDOM = 3,          /* random control: score tiles, strict
                                      counts, hash selection, recompute,
                                      finish                                  */
    LAMP_IMPL_RELAXED_FUSED = 4,   /* relaxed, the fused one-pass kernel (online
                                      softmax) [+ probabilities pass]         */
    LAMP_IMPL_RELAXED_ROWS = 5,    /* relaxed, two passes over rows of <= 1024
                                      keys: score tiles, row pass, P.V        */
    LAMP_IMPL_RELAXED_STREAM = 6,  /* relaxed, two passes over longer rows:
                                      score tiles, streaming row pass, finish */
    LAMP_IMPL_DECODE = 7,          /* lamp_decode_fwd                         */
    LAMP_IMPL_GELU = 8,            /* lamp_gelu_fwd                           */
    LAMP_IMPL_LAYERNORM = 9        /* lamp_layernorm_fwd                      */
};

/* Optional extras for lamp_attention_fwd_ex.  Zero-initialise and set what
 * you need; every pointer may be NULL. */
typedef struct {
    void *stream;             /* hipStream_t to enqueue on; NULL = default    */
    void *workspace;          /* device scratch of workspace_bytes, or NULL:
                                 the library keeps a per-device pool, grown
                                 on demand and shared by every call on that
                                 device; a call that uses it first makes its
                                 stream wait for the previous user's work
                                 (an event), so calls on different streams
                                 never overlap on the pool.  Pass a
                                 workspace per stream to let them overlap    */
    size_t workspace_bytes;   /* >= lamp_workspace_bytes(...) when given      */
    uint64_t seed;            /* LAMP_RANDOM seed                             */
    double *row_kl;           /* device [B,H,S]: KL(P_FP32 || P_LAMP) per row */
    double *row_kl_lowp;      /* device [B,H,S]: KL(P_FP32 || P_lowp) per row */
    uint32_t *row_count;      /* device [B,H,S]: selected keys per row        */
    float *scores_mix;        /* device [B,H,S,S]: y^mix (selected entries
                                 hold the FP32 recompute, others y^lo); valid
                                 entries only, others untouched.  Strict and
                                 random modes, and relaxed when non-NULL      */
    float *scores_ref;        /* device [B,H,S,S]: uniform FP32 scores y^ref  */
    void **stage_events;      /* NULL or 2*LAMP_N_STAGES hipEvent_t created by
                                 the caller; event 2s / 2s+1 are recorded on
                                 the stream before / after stage s when that
                                 stage runs (profiling); a NULL entry is not
                                 recorded.  Each record of an event created
                                 without hipEventDisableSystemFence writes
                                 back and invalidates the caches, which slows
                                 the stage after it                           */
    int ps_block;             /* PS(mu) accumulation order: 0 or 1 = the
                                 sequential order (default); a power of two
                                 b >= 4 (<= 2^24) = the blocked ("packed")
                                 order of a native low-precision dot unit
                                 (LAMP summary, "Significance"): the products
                                 of each run of b consecutive terms are summed
                                 from +0 in PS(mu), and each run's sum is added
                                 to the running accumulator with one more
                                 PS(mu) rounding.  Only y^lo changes; the FP32
                                 reference and recompute stay sequential.
                                 Other values: LAMP_ERR_INVALID_ARG (< 0) or
                                 LAMP_ERR_UNSUPPORTED                         */
    int relaxed_path;         /* LAMP_RELAXED only: which implementation.
                                 0 = the library's choice: rows of <= 1024
                                 keys with probs written run in two passes
                                 (score tiles, then one wave per row: the
                                 relaxed rule, FP32 recompute, softmax,
                                 probabilities; then P.V), other rows of
                                 <= 1024 keys in the fused one-pass kernel
                                 (online softmax); longer rows in two passes
                                 (below) when their dense score buffers fit
                                 the caller's workspace or the library's
                                 pool can allocate them, else in the fused
                                 kernel.
                                 1 = always the fused one-pass kernel.
                                 2 = always two passes.  Rows longer than
                                 1024 keys: score tiles keeping y^lo, y^ref
                                 and per-tile partials, one streaming pass
                                 per row (relaxed rule, y^mix in place,
                                 softmax sums, KL), then probabilities and
                                 P.V; the workspace then holds the dense
                                 score buffers the caller does not pass.
                                 Masks, counts and y^mix are the same either
                                 way; probabilities, out and KL agree within
                                 the stated tolerances.  Other values:
                                 LAMP_ERR_INVALID_ARG                         */
    int block_k;              /* LAMP_RELAXED: the key-block width of the
                                 relaxed rule's running maximum m_t (part of
                                 the rule's definition).  0 = 64, the default
                                 and the only width implemented; any other
                                 value: LAMP_ERR_UNSUPPORTED (< 0:
                                 LAMP_ERR_INVALID_ARG).  Ignored by the other
                                 modes                                        */
} lamp_params;

/* Stages, for lamp_params.stage_events. */
enum {
    LAMP_STAGE_SCAN = 0,      /* operand range scan (fast/exact path choice)  */
    LAMP_STAGE_SCORES = 1,    /* PS(mu) + FP32 score tiles on the FP32 fast
                                 path (strict, random); the fused one-pass
                                 kernel on the fast path (relaxed)            */
    LAMP_STAGE_SELECT = 2,    /* row softmax + selection + compaction         */
    LAMP_STAGE_RECOMPUTE = 3, /* gather FP32 recompute + scatter              */
    LAMP_STAGE_FINISH = 4,    /* softmax, probs, P.V, KL (strict, random);
                                 probs normalise pass (relaxed)               */
    LAMP_STAGE_STATS = 5,     /* row reductions into lamp_stats               */
    LAMP_STAGE_EXACT = 6,     /* score tiles / query blocks outside the FP32
                                 fast path (exact double path; FP32 at mu=23) */
    LAMP_N_STAGES = 7
};

/*
 * lamp_attention_fwd -- LAMP attention forward (the whole hot path).
 *   q, k, v         [B,H,S,D] inputs (required).
 *   B, H, S, D      sizes, >= 1; D % 4 == 0 and D <= 256.
 *   causal          0 or 1.
 *   mu              PS(mu) fraction bits, 1..23.
 *   tau             selection threshold, >= 0 (+inf selects nothing).
 *   mode            LAMP_STRICT, LAMP_RELAXED or LAMP_RANDOM.
 *   out             [B,H,S,D] attention output (required).
 *   probs           [B,H,S,S] final softmax, or NULL; invalid keys are 0.
 *   recompute_mask  [B,H,S,ceil(S/32)] uint32 or NULL: bit (j % 32) of word
 *                   j / 32 is set iff score (i, j) was recomputed; all other
 *                   bits (invalid keys, padding) are 0.
 *   stats           host lamp_stats or NULL (non-NULL synchronises).
 * Uses the default stream and the library-managed workspace.
 */
int lamp_attention_fwd(const float *q, const float *k, const float *v,
                       int B, int H, int S, int D, int causal, int mu, float tau, int mode,
                       float *out, float *probs, uint32_t *recompute_mask, lamp_stats *stats);

/* Same, with the optional extras of lamp_params (p may be NULL). */
int lamp_attention_fwd_ex(const float *q, const float *k, const float *v,
                          int B, int H, int S, int D, int causal, int mu, float tau, int mode,
                          float *out, float *probs, uint32_t *recompute_mask, lamp_stats *stats,
                          const lamp_params *p);

/*
 * lamp_attention_fwd_noalloc -- lamp_attention_fwd_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc /
 * hipFree, no library allocation): its scratch is a fixed device array of
 * LAMP_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The caller still passes all inputs and outputs.
 *   Arguments as for lamp_attention_fwd_ex; p->workspace must be NULL
 *   (LAMP_ERR_INVALID_ARG otherwise).
 *   A call whose scratch need (lamp_workspace_bytes_ex with the same
 *   arguments; relaxed rows longer than 1024 keys fall back to the fused
 *   one-pass kernel first) exceeds LAMP_NOALLOC_SCRATCH_BYTES is refused
 *   with LAMP_ERR_UNSUPPORTED before any HIP call.  Passing the optional
 *   buffers (probs, scores_ref, row_count, row_kl) keeps them out of the
 *   scratch.
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind (each call clears what it needs cleared): calls that overlap on
 *   one GPU -- different streams or host threads without ordering between
 *   them -- race and give undefined results.  Order them (one stream, or
 *   events), or use lamp_attention_fwd_ex.
 *   A non-NULL `stats` still synchronises the stream.
 */
#define LAMP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int lamp_attention_fwd_noalloc(const float *q, const float *k, const float *v,
                               int B, int H, int S, int D, int causal, int mu, float tau,
                               int mode, float *out, float *probs, uint32_t *recompute_mask,
                               lamp_stats *stats, const lamp_params *p);

/*
 * lamp_workspace_bytes -- device scratch that lamp_attention_fwd_ex needs for
 * these sizes and mode when probs / scores_mix / scores_ref are not given by
 * the caller (an upper bound: it assumes none of them is).  Returns 0 on
 * invalid sizes.
 */
size_t lamp_workspace_bytes(int B, int H, int S, int D, int mode, int want_probs);

/*
 * lamp_workspace_bytes_ex -- the exact device scratch of one
 * lamp_attention_fwd_ex call: the same sizes, causal flag and mode, whether
 * probs is given (want_probs) and stats requested (want_stats), and the
 * call's lamp_params p (may be NULL), whose scores_mix, scores_ref, row_kl,
 * row_kl_lowp, row_count and relaxed_path decide what the library keeps in
 * the workspace.  Relaxed rows longer than 1024 keys with relaxed_path 0:
 * the size of the two-pass form (dense score buffers); a workspace smaller
 * than that but at least the relaxed_path = 1 size runs the fused one-pass
 * kernel instead (per-row state only).  Returns 0 on invalid arguments
 * (lamp_last_error() says which).
 */
size_t lamp_workspace_bytes_ex(int B, int H, int S, int D, int causal, int mode, int want_probs,
                               int want_stats, const lamp_params *p);

/*
 * lamp_ps_scores -- step 1 alone: the PS(mu) scores y^lo and the uniform FP32
 * scores y^ref of every valid (i, j), written into [B,H,S,S] buffers (invalid
 * entries untouched).  Either output may be NULL (not both).  Enqueued on
 * `stream` (NULL = default); no synchronisation; no workspace beyond a small
 * library-managed flag array.
 */
int lamp_ps_scores(const float *q, const float *k, int B, int H, int S, int D, int causal, int mu,
                   float *ylo, float *yref, void *stream);

/*
 * lamp_decode_fwd -- relaxed LAMP at decode shapes: Nq new queries per (batch,
 * head) against a cache of S keys (LAMP summary, "Experimental results": the
 * relaxed relative-threshold rule, which needs no look-ahead over the row, so
 * the keys can be split across the GPU; "Implementation strategy" steps 1-3).
 * The queries are the last Nq positions of the sequence: with causal = 1,
 * query t sees keys 0 .. S - Nq + t; with causal = 0 every query sees all S
 * keys.  Every result equals rows S - Nq .. S - 1 of lamp_attention_fwd in
 * LAMP_RELAXED mode on the full sequence (same PS(mu) scores, the same
 * canonical 64-key running maximum for the rule, bit-exact masks).
 *   q               [B,H,Nq,D] queries (required).
 *   k, v            [B,H,S,D] key / value cache (required).
 *   B, H, Nq, S, D  sizes, >= 1; Nq <= 16 and Nq <= S; D % 4 == 0, D <= 256;
 *                   B*H*Nq <= 65535.
 *   causal, mu, tau as for lamp_attention_fwd.
 *   out             [B,H,Nq,D] (required).
 *   probs           [B,H,Nq,S] or NULL; keys a query does not see are 0.
 *   recompute_mask  [B,H,Nq,ceil(S/32)] uint32 or NULL, encoded as above.
 *   stats           host lamp_stats or NULL (non-NULL synchronises); n_rows is
 *                   B*H*Nq and n_exact_tiles counts 256-key chunks that took
 *                   the exact double-precision path.
 *   p               NULL or extras: stream, workspace (see
 *                   lamp_decode_workspace_bytes), row_kl / row_kl_lowp /
 *                   row_count per query row ([B,H,Nq]), scores_mix / scores_ref
 *                   ([B,H,Nq,S]: y^mix and y^ref of the valid keys), and
 *                   stage_events (LAMP_STAGE_SCORES: score pass;
 *                   LAMP_STAGE_SELECT: rule, softmax and P.V partials per
 *                   chunk; LAMP_STAGE_FINISH: combine and probabilities;
 *                   LAMP_STAGE_STATS).  seed is unused.
 * Errors and ownership as for lamp_attention_fwd.
 */
int lamp_decode_fwd(const float *q, const float *k, const float *v,
                    int B, int H, int Nq, int S, int D, int causal, int mu, float tau,
                    float *out, float *probs, uint32_t *recompute_mask, lamp_stats *stats,
                    const lamp_params *p);

/* Device scratch lamp_decode_fwd needs when none of scores_mix, scores_ref,
 * row_count, row_kl, row_kl_lowp is given (an upper bound); 0 on invalid
 * sizes. */
size_t lamp_decode_workspace_bytes(int B, int H, int Nq, int S, int D);

/*
 * LAMP after a matrix product y = x W^T accumulated in PS(mu) (LAMP summary,
 * "Theoretical foundation" item 3: an activation function and layer
 * normalisation have closed-form sensitivities too; "Implementation strategy"
 * steps 1-3).  x is [M,K] and W is [N,K], both row-major FP32; y^lo[i][j] is
 * the PS(mu) dot of row i of x and row j of W in k order (rounded after every
 * multiply and add), y^ref[i][j] the plain FP32 dot in the same order.
 *
 * lamp_gelu_fwd -- GELU (tanh form) on y with the activation rule: y_ij is
 *   recomputed in FP32 iff |GELU'(y^lo_ij) y^lo_ij| > tau (evaluated in
 *   double), out = GELU(y^mix) rounded to FP32.
 *   x, w            inputs (required, 16-byte aligned).
 *   M, N, K         sizes, >= 1; K % 4 == 0, K <= 2^24.
 *   mu              PS(mu) fraction bits, 1..23.
 *   tau             threshold, >= 0 (+inf selects nothing).
 *   out             [M,N] (required, 16-byte aligned).
 *   recompute_mask  [M,ceil(N/32)] uint32 or NULL, bit j % 32 of word j / 32
 *                   set iff y_ij was recomputed (padding bits 0).
 *   stats           host lamp_stats or NULL (non-NULL synchronises): n_rows M,
 *                   n_valid M*N, n_selected, n_exact_tiles (64x64 tiles on the
 *                   exact path), kl_sum / kl_max / kl_lowp_sum hold the row
 *                   error measures below instead of KL.
 *   p               NULL or extras: stream, workspace (lamp_mlp_workspace_bytes),
 *                   row_kl [M] (double): sum_j |out_ij - GELU(y^ref_ij)| in
 *                   double before the final rounding; row_kl_lowp [M]: the same
 *                   for the all-PS(mu) output; row_count [M]; scores_mix /
 *                   scores_ref [M,N]: y^mix and y^ref; stage_events
 *                   (LAMP_STAGE_SCAN, LAMP_STAGE_SCORES: fast-path tiles with the
 *                   rule fused, LAMP_STAGE_EXACT, LAMP_STAGE_FINISH: row sums).
 *
 * lamp_layernorm_fwd -- layer normalisation of each row of y with the greedy
 *   rule: with sigma^2 = var(y^lo_i) + eps, the components of largest |y^lo_ij|
 *   (ties to the lower j) are recomputed until the others have
 *   sum y_j^2 <= tau^2 sigma^2 N; out = gamma (y^mix - mean) / sqrt(var + eps)
 *   + beta over y^mix, in double, rounded to FP32.  N <= 8192.
 *   gamma, beta     [N] (required).  eps >= 0.
 *   Other arguments as for lamp_gelu_fwd; row_kl / row_kl_lowp hold the l2
 *   distances ||LN(y^mix) - LN(y^ref)|| and ||LN(y^lo) - LN(y^ref)|| per row.
 *
 * Errors and ownership as for lamp_attention_fwd.
 */
int lamp_gelu_fwd(const float *x, const float *w, int M, int N, int K, int mu, float tau,
                  float *out, uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p);

int lamp_layernorm_fwd(const float *x, const float *w, const float *gamma, const float *beta,
                       int M, int N, int K, int mu, float eps, float tau, float *out,
                       uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p);

/* Device scratch lamp_gelu_fwd (op 1) or lamp_layernorm_fwd (op 2) needs when
 * none of the optional outputs is given (an upper bound); 0 on invalid
 * sizes. */
size_t lamp_mlp_workspace_bytes(int M, int N, int K, int op);

/*
 * lamp_gemm_scores -- the matrix product alone: y^lo (PS(mu)) and y^ref (FP32)
 * of x [M,K] and W [N,K] into [M,N] buffers; either may be NULL (not both).
 * Enqueued on `stream`; no synchronisation.
 */
int lamp_gemm_scores(const float *x, const float *w, int M, int N, int K, int mu, float *ylo,
                     float *yref, void *stream);

/*
 * lamp_diag_exp -- diagnostic: evaluates the library's two device exponentials
 * (the double one used for the selection criterion and the KL sums, the
 * FP32-accurate one used for probabilities) on n device doubles x, writing
 * y64[e] and y32[e].  For accuracy tests; enqueued on `stream`.  Returns 0,
 * -1 on NULL pointers or n < 0, -3 on a launch failure.
 */
int lamp_diag_exp(const double *x, double *y64, float *y32, int n, void *stream);

/* The implementation (LAMP_IMPL_*) that the calling thread's last
 * successful lamp_attention_fwd[_ex], lamp_decode_fwd, lamp_gelu_fwd or
 * lamp_layernorm_fwd call ran; LAMP_IMPL_NONE before the first one.  The
 * same value lamp_stats.impl reports, without the synchronisation that
 * filling lamp_stats costs. */
int lamp_last_impl(void);

/* Static text for a return code. */
const char *lamp_strerror(int code);

/* Thread-local detail of this thread's last failing call ("" if none). */
const char *lamp_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int lamp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAMP_H */
