// lamp_api.cpp -- the C ABI declared in include/lamp.h: argument checks,
// workspace layout, launch sequence, errors.
//
// Launch sequence of one call (LAMP summary, "Implementation strategy"):
//   strict, S <= 1024: operand scan -> PS(mu) score tiles (+ per-tile FP32
//                     reference statistics) -> fused row pass (softmax
//                     statistics, selection, compaction, gather FP32
//                     recompute, probabilities, KL) -> P.V -> [stats]
//   strict (longer rows) / random: operand scan -> PS(mu) + FP32 score
//                     tiles -> row softmax + selection + compaction (random:
//                     strict counts, then hash selection) -> gather FP32
//                     recompute -> softmax + P.V + KL -> [stats]
//   relaxed:          operand scan -> fused one-pass kernel -> [probs pass]
//                     -> [stats]; rows of <= 1024 keys with probs: the strict
//                     sequence with the relaxed rule in the row pass
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "lamp.h"
#include "lamp_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local int g_last_impl = LAMP_IMPL_NONE;

int set_error(int code, const std::string &msg)
{
    g_last_error = msg;
    return code;
}

int hip_error(hipError_t e, const char *what)
{
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return LAMP_ERR_HIP;
}

#define LAMP_HIP_TRY(expr, what)                  \
    do {                                          \
        hipError_t e_ = (expr);                   \
        if (e_ != hipSuccess)                     \
            return hip_error(e_, what);           \
    } while (0)

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Library-managed workspace, one per device, grow-only.  Calls that use it
// are serialised on the device: a call holds the pool's lock while it
// enqueues its work, first makes its stream wait for the event the previous
// user recorded after its last launch, and records that event again after
// its own (PoolLease's destructor), so work on different streams never runs
// over the same pool memory at the same time.
struct Pool {
    void *ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;   // recorded after the last user's launches
    bool pending = false;        // `done` has been recorded at least once
};
std::mutex g_pool_mutex;
std::vector<Pool> g_pools;

class PoolLease {
  public:
    PoolLease() = default;
    PoolLease(const PoolLease &) = delete;
    PoolLease &operator=(const PoolLease &) = delete;
    ~PoolLease()
    {
        if (pool_ && pool_->done && hipEventRecord(pool_->done, st_) == hipSuccess)
            pool_->pending = true;
    }
    // The pool of the current device, at least `bytes` large, in *out; the
    // lock is held until this lease ends.
    int acquire(size_t bytes, hipStream_t st, void **out)
    {
        int dev = 0;
        LAMP_HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
        lock_ = std::unique_lock<std::mutex>(g_pool_mutex);
        if ((size_t)dev >= g_pools.size())
            g_pools.resize(dev + 1);
        Pool &p = g_pools[dev];
        if (!p.done)
            LAMP_HIP_TRY(hipEventCreateWithFlags(&p.done, hipEventDisableTiming),
                         "hipEventCreateWithFlags");
        if (p.bytes < bytes) {
            if (p.ptr) {
                // in-flight work may still use the old block
                LAMP_HIP_TRY(hipDeviceSynchronize(), "hipDeviceSynchronize");
                LAMP_HIP_TRY(hipFree(p.ptr), "hipFree");
                p.ptr = nullptr;
                p.bytes = 0;
            }
            void *ptr = nullptr;
            hipError_t e = hipMalloc(&ptr, bytes);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return set_error(LAMP_ERR_NO_MEMORY,
                                 "hipMalloc of " + std::to_string(bytes) + " bytes failed: " +
                                     hipGetErrorString(e));
            }
            p.ptr = ptr;
            p.bytes = bytes;
        } else if (p.pending) {
            LAMP_HIP_TRY(hipStreamWaitEvent(st, p.done, 0), "hipStreamWaitEvent");
        }
        pool_ = &p;
        st_ = st;
        *out = p.ptr;
        return LAMP_OK;
    }

  private:
    std::unique_lock<std::mutex> lock_;
    Pool *pool_ = nullptr;
    hipStream_t st_ = nullptr;
};

struct Sizes {
    uint64_t BH, n_rows, n_valid, n_scores;
    int tiles, W;
};

int check_sizes(int B, int H, int S, int D, Sizes *z)
{
    if (B < 1 || H < 1 || S < 1 || D < 1)
        return set_error(LAMP_ERR_INVALID_ARG, "B, H, S and D must be >= 1");
    if (D % 4 != 0 || D > 256)
        return set_error(LAMP_ERR_UNSUPPORTED, "D must be a multiple of 4 and at most 256");
    z->BH = (uint64_t)B * (uint64_t)H;
    z->n_rows = z->BH * (uint64_t)S;
    z->tiles = (S + lamp::kTile - 1) / lamp::kTile;
    z->W = (S + 31) / 32;
    z->n_scores = z->n_rows * (uint64_t)S;
    if (z->BH > (1ull << 31) || z->n_rows >= (1ull << 31) ||
        z->BH * (uint64_t)z->tiles * (uint64_t)z->tiles >= (1ull << 31) ||
        z->n_scores > (1ull << 40))
        return set_error(LAMP_ERR_UNSUPPORTED, "problem size overflows the launch geometry");
    return LAMP_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_args(const float *q, const float *k, const float *v, int causal, int mu, float tau,
               int mode, const float *out)
{
    if (!q || !k || !v || !out)
        return set_error(LAMP_ERR_INVALID_ARG, "q, k, v and out are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return set_error(LAMP_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (causal != 0 && causal != 1)
        return set_error(LAMP_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (mu < 1 || mu > 23)
        return set_error(LAMP_ERR_INVALID_ARG, "mu must be in [1, 23]");
    if (isnan(tau) || tau < 0.0f)
        return set_error(LAMP_ERR_INVALID_ARG, "tau must be >= 0 and not NaN");
    if (mode != LAMP_STRICT && mode != LAMP_RELAXED && mode != LAMP_RANDOM)
        return set_error(LAMP_ERR_INVALID_ARG, "unknown mode");
    return LAMP_OK;
}

// Workspace carve-up; offsets of pieces that are not needed stay SIZE_MAX.
struct Layout {
    size_t ymix = SIZE_MAX, yref = SIZE_MAX, list = SIZE_MAX, row_count = SIZE_MAX,
           row_kl = SIZE_MAX, row_kl_lowp = SIZE_MAX, unsafe = SIZE_MAX, dstats = SIZE_MAX,
           row_m = SIZE_MAX, row_l = SIZE_MAX, rowstats = SIZE_MAX, pbuf = SIZE_MAX,
           part = SIZE_MAX;
    size_t total = 0;
    size_t take(size_t bytes)
    {
        size_t off = total;
        total += align_up(bytes);
        return off;
    }
};

struct Needs {
    bool ymix, yref, row_count, row_kl, row_kl_lowp;
    bool fused;   // rows of <= 1024 keys through the fused row pass (strict;
                  // relaxed in two passes)
    bool pbuf;    // fused: probabilities need their own buffer
    bool part;    // fused: per-tile partials (KL wanted; relaxed rule)
    bool rowkl;   // fused: the row KLs are formed (KL wanted)
    bool relaxed_long;   // relaxed in two passes over rows longer than 1024 keys
};

constexpr int kFusedMaxS = 1024;

Layout plan(const Sizes &z, int mode, const Needs &n)
{
    Layout L;
    L.dstats = L.take(sizeof(lamp::DevStats));
    L.unsafe = L.take(2 * z.BH * (uint64_t)z.tiles);
    if (n.row_count)
        L.row_count = L.take(4 * z.n_rows);
    if (n.row_kl)
        L.row_kl = L.take(8 * z.n_rows);
    if (n.row_kl_lowp)
        L.row_kl_lowp = L.take(8 * z.n_rows);
    if (n.relaxed_long) {
        if (n.ymix)
            L.ymix = L.take(4 * z.n_scores);
        if (n.yref)
            L.yref = L.take(4 * z.n_scores);
        L.part = L.take(sizeof(lamp::RefPartial) * z.n_rows * (uint64_t)z.tiles);
        L.rowstats = L.take(sizeof(lamp::RowStats) * z.n_rows);
    } else if (mode == LAMP_RELAXED && !n.fused) {
        if (n.ymix) {   // probs requested: per-row statistics for the probs pass
            L.row_m = L.take(4 * z.n_rows);
            L.row_l = L.take(8 * z.n_rows);
        }
    } else if (n.fused) {
        if (n.ymix)
            L.ymix = L.take(4 * z.n_scores);
        if (n.yref)
            L.yref = L.take(4 * z.n_scores);
        if (n.pbuf)
            L.pbuf = L.take(4 * z.n_scores);
        if (n.part)
            L.part = L.take(sizeof(lamp::RefPartial) * z.n_rows * (uint64_t)z.tiles);
    } else {
        if (n.ymix)
            L.ymix = L.take(4 * z.n_scores);
        if (n.yref)
            L.yref = L.take(4 * z.n_scores);
        L.list = L.take(4 * z.n_valid);
        L.rowstats = L.take(sizeof(lamp::RowStats) * z.n_rows);
    }
    return L;
}

// What a call needs in its workspace, given the optional buffers the caller
// passes.  relaxed_long: relaxed rows longer than 1024 keys in two passes.
Needs make_needs(const lamp_params &p, int mode, int S, bool probs, bool want_stats,
                 bool relaxed_long)
{
    Needs need{};
    need.row_count = p.row_count == nullptr;
    need.row_kl = p.row_kl == nullptr && want_stats;
    need.row_kl_lowp = p.row_kl_lowp == nullptr && want_stats;
    // relaxed rows of <= 1024 keys in two passes (score tiles, row pass)
    const bool relaxed_rows = mode == LAMP_RELAXED && S <= kFusedMaxS &&
                              (p.relaxed_path == 2 || (p.relaxed_path == 0 && probs));
    need.fused = (mode == LAMP_STRICT && S <= kFusedMaxS) || relaxed_rows;
    need.relaxed_long = relaxed_long;
    const bool want_kl = want_stats || p.row_kl || p.row_kl_lowp;
    if (need.relaxed_long) {
        need.ymix = p.scores_mix == nullptr && !probs;
        need.yref = p.scores_ref == nullptr;
    } else if (mode == LAMP_RELAXED && !need.fused) {
        need.ymix = probs;
        need.yref = false;
    } else if (need.fused) {
        need.ymix = p.scores_mix == nullptr && !probs;
        need.pbuf = p.scores_mix != nullptr && !probs;
        need.part = want_kl || relaxed_rows;
        need.rowkl = want_kl;
        // the score tiles form y^ref for every pair when they form the
        // partials: kept, the row pass takes the selected scores' FP32 values
        // from it instead of forming each dot again (a gather dot per
        // selected key costs the row pass more than the dense store costs the
        // score tiles)
        need.yref = need.part && p.scores_ref == nullptr;
    } else {
        // longer strict rows and the random control: y^ref only for the row
        // KLs (without them the recompute forms each selected key's FP32 dot
        // from the gathered query and key rows)
        need.ymix = p.scores_mix == nullptr && !probs;
        need.yref = p.scores_ref == nullptr && want_kl;
    }
    return need;
}

template <typename T>
T *at(void *base, size_t off)
{
    return off == SIZE_MAX ? nullptr : reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

struct StageTimer {
    void **ev;
    hipStream_t st;
    hipError_t begin(int s) { return rec(2 * s); }
    hipError_t end(int s) { return rec(2 * s + 1); }
    hipError_t rec(int i)
    {   // (a NULL entry: that stage is not timed)
        return ev && ev[i] ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
    }
};

}  // namespace

// ---------------------------------------------------------------------------
// Decode shapes (relaxed rule).
// ---------------------------------------------------------------------------
namespace {

struct DecodeLayout {
    size_t ylo = SIZE_MAX, yref = SIZE_MAX, bmax = SIZE_MAX, unsafe = SIZE_MAX, part = SIZE_MAX,
           acc = SIZE_MAX,
           row_lse = SIZE_MAX, row_count = SIZE_MAX, row_kl = SIZE_MAX, row_kl_lowp = SIZE_MAX,
           dstats = SIZE_MAX;
    size_t total = 0;
    size_t take(size_t bytes)
    {
        size_t off = total;
        total += align_up(bytes);
        return off;
    }
};

constexpr int kDecodeMaxQ = 16;

int check_decode(int B, int H, int Nq, int S, int D)
{
    if (B < 1 || H < 1 || Nq < 1 || S < 1 || D < 1)
        return set_error(LAMP_ERR_INVALID_ARG, "B, H, Nq, S and D must be >= 1");
    if (Nq > kDecodeMaxQ)
        return set_error(LAMP_ERR_UNSUPPORTED, "Nq must be at most 16");
    if (Nq > S)
        return set_error(LAMP_ERR_INVALID_ARG, "Nq must not exceed S");
    if (D % 4 != 0 || D > 256)
        return set_error(LAMP_ERR_UNSUPPORTED, "D must be a multiple of 4 and at most 256");
    const uint64_t BH = (uint64_t)B * (uint64_t)H;
    if (BH * (uint64_t)Nq > 65535 || (uint64_t)S > (1ull << 30) ||
        BH * (uint64_t)Nq * (uint64_t)S > (1ull << 40))
        return set_error(LAMP_ERR_UNSUPPORTED, "problem size overflows the launch geometry");
    return LAMP_OK;
}

DecodeLayout decode_plan(uint64_t BH, int Nq, int S, int D, bool need_ylo, bool need_yref,
                         bool need_count, bool need_kl, bool need_kl_lowp)
{
    DecodeLayout L;
    const uint64_t rows = BH * (uint64_t)Nq;
    L.dstats = L.take(sizeof(lamp::DevStats));
    if (need_ylo)
        L.ylo = L.take(4 * rows * (uint64_t)S);
    if (need_yref)
        L.yref = L.take(4 * rows * (uint64_t)S);
    const uint64_t blocks = (S + 63) / 64;
    L.bmax = L.take(4 * rows * blocks);
    L.unsafe = L.take(BH * (uint64_t)((S + 255) / 256));
    L.part = L.take(sizeof(lamp::DecPartial) * rows * blocks);
    L.acc = L.take(4 * rows * blocks * (uint64_t)D);
    L.row_lse = L.take(8 * rows);
    if (need_count)
        L.row_count = L.take(4 * rows);
    if (need_kl)
        L.row_kl = L.take(8 * rows);
    if (need_kl_lowp)
        L.row_kl_lowp = L.take(8 * rows);
    return L;
}

// The accumulation order of lamp_params.ps_block: 0, 1 or a power of two
// in [4, 2^24].
int check_ps_block(int b)
{
    if (b < 0)
        return set_error(LAMP_ERR_INVALID_ARG, "ps_block must be >= 0");
    if (b <= 1)
        return LAMP_OK;
    if (b < 4 || b > (1 << 24) || (b & (b - 1)) != 0)
        return set_error(LAMP_ERR_UNSUPPORTED,
                         "ps_block must be 0, 1 or a power of two in [4, 2^24]");
    return LAMP_OK;
}

// The relaxed rule's block width (lamp_params.block_k): 0 or 64.
int check_block_k(int b)
{
    if (b < 0)
        return set_error(LAMP_ERR_INVALID_ARG, "block_k must be >= 0");
    if (b != 0 && b != 64)
        return set_error(LAMP_ERR_UNSUPPORTED,
                         "block_k: only the 64-key block of the relaxed rule is implemented");
    return LAMP_OK;
}

// the summary fields of DevStats (the work-group partials stay on the device)
constexpr size_t kStatsHead = offsetof(lamp::DevStats, blocks_done);

void fill_stats(lamp_stats *stats, uint64_t n_rows, uint64_t n_valid, const lamp::DevStats &ds,
                int impl)
{
    stats->n_rows = n_rows;
    stats->n_valid = n_valid;
    stats->n_selected = ds.n_selected;
    stats->n_exact_tiles = ds.n_exact_tiles;
    stats->kl_sum = ds.kl_sum;
    stats->kl_max = ds.kl_max;
    stats->kl_lowp_sum = ds.kl_lowp_sum;
    stats->n_tie_band = ds.n_tie_band;
    stats->impl = impl;
    stats->reserved = 0;
}

int run_decode(const float *q, const float *k, const float *v, int B, int H, int Nq, int S, int D,
               int causal, int mu, float tau, float *out, float *probs, uint32_t *mask,
               lamp_stats *stats, const lamp_params *pp)
{
    g_last_error.clear();
    int rc = check_args(q, k, v, causal, mu, tau, LAMP_RELAXED, out);
    if (rc != LAMP_OK)
        return rc;
    rc = check_decode(B, H, Nq, S, D);
    if (rc != LAMP_OK)
        return rc;
    lamp_params none{};
    const lamp_params &p = pp ? *pp : none;
    rc = check_ps_block(p.ps_block);
    if (rc != LAMP_OK)
        return rc;
    rc = check_block_k(p.block_k);
    if (rc != LAMP_OK)
        return rc;
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)p.stream;
    const bool want_stats = stats != nullptr;
    const uint64_t BH = (uint64_t)B * (uint64_t)H;
    const DecodeLayout L =
        decode_plan(BH, Nq, S, D, p.scores_mix == nullptr, p.scores_ref == nullptr,
                    p.row_count == nullptr, p.row_kl == nullptr && want_stats,
                    p.row_kl_lowp == nullptr && want_stats);
    PoolLease lease;
    void *ws = nullptr;
    if (p.workspace) {
        if (p.workspace_bytes < L.total)
            return set_error(LAMP_ERR_INVALID_ARG,
                             "workspace too small: need " + std::to_string(L.total) + " bytes");
        if (((uintptr_t)p.workspace & (kAlign - 1)) != 0)
            return set_error(LAMP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        ws = p.workspace;
    } else {
        rc = lease.acquire(L.total, st, &ws);
        if (rc != LAMP_OK)
            return rc;
    }
    auto *dstats = at<lamp::DevStats>(ws, L.dstats);
    lamp::DecodeProblem P;
    P.q = q;
    P.k = k;
    P.v = v;
    P.BH = (int)BH;
    P.S = S;
    P.D = D;
    P.nq = Nq;
    P.causal = causal;
    P.mu = mu;
    P.tau = tau;
    P.ps_block = p.ps_block;
    P.n_band = want_stats ? &dstats->n_tie_band : nullptr;
    lamp::DecodeBuffers b;
    b.ylo = p.scores_mix ? p.scores_mix : at<float>(ws, L.ylo);
    b.yref = p.scores_ref ? p.scores_ref : at<float>(ws, L.yref);
    b.bmax = at<float>(ws, L.bmax);
    b.unsafe = at<uint8_t>(ws, L.unsafe);
    b.mask = mask;
    b.part = at<lamp::DecPartial>(ws, L.part);
    b.acc = at<float>(ws, L.acc);
    b.out = out;
    b.row_lse = at<double>(ws, L.row_lse);
    b.row_count = p.row_count ? p.row_count : at<uint32_t>(ws, L.row_count);
    b.row_kl = p.row_kl ? p.row_kl : at<double>(ws, L.row_kl);
    b.row_kl_lowp = p.row_kl_lowp ? p.row_kl_lowp : at<double>(ws, L.row_kl_lowp);
    b.probs = probs;
    b.exact_chunks = &dstats->n_exact_tiles;
    LAMP_HIP_TRY(lamp::launch_zero(dstats, sizeof(lamp::DevStats), st), "zero stats");
    LAMP_HIP_TRY(lamp::launch_decode(P, b, st, p.stage_events), "decode kernels launch");
    if (want_stats) {
        lamp::Problem Ps{};
        Ps.n_rows = BH * (uint64_t)Nq;
        StageTimer tm{p.stage_events, st};
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_STATS), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_stats(Ps, b.row_kl, b.row_kl_lowp, b.row_count, dstats, st),
                     "stats launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_STATS), "hipEventRecord");
        lamp::DevStats ds;
        LAMP_HIP_TRY(hipMemcpyAsync(&ds, dstats, kStatsHead, hipMemcpyDeviceToHost, st),
                     "hipMemcpyAsync stats");
        LAMP_HIP_TRY(hipStreamSynchronize(st), "hipStreamSynchronize");
        const uint64_t per_head = causal ? (uint64_t)Nq * (uint64_t)(S - Nq) +
                                               (uint64_t)Nq * (uint64_t)(Nq + 1) / 2
                                         : (uint64_t)Nq * (uint64_t)S;
        fill_stats(stats, BH * (uint64_t)Nq, BH * per_head, ds, LAMP_IMPL_DECODE);
    }
    g_last_impl = LAMP_IMPL_DECODE;
    return LAMP_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Matrix product + activation / layer normalisation.
// ---------------------------------------------------------------------------
namespace {

constexpr int kLnMaxN = 8192;

struct MlpLayout {
    size_t unsafe = SIZE_MAX, ylo = SIZE_MAX, yref = SIZE_MAX, mask = SIZE_MAX,
           err_part = SIZE_MAX, errl_part = SIZE_MAX, err = SIZE_MAX, errl = SIZE_MAX,
           count = SIZE_MAX, dstats = SIZE_MAX;
    size_t total = 0;
    size_t take(size_t bytes)
    {
        size_t off = total;
        total += align_up(bytes);
        return off;
    }
};

int check_mlp(int M, int N, int K, int op)
{
    if (M < 1 || N < 1 || K < 1)
        return set_error(LAMP_ERR_INVALID_ARG, "M, N and K must be >= 1");
    if (K % 4 != 0)
        return set_error(LAMP_ERR_UNSUPPORTED, "K must be a multiple of 4");
    if (K > (1 << 24))
        return set_error(LAMP_ERR_UNSUPPORTED, "K must be <= 2^24");
    if (op == lamp::MLP_LAYERNORM && N > kLnMaxN)
        return set_error(LAMP_ERR_UNSUPPORTED, "layer normalisation supports N <= 8192");
    const uint64_t tm = (M + 63) / 64, tn = (N + 63) / 64;
    if (tm * tn >= (1ull << 31) || (uint64_t)M * (uint64_t)N > (1ull << 40) ||
        (uint64_t)M * (uint64_t)K > (1ull << 40) || (uint64_t)N * (uint64_t)K > (1ull << 40))
        return set_error(LAMP_ERR_UNSUPPORTED, "problem size overflows the launch geometry");
    return LAMP_OK;
}

MlpLayout mlp_plan(int M, int N, int op, bool need_ylo, bool need_yref, bool need_mask,
                   bool need_err, bool need_errl, bool need_count)
{
    MlpLayout L;
    const uint64_t tm = (M + 63) / 64, tn = (N + 63) / 64;
    L.dstats = L.take(sizeof(lamp::DevStats));
    L.unsafe = L.take(4 * (tm + tn));
    if (op == lamp::MLP_LAYERNORM) {
        if (need_ylo)
            L.ylo = L.take(4 * (uint64_t)M * N);
        if (need_yref)
            L.yref = L.take(4 * (uint64_t)M * N);
    }
    if (op == lamp::MLP_GELU) {
        const uint64_t nb = (uint64_t)(N + 31) / 32;   // 32-column blocks
        L.err_part = L.take(8 * (uint64_t)M * nb);
        L.errl_part = L.take(8 * (uint64_t)M * nb);
        if (need_mask)
            L.mask = L.take(4 * (uint64_t)M * ((N + 31) / 32));
    }
    if (need_err)
        L.err = L.take(8 * (uint64_t)M);
    if (need_errl)
        L.errl = L.take(8 * (uint64_t)M);
    if (need_count)
        L.count = L.take(4 * (uint64_t)M);
    return L;
}

int run_mlp(int op, const float *x, const float *w, const float *gamma, const float *beta, int M,
            int N, int K, int mu, float eps, float tau, float *out, uint32_t *mask,
            lamp_stats *stats, const lamp_params *pp)
{
    g_last_error.clear();
    if (!x || !w || !out || (op == lamp::MLP_LAYERNORM && (!gamma || !beta)))
        return set_error(LAMP_ERR_INVALID_ARG, "x, w, out (and gamma, beta) are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out))
        return set_error(LAMP_ERR_INVALID_ARG, "x, w and out must be 16-byte aligned");
    if (mu < 1 || mu > 23)
        return set_error(LAMP_ERR_INVALID_ARG, "mu must be in [1, 23]");
    if (isnan(tau) || tau < 0.0f)
        return set_error(LAMP_ERR_INVALID_ARG, "tau must be >= 0 and not NaN");
    if (op == lamp::MLP_LAYERNORM && (isnan(eps) || eps < 0.0f))
        return set_error(LAMP_ERR_INVALID_ARG, "eps must be >= 0 and not NaN");
    int rc = check_mlp(M, N, K, op);
    if (rc != LAMP_OK)
        return rc;
    lamp_params none{};
    const lamp_params &p = pp ? *pp : none;
    rc = check_ps_block(p.ps_block);
    if (rc != LAMP_OK)
        return rc;
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)p.stream;
    const bool want_stats = stats != nullptr;
    const MlpLayout L = mlp_plan(M, N, op, true, p.scores_ref == nullptr, mask == nullptr,
                                 p.row_kl == nullptr, p.row_kl_lowp == nullptr,
                                 p.row_count == nullptr);
    PoolLease lease;
    void *ws = nullptr;
    if (p.workspace) {
        if (p.workspace_bytes < L.total)
            return set_error(LAMP_ERR_INVALID_ARG,
                             "workspace too small: need " + std::to_string(L.total) + " bytes");
        if (((uintptr_t)p.workspace & (kAlign - 1)) != 0)
            return set_error(LAMP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        ws = p.workspace;
    } else {
        rc = lease.acquire(L.total, st, &ws);
        if (rc != LAMP_OK)
            return rc;
    }
    const int impl = op == lamp::MLP_GELU ? LAMP_IMPL_GELU : LAMP_IMPL_LAYERNORM;
    auto *dstats = at<lamp::DevStats>(ws, L.dstats);
    lamp::MlpProblem P;
    P.x = x;
    P.w = w;
    P.gamma = gamma;
    P.beta = beta;
    P.M = M;
    P.N = N;
    P.K = K;
    P.mu = mu;
    P.op = op;
    P.tau = tau;
    P.ps_block = p.ps_block;
    P.eps = eps;
    P.n_band = &dstats->n_tie_band;
    lamp::MlpBuffers b{};
    b.unsafe = at<uint32_t>(ws, L.unsafe);
    if (op == lamp::MLP_LAYERNORM) {
        b.ylo = at<float>(ws, L.ylo);
        b.yref = p.scores_ref ? p.scores_ref : at<float>(ws, L.yref);
        b.ymix = p.scores_mix;
    } else {
        b.ylo = p.scores_mix;   // y^mix, when asked for
        b.yref = p.scores_ref;
    }
    b.out = out;
    b.mask = mask ? mask : at<uint32_t>(ws, L.mask);
    b.err_part = at<double>(ws, L.err_part);
    b.errl_part = at<double>(ws, L.errl_part);
    b.err = p.row_kl ? p.row_kl : at<double>(ws, L.err);
    b.errl = p.row_kl_lowp ? p.row_kl_lowp : at<double>(ws, L.errl);
    uint32_t *count = p.row_count ? p.row_count : at<uint32_t>(ws, L.count);
    b.row_count = count;
    b.exact_tiles = &dstats->n_exact_tiles;
    LAMP_HIP_TRY(lamp::launch_zero(dstats, sizeof(lamp::DevStats), st), "zero stats");
    LAMP_HIP_TRY(lamp::launch_mlp(P, b, st, p.stage_events), "matrix product launch");
    if (op == lamp::MLP_GELU)
        LAMP_HIP_TRY(lamp::launch_mask_count(b.mask, M, N, count, st), "count launch");
    if (want_stats) {
        lamp::Problem Ps{};
        Ps.n_rows = (uint64_t)M;
        LAMP_HIP_TRY(lamp::launch_stats(Ps, b.err, b.errl, count, dstats, st), "stats launch");
        lamp::DevStats ds;
        LAMP_HIP_TRY(hipMemcpyAsync(&ds, dstats, kStatsHead, hipMemcpyDeviceToHost, st),
                     "hipMemcpyAsync stats");
        LAMP_HIP_TRY(hipStreamSynchronize(st), "hipStreamSynchronize");
        fill_stats(stats, (uint64_t)M, (uint64_t)M * (uint64_t)N, ds, impl);
    }
    g_last_impl = impl;
    return LAMP_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: a fixed device array, one per
// GPU (the code object's copy on each device), held until the process ends.
// Host code never uses the array's name as an address: its device address is
// looked up once per device with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = LAMP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device

int scratch_address(void **out)
{
    int dev = 0;
    LAMP_HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(LAMP_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        LAMP_HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress");
        if (!ptr || ((uintptr_t)ptr & (kAlign - 1)) != 0)
            return set_error(LAMP_ERR_HIP, "scratch array without a 256-byte aligned address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LAMP_OK;
}

}  // namespace

extern "C" {

const char *lamp_strerror(int code)
{
    switch (code) {
    case LAMP_OK: return "success";
    case LAMP_ERR_INVALID_ARG: return "invalid argument";
    case LAMP_ERR_UNSUPPORTED: return "unsupported problem shape";
    case LAMP_ERR_HIP: return "HIP runtime error";
    case LAMP_ERR_NO_MEMORY: return "out of device memory";
    default: return "unknown error";
    }
}

const char *lamp_last_error(void) { return g_last_error.c_str(); }

int lamp_version(void) { return 10100; }

int lamp_last_impl(void) { return g_last_impl; }

size_t lamp_workspace_bytes(int B, int H, int S, int D, int mode, int want_probs)
{
    Sizes z;
    if (check_sizes(B, H, S, D, &z) != LAMP_OK)
        return 0;
    if (mode != LAMP_STRICT && mode != LAMP_RELAXED && mode != LAMP_RANDOM)
        return 0;
    z.n_valid = 0;
    z.n_valid = z.BH * (uint64_t)S * (uint64_t)(S + 1) / 2;   // causal-agnostic bound below
    z.n_valid = z.n_scores > z.n_valid ? z.n_scores : z.n_valid;
    Needs n{mode == LAMP_RELAXED ? want_probs != 0 : want_probs == 0, true, true, true, true,
            false, false, false, false, false};
    size_t total = plan(z, mode, n).total;
    if ((mode == LAMP_STRICT || mode == LAMP_RELAXED) && S <= kFusedMaxS) {
        Needs f{want_probs == 0, true, true, true, true, true, false, true, true, false};
        const size_t tf = plan(z, mode, f).total;
        total = tf > total ? tf : total;
    }
    if (mode == LAMP_RELAXED && S > kFusedMaxS) {
        Needs f{want_probs == 0, true, true, true, true, false, false, false, false, true};
        const size_t tf = plan(z, mode, f).total;
        total = tf > total ? tf : total;
    }
    return total;
}

size_t lamp_workspace_bytes_ex(int B, int H, int S, int D, int causal, int mode, int want_probs,
                               int want_stats, const lamp_params *pp)
{
    try {
        Sizes z;
        if (check_sizes(B, H, S, D, &z) != LAMP_OK)
            return 0;
        if (mode != LAMP_STRICT && mode != LAMP_RELAXED && mode != LAMP_RANDOM) {
            set_error(LAMP_ERR_INVALID_ARG, "unknown mode");
            return 0;
        }
        if (causal != 0 && causal != 1) {
            set_error(LAMP_ERR_INVALID_ARG, "causal must be 0 or 1");
            return 0;
        }
        if (mode == LAMP_RELAXED && D > 128) {
            set_error(LAMP_ERR_UNSUPPORTED, "relaxed mode supports D <= 128");
            return 0;
        }
        lamp_params none{};
        const lamp_params &p = pp ? *pp : none;
        if (p.relaxed_path < 0 || p.relaxed_path > 2) {
            set_error(LAMP_ERR_INVALID_ARG, "relaxed_path must be 0, 1 or 2");
            return 0;
        }
        if (check_ps_block(p.ps_block) != LAMP_OK)
            return 0;
        if (mode == LAMP_RELAXED && check_block_k(p.block_k) != LAMP_OK)
            return 0;
        z.n_valid = causal ? z.BH * (uint64_t)S * (uint64_t)(S + 1) / 2 : z.n_scores;
        const bool relaxed_long = mode == LAMP_RELAXED && S > kFusedMaxS && p.relaxed_path != 1;
        return plan(z, mode,
                    make_needs(p, mode, S, want_probs != 0, want_stats != 0, relaxed_long))
            .total;
    } catch (...) {
        return 0;
    }
}

// Workspace of a call: the caller's (lamp_params.workspace), the library's
// pool, or -- for lamp_attention_fwd_noalloc -- the fixed scratch array.
enum class WsSource { kCallerOrPool, kScratch };

static int run(const float *q, const float *k, const float *v, int B, int H, int S, int D,
               int causal, int mu, float tau, int mode, float *out, float *probs,
               uint32_t *mask, lamp_stats *stats, const lamp_params *pp,
               WsSource src = WsSource::kCallerOrPool)
{
    g_last_error.clear();
    int rc = check_args(q, k, v, causal, mu, tau, mode, out);
    if (rc != LAMP_OK)
        return rc;
    Sizes z;
    rc = check_sizes(B, H, S, D, &z);
    if (rc != LAMP_OK)
        return rc;
    if (mode == LAMP_RELAXED && D > 128)
        return set_error(LAMP_ERR_UNSUPPORTED, "relaxed mode supports D <= 128");
    z.n_valid = causal ? z.BH * (uint64_t)S * (uint64_t)(S + 1) / 2 : z.n_scores;

    lamp_params none{};
    const lamp_params &p = pp ? *pp : none;
    rc = check_ps_block(p.ps_block);
    if (rc != LAMP_OK)
        return rc;
    if (p.relaxed_path < 0 || p.relaxed_path > 2)
        return set_error(LAMP_ERR_INVALID_ARG, "relaxed_path must be 0, 1 or 2");
    if (mode == LAMP_RELAXED) {
        rc = check_block_k(p.block_k);
        if (rc != LAMP_OK)
            return rc;
    }
    hipStream_t st = (hipStream_t)p.stream;
    const bool want_stats = stats != nullptr;

    // relaxed rows longer than 1024 keys: two passes when asked for, and by
    // default when their dense score buffers fit (the caller's workspace, or
    // what the pool can allocate); the fused one-pass kernel otherwise
    bool relaxed_long = mode == LAMP_RELAXED && S > kFusedMaxS && p.relaxed_path != 1;
    Needs need = make_needs(p, mode, S, probs != nullptr, want_stats, relaxed_long);
    Layout L = plan(z, mode, need);
    const bool may_fall_back = relaxed_long && p.relaxed_path == 0;
    auto fall_back = [&]() {
        relaxed_long = false;
        need = make_needs(p, mode, S, probs != nullptr, want_stats, false);
        L = plan(z, mode, need);
    };
    if (p.workspace && p.workspace_bytes < L.total && may_fall_back)
        fall_back();
    if (src == WsSource::kScratch) {
        if (p.workspace)
            return set_error(LAMP_ERR_INVALID_ARG,
                             "lamp_attention_fwd_noalloc takes no workspace (it uses the "
                             "library's scratch array)");
        if (L.total > kScratchBytes && may_fall_back)
            fall_back();
        if (L.total > kScratchBytes)
            return set_error(LAMP_ERR_UNSUPPORTED,
                             "this call needs " + std::to_string(L.total) +
                                 " bytes of scratch; lamp_attention_fwd_noalloc holds " +
                                 std::to_string(kScratchBytes) +
                                 " (pass buffers such as probs / scores_ref / row_count, or "
                                 "use lamp_attention_fwd_ex)");
    }

    PoolLease lease;
    void *ws = nullptr;
    if (src == WsSource::kScratch) {
        rc = scratch_address(&ws);
        if (rc != LAMP_OK)
            return rc;
    } else if (p.workspace) {
        if (p.workspace_bytes < L.total)
            return set_error(LAMP_ERR_INVALID_ARG,
                             "workspace too small: need " + std::to_string(L.total) + " bytes");
        if (((uintptr_t)p.workspace & (kAlign - 1)) != 0)
            return set_error(LAMP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        ws = p.workspace;
    } else {
        rc = lease.acquire(L.total, st, &ws);
        if (rc == LAMP_ERR_NO_MEMORY && may_fall_back) {
            fall_back();
            rc = lease.acquire(L.total, st, &ws);
            if (rc == LAMP_OK)
                g_last_error.clear();
        }
        if (rc != LAMP_OK)
            return rc;
    }
    (void)hipGetLastError();   // launches below are checked with hipGetLastError

    lamp::Problem P;
    P.q = q;
    P.k = k;
    P.v = v;
    P.BH = (int)z.BH;
    P.S = S;
    P.D = D;
    P.causal = causal;
    P.mu = mu;
    P.tau = tau;
    P.pc = lamp::make_ps_const(mu, D);
    lamp::set_ps_block(P.pc, p.ps_block, D);
    P.tiles = z.tiles;
    P.n_rows = z.n_rows;
    P.head_valid = z.n_valid / z.BH;
    // the partials' reference sums serve only the row KL, their y^lo block
    // maxima only the relaxed rule
    P.ref_sums = want_stats || p.row_kl || p.row_kl_lowp;
    P.lo_max = mode == LAMP_RELAXED;

    // the device summary's counters are kept (and zeroed) only for a summary
    auto *dstats = at<lamp::DevStats>(ws, L.dstats);
    unsigned long long *n_exact = want_stats ? &dstats->n_exact_tiles : nullptr;
    P.n_band = want_stats ? &dstats->n_tie_band : nullptr;
    auto *unsafe = at<uint8_t>(ws, L.unsafe);
    uint32_t *row_count = p.row_count ? p.row_count : at<uint32_t>(ws, L.row_count);
    double *row_kl = p.row_kl ? p.row_kl : at<double>(ws, L.row_kl);
    double *row_kl_lowp = p.row_kl_lowp ? p.row_kl_lowp : at<double>(ws, L.row_kl_lowp);
    StageTimer tm{p.stage_events, st};

    const int impl = need.relaxed_long ? LAMP_IMPL_RELAXED_STREAM
                     : (mode == LAMP_RELAXED && !need.fused) ? LAMP_IMPL_RELAXED_FUSED
                     : need.fused ? (mode == LAMP_RELAXED ? LAMP_IMPL_RELAXED_ROWS
                                                          : LAMP_IMPL_STRICT_ROWS)
                     : mode == LAMP_RANDOM ? LAMP_IMPL_RANDOM
                                           : LAMP_IMPL_STRICT_STREAM;
    if (want_stats)
        LAMP_HIP_TRY(lamp::launch_zero(dstats, sizeof(lamp::DevStats), st), "zero stats");
    LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SCAN), "hipEventRecord");
    LAMP_HIP_TRY(lamp::launch_operand_scan(P, unsafe, st), "operand scan launch");
    LAMP_HIP_TRY(tm.end(LAMP_STAGE_SCAN), "hipEventRecord");

    if (need.relaxed_long) {
        float *ymix = p.scores_mix ? p.scores_mix : (probs ? probs : at<float>(ws, L.ymix));
        float *yref = p.scores_ref ? p.scores_ref : at<float>(ws, L.yref);
        auto *part = at<lamp::RefPartial>(ws, L.part);
        auto *rs = at<lamp::RowStats>(ws, L.rowstats);
        // causal, probabilities asked for: their zeros above the diagonal
        // tiles come from the score tiles
        float *pzero = P.causal && probs ? probs : nullptr;
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ymix, yref, part,
                                            n_exact, false, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ymix, yref, part,
                                            n_exact, true, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SELECT), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_relaxed_select(P, ymix, yref, part, mask, row_count, rs,
                                                 row_kl, row_kl_lowp, st),
                     "relaxed select launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SELECT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_FINISH), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_finish(P, ymix, rs, probs, out, row_kl, st, pzero != nullptr),
                     "finish launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_FINISH), "hipEventRecord");
    } else if (mode == LAMP_RELAXED && !need.fused) {
        float *ymix_raw = p.scores_mix ? p.scores_mix : probs;
        float *row_m = at<float>(ws, L.row_m);
        double *row_l = at<double>(ws, L.row_l);
        // causal, probabilities asked for: each query block's zero tails come
        // from the fused kernel
        float *pzero = P.causal && probs ? probs : nullptr;
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_relaxed(P, unsafe, out, mask, row_count, row_kl, row_kl_lowp,
                                          ymix_raw, p.scores_ref, row_m, row_l,
                                          n_exact, false, st, pzero),
                     "relaxed kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_relaxed(P, unsafe, out, mask, row_count, row_kl, row_kl_lowp,
                                          ymix_raw, p.scores_ref, row_m, row_l,
                                          n_exact, true, st, pzero),
                     "relaxed kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SCORES), "hipEventRecord");
        if (probs) {
            LAMP_HIP_TRY(tm.begin(LAMP_STAGE_FINISH), "hipEventRecord");
            LAMP_HIP_TRY(lamp::launch_normalise(P, ymix_raw, row_m, row_l, probs, st,
                                                pzero != nullptr),
                         "normalise launch");
            LAMP_HIP_TRY(tm.end(LAMP_STAGE_FINISH), "hipEventRecord");
        }
    } else if (need.fused) {
        // y^lo lands in its final buffer: scores_mix (y^mix in place), else
        // probs (probabilities in place), else the workspace
        float *ybuf = p.scores_mix ? p.scores_mix : (probs ? probs : at<float>(ws, L.ymix));
        float *pbuf = probs ? probs : (p.scores_mix ? at<float>(ws, L.pbuf) : ybuf);
        float *yref = p.scores_ref ? p.scores_ref : at<float>(ws, L.yref);
        auto *part = at<lamp::RefPartial>(ws, L.part);
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_EXACT), "hipEventRecord");
        // causal, probabilities asked for: the score tiles write their zeros
        // above the diagonal tiles (probs never aliases y^ref or the
        // partials; where it is y^lo's buffer those entries are not scores).
        // Without probs no zero tail is written at all: P.V reads no key past
        // a group's diagonal block.
        float *pzero = P.causal && probs ? pbuf : nullptr;
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ybuf, yref, part,
                                            n_exact, false, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ybuf, yref, part,
                                            n_exact, true, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SCORES), "hipEventRecord");
        const bool kl = need.rowkl;
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SELECT), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_rows_pv(P, ybuf, yref, part, mask, row_count, pbuf,
                                          p.scores_mix, out, kl ? row_kl : nullptr,
                                          kl ? row_kl_lowp : nullptr, mode == LAMP_RELAXED, st,
                                          pzero != nullptr || probs == nullptr),
                     "row kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SELECT), "hipEventRecord");
    } else {
        float *ymix = p.scores_mix ? p.scores_mix : (probs ? probs : at<float>(ws, L.ymix));
        float *yref = p.scores_ref ? p.scores_ref : at<float>(ws, L.yref);
        uint32_t *list = at<uint32_t>(ws, L.list);
        // causal, probabilities asked for: their zeros above the diagonal
        // tiles come from the score tiles
        float *pzero = P.causal && probs ? probs : nullptr;
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ymix, yref, nullptr,
                                            n_exact, false, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_EXACT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, unsafe, ymix, yref, nullptr,
                                            n_exact, true, st, pzero),
                     "score kernel launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SCORES), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_SELECT), "hipEventRecord");
        auto *rs = at<lamp::RowStats>(ws, L.rowstats);
        if (mode == LAMP_STRICT) {
            LAMP_HIP_TRY(lamp::launch_strict_select(P, ymix, yref, mask, list, row_count, rs,
                                                    row_kl, row_kl_lowp, 0, st),
                         "select kernel launch");
        } else if (S <= 1024) {
            // counts and the random selection in one pass (one wave per row)
            const uint64_t seed = p.seed;
            LAMP_HIP_TRY(lamp::launch_strict_select(P, ymix, yref, mask, list, row_count, rs,
                                                    row_kl, row_kl_lowp, 1, st, &seed),
                         "count + random select launch");
        } else {
            LAMP_HIP_TRY(lamp::launch_strict_select(P, ymix, yref, nullptr, nullptr, row_count, rs,
                                                    row_kl, row_kl_lowp, 1, st),
                         "count kernel launch");
            LAMP_HIP_TRY(lamp::launch_random_select(P, p.seed, mask, list, row_count, st),
                         "random select launch");
        }
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_SELECT), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_RECOMPUTE), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_recompute(P, list, row_count, yref, ymix, rs, row_kl, st),
                     "recompute launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_RECOMPUTE), "hipEventRecord");
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_FINISH), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_finish(P, ymix, rs, probs, out, row_kl, st, pzero != nullptr),
                     "finish launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_FINISH), "hipEventRecord");
    }

    if (want_stats) {
        LAMP_HIP_TRY(tm.begin(LAMP_STAGE_STATS), "hipEventRecord");
        LAMP_HIP_TRY(lamp::launch_stats(P, row_kl, row_kl_lowp, row_count, dstats, st),
                     "stats launch");
        LAMP_HIP_TRY(tm.end(LAMP_STAGE_STATS), "hipEventRecord");
        lamp::DevStats ds;
        LAMP_HIP_TRY(hipMemcpyAsync(&ds, dstats, kStatsHead, hipMemcpyDeviceToHost, st),
                     "hipMemcpyAsync stats");
        LAMP_HIP_TRY(hipStreamSynchronize(st), "hipStreamSynchronize");
        fill_stats(stats, z.n_rows, z.n_valid, ds, impl);
    }
    g_last_impl = impl;
    return LAMP_OK;
}

int lamp_attention_fwd_ex(const float *q, const float *k, const float *v, int B, int H, int S,
                          int D, int causal, int mu, float tau, int mode, float *out, float *probs,
                          uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p)
{
    try {
        return run(q, k, v, B, H, S, D, causal, mu, tau, mode, out, probs, recompute_mask, stats, p);
    } catch (const std::bad_alloc &) {
        return set_error(LAMP_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

int lamp_attention_fwd_noalloc(const float *q, const float *k, const float *v, int B, int H,
                               int S, int D, int causal, int mu, float tau, int mode, float *out,
                               float *probs, uint32_t *recompute_mask, lamp_stats *stats,
                               const lamp_params *p)
{
    try {
        return run(q, k, v, B, H, S, D, causal, mu, tau, mode, out, probs, recompute_mask, stats,
                   p, WsSource::kScratch);
    } catch (const std::bad_alloc &) {
        return set_error(LAMP_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

int lamp_attention_fwd(const float *q, const float *k, const float *v, int B, int H, int S, int D,
                       int causal, int mu, float tau, int mode, float *out, float *probs,
                       uint32_t *recompute_mask, lamp_stats *stats)
{
    return lamp_attention_fwd_ex(q, k, v, B, H, S, D, causal, mu, tau, mode, out, probs,
                                 recompute_mask, stats, nullptr);
}

size_t lamp_decode_workspace_bytes(int B, int H, int Nq, int S, int D)
{
    if (check_decode(B, H, Nq, S, D) != LAMP_OK)
        return 0;
    return decode_plan((uint64_t)B * (uint64_t)H, Nq, S, D, true, true, true, true, true).total;
}

int lamp_decode_fwd(const float *q, const float *k, const float *v, int B, int H, int Nq, int S,
                    int D, int causal, int mu, float tau, float *out, float *probs,
                    uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p)
{
    try {
        return run_decode(q, k, v, B, H, Nq, S, D, causal, mu, tau, out, probs, recompute_mask,
                          stats, p);
    } catch (const std::bad_alloc &) {
        return set_error(LAMP_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

int lamp_gelu_fwd(const float *x, const float *w, int M, int N, int K, int mu, float tau,
                  float *out, uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p)
{
    try {
        return run_mlp(lamp::MLP_GELU, x, w, nullptr, nullptr, M, N, K, mu, 0.0f, tau, out,
                       recompute_mask, stats, p);
    } catch (const std::bad_alloc &) {
        return set_error(LAMP_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

int lamp_layernorm_fwd(const float *x, const float *w, const float *gamma, const float *beta,
                       int M, int N, int K, int mu, float eps, float tau, float *out,
                       uint32_t *recompute_mask, lamp_stats *stats, const lamp_params *p)
{
    try {
        return run_mlp(lamp::MLP_LAYERNORM, x, w, gamma, beta, M, N, K, mu, eps, tau, out,
                       recompute_mask, stats, p);
    } catch (const std::bad_alloc &) {
        return set_error(LAMP_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

size_t lamp_mlp_workspace_bytes(int M, int N, int K, int op)
{
    if (op != lamp::MLP_GELU && op != lamp::MLP_LAYERNORM)
        return 0;
    if (check_mlp(M, N, K, op) != LAMP_OK)
        return 0;
    return mlp_plan(M, N, op, true, true, true, true, true, true).total;
}

int lamp_gemm_scores(const float *x, const float *w, int M, int N, int K, int mu, float *ylo,
                     float *yref, void *stream)
{
    try {
        g_last_error.clear();
        if (!x || !w || (!ylo && !yref))
            return set_error(LAMP_ERR_INVALID_ARG, "x, w and one of ylo, yref are required");
        if (!aligned16(x) || !aligned16(w))
            return set_error(LAMP_ERR_INVALID_ARG, "x and w must be 16-byte aligned");
        if (mu < 1 || mu > 23)
            return set_error(LAMP_ERR_INVALID_ARG, "mu must be in [1, 23]");
        int rc = check_mlp(M, N, K, lamp::MLP_GEMM);
        if (rc != LAMP_OK)
            return rc;
        void *ws = nullptr;
        const size_t flags = 4 * ((size_t)(M + 63) / 64 + (size_t)(N + 63) / 64);
        PoolLease lease;
        rc = lease.acquire(align_up(flags), (hipStream_t)stream, &ws);
        if (rc != LAMP_OK)
            return rc;
        (void)hipGetLastError();
        lamp::MlpProblem P{};
        P.x = x;
        P.w = w;
        P.M = M;
        P.N = N;
        P.K = K;
        P.mu = mu;
        P.op = lamp::MLP_GEMM;
        lamp::MlpBuffers b{};
        b.unsafe = (uint32_t *)ws;
        b.ylo = ylo;
        b.yref = yref;
        LAMP_HIP_TRY(lamp::launch_mlp(P, b, (hipStream_t)stream, nullptr), "matrix product launch");
        return LAMP_OK;
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

int lamp_ps_scores(const float *q, const float *k, int B, int H, int S, int D, int causal, int mu,
                   float *ylo, float *yref, void *stream)
{
    try {
        g_last_error.clear();
        if (!q || !k)
            return set_error(LAMP_ERR_INVALID_ARG, "q and k are required");
        if (!ylo && !yref)
            return set_error(LAMP_ERR_INVALID_ARG, "at least one of ylo, yref is required");
        if (!aligned16(q) || !aligned16(k))
            return set_error(LAMP_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
        if (causal != 0 && causal != 1)
            return set_error(LAMP_ERR_INVALID_ARG, "causal must be 0 or 1");
        if (mu < 1 || mu > 23)
            return set_error(LAMP_ERR_INVALID_ARG, "mu must be in [1, 23]");
        Sizes z;
        int rc = check_sizes(B, H, S, D, &z);
        if (rc != LAMP_OK)
            return rc;
        void *ws = nullptr;
        hipStream_t st = (hipStream_t)stream;
        PoolLease lease;
        rc = lease.acquire(align_up(2 * z.BH * (uint64_t)z.tiles), st, &ws);
        if (rc != LAMP_OK)
            return rc;
        lamp::Problem P{};
        P.q = q;
        P.k = k;
        P.BH = (int)z.BH;
        P.S = S;
        P.D = D;
        P.causal = causal;
        P.mu = mu;
        P.pc = lamp::make_ps_const(mu, D);
        P.tiles = z.tiles;
        P.n_rows = z.n_rows;
        (void)hipGetLastError();
        LAMP_HIP_TRY(lamp::launch_operand_scan(P, (uint8_t *)ws, st), "operand scan launch");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, (uint8_t *)ws, ylo, yref, nullptr, nullptr, false, st),
                     "score kernel launch");
        LAMP_HIP_TRY(lamp::launch_ps_scores(P, (uint8_t *)ws, ylo, yref, nullptr, nullptr, true, st),
                     "score kernel launch");
        return LAMP_OK;
    } catch (...) {
        return set_error(LAMP_ERR_HIP, "unexpected exception");
    }
}

}  // extern "C"
