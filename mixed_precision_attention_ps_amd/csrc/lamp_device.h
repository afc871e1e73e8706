// lamp_device.h -- device helpers shared by the LAMP kernels: PS(mu)
// arithmetic, the score micro-tile, wave reductions, the SplitMix64 hash.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lamp_exp.h"
#include "lamp_internal.h"

namespace lamp {

// ---------------------------------------------------------------------------
// PS(mu) arithmetic.  PS(mu) is the custom float of the LAMP summary's
// "Experimental results" (mu mantissa bits); here: mu stored fraction bits,
// FP32 exponent range, round to nearest even after every multiply and add.
//
// Fast path (mu <= 10, every nonzero operand magnitude in [2^-40, 2^40]):
//  * product: p = fl(q k) gives the sign and binade of the exact product (up
//    to a round-up into the next binade, which rounds identically).  With
//    C = sign(p) * 2^exponent(p) (p's sign and exponent bits), fma(q *
//    2^(mu-23), k, C) adds the EXACT scaled product to C -- same sign, so the
//    magnitude stays in C's binade -- and rounds once at C's ulp, which is
//    the PS(mu) ulp of the scaled product; C is 2^23 ulps (even), so ties go
//    to even.  r = fma(...) - C is exact (Sterbenz).  Cost: mul, and, fma, sub.
//  * sum: s = fl(acc + r) of two PS(mu) values, then RNE of s to mu fraction
//    bits; double rounding through FP32 is innocuous for 24 >= 2(mu+1)+2,
//    i.e. mu <= 10.  The RNE is Veltkamp's splitting with the constant
//    2^(23-mu) + 1: g = fl(C s), hi = fl(g + fl(s - g)) (three FP32 ops with
//    the short encoding, which issue at twice the rate of the three-operand
//    integer ones of the bit-level form); for every normal s below 2^100 and
//    mu = 1..10 it gives the bits of the bit-level RNE (checked exhaustively
//    over all FP32 inputs by a CPU test).  The fast path's sums are normal
//    (nonzero magnitudes >= 2^-103 in the scaled domain), below 2^75 and
//    never -0.  Cost: add, mul, sub, add.
//  The accumulator lives in the scaled domain (x 2^(mu-23)); rounding to a
//  number of significant bits commutes with power-of-two scaling while
//  values stay normal, which the operand range guarantees.
// Exact path (any input, any mu): products exact in double, RN_mu in double
// with FP32 range; double add then RN_mu (53 >= 2*24+2).
// ---------------------------------------------------------------------------

// RNE of a fast-path sum to mu fraction bits (split = 2^(23-mu) + 1).
__device__ __forceinline__ float ps_round_split(float x, float split)
{
    const float g = split * x;
    const float d = x - g;
    return g + d;
}

// One fast-path multiply-accumulate of PS(mu) (scaled domain) and of the
// sequential FP32 reference, sharing the FP32 product.
__device__ __forceinline__ void ps_mac_fast(float q, float qs, float k, float &acc_s,
                                            float &acc_r, float split)
{
    float p = q * k;
    float C = __uint_as_float(__float_as_uint(p) & 0xff800000u);
    float t = __builtin_fmaf(qs, k, C);
    float r = t - C;
    float s = acc_s + r;
    acc_s = ps_round_split(s, split);
    acc_r = acc_r + p;
}

// RN_mu of a double with FP32 exponent range (exact path).
__device__ __forceinline__ double ps_rn64(double x, int mu)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    int b = ilogb(x);
    b = b < -126 ? -126 : b;
    double r = ldexp(rint(ldexp(x, mu - b)), b - mu);
    if (fabs(r) >= 0x1p128)
        r = copysign(__builtin_inf(), x);
    return r;
}

// ---------------------------------------------------------------------------
// Score micro-tile.  A work-group owns a 64 x 64 tile (64 query rows, 64
// keys); thread (ty = tid / 16, tx = tid % 16) owns rows ty*4 + r and keys
// tx + 16*c (r, c in 0..3).  The head dimension is staged through LDS in
// 16-wide slices: sQ / sQs hold q and q * 2^(mu-23) as [d][row]; sK holds k as
// [d][slot] with key j in slot (j % 16) * 4 + j / 16, so that each thread
// reads its four keys as one 16-byte LDS load.
// ---------------------------------------------------------------------------
enum { PATH_FAST = 0, PATH_EXACT = 1, PATH_FP32 = 2 };

struct alignas(16) TileSmem {
    float q[kDChunk][kTile];
    float qs[kDChunk][kTile];
    float k[kDChunk][kTile];
};

struct TileAcc {
    float lo[4][4];     // fast path: scaled-domain PS accumulator (blocked FP32:
                        // the blocked FP32 sum)
    double lod[4][4];   // exact path: PS accumulator in double
    float ref[4][4];    // sequential FP32 accumulator
    float blk[4][4];    // blocked order: the current run's sum (fast, FP32)
    double blkd[4][4];  // blocked order: the current run's sum (exact path)
};

__device__ __forceinline__ int key_slot(int j) { return (j & 15) * 4 + (j >> 4); }

// Global -> register slice loads: with kSliceV4 = kDChunk / 16 float4 per
// thread, thread tid loads row (tid >> 2), d offsets (tid & 3) * 4 + 16 u of
// the Q and K blocks.  Rows past S and d past D read 0.
constexpr int kSliceV4 = kDChunk / 16;

__device__ __forceinline__ float4 load_slice(const float *base, int row, int nrows, int D, int d)
{
    if (row < nrows && d < D)
        return *reinterpret_cast<const float4 *>(base + (size_t)row * D + d);
    return make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int PATH>
__device__ __forceinline__ void stage_slice(TileSmem &sm, const float4 (&qv)[kSliceV4],
                                            const float4 (&kv)[kSliceV4], int tid, float qscale)
{
    const int row = tid >> 2, slot = key_slot(row);
#pragma unroll
    for (int u = 0; u < kSliceV4; ++u) {
        const int d = (tid & 3) * 4 + 16 * u;
        const float qa[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
        const float ka[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.q[d + e][row] = qa[e];
            if (PATH == PATH_FAST)
                sm.qs[d + e][row] = qa[e] * qscale;
            sm.k[d + e][slot] = ka[e];
        }
    }
}

// compute_slice's run width for a blocked order with runs of blk products
// (0: sequential).
__host__ __device__ constexpr int run_width(int blk) { return blk == 0 ? 0 : blk < 32 ? blk : 32; }

// Blocked ("packed") accumulation order: the current run's sum is added to
// the accumulator (one PS(mu) add) and restarted from +0.  NC: the key
// groups c < NC the thread accumulates (see compute_slice).
template <int PATH, int NC = 4>
__device__ __forceinline__ void flush_runs(TileAcc &acc, const PsConst &pc)
{
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (PATH == PATH_FAST) {
                acc.lo[r][c] = ps_round_split(acc.lo[r][c] + acc.blk[r][c], pc.split);
                acc.blk[r][c] = 0.0f;
            } else if (PATH == PATH_EXACT) {
                acc.lod[r][c] = ps_rn64(acc.lod[r][c] + acc.blkd[r][c], pc.mu);
                acc.blkd[r][c] = 0.0;
            } else {
                acc.lo[r][c] = acc.lo[r][c] + acc.blk[r][c];
                acc.blk[r][c] = 0.0f;
            }
        }
}

// One 32-wide slice of the head dimension.  Sequential order (P = 0): every
// product goes into the accumulator.  Blocked order with runs of P = 4, 8 or
// 16 products: products go into the run sum, which is flushed after every
// P-th position (compile-time positions, no branch).  P = 32 stands for runs
// of 32 or more products, whole slices: the caller flushes after a run's
// last slice.  (A flush that depends on a run-time condition inside or at
// the end of the unrolled slice makes the compiler hoist all of the slice's
// LDS reads and spill.)  NC: only the keys tx + 16 c with c < NC are
// accumulated (a causal diagonal tile's rows 16 w .. 16 w + 15 see no key
// past 16 w + 15: wave w needs c <= w); the others stay +0.
template <int PATH, int P, int NC = 4>
__device__ __forceinline__ void compute_slice(const TileSmem &sm, TileAcc &acc, int tx, int ty,
                                              const PsConst &pc)
{
    static_assert(P == 0 || P == 4 || P == 8 || P == 16 || P == 32, "run width");
    static_assert(NC >= 1 && NC <= 4, "key groups");
    constexpr bool BLOCKED = P != 0;
#pragma unroll
    for (int dd = 0; dd < kDChunk; ++dd) {
        const float4 qv = *reinterpret_cast<const float4 *>(&sm.q[dd][ty * 4]);
        const float4 kv = *reinterpret_cast<const float4 *>(&sm.k[dd][tx * 4]);
        const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
        const float ka[4] = {kv.x, kv.y, kv.z, kv.w};
        if (PATH == PATH_FAST) {
            const float4 sv = *reinterpret_cast<const float4 *>(&sm.qs[dd][ty * 4]);
            const float sa[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    ps_mac_fast(qa[r], sa[r], ka[c], BLOCKED ? acc.blk[r][c] : acc.lo[r][c],
                                acc.ref[r][c], pc.split);
        } else if (PATH == PATH_EXACT) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    double t = (double)qa[r] * (double)ka[c];
                    double &a = BLOCKED ? acc.blkd[r][c] : acc.lod[r][c];
                    a = ps_rn64(a + ps_rn64(t, pc.mu), pc.mu);
                    float p = qa[r] * ka[c];
                    acc.ref[r][c] = acc.ref[r][c] + p;
                }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float p = qa[r] * ka[c];
                    if (BLOCKED)
                        acc.blk[r][c] = acc.blk[r][c] + p;
                    acc.ref[r][c] = acc.ref[r][c] + p;
                }
        }
        if (BLOCKED && P < kDChunk && dd % (P ? P : 1) == (P ? P : 1) - 1)
            flush_runs<PATH, NC>(acc, pc);
    }
}

// Full-D accumulation of one 64x64 tile: rows row0.. of Qh (nq rows), keys
// col0.. of Kh (nk rows); both row-major with D columns.
// Issue priority from a wave's progress through a long dot: the waves that
// are behind (first quarter of D) get the highest priority.  The arbiter
// otherwise favours the oldest waves, which then finish first and leave the
// last stretch of a one-round launch to one or two waves per SIMD, where the
// FP32 and integer halves of the multiply-add no longer issue side by side.
// Measured on a 1024 x 1600 x 6400 product: 2.07 -> 1.90 ms.
__device__ __forceinline__ void progress_priority(int d0, int D)
{
    switch ((int)(((long long)d0 * 4) / D)) {
    case 0: __builtin_amdgcn_s_setprio(3); break;
    case 1: __builtin_amdgcn_s_setprio(2); break;
    case 2: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
    }
}

// P: the run width of the blocked order as compute_slice takes it (0 =
// sequential; 4, 8, 16; 32 for runs of pc.blk >= 32).  PRIO: progress-based
// issue priority (long dots: the matrix product).  NC: key groups per thread
// (compute_slice).
template <int PATH, int P = 0, bool PRIO = false, int NC = 4>
__device__ __forceinline__ void score_tile(TileSmem &sm, TileAcc &acc, const float *Qh,
                                           const float *Kh, int row0, int col0, int nq, int nk,
                                           int D, const PsConst &pc)
{
    constexpr bool BLOCKED = P != 0;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc.lo[r][c] = 0.0f;
            acc.lod[r][c] = 0.0;
            acc.ref[r][c] = 0.0f;
            if (BLOCKED) {
                acc.blk[r][c] = 0.0f;
                acc.blkd[r][c] = 0.0;
            }
        }
    const int lrow = tid >> 2, ld = (tid & 3) * 4;
    const float *Qb = Qh + (size_t)row0 * D;
    const float *Kb = Kh + (size_t)col0 * D;
    const int qrows = nq - row0, krows = nk - col0;
    float4 qv[kSliceV4], kv[kSliceV4];
#pragma unroll
    for (int u = 0; u < kSliceV4; ++u) {
        qv[u] = load_slice(Qb, lrow, qrows, D, ld + 16 * u);
        kv[u] = load_slice(Kb, lrow, krows, D, ld + 16 * u);
    }
    // runs of >= 32 products (P = 32) cover whole slices: the slice loop
    // is cut into runs of pc.blk positions with a flush after each; otherwise
    // one run spans the whole loop
    const int run = P == kDChunk ? pc.blk : D;
    for (int r0 = 0; r0 < D; r0 += run) {
        const int r1 = min(D, r0 + run);
        for (int d0 = r0; d0 < r1; d0 += kDChunk) {
            __syncthreads();
            stage_slice<PATH>(sm, qv, kv, tid, pc.qscale);
            __syncthreads();
            if (PRIO)
                progress_priority(d0, D);
            if (d0 + kDChunk < D) {
#pragma unroll
                for (int u = 0; u < kSliceV4; ++u) {
                    qv[u] = load_slice(Qb, lrow, qrows, D, d0 + kDChunk + ld + 16 * u);
                    kv[u] = load_slice(Kb, lrow, krows, D, d0 + kDChunk + ld + 16 * u);
                }
            }
            compute_slice<PATH, P, NC>(sm, acc, tx, ty, pc);
        }
        // the end of a run (P = 32), or of the last run (zero padding past D
        // leaves run sums unchanged)
        if (BLOCKED)
            flush_runs<PATH, NC>(acc, pc);
    }
}

// Final scaled scores of the micro-tile.
template <int PATH, int P = 0>
__device__ __forceinline__ void tile_scores(const TileAcc &acc, const PsConst &pc, float lo[4][4],
                                            float ref[4][4])
{
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ref[r][c] = acc.ref[r][c] * pc.s;
            if (PATH == PATH_FAST)
                lo[r][c] = acc.lo[r][c] * pc.out_scale;
            else if (PATH == PATH_EXACT)
                lo[r][c] = (float)acc.lod[r][c] * pc.s;
            else if (P != 0)   // mu = 23 in the blocked order: the blocked FP32 sum
                lo[r][c] = acc.lo[r][c] * pc.s;
            else
                lo[r][c] = ref[r][c];
        }
}

// ---------------------------------------------------------------------------
// Wave reductions (wave64).
//
// Within each row of 16 lanes the partners are exchanged through DPP
// (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror): after the
// four steps every lane of a row holds the row's reduction.  A wave reduction
// then folds the rows with row_bcast:15 (lane 15 of each row into rows 1 and
// 3) and row_bcast:31 (lane 31 into rows 2 and 3), which leaves the total in
// lane 63, and reads it with readlane, so the result is wave-uniform.  No
// LDS traffic, no waits on it.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- lane 15 - i within 16
constexpr int kDppBcast15 = 0x142;      // row r <- lane 15 of row r - 1
constexpr int kDppBcast31 = 0x143;      // rows 2, 3 <- lane 31

// A DPP move over all rows and banks (every lane has a source).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// A DPP move into the rows of ROW_MASK; the other rows keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32_rows(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v, float old = 0.0f)
{
    if (ROW_MASK == 0xf)
        return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
    return __uint_as_float(dpp_u32_rows<CTRL, ROW_MASK>(__float_as_uint(old), __float_as_uint(v)));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp(double v, double old = 0.0)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t o = (uint64_t)__double_as_longlong(old);
    uint64_t lo, hi;
    if (ROW_MASK == 0xf) {
        lo = dpp_u32<CTRL>((uint32_t)u);
        hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    } else {
        lo = dpp_u32_rows<CTRL, ROW_MASK>((uint32_t)o, (uint32_t)u);
        hi = dpp_u32_rows<CTRL, ROW_MASK>((uint32_t)(o >> 32), (uint32_t)(u >> 32));
    }
    return __longlong_as_double((long long)((hi << 32) | lo));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t v, uint32_t old = 0u)
{
    if (ROW_MASK == 0xf)
        return dpp_u32<CTRL>(v);
    return dpp_u32_rows<CTRL, ROW_MASK>(old, v);
}

template <typename T, typename Op>
__device__ __forceinline__ T row16_reduce(T v, Op op)
{
    v = op(v, dpp<kDppQuadXor1>(v));
    v = op(v, dpp<kDppQuadXor2>(v));
    v = op(v, dpp<kDppHalfMirror>(v));
    v = op(v, dpp<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float lane_read(float v, int l)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), l));
}

__device__ __forceinline__ uint32_t lane_read(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ double lane_read(double v, int l)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)((hi << 32) | lo));
}

// `id` is the identity of `op` (what rows outside a broadcast's mask add).
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op, T id)
{
    v = row16_reduce(v, op);
    v = op(v, dpp<kDppBcast15, 0xA>(v, id));
    v = op(v, dpp<kDppBcast31, 0xC>(v, id));
    return lane_read(v, 63);
}

struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpAdd {
    template <typename T>
    __device__ T operator()(T a, T b) const { return a + b; }
};

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax{}, -INFINITY); }
__device__ __forceinline__ double wave_sum(double v) { return wave_reduce(v, OpAdd{}, 0.0); }
__device__ __forceinline__ int wave_sum_int(int v)
{
    return (int)wave_reduce((uint32_t)v, OpAdd{}, 0u);
}

// Max / sum over the 16 lanes that share a row (lane groups of 16).
__device__ __forceinline__ float group16_max(float v) { return row16_reduce(v, OpMax{}); }
__device__ __forceinline__ double group16_sum(double v) { return row16_reduce(v, OpAdd{}); }
__device__ __forceinline__ uint32_t group16_sum_u(uint32_t v) { return row16_reduce(v, OpAdd{}); }

// Zeros over rows row0 .. row0 + nrows - 1, keys k0 .. k1 - 1 of head bh of a
// [BH, S, S] buffer, by the whole work-group (nt threads).  Under a causal
// mask these are probabilities past every row's last key when k0 is past the
// last row: the zero tails of the rows, written by a kernel whose own work
// is ALU-bound instead of by the memory-bound one after it.  16-byte stores
// when S and k0 are multiples of 4 (a float4 then lies wholly inside or past
// the range), else 4-byte ones.
__device__ __forceinline__ void zero_block(float *pz, int S, int bh, int row0, int nrows, int k0,
                                           int k1, int nt)
{
    float *base = pz + ((size_t)bh * S + (size_t)row0) * S;
    const int w = k1 - k0;
    if (w <= 0 || nrows <= 0)
        return;
    if ((S & 3) == 0 && (k0 & 3) == 0) {
        const int w4 = (w + 3) / 4;
        for (int e = threadIdx.x; e < nrows * w4; e += nt) {
            const int r = e / w4, c = k0 + 4 * (e % w4);
            *reinterpret_cast<float4 *>(base + (size_t)r * S + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        for (int e = threadIdx.x; e < nrows * w; e += nt) {
            const int r = e / w, c = k0 + e % w;
            base[(size_t)r * S + c] = 0.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// Buffer (range-checked) access to one row: a buffer resource over `bytes`
// bytes at a wave-uniform base; lanes whose byte offset falls outside the
// range read 0 and their stores are dropped.  Offsets are 32-bit, so a row's
// 16 per-lane chunks share one offset register plus immediate offsets.
// ---------------------------------------------------------------------------
constexpr int kBufferRsrcWord3 = 0x00020000;   // gfx9: 32-bit data, raw buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufferRsrcWord3);
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, 0));
}

// 16 bytes at byte_off (a multiple of 16 here); out of range: zeros
__device__ __forceinline__ float4 buf_load_f32x4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off)
{
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
    return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                       __uint_as_float(u[3]));
}

__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, byte_off, 0, 0);
}

// Work-group b of a launch over BH x nblk (head, block) pairs -> head bh and
// block k, counted from the last block (the heaviest one under a causal
// mask).  Work-groups go to the GPU's eight XCDs in turn (b mod 8), each XCD
// with its own L2.  When the heads split evenly over the XCDs in batches of
// hb, XCD x takes heads x, x + 8, ... in batches of hb and walks a batch's
// blocks heaviest first with the batch's heads side by side, so that the
// batch's K or V rows, read by every block of a head, stay in the XCD's L2
// between its blocks (hb: the largest divisor of an XCD's head count not
// above hb_max).  Otherwise heaviest blocks first over all heads.
__device__ __forceinline__ void xcd_head_batches(unsigned b, int BH, int nblk, int hb_max,
                                                 int &bh, int &k)
{
    constexpr int kXcd = 8;
    int hb = hb_max;
    while (hb > 1 && (BH / kXcd) % hb != 0)
        --hb;
    if (BH % kXcd == 0 && BH >= kXcd) {
        const int x = (int)(b % kXcd);
        const int l = (int)(b / kXcd);
        const int batch = l / (hb * nblk);
        const int j = l % (hb * nblk);
        k = nblk - 1 - j / hb;
        bh = (batch * hb + j % hb) * kXcd + x;
    } else {
        bh = (int)(b % (unsigned)BH);
        k = nblk - 1 - (int)(b / (unsigned)BH);
    }
}

// Wave ballot: bit l is set iff `c` holds on (active) lane l.  The compare's
// own lane mask, with no round trip through a vector register (HIP's
// __ballot goes through one: a select and a compare per call).
__device__ __forceinline__ uint64_t ballot(bool c) { return __builtin_amdgcn_ballot_w64(c); }

// Lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// All four values finite; and the same values with every non-finite one
// replaced by 0 (V tiles of causal P.V steps, where a key past a row's
// limit carries probability 0).
__device__ __forceinline__ bool finite4(float4 x)
{
    return isfinite(x.x) && isfinite(x.y) && isfinite(x.z) && isfinite(x.w);
}

__device__ __forceinline__ float4 finite_or_zero(float4 x)
{
    return make_float4(isfinite(x.x) ? x.x : 0.0f, isfinite(x.y) ? x.y : 0.0f,
                       isfinite(x.z) ? x.z : 0.0f, isfinite(x.w) ? x.w : 0.0f);
}

// Near tie of a criterion decided as c > t: |c - t| <= 2^-16 t with t
// finite, the band where a single-precision evaluation of c could not decide
// (the library decides every key in double precision).
__device__ __forceinline__ bool near_tie(double c, double t)
{
    return fabs(c - t) <= 0x1p-16 * t && t < INFINITY;
}

// Adds a wave's count of near ties to the call's total: one atomic per wave
// that has any (wave-uniform count).
__device__ __forceinline__ void add_ties(unsigned long long *n, uint32_t cnt)
{
    if (n && cnt && (threadIdx.x & 63) == 0)
        atomicAdd(n, (unsigned long long)cnt);
}

// SplitMix64 output for a state (Steele, Lea & Flood, OOPSLA 2014): add the
// golden gamma, then two xor-shift-multiply mixing rounds and a final
// xor-shift.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x)
{
    uint64_t z = x + 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

}  // namespace lamp
