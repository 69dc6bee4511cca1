// gear_compress.hip -- GEAR compression of stacks of per-head K/V matrices on
// gfx950.
//
// What is computed (GEAR pages: "GEAR: Efficient KV Cache Compression for LLM
// Inference", Q3; app.cochat.ai "Cites" list, sentences quoted under the
// SqueezeLLM, ZeroQuant, FlexGen and PowerSGD entries):
//   S = the k largest-|x| entries (ties: lower flat index), kept exactly;
//   Q = b-bit codes of D = X - S, per group of g columns of a token
//       (zero-point = group min, scale = (max-min)/(2^b-1), round half even);
//   A, B = t PowerSGD steps on R = D - deq(Q) from a fixed B0, L = A B^T.
//
// Design (MI355X):
//   * One workgroup (4 waves) owns one matrix and streams its rows in passes;
//     each wave owns a contiguous quarter of the rows, 8 columns per lane and
//     D/8 lanes per token row.  Nothing is exchanged between workgroups, so
//     no grid-level synchronisation or device-scope fence is needed, and
//     thousands of entries are processed between the few workgroup barriers.
//   * Pass 1: 4096-bin histogram of |x| >> 3 in LDS -> the coarse bin of the
//     k-th largest magnitude.  Pass 2: per-wave 8-bin histograms inside that
//     bin -> the exact threshold key, the number of ties to take, and every
//     wave's CSR start and tie quota (flat order = wave order, then row, lane).
//   * Pass 3: outlier mask, CSR emit (wave-level prefix sums), bit-exact fp32
//     group quantization (rint of the correctly rounded quotient, taken from a
//     reciprocal product away from rounding ties) with codes packed
//     in registers and stored as one 32- or 16-bit word per lane per token,
//     and the first power-iteration product.  Passes 4..: the remaining power
//     steps, with R = D - deq(Q) recomputed from X and the stored codes.
//   * A power step is one pass: P = R B and W = R^T P together, G = P^T P in
//     fp64 from a small per-wave LDS ring of P rows; then G = C^T C (Cholesky,
//     one thread), M = C^-1, B' = W M, and after the last step A = P M.  In
//     exact arithmetic this equals modified Gram-Schmidt on P, B = R^T A.
//   * The products are bandwidth-shaped (r <= 8 columns): plain fp32 VALU
//     FMAs; a token's dot product is finished with a butterfly over its lanes.
#include "gear_internal.h"

namespace gear {
namespace {

constexpr int kRing = 64;   // P rows buffered per wave before the fp64 Gram update

__device__ __forceinline__ float h2f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ uint32_t half_of(const uint4& w, int e) {
    const uint32_t v = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
    return (v >> (16 * (e & 1))) & 0xffffu;
}

// DPP lane exchange (no LDS traffic).  quad_perm(1,0,3,2) = 0xB1,
// quad_perm(2,3,0,1) = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over each aligned group of N lanes (N = 8 or 16), result in every lane:
// pairs, then quads, then the mirrored quad, then the mirrored half-row.
template <int N>
__device__ __forceinline__ float row_allreduce(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    if (N >= 8) v += dpp<0x141>(v);
    if (N >= 16) v += dpp<0x140>(v);
    return v;
}

// min and max over each aligned group of g lanes, g in {1, 2, 4, 8, 16}.
__device__ __forceinline__ void group_minmax(float& mn, float& mx, int g) {
    if (g >= 2) { mn = fminf(mn, dpp<0xB1>(mn)); mx = fmaxf(mx, dpp<0xB1>(mx)); }
    if (g >= 4) { mn = fminf(mn, dpp<0x4E>(mn)); mx = fmaxf(mx, dpp<0x4E>(mx)); }
    if (g >= 8) { mn = fminf(mn, dpp<0x141>(mn)); mx = fmaxf(mx, dpp<0x141>(mx)); }
    if (g >= 16) { mn = fminf(mn, dpp<0x140>(mn)); mx = fmaxf(mx, dpp<0x140>(mx)); }
}

// Exclusive prefix sum over the 256 threads of the block; *total = full sum.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    __syncthreads();
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t t = s_tmp[i];
        base += (i < w) ? t : 0u;
        tot += t;
    }
    *total = tot;
    return base + x - v;
}

// Exclusive prefix sum over the 64 lanes of the wave (lane order).
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, int lane, uint32_t* total) {
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    *total = __shfl(x, 63, 64);
    return x - v;
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + i * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// M (RK x RK upper triangular; column c holds the coefficients of A[:,c] in
// the columns of P) from the Gram matrix G = P^T P.  Gram-Schmidt expressed
// through G is a Cholesky factorisation G = C^T C followed by M = C^-1:
//   C[i][j] = (G[i][j] - sum_{k<i} C[k][i] C[k][j]) / C[i][i]     (i < j)
//   C[j][j]^2 = G[j][j] - sum_{k<j} C[k][j]^2 = |P_j after projection|^2
// A column whose squared norm after projection is at most 1e-12 of its squared
// norm before (G[j][j]), or zero, is dead: its row of C and column of M are
// zero, so later columns do not project on it (the modified Gram-Schmidt zero
// rule with threshold 1e-6 on norms).  fp64, fully unrolled, one thread.
template <int RK>
__device__ void gram_to_m(const double* G /* RK*RK symmetric, LDS */, float* Mout /* LDS */) {
    double c[RK][RK];
    bool alive[RK];
#pragma unroll
    for (int i = 0; i < RK; ++i)
#pragma unroll
        for (int j = i; j < RK; ++j) c[i][j] = G[i * RK + j];
#pragma unroll
    for (int j = 0; j < RK; ++j) {
#pragma unroll
        for (int i = 0; i < j; ++i) {
            double v = c[i][j];
#pragma unroll
            for (int k = 0; k < i; ++k) v -= c[k][i] * c[k][j];
            c[i][j] = alive[i] ? v / c[i][i] : 0.0;
        }
        const double pre2 = c[j][j];
        double post2 = pre2;
#pragma unroll
        for (int k = 0; k < j; ++k) post2 -= c[k][j] * c[k][j];
        alive[j] = (pre2 > 0.0) && (post2 > 1e-12 * pre2);
        c[j][j] = alive[j] ? sqrt(post2) : 0.0;
    }
    // M = C^-1 in place (upper triangular; column j only needs columns < j of
    // the inverse and column j of C, overwritten top to bottom); a dead pivot
    // gives a zero row and column.
#pragma unroll
    for (int j = 0; j < RK; ++j) {
        const double inv = alive[j] ? 1.0 / c[j][j] : 0.0;
#pragma unroll
        for (int i = 0; i < j; ++i) {
            double v = 0.0;
#pragma unroll
            for (int k = i; k < j; ++k) v += c[i][k] * c[k][j];
            c[i][j] = -v * inv;
        }
        c[j][j] = inv;
    }
#pragma unroll
    for (int a = 0; a < RK; ++a)
#pragma unroll
        for (int j = 0; j < RK; ++j) Mout[a * RK + j] = a <= j ? (float)c[a][j] : 0.0f;
}

template <int RK>
struct PairLanes {
    static constexpr int NP = RK * (RK + 1) / 2;
    // lanes per Gram pair: the largest power of two with NP * LP <= 64
    static constexpr int LP = NP <= 1 ? 64 : NP <= 2 ? 32 : NP <= 4 ? 16 : NP <= 8 ? 8
                            : NP <= 16 ? 4 : NP <= 32 ? 2 : 1;
};

constexpr int kCoarse = 4096;   // pass-1 bins: |x| bit pattern >> 3
constexpr int kFine = 8;        // pass-2 bins inside the chosen coarse bin
constexpr int kFineSlot = kFine + 1;
constexpr int kSelThreads = 1024;

// U consecutive row steps of one wave: the X words, and (after the first
// pass) the stored code word and the group's scale and zero of each row.
template <int U>
struct StepBuf {
    uint4 x[U];
    uint32_t cw[U];
    float sc[U], zp[U];
};

template <int D, int U, int RPS>
__device__ __forceinline__ void load_steps(StepBuf<U>& b, const uint16_t* xm, const Packed& o,
                                           int64_t mm, int rows, int wr0, int s0, int steps,
                                           int rl, int colq, bool with_codes) {
    const int ngr = D / o.group, gl = o.group / 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = wr0 + (s0 + u) * RPS + rl;
        const bool ok = s0 + u < steps && row < rows;
        b.x[u] = ok ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                    : make_uint4(0u, 0u, 0u, 0u);
        b.cw[u] = 0u;
        b.sc[u] = 0.0f;
        b.zp[u] = 0.0f;
        if (with_codes && ok) {
            const size_t grow = (size_t)mm * rows + row;
            b.cw[u] = o.bits == 4 ? reinterpret_cast<const uint32_t*>(o.codes)[grow * (D / 8) + colq]
                                  : reinterpret_cast<const uint16_t*>(o.codes)[grow * (D / 8) + colq];
            b.sc[u] = o.scale[grow * ngr + colq / gl];
            b.zp[u] = o.zero[grow * ngr + colq / gl];
        }
    }
}

// ---------------------------------------------------------------------------
// Outlier threshold: the k-th largest |x| of a matrix, with ties broken by
// the lower flat index.  One 16-wave workgroup per matrix.  The rows are split
// exactly as the compress kernel splits them over its 4 waves; each of those
// row blocks is read here by 4 consecutive waves.  Output per matrix
// (kSelStride words): threshold key, then for each of the 4 row blocks the
// number of ties at the threshold it takes, then its first CSR position.
//
// Common path (one pass over X plus a 1/16 sample): a histogram of a sample
// of rows gives a key L0 that at least ~1.25 k entries reach; one pass then
// counts, per row block, every key in the window [L0, L0 + 4096) exactly and
// every key above it.  If the k-th largest key lies in the window this is
// the exact answer (checked from the counts); otherwise a two-pass radix
// select over all keys (4096 coarse bins, then 8 fine bins) is used.
template <int D, int U>
__global__ void __launch_bounds__(kSelThreads) select_kernel(CompressArgs a) {
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int NW = kSelThreads / 64;       // 16 waves
    constexpr int kWin = 4096;                 // exact window of keys
    constexpr int kSampleEvery = 16;           // sample = every 16th step
    __shared__ uint32_t s_hist[kCoarse];
    __shared__ uint32_t s_win[4 * kWin];
    __shared__ uint32_t s_cnt[2 * NW];
    __shared__ uint32_t s_fine[NW * kFineSlot];
    __shared__ uint32_t s_tmp[NW];
    __shared__ uint32_t s_res[12];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const Packed& o = a.out;
    const int64_t mm = blockIdx.x;
    const int rows = o.rows;
    const uint32_t kk = (uint32_t)o.k;
    uint32_t* sel = a.sel + (size_t)mm * kSelStride;
    if (kk == 0) {
        if (tid < kSelStride) sel[tid] = tid == 0 ? 0x8000u : 0u;
        return;
    }
    const int rw = ((rows + 3) / 4 + RPS - 1) / RPS * RPS;
    const int steps = rw / RPS;
    const int mb = wv / 4, sub = wv % 4;
    const int per = (steps + 3) / 4;
    const int sb = min(steps, sub * per), se = min(steps, sb + per);
    const int wr0 = mb * rw;
    const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * rows * D
                                         : a.x2 + (size_t)(mm - a.m_split) * rows * D;
    for (int i = tid; i < kCoarse; i += kSelThreads) s_hist[i] = 0u;
    for (int i = tid; i < 4 * kWin; i += kSelThreads) s_win[i] = 0u;
    if (tid < NW * kFineSlot) s_fine[tid] = 0u;
    if (tid < 12) s_res[tid] = 0u;
    __syncthreads();

    auto load = [&](uint4 (&xr)[U], bool (&ok)[U], int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = wr0 + (s0 + u) * RPS + rl;
            ok[u] = s0 + u < se && row < rows;
            xr[u] = ok[u] ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // Thread t owns 4 consecutive bins of a 4096-bin table, the top ones first;
    // returns the bin where the count from the top, started at `base`,
    // reaches `target` (writes it to *out; no write if never reached).
    auto find_bin = [&](const uint32_t (&h)[4], uint32_t base, uint32_t target, uint32_t* out) {
        const int b0 = (kSelThreads - 1 - tid) * 4;
        const uint32_t sum = h[0] + h[1] + h[2] + h[3];
        uint32_t x = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        __syncthreads();
        if (lane == 63) s_tmp[wv] = x;
        __syncthreads();
        uint32_t cum = base + x - sum;
        for (int w = 0; w < wv; ++w) cum += s_tmp[w];
#pragma unroll
        for (int q = 3; q >= 0; --q) {
            if (cum < target && cum + h[q] >= target) *out = (uint32_t)(b0 + q);
            cum += h[q];
        }
    };

    // ---- sample: every 16th step of each wave's range
    uint32_t nsamp = 0;
    for (int s0 = sb; s0 < se; s0 += kSampleEvery) {
        const int row = wr0 + s0 * RPS + rl;
        if (row < rows) {
            const uint4 xr = *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8);
            const uint32_t w4[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                atomicAdd(&s_hist[__builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 19u : 3u, 12u)], 1u);
            nsamp += 8;
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) nsamp += __shfl_xor(nsamp, off, 64);
    if (lane == 0) s_cnt[wv] = nsamp;
    __syncthreads();
    uint32_t total_samp = 0;
    for (int w = 0; w < NW; ++w) total_samp += s_cnt[w];
    const double frac = (double)total_samp / ((double)rows * D);
    const double expect = (double)kk * frac;
    const uint32_t target = (uint32_t)(1.25 * expect + 4.0 * sqrt(expect) + 8.0);
    uint32_t L0 = 0;
    if (target <= total_samp) {
        uint32_t h[4];
        const int b0 = (kSelThreads - 1 - tid) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = s_hist[b0 + q];
        find_bin(h, 0u, target, &s_res[0]);
        __syncthreads();
        L0 = s_res[0] << 3;
    }

    // ---- window pass: exact counts of keys in [L0, L0 + kWin), count above
    uint32_t above = 0;
    auto window = [&](const uint4 (&xr)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u]) continue;
            const uint32_t w4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
            bool any = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t key = __builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 16u : 0u, 15u);
                const uint32_t dlt = key - L0;
                above += (key >= L0 + kWin) ? 1u : 0u;
                any |= dlt < (uint32_t)kWin;
            }
            if (any) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t key = __builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 16u : 0u, 15u);
                    const uint32_t dlt = key - L0;
                    if (dlt < (uint32_t)kWin) atomicAdd(&s_win[mb * kWin + dlt], 1u);
                }
            }
        }
    };
    {
        uint4 xa[U], xb[U];
        bool oka[U], okb[U];
        load(xa, oka, sb);
        for (int s0 = sb; s0 < se; s0 += 2 * U) {
            load(xb, okb, s0 + U);
            window(xa, oka);
            load(xa, oka, s0 + 2 * U);
            window(xb, okb);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) above += __shfl_xor(above, off, 64);
    if (lane == 0) s_cnt[NW + wv] = above;
    __syncthreads();
    uint32_t above_b[4], above_tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        above_b[b] = s_cnt[NW + 4 * b] + s_cnt[NW + 4 * b + 1] + s_cnt[NW + 4 * b + 2] + s_cnt[NW + 4 * b + 3];
        above_tot += above_b[b];
    }
    {
        uint32_t h[4];
        const int b0 = (kSelThreads - 1 - tid) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            h[q] = s_win[b0 + q] + s_win[kWin + b0 + q] + s_win[2 * kWin + b0 + q] + s_win[3 * kWin + b0 + q];
        s_res[1] = 0xffffffffu;
        __syncthreads();
        if (above_tot < kk) find_bin(h, above_tot, kk, &s_res[1]);
        __syncthreads();
    }
    const uint32_t jstar = s_res[1];
    if (jstar != 0xffffffffu) {
        // exact threshold T = L0 + j*; per block: ties at T, count above T
        const int b0 = (kSelThreads - 1 - tid) * 4;
        uint32_t gtp[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if ((uint32_t)(b0 + q) > jstar) {
#pragma unroll
                for (int b = 0; b < 4; ++b) gtp[b] += s_win[b * kWin + b0 + q];
            }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) gtp[b] += __shfl_xor(gtp[b], off, 64);
            if (lane == 0 && gtp[b]) atomicAdd(&s_res[4 + b], gtp[b]);
        }
        __syncthreads();
        if (wv == 0) {
            const uint32_t eq = lane < 4 ? s_win[lane * kWin + jstar] : 0u;
            uint32_t gt = 0;
            if (lane < 4) gt = s_res[4 + lane] + (lane == 0 ? above_b[0] : lane == 1 ? above_b[1]
                                                 : lane == 2 ? above_b[2] : above_b[3]);
            uint32_t tot_gt = gt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) tot_gt += __shfl_xor(tot_gt, off, 64);
            const uint32_t need = kk - tot_gt;   // ties to take, >= 1
            uint32_t tt;
            const uint32_t ties_before = wave_excl_scan(eq, lane, &tt);
            const uint32_t take = (need > ties_before) ? min(eq, need - ties_before) : 0u;
            const uint32_t before = wave_excl_scan(gt + take, lane, &tt);
            if (lane == 0) sel[0] = L0 + jstar;
            if (lane < 4) {
                sel[1 + lane] = take;
                sel[5 + lane] = before;
            }
        }
        return;
    }

    // ---- fallback: radix select over all keys (4096 coarse bins, then 8 fine)
    for (int i = tid; i < kCoarse; i += kSelThreads) s_hist[i] = 0u;
    __syncthreads();
    auto hist = [&](const uint4 (&xr)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) {
                const uint32_t w4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    atomicAdd(&s_hist[__builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 19u : 3u, 12u)], 1u);
            }
    };
    {
        uint4 xa[U], xb[U];
        bool oka[U], okb[U];
        load(xa, oka, sb);
        for (int s0 = sb; s0 < se; s0 += 2 * U) {
            load(xb, okb, s0 + U);
            hist(xa, oka);
            load(xa, oka, s0 + 2 * U);
            hist(xb, okb);
        }
    }
    __syncthreads();
    {
        uint32_t h[4];
        const int b0 = (kSelThreads - 1 - tid) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = s_hist[b0 + q];
        find_bin(h, 0u, kk, &s_res[2]);
        __syncthreads();
    }
    const uint32_t bstar = s_res[2];
    uint32_t my_above = 0;
    auto fine = [&](const uint4 (&xr)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t w4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
            bool any = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t kb = __builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 19u : 3u, 12u);
                my_above += (ok[u] && kb > bstar) ? 1u : 0u;
                any |= kb == bstar;
            }
            if (__ballot(ok[u] && any) != 0ull && ok[u] && any) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t key = half_of(xr[u], e) & 0x7fffu;
                    if ((key >> 3) == bstar) atomicAdd(&s_fine[wv * kFineSlot + (key & 7u)], 1u);
                }
            }
        }
    };
    {
        uint4 xa[U], xb[U];
        bool oka[U], okb[U];
        load(xa, oka, sb);
        for (int s0 = sb; s0 < se; s0 += 2 * U) {
            load(xb, okb, s0 + U);
            fine(xa, oka);
            load(xa, oka, s0 + 2 * U);
            fine(xb, okb);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) my_above += __shfl_xor(my_above, off, 64);
    if (lane == 0) s_fine[wv * kFineSlot + kFine] = my_above;
    __syncthreads();
    if (wv == 0) {
        uint32_t F = 0, abv = 0;
        for (int w = 0; w < NW; ++w) {
            if (lane < kFine) F += s_fine[w * kFineSlot + lane];
            abv += s_fine[w * kFineSlot + kFine];
        }
        const uint32_t needk = kk - abv;   // >= 1 by the choice of the coarse bin
        uint32_t suf = (lane < kFine) ? F : 0u;  // lane f: sum of F[f'] for f' >= f
#pragma unroll
        for (int off = 1; off < kFine; off <<= 1) {
            const uint32_t y = __shfl_down(suf, off, 64);
            if (lane + off < kFine) suf += y;
        }
        const uint32_t strictly_above = suf - ((lane < kFine) ? F : 0u);
        const uint64_t bal = __ballot(lane < kFine && strictly_above < needk && suf >= needk);
        const int fstar = bal ? (int)__builtin_ctzll(bal) : 0;
        const uint32_t need = needk - __shfl(strictly_above, fstar, 64);   // ties to take
        uint32_t eq = 0, gt = 0;
        if (lane < 4) {
            for (int j = 0; j < 4; ++j) {
                const uint32_t* f = s_fine + (lane * 4 + j) * kFineSlot;
                eq += f[fstar];
                gt += f[kFine];
                for (int q = fstar + 1; q < kFine; ++q) gt += f[q];
            }
        }
        uint32_t tt;
        const uint32_t ties_before = wave_excl_scan(eq, lane, &tt);
        const uint32_t take = (need > ties_before) ? min(eq, need - ties_before) : 0u;
        const uint32_t before = wave_excl_scan(gt + take, lane, &tt);
        if (lane == 0) sel[0] = (bstar << 3) | (uint32_t)fstar;
        if (lane < 4) {
            sel[1 + lane] = take;
            sel[5 + lane] = before;
        }
    }
}

template <int D, int RK, int U>
__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPS = 64 / LPR;           // rows per wave per step
    constexpr int RKX = RK > 0 ? RK : 1;
    constexpr int NP = RKX * (RKX + 1) / 2;
    constexpr int LP = PairLanes<RKX>::LP;
    constexpr int RING_STEPS = kRing / RPS;
    static_assert(RING_STEPS % (2 * U) == 0 || (2 * U) % RING_STEPS == 0, "ring/step blocking");

    __shared__ float s_b0[D * RKX];
    __shared__ float s_w[4 * D * RKX];
    __shared__ float s_ring[4 * kRing * RKX];
    __shared__ double s_g[4 * NP];
    __shared__ double s_gt[RKX * RKX];
    __shared__ float s_m[RKX * RKX];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const Packed& o = a.out;
    const int64_t mm = blockIdx.x;
    const int rows = o.rows;
    const int bits = o.bits, gl = o.group / 8, ngr = D / o.group;
    const uint32_t kk = (uint32_t)o.k;
    const uint32_t cmask = (1u << bits) - 1u;
    const float qmax = (float)cmask;
    const int rank = o.rank;
    // each wave owns rows [wr0, wr0 + rw); rw is a multiple of RPS
    const int rw = ((rows + 3) / 4 + RPS - 1) / RPS * RPS;
    const int steps = rw / RPS;
    const int wr0 = wv * rw;
    const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * rows * D
                                         : a.x2 + (size_t)(mm - a.m_split) * rows * D;

    if (mm == 0 && tid == 0) *a.err = 0u;
    if (RK > 0) {
        for (int i = tid; i < D * RKX; i += kThreads) {
            const int j = i / RKX, c = i % RKX;
            float v = 0.0f;
            if (c < rank) {
                const uint64_t u = splitmix64(a.seed, (uint64_t)(j * rank + c + 1)) >> 40;
                v = (float)u * 0x1p-23f - 1.0f;
            }
            s_b0[i] = v;
        }
    }

    StepBuf<U> ba, bb;

    // ============ outlier threshold, from the select kernel ===================
    uint32_t tkey = 0x8000u;      // above every finite key: nothing selected
    float tf = __builtin_inff();   // |x| threshold as fp32
    uint32_t take_w = 0, csr_w = 0;
    if (kk > 0) {
        const uint32_t* sel = a.sel + (size_t)mm * kSelStride;
        tkey = sel[0];
        tf = h2f(tkey);
        take_w = sel[1 + wv];
        csr_w = sel[5 + wv];
    }

    // ============ quantization pass, then the power-iteration passes =========
    int32_t* rp = o.row_ptr + (size_t)mm * (rows + 1);
    uint16_t* cm = o.col + (size_t)mm * kk;
    uint16_t* vm = o.val + (size_t)mm * kk;
    float* Am = o.A + (size_t)mm * rows * rank;
    const bool lowrank = RK > 0 && rank > 0 && a.iters > 0;
    const int passes = lowrank ? a.iters : 1;

    float Bm[8][RKX];
    if (RK > 0) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int c = 0; c < RKX; ++c) Bm[e][c] = s_b0[(colq * 8 + e) * RKX + c];
    }

    for (int pass = 0; pass < passes; ++pass) {
        const bool first = pass == 0, last = pass == passes - 1;
        float W[8][RKX];
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int c = 0; c < RKX; ++c) W[e][c] = 0.0f;
        double gacc = 0.0;
        uint32_t ties_seen = 0, csr = csr_w;

        auto step_block = [&](const StepBuf<U>& b, int s0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u;
                if (s >= steps) break;   // wave-uniform
                const int row = wr0 + s * RPS + rl;
                const bool valid = row < rows;   // rows past the end hold zeros
                const size_t grow = (size_t)mm * rows + (valid ? row : 0);
                // ---- outliers: |x| > T, or |x| == T within the wave's tie quota
                // (|x| compared in fp32: fp16 -> fp32 is exact and monotone)
                float xf[8];
                bool gt[8];
                bool any_eq = false;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xf[e] = h2f(half_of(b.x[u], e));
                    gt[e] = fabsf(xf[e]) > tf;
                    any_eq |= fabsf(xf[e]) == tf;
                }
                if (__ballot(any_eq) != 0ull && ties_seen < take_w) {   // rare
                    uint32_t eqm = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) eqm |= (fabsf(xf[e]) == tf) ? (1u << e) : 0u;
                    uint32_t tot;
                    uint32_t rank0 = ties_seen + wave_excl_scan(__builtin_popcount(eqm), lane, &tot);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if ((eqm >> e) & 1u) {
                            gt[e] = gt[e] || rank0 < take_w;
                            ++rank0;
                        }
                    ties_seen += tot;
                }
                // ---- CSR (first pass only)
                if (first && kk > 0) {
                    uint32_t om = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) om |= gt[e] ? (1u << e) : 0u;
                    uint32_t pre = 0, tot = 0;
                    if (__ballot(om != 0u) != 0ull) pre = wave_excl_scan(__builtin_popcount(om), lane, &tot);
                    if (valid && colq == 0) rp[row] = (int32_t)(csr + pre);
                    if (om) {
                        uint32_t pos = csr + pre;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (((om >> e) & 1u) && pos < kk) {
                                cm[pos] = (uint16_t)(colq * 8 + e);
                                vm[pos] = (uint16_t)half_of(b.x[u], e);
                                ++pos;
                            }
                    }
                    csr += tot;
                } else if (first && valid && colq == 0) {
                    rp[row] = 0;
                }
                // ---- D = X - S; quantize (first pass) or reload codes; R
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = gt[e] ? 0.0f : xf[e];
                float R[8];
                if (first) {
                    float mn = fminf(fminf(fminf(v[0], v[1]), fminf(v[2], v[3])),
                                     fminf(fminf(v[4], v[5]), fminf(v[6], v[7])));
                    float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                                     fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
                    group_minmax(mn, mx, gl);
                    const float sc = (mx - mn) / qmax;
                    const float inv = sc != 0.0f ? __builtin_amdgcn_rcpf(sc) : 0.0f;
                    float t[8], cf[8];
                    bool near_tie = false;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        t[e] = v[e] - mn;
                        const float q = t[e] * inv;
                        cf[e] = rintf(q);
                        near_tie |= fabsf(q - cf[e]) > 0.49999f;
                    }
                    if (__ballot(near_tie) != 0ull && near_tie) {
                        // within 1e-5 of a half-integer: round the exact quotient
#pragma unroll
                        for (int e = 0; e < 8; ++e) cf[e] = rintf(t[e] / sc);
                    }
                    uint32_t word = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        cf[e] = __builtin_amdgcn_fmed3f(cf[e], 0.0f, qmax);
                        word |= (uint32_t)cf[e] << (e * bits);
                        R[e] = fmaf(-cf[e], sc, t[e]);
                    }
                    if (valid) {
                        if (bits == 4)
                            reinterpret_cast<uint32_t*>(o.codes)[grow * (D / 8) + colq] = word;
                        else
                            reinterpret_cast<uint16_t*>(o.codes)[grow * (D / 8) + colq] = (uint16_t)word;
                        if ((colq % gl) == 0) {
                            o.scale[grow * ngr + colq / gl] = sc;
                            o.zero[grow * ngr + colq / gl] = mn;
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float c = (float)((b.cw[u] >> (e * bits)) & cmask);
                        R[e] = fmaf(-c, b.sc[u], v[e] - b.zp[u]);
                    }
                }
                if (!lowrank) continue;
                // ---- P = R B (row dot products), W += R^T P, ring of P rows
                float p[RKX];
#pragma unroll
                for (int c = 0; c < RKX; ++c) {
                    float acc = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = fmaf(R[e], Bm[e][c], acc);
                    p[c] = row_allreduce<LPR>(acc);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int c = 0; c < RKX; ++c) W[e][c] = fmaf(R[e], p[c], W[e][c]);
                const int slot = s % RING_STEPS;
                if (colq == 0) {
#pragma unroll
                    for (int c = 0; c < RKX; ++c) s_ring[(wv * kRing + slot * RPS + rl) * RKX + c] = p[c];
                    if (last && valid) {
#pragma unroll
                        for (int c = 0; c < RKX; ++c)
                            if (c < rank) Am[(size_t)row * rank + c] = p[c];
                    }
                }
                if (slot == RING_STEPS - 1 || s == steps - 1) {
                    // fp64 Gram update from the ring (wave-local LDS, in order)
                    __builtin_amdgcn_wave_barrier();
                    const int nr = (slot + 1) * RPS;
                    const int q = lane / LP, sub = lane % LP;
                    if (q < NP) {
                        int c1 = 0, rem = q;
                        while (rem >= RKX - c1) {
                            rem -= RKX - c1;
                            ++c1;
                        }
                        const int c2 = c1 + rem;
                        const float* rg = s_ring + wv * kRing * RKX;
                        for (int r2 = sub; r2 < nr; r2 += LP)
                            gacc += (double)rg[r2 * RKX + c1] * (double)rg[r2 * RKX + c2];
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        };
        load_steps<D, U, RPS>(ba, xm, o, mm, rows, wr0, 0, steps, rl, colq, !first);
        for (int s0 = 0; s0 < steps; s0 += 2 * U) {
            load_steps<D, U, RPS>(bb, xm, o, mm, rows, wr0, s0 + U, steps, rl, colq, !first);
            step_block(ba, s0);
            load_steps<D, U, RPS>(ba, xm, o, mm, rows, wr0, s0 + 2 * U, steps, rl, colq, !first);
            step_block(bb, s0 + U);
        }
        if (first && tid == 0) rp[rows] = (int32_t)kk;
        if (!lowrank) break;

        // ---- end of a power step: reduce W and G over the workgroup
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int c = 0; c < RKX; ++c) W[e][c] += __shfl_xor(W[e][c], off, 64);
        if (rl == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int c = 0; c < RKX; ++c) s_w[(wv * D + colq * 8 + e) * RKX + c] = W[e][c];
        }
#pragma unroll
        for (int off = 1; off < LP; off <<= 1) gacc += __shfl_xor(gacc, off, 64);
        if ((lane % LP) == 0 && lane / LP < NP) s_g[wv * NP + lane / LP] = gacc;
        __syncthreads();
        for (int i = tid; i < D * RKX; i += kThreads)
            s_w[i] = s_w[i] + s_w[D * RKX + i] + s_w[2 * D * RKX + i] + s_w[3 * D * RKX + i];
        if (tid == 0) {
            int q = 0;
            for (int c1 = 0; c1 < RKX; ++c1)
                for (int c2 = c1; c2 < RKX; ++c2) {
                    const double v = s_g[q] + s_g[NP + q] + s_g[2 * NP + q] + s_g[3 * NP + q];
                    ++q;
                    s_gt[c1 * RKX + c2] = v;
                    s_gt[c2 * RKX + c1] = v;
                }
            gram_to_m<RKX>(s_gt, s_m);
        }
        __syncthreads();
        // B' = W M for this lane's 8 columns
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float wrow[RKX];
#pragma unroll
            for (int c = 0; c < RKX; ++c) wrow[c] = s_w[(colq * 8 + e) * RKX + c];
#pragma unroll
            for (int c = 0; c < RKX; ++c) {
                float acc = 0.0f;
#pragma unroll
                for (int c2 = 0; c2 < RKX; ++c2) acc = fmaf(wrow[c2], s_m[c2 * RKX + c], acc);
                Bm[e][c] = acc;
            }
        }
        if (last) {
            // A = P M in place, by the lanes that stored the P rows; B out
            if (colq == 0) {
                for (int s = 0; s < steps; ++s) {
                    const int row = wr0 + s * RPS + rl;
                    if (row >= rows) break;
                    float pr[RKX];
#pragma unroll
                    for (int c = 0; c < RKX; ++c) pr[c] = c < rank ? Am[(size_t)row * rank + c] : 0.0f;
#pragma unroll
                    for (int c = 0; c < RKX; ++c) {
                        if (c >= rank) continue;
                        float acc = 0.0f;
#pragma unroll
                        for (int c2 = 0; c2 < RKX; ++c2) acc = fmaf(pr[c2], s_m[c2 * RKX + c], acc);
                        Am[(size_t)row * rank + c] = acc;
                    }
                }
            }
            if (wv == 0 && rl == 0) {
                float* Bo = o.B + (size_t)mm * D * rank;
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int c = 0; c < RKX; ++c)
                        if (c < rank) Bo[(colq * 8 + e) * rank + c] = Bm[e][c];
            }
        }
        __syncthreads();
    }
}

template <int D, int RK>
hipError_t launch_d_rk(const CompressArgs& a, hipStream_t st) {
    if (a.out.k > 0) {
        hipLaunchKernelGGL((select_kernel<D, 4>), dim3((unsigned)a.out.M), dim3(kSelThreads), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int U = RK >= 8 ? 1 : 4;
    hipLaunchKernelGGL((compress_kernel<D, RK, U>), dim3((unsigned)a.out.M), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const CompressArgs& a, hipStream_t st) {
    const int r = a.out.rank;
    const int rk = r == 0 ? 0 : r <= 2 ? 2 : r <= 4 ? 4 : 8;
    switch (rk) {
        case 0: return launch_d_rk<D, 0>(a, st);
        case 2: return launch_d_rk<D, 2>(a, st);
        case 4: return launch_d_rk<D, 4>(a, st);
        default: return launch_d_rk<D, 8>(a, st);
    }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
    if (a.out.M <= 0) return hipSuccess;
    if (a.out.M > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.out.d == 64) return launch_d<64>(a, st);
    if (a.out.d == 128) return launch_d<128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace gear
