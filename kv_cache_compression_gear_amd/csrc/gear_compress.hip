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
// Design (MI355X): three launches per call.
//   * select_kernel (8 or 16 waves per matrix): the threshold key T of the k-th
//     largest |x|, each row block's share of the ties at T and its first CSR
//     position.  A 1/16 row sample places a 1024-key window that one exact
//     counting pass resolves; a two-pass radix select is the fallback.
//   * compress_kernel (8 waves per matrix, one pass over X): outlier mask, CSR
//     emit (DPP prefix sums), bit-exact fp32 group quantization (rint of the
//     correctly rounded quotient, taken from a reciprocal product away from
//     rounding ties), codes packed in registers, and C = R^T R on the matrix
//     cores from an fp16 hi/lo split of the scaled residual; then the t power
//     steps on C in fp64 and the output B.
//   * lowrank_a_kernel (many workgroups per matrix): A = R (B_prev M), the
//     one product that needs R itself after the power steps.
//   The power steps are those of PowerSGD, with P = R B, A = orth(P),
//   B = R^T A; orth is a Cholesky factorisation of P^T P = B^T C B, which in
//   exact arithmetic is modified Gram-Schmidt on P, so L = A B^T is the same.
#include <atomic>

#include "gear_internal.h"

namespace gear {
namespace {

// Raw buffer view of [base, base + bytes) for stores: a store at an offset
// past the end (kDrop) is dropped by the hardware, so a lane with nothing to
// store still issues it.  Stores issued on every path let the compiler wait
// for older loads without waiting for the stores issued after them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kDrop = 0x80000000u;

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

// fp64 lane exchange: the two halves through DPP
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
// fp64 sum over each aligned group of N lanes (N = 8 or 16), result in every lane
template <int N>
__device__ __forceinline__ double row_sum64(double v) {
    v += dpp64<0xB1>(v);
    v += dpp64<0x4E>(v);
    v += dpp64<0x141>(v);
    if (N >= 16) v += dpp64<0x140>(v);
    return v;
}

// min and max over each aligned group of g lanes, g in {1, 2, 4, 8, 16}
// (g = G when G > 0).
template <int G>
__device__ __forceinline__ void group_minmax(float& mn, float& mx, int g) {
    if (G > 0) g = G;
    if (g >= 2) { mn = fminf(mn, dpp<0xB1>(mn)); mx = fmaxf(mx, dpp<0xB1>(mx)); }
    if (g >= 4) { mn = fminf(mn, dpp<0x4E>(mn)); mx = fmaxf(mx, dpp<0x4E>(mx)); }
    if (g >= 8) { mn = fminf(mn, dpp<0x141>(mn)); mx = fmaxf(mx, dpp<0x141>(mx)); }
    if (g >= 16) { mn = fminf(mn, dpp<0x140>(mn)); mx = fmaxf(mx, dpp<0x140>(mx)); }
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
__device__ void gram_to_m(const double* G /* RK*RK symmetric, LDS */, double* Mout /* LDS */) {
    double c[RK][RK];
    double rinv[RK];   // 1 / C[i][i], 0 for a dead pivot
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
            c[i][j] = v * rinv[i];
        }
        const double pre2 = c[j][j];
        double post2 = pre2;
#pragma unroll
        for (int k = 0; k < j; ++k) post2 -= c[k][j] * c[k][j];
        alive[j] = (pre2 > 0.0) && (post2 > 1e-12 * pre2);
        const double sq = alive[j] ? sqrt(post2) : 0.0;
        c[j][j] = sq;
        rinv[j] = alive[j] ? 1.0 / sq : 0.0;
    }
    // M = C^-1 in place (upper triangular; column j only needs columns < j of
    // the inverse and column j of C, overwritten top to bottom); a dead pivot
    // gives a zero row and column.
#pragma unroll
    for (int j = 0; j < RK; ++j) {
        const double inv = rinv[j];
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
        for (int j = 0; j < RK; ++j) Mout[a * RK + j] = a <= j ? c[a][j] : 0.0;
}

constexpr int kCoarse = 4096;   // pass-1 bins: |x| bit pattern >> 3
constexpr int kFine = 8;        // pass-2 bins inside the chosen coarse bin
constexpr int kFineSlot = kFine + 1;

// ---------------------------------------------------------------------------
// Outlier threshold: the k-th largest |x| of a matrix, with ties broken by
// the lower flat index.  One workgroup per matrix, of NT = 512 or 1024
// threads (8 or 16 waves).  The rows are split exactly as the compress
// kernel splits them over its 8 waves (wave_rows); row block b is read by
// NT / 512 waves.  Output per
// matrix (kSelStride words, layout in gear_internal.h): the threshold key T,
// per row block the ties at T it takes, its first CSR position and the ties it
// holds, and a key bounding |x| over the entries that are not outliers (T, or
// the largest key when k = 0, which only the low-rank fit needs).
//
// Common path (one pass over X plus a 1/16 sample): a histogram of a sample
// of rows gives a key L0 that at least ~1.25 k entries reach; one pass then
// counts, per row block, every key in the window [L0, L0 + 1024) exactly and
// every key above it.  If the k-th largest key lies in the window this is
// the exact answer (checked from the counts); otherwise a two-pass radix
// select over all keys (4096 coarse bins, then 8 fine bins) is used.
template <int D, int U, int NT>
__global__ void __launch_bounds__(NT, NT / 128) select_kernel(CompressArgs a) {
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int NW = NT / 64;       // 8 or 16 waves
    constexpr int NB = kCompressWaves;         // row blocks
    constexpr int WPB = NW / NB;               // waves per row block
    // exact window of keys: one binade of fp16 (a factor of 2 in |x|); the
    // sample places L0 where ~25% more than k entries lie above, typically a
    // few dozen keys below the threshold.  A miss takes the radix path.
    constexpr int kWin = 1024;
    constexpr int BPC = kCoarse / NT;   // coarse bins per thread
    constexpr int BPW = kWin / NT;      // window bins per thread
    constexpr int kSampleEvery = 16;           // sample = every 16th step
    __shared__ uint32_t s_hist[kCoarse];
    __shared__ __attribute__((aligned(16))) uint32_t s_win[NB * kWin];
    __shared__ uint32_t s_cnt[2 * NW];
    __shared__ uint32_t s_fine[NW * kFineSlot];
    __shared__ uint32_t s_tmp[NW];
    __shared__ uint32_t s_res[4 + kCompressWaves];

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const Packed& o = a.out;
    const int64_t mm = a.m0 + group_id_x();
    const int rows = o.rows;
    const uint32_t kk = (uint32_t)o.k;
    uint32_t* sel = a.sel + (size_t)mm * kSelStride;
    const int rw = wave_rows(rows);
    const int steps = rw / RPS;
    const int mb = wv / WPB, sub = wv % WPB;
    const int per = (steps + WPB - 1) / WPB;
    const int sb = min(steps, sub * per), se = min(steps, sb + per);
    const int wr0 = mb * rw;
    const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * rows * D
                                         : a.x2 + (size_t)(mm - a.m_split) * rows * D;
    if (kk == 0) {
        // no outliers: only the largest key, which bounds |R| for the low-rank fit
        uint32_t mx = 0;
        for (int s = sb; s < se; ++s) {
            const int row = wr0 + s * RPS + rl;
            if (row >= rows) break;
            const uint4 xr = *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8);
            const uint32_t w4[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mx = max(mx, max(w4[q] & 0x7fffu, (w4[q] >> 16) & 0x7fffu));
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        if (lane == 0) s_tmp[wv] = mx;
        __syncthreads();
        if (tid < kSelStride) {
            uint32_t v = tid == 0 ? 0x8000u : 0u;
            if (tid == kSelBound)
                for (int w = 0; w < NW; ++w) v = max(v, s_tmp[w]);
            sel[tid] = v;
        }
        return;
    }
    for (int i = tid; i < kCoarse; i += NT) s_hist[i] = 0u;
    for (int i = tid; i < NB * kWin / 4; i += NT)
        reinterpret_cast<uint4*>(s_win)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < NW * kFineSlot) s_fine[tid] = 0u;
    if (tid < 4 + NB) s_res[tid] = 0u;
    __syncthreads();

    // Loads are issued unconditionally (steps past the range read a valid row
    // and are flagged), so that the compiler can count them and wait for one
    // batch while the next is in flight; 32-bit offsets from the matrix base
    // (rows * D * 2 < 2^32).
    auto load = [&](auto& xr, auto& ok, int s0) {
        constexpr int UU = sizeof(ok) / sizeof(ok[0]);
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            const int row = wr0 + (s0 + u) * RPS + rl;
            ok[u] = s0 + u < se && row < rows;
            const uint32_t rc = (uint32_t)min(row, rows - 1);
            xr[u] = ld_at<uint4>(xm, (rc * D + colq * 8) * 2);
        }
    };
    // Thread t owns the BP consecutive bins (BP = elements of h) of a table of
    // BP * NT bins, the top ones first; returns the bin where the
    // count from the top, started at `base`, reaches `target` (writes it to
    // *out; no write if never reached).
    auto find_bin = [&](const auto& h, uint32_t base, uint32_t target, uint32_t* out) {
        constexpr int BP = sizeof(h) / sizeof(h[0]);
        const int b0 = (NT - 1 - tid) * BP;
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < BP; ++q) sum += h[q];
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
        for (int q = BP - 1; q >= 0; --q) {
            if (cum < target && cum + h[q] >= target) *out = (uint32_t)(b0 + q);
            cum += h[q];
        }
    };

    // ---- sample: every 16th step of each wave's range.  The window pass's
    // first batch is issued here too, so that it is in flight while the
    // sample's histogram is built and searched.
    uint4 xw0[U];
    bool okw0[U];
    uint32_t nsamp = 0;
    for (int s0 = sb; s0 < se; s0 += 4 * kSampleEvery) {   // 4 sampled rows in flight
        uint4 xr[4];
        bool ok[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s = s0 + q * kSampleEvery;
            const int row = wr0 + s * RPS + rl;
            ok[q] = s < se && row < rows;
            const uint32_t rc = (uint32_t)min(row, rows - 1);
            xr[q] = ld_at<uint4>(xm, (rc * D + colq * 8) * 2);
        }
        if (s0 == sb) load(xw0, okw0, sb);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (!ok[q]) continue;
            const uint32_t w4[4] = {xr[q].x, xr[q].y, xr[q].z, xr[q].w};
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
        uint32_t h[BPC];
        const int b0 = (NT - 1 - tid) * BPC;
#pragma unroll
        for (int q = 0; q < BPC; ++q) h[q] = s_hist[b0 + q];
        find_bin(h, 0u, target, &s_res[0]);
        __syncthreads();
        L0 = s_res[0] << 3;
    }

    // ---- window pass: exact counts of keys in [L0, L0 + kWin), count above.
    // On the two keys of a dword at once: adding 0x8000 - L to each 15-bit key
    // sets its bit 15 exactly when key >= L (no carry leaves a half).
    uint32_t above = 0;
    const uint32_t thw = L0 + kWin;
    const uint32_t add_l = (0x8000u - L0) * 0x10001u;
    const uint32_t add_t = thw < 0x8000u ? (0x8000u - thw) * 0x10001u : 0u;
    const uint32_t msk_t = thw < 0x8000u ? 0x80008000u : 0u;   // no key reaches 0x8000
    auto window = [&](const uint4 (&xr)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u]) continue;
            const uint32_t w4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
            uint32_t ge_l = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t k2 = w4[i] & 0x7fff7fffu;
                ge_l |= (k2 + add_l) & 0x80008000u;
                above += __builtin_popcount((k2 + add_t) & msk_t);
            }
            // keys >= L0 + kWin also set ge_l: the loop below re-checks the window
            if (ge_l != 0u) {
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
        if (sb >= se) load(xw0, okw0, sb);   // (no sample loop ran: an empty range)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xa[u] = xw0[u];
            oka[u] = okw0[u];
        }
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
    uint32_t above_tot = 0;
    for (int w = 0; w < NW; ++w) above_tot += s_cnt[NW + w];
    {
        uint32_t h[BPW];
        const int b0 = (NT - 1 - tid) * BPW;
#pragma unroll
        for (int q = 0; q < BPW; ++q) {
            h[q] = 0u;
#pragma unroll
            for (int b = 0; b < NB; ++b) h[q] += s_win[b * kWin + b0 + q];
        }
        s_res[1] = 0xffffffffu;
        __syncthreads();
        if (above_tot < kk) find_bin(h, above_tot, kk, &s_res[1]);
        __syncthreads();
    }
    const uint32_t jstar = s_res[1];
    if (jstar != 0xffffffffu) {
        // exact threshold T = L0 + j*; per block: ties at T, count above T
        const int b0 = (NT - 1 - tid) * BPW;
        uint32_t gtp[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) gtp[b] = 0u;
#pragma unroll
        for (int q = 0; q < BPW; ++q)
            if ((uint32_t)(b0 + q) > jstar) {
#pragma unroll
                for (int b = 0; b < NB; ++b) gtp[b] += s_win[b * kWin + b0 + q];
            }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) gtp[b] += __shfl_xor(gtp[b], off, 64);
            if (lane == 0 && gtp[b]) atomicAdd(&s_res[4 + b], gtp[b]);
        }
        __syncthreads();
        if (wv == 0) {
            const uint32_t eq = lane < NB ? s_win[lane * kWin + jstar] : 0u;
            uint32_t gt = 0;
            if (lane < NB) {
                gt = s_res[4 + lane];
                for (int j = 0; j < WPB; ++j) gt += s_cnt[NW + lane * WPB + j];
            }
            uint32_t tot_gt = gt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) tot_gt += __shfl_xor(tot_gt, off, 64);
            const uint32_t need = kk - tot_gt;   // ties to take, >= 1
            uint32_t tt;
            const uint32_t ties_before = wave_excl_scan(eq, lane, &tt);
            const uint32_t take = (need > ties_before) ? min(eq, need - ties_before) : 0u;
            const uint32_t before = wave_excl_scan(gt + take, lane, &tt);
            if (lane == 0) {
                sel[0] = L0 + jstar;
                sel[kSelBound] = L0 + jstar;
            }
            if (lane < NB) {
                sel[kSelTake + lane] = take;
                sel[kSelCsr + lane] = before;
                sel[kSelEq + lane] = eq;
            }
        }
        return;
    }

    // ---- fallback: radix select over all keys (4096 coarse bins, then 8 fine)
    for (int i = tid; i < kCoarse; i += NT) s_hist[i] = 0u;
    __syncthreads();
    // (the fallback is rare: its passes take one step at a time, so that its
    // registers do not set the common path's register budget)
    constexpr int UF = 1;
    auto hist = [&](const uint4 (&xr)[UF], const bool (&ok)[UF]) {
#pragma unroll
        for (int u = 0; u < UF; ++u)
            if (ok[u]) {
                const uint32_t w4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    atomicAdd(&s_hist[__builtin_amdgcn_ubfe(w4[e >> 1], (e & 1) ? 19u : 3u, 12u)], 1u);
            }
    };
    for (int s0 = sb; s0 < se; s0 += UF) {
        uint4 xa[UF];
        bool oka[UF];
        load(xa, oka, s0);
        hist(xa, oka);
    }
    __syncthreads();
    {
        uint32_t h[BPC];
        const int b0 = (NT - 1 - tid) * BPC;
#pragma unroll
        for (int q = 0; q < BPC; ++q) h[q] = s_hist[b0 + q];
        find_bin(h, 0u, kk, &s_res[2]);
        __syncthreads();
    }
    const uint32_t bstar = s_res[2];
    uint32_t my_above = 0;
    auto fine = [&](const uint4 (&xr)[UF], const bool (&ok)[UF]) {
#pragma unroll
        for (int u = 0; u < UF; ++u) {
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
    for (int s0 = sb; s0 < se; s0 += UF) {
        uint4 xa[UF];
        bool oka[UF];
        load(xa, oka, s0);
        fine(xa, oka);
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
        if (lane < NB) {
            for (int j = 0; j < WPB; ++j) {
                const uint32_t* f = s_fine + (lane * WPB + j) * kFineSlot;
                eq += f[fstar];
                gt += f[kFine];
                for (int q = fstar + 1; q < kFine; ++q) gt += f[q];
            }
        }
        uint32_t tt;
        const uint32_t ties_before = wave_excl_scan(eq, lane, &tt);
        const uint32_t take = (need > ties_before) ? min(eq, need - ties_before) : 0u;
        const uint32_t before = wave_excl_scan(gt + take, lane, &tt);
        if (lane == 0) {
            sel[0] = (bstar << 3) | (uint32_t)fstar;
            sel[kSelBound] = (bstar << 3) | (uint32_t)fstar;
        }
        if (lane < NB) {
            sel[kSelTake + lane] = take;
            sel[kSelCsr + lane] = before;
            sel[kSelEq + lane] = eq;
        }
    }
}

// ---------------------------------------------------------------------------
// Compress: one workgroup (8 waves) per matrix, one pass over its rows.
//
// Wave w owns rows [w * wave_rows(n), (w + 1) * wave_rows(n)); a lane holds 8
// consecutive columns of a token row, D/8 lanes per row.  The rows are taken
// in slabs of 8 rows per wave (64 per workgroup).  For each row the wave
// applies the outlier mask, emits the row's CSR entries, quantizes the groups
// and forms the residual R = D - deq(Q).  With a low-rank term, R (scaled by
// 2^ex so that fp16 covers it) is split into fp16 hi + lo parts and written
// row-major into an LDS slab; after a workgroup barrier, and issued among the
// next slab's vector work, every wave adds its share of the 16x16 blocks of
// C = R^T R over the slab with
// v_mfma_f32_16x16x32_f16 (hi*hi + hi*lo + lo*hi; the products are exact in
// fp32, lo*lo is below 2^-22 of the total), nine blocks per SIMD at d = 128.
// The operands are read with ds_read_b64_tr_b16, which turns the row-major
// slab into the MFMA's "8 consecutive k per lane" layout; chunks of 8 bytes
// are XOR-swizzled by row so that the transposing reads hit distinct LDS
// banks.
//
// After the pass C is in LDS and the t power steps of the PowerSGD-style fit
// run on it in fp64: W = C B (= R^T P with P = R B), G = B^T W (= P^T P),
// Cholesky G = C_g^T C_g with the dead-column rule, M = C_g^-1, B' = W M.
// The last step's B' is the output B; A = P M = R (B_prev M) needs R once more
// and is formed by lowrank_a_kernel from the d x r matrix B_prev M left in the
// workspace.
// ---------------------------------------------------------------------------

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef short s4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef short s2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s4v lds_s4v;

constexpr int kSlabRows = 64;     // 8 rows from each of the 8 waves
constexpr int kWaveSlab = kSlabRows / kCompressWaves;
constexpr int kCompressThreads = kCompressWaves * 64;

// 8-byte chunk c8 of slab row `row`, XOR-swizzled so that the transposing
// loads below are free of bank conflicts: at d = 128 the 16 lanes of a group
// read 16 distinct chunks of 4 rows, and the two groups of a half-wave
// (rows 8 apart) the other half of the banks (bit 2 of the chunk flipped
// by bit 3 of the row).  Bit 0 is never changed, so a lane's 16-byte store
// of chunks 2c, 2c + 1 stays contiguous.
template <int D>
__device__ __forceinline__ int swz_chunk(int row, int c8) {
    return D == 128 ? (c8 ^ ((row & 3) << 3) ^ (((row >> 3) & 1) << 2)) : (c8 ^ (((row >> 1) & 1) << 3));
}

// Operand of v_mfma_f32_16x16x32_f16 (either side) for columns [16 X,
// 16 X + 16) over slab rows [kb, kb + 32): lane l receives
// R[kb + 8 (l / 16) + i][16 X + l % 16], i = 0..7.  Each transposing load
// serves 4 rows: within a group of 16 lanes, lane p supplies the address of 4
// consecutive columns of row p / 4 and receives column p of the 4 rows.
template <int D>
__device__ __forceinline__ h8v read_operand(const unsigned char* plane, int kb, int X, int lane) {
    const int g = lane >> 4, p = lane & 15;
    const int c8 = 4 * X + (p & 3);
    const int r0 = kb + 8 * g + (p >> 2);
    const int r1 = r0 + 4;
    const s4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4v*)(plane + r0 * (D * 2) + swz_chunk<D>(r0, c8) * 8));
    const s4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4v*)(plane + r1 * (D * 2) + swz_chunk<D>(r1, c8) * 8));
    return __builtin_shufflevector(__builtin_bit_cast(h4v, v0), __builtin_bit_cast(h4v, v1),
                                   0, 1, 2, 3, 4, 5, 6, 7);
}

// The three products that make R_I^T R_J exact in fp32 from the hi and lo
// parts (lo^T lo is below 2^-22 of the total).
__device__ __forceinline__ f4v mma3(const h8v& hi_i, const h8v& lo_i, const h8v& hi_j,
                                    const h8v& lo_j, f4v acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi_i, hi_j, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi_i, lo_j, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo_i, hi_j, acc, 0, 0, 0);
    return acc;
}

// Gram blocks of 16 x 16 over NCB = D / 16 column blocks: the NCB (NCB + 1) / 2
// unordered pairs {i, j}, taken as {q, q + b mod NCB}.  Wave q < NCB takes
// b = 0 .. NCB / 2 - 1, and the waves q < NCB / 2 also {q, q + NCB / 2}: at
// d = 128 five or four blocks per wave, nine per SIMD (waves q and q + 4
// share one).  A wave's first operand (column block q) is read once per
// 32-row chunk and serves all of its blocks.
template <int D>
struct GramPlan {
    static constexpr int NCB = D / 16, HC = NCB / 2, NBW = HC + 1;
};
// Block b of wave q: rows i, columns j; false if the wave has no block b.
template <int D>
__device__ __forceinline__ bool gram_block(int q, int b, int& i, int& j) {
    constexpr int NCB = GramPlan<D>::NCB, HC = GramPlan<D>::HC;
    i = q;
    j = (q + b) % NCB;
    return q < NCB && (b < HC || q < HC);
}

// This wave's Gram blocks over one 64-row slab (two 32-row chunks).
template <int D>
__device__ __forceinline__ void slab_mma(const unsigned char* slab, int wv, int lane,
                                         f4v (&acc)[GramPlan<D>::NBW]) {
    constexpr int kPlane = kSlabRows * D * 2;
    constexpr int NCB = GramPlan<D>::NCB, HC = GramPlan<D>::HC;
    const unsigned char* hi = slab;
    const unsigned char* lo = slab + kPlane;
    const int q = wv;
    if (q >= NCB) return;   // wave-uniform
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int kb = 32 * kc;
        const h8v ah = read_operand<D>(hi, kb, q, lane), al = read_operand<D>(lo, kb, q, lane);
        acc[0] = mma3(ah, al, ah, al, acc[0]);
#pragma unroll
        for (int b = 1; b < HC; ++b) {
            const int j = (q + b) % NCB;
            const h8v bh = read_operand<D>(hi, kb, j, lane), bl = read_operand<D>(lo, kb, j, lane);
            acc[b] = mma3(ah, al, bh, bl, acc[b]);
        }
        if (q < HC) {   // wave-uniform
            const int j = q + HC;
            const h8v bh = read_operand<D>(hi, kb, j, lane), bl = read_operand<D>(lo, kb, j, lane);
            acc[HC] = mma3(ah, al, bh, bl, acc[HC]);
        }
    }
}

// Inclusive prefix sum over the wave in lane order with DPP only: shifts of
// 1, 2, 4, 8 within rows of 16 lanes, then row_bcast:15 and row_bcast:31.
// Lanes with no source lane read 0 (bound_ctrl), rows outside the row mask
// keep x, so every step is a single v_add_u32_dpp.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
    return x;
}

// Largest power-of-two exponent e with bound * 2^e < 2^14 (0 for bound 0):
// every |R| <= bound / (2^b - 1) then scales into fp16's normal range.
__device__ __forceinline__ int residual_exponent(float bound) {
    if (!(bound > 0.0f)) return 0;
    int E;
    frexpf(bound, &E);
    return 14 - E;
}

// Exponent of a slab that holds only zeros: larger than any finite slab's
// (whose keys are at least the smallest fp16 subnormal, exponent 14 + 23), so
// that it never lowers the running minimum.
constexpr int kExNone = 40;

// Largest key (|x| bit pattern) in the rows of xr, over the whole wave, as a
// wave-uniform value: keys two at a time with packed 16-bit max, then DPP
// within rows of 16 lanes and the four rows' maxima read out.
template <int SS>
__device__ __forceinline__ uint32_t wave_max_key(const uint4 (&xr)[SS]) {
    typedef unsigned short u2v __attribute__((ext_vector_type(2)));
    u2v m2 = {0, 0};
#pragma unroll
    for (int u = 0; u < SS; ++u) {
        const uint32_t w[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u2v, w[i] & 0x7fff7fffu));
    }
    uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
    return max(max(a, b), max(c, d));
}

// 2^e as an fp32 bit pattern, for |e| <= 126
__device__ __forceinline__ float pow2f(int e) { return __builtin_bit_cast(float, (uint32_t)(127 + e) << 23); }

// GL: lanes per quantization group when fixed at compile time (D/8: a group
// is a whole token row), 0 for the group size of the call.  CH: keys quantized
// per channel (groups of out.group tokens; their scales and zeros already in
// the packed buffer, [rows / group][D]); the matrices have no outliers then.
template <int D, int RK, int GL, bool CH = false>
__global__ void __launch_bounds__(kCompressThreads, 4) compress_kernel(CompressArgs a) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPS = 64 / LPR;           // rows per wave per step
    constexpr int SS = kWaveSlab / RPS;     // steps per slab slice of a wave
    constexpr bool LR = RK > 0;
    constexpr int RKX = LR ? RK : 1;
    constexpr int NP = RKX * (RKX + 1) / 2;
    // threads taking part in the power steps: all of them, except at D = 128
    // with rank 8, where their partial sums would not fit the LDS budget of
    // two workgroups per CU
    constexpr int PT = (D == 128 && RK == 8) ? 256 : kCompressThreads;
    constexpr int NH = PT / D;              // threads per row of C in the power steps
    constexpr int kPlane = kSlabRows * D * 2;
    constexpr int kBig = LR ? (4 * kPlane > D * D * 4 ? 4 * kPlane : D * D * 4) : 16;
    __shared__ __attribute__((aligned(16))) unsigned char s_big[kBig];  // 2 slabs, then C
    __shared__ float s_b[LR ? D * RKX : 1];
    __shared__ double s_w[LR ? (NH - 1) * D * RKX : 1];   // [part][c][j]: a wave's j contiguous
    __shared__ double s_g[RKX * RKX];
    __shared__ double s_m[RKX * RKX];
    __shared__ uint32_t s_ex[2][kCompressWaves];   // per slab: each wave's largest key

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const Packed& o = a.out;
    const int64_t mm = a.m0 + group_id_x();
    const int rows = o.rows;
    const int bits = o.bits;
    const int gl = GL > 0 ? GL : o.group / 8, ngr = D / (8 * gl);
    const uint32_t kk = CH ? 0u : (uint32_t)o.k;
    const float qmax = (float)((1 << bits) - 1);
    // 1/qmax rounded to nearest: with one fma correction the quotient
    // y / qmax is correctly rounded for every fp32 y (checked exhaustively
    // over all significands for qmax = 3 and 15)
    const float rq = bits == 4 ? 0x1.111112p-4f : 0x1.555556p-2f;
    const int rank = o.rank;
    const int rw = wave_rows(rows);
    const int nslab = rw / kWaveSlab;
    const int wr0 = wv * rw;
    // per-matrix bases; 32-bit offsets below (rows * D * 2 < 2^32)
    const unsigned char* xb = reinterpret_cast<const unsigned char*>(
        mm < a.m_split ? a.x + (size_t)mm * rows * D : a.x2 + (size_t)(mm - a.m_split) * rows * D);
    unsigned char* codes_m = o.codes + (size_t)mm * rows * (D * bits / 8);
    float* scale_m = o.scale + (size_t)mm * rows * ngr;
    float* zero_m = o.zero + (size_t)mm * rows * ngr;
    const auto codes_r = buffer_of(codes_m, (uint32_t)rows * (D * bits / 8));
    const auto scale_r = buffer_of(scale_m, (uint32_t)rows * ngr * 4);
    const auto zero_r = buffer_of(zero_m, (uint32_t)rows * ngr * 4);

    // ---- outlier rule from the selection, on keys (|x| bit patterns, monotone
    // in |x|): key > thrk, plus (in the one row block whose quota splits the
    // ties at key T) ties ranked in flat order.  thrk = 0x7fff: none.
    uint32_t take_w = 0, csr = 0;
    int thrk = 0x7fff, tk = -1;
    bool split = false;
    float bound = 0.0f;
    const uint32_t* sel = a.sel + (size_t)mm * kSelStride;
    if (kk > 0) {
        const uint32_t tkey = sel[0];
        take_w = sel[kSelTake + wv];
        csr = sel[kSelCsr + wv];
        const uint32_t eq_w = sel[kSelEq + wv];
        split = take_w > 0 && take_w < eq_w;
        tk = (int)tkey;
        thrk = (take_w > 0 && take_w == eq_w) ? (int)tkey - 1 : (int)tkey;
    }
    // both 16-bit halves hold thrk (thrk in [-1, 0x7fff], so thrk - key fits
    // an int16 and is negative exactly for the outliers)
    const uint32_t thr2 = ((uint32_t)thrk & 0xffffu) * 0x10001u;
    // R is formed in units of 2^ex so that fp16 covers it.  With outliers the
    // exponent comes from the selection's bound on the non-outliers; without
    // them (no selection pass is run) from each 64-row slab's largest key,
    // made known one slab ahead through s_ex: the running exponent only
    // decreases, and when it does the Gram accumulators are rescaled by the
    // exact power of two.  Codes, scales and zeros do not depend on it.
    constexpr bool kSlabExp = true;
    const bool slab_ex = LR && kSlabExp && kk == 0;
    if (LR && !slab_ex) bound = h2f(sel[kSelBound]);
    int ex = LR && !slab_ex ? residual_exponent(bound) : slab_ex ? kExNone : 0;
    float sx = pow2f(ex), rsx = pow2f(-ex);
    float m1 = -(sx * rsx);   // -1, opaque to the compiler: keeps fma_mix below

    int32_t* rp = o.row_ptr + (size_t)mm * (rows + 1);
    uint16_t* cm = o.col + (size_t)mm * kk;
    uint16_t* vm = o.val + (size_t)mm * kk;
    constexpr int NBW = GramPlan<D>::NBW;
    f4v acc[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) acc[b] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t ties_seen = 0;

    // per-channel parameters (CH) of the group the wave's slab slice lies in
    // (its 8 rows are in one group: groups are multiples of 16 tokens)
    const float* chs = o.scale + (size_t)mm * (CH ? rows / o.group : 0) * D + colq * 8;
    const float* chz = o.zero + (size_t)mm * (CH ? rows / o.group : 0) * D + colq * 8;
    auto load_chp = [&](float (&cs)[8], float (&cz)[8], int sl) {
        const int row = min(wr0 + sl * kWaveSlab, rows - 1);
        const uint32_t off = (uint32_t)(row / o.group) * D * 4;
        const float4 s0 = ld_at<float4>(chs, off), s1 = ld_at<float4>(chs, off + 16);
        const float4 z0 = ld_at<float4>(chz, off), z1 = ld_at<float4>(chz, off + 16);
        cs[0] = s0.x, cs[1] = s0.y, cs[2] = s0.z, cs[3] = s0.w, cs[4] = s1.x, cs[5] = s1.y, cs[6] = s1.z, cs[7] = s1.w;
        cz[0] = z0.x, cz[1] = z0.y, cz[2] = z0.z, cz[3] = z0.w, cz[4] = z1.x, cz[5] = z1.y, cz[6] = z1.z, cz[7] = z1.w;
    };
    auto load_slab = [&](uint4 (&xr)[SS], int sl) {
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            const int row = wr0 + sl * kWaveSlab + u * RPS + rl;
            const bool ok = sl < nslab && row < rows;
            const uint32_t rc = (uint32_t)min(row, rows - 1);   // always a valid address
            const uint4 xv = ld_at<uint4>(xb, (rc * D + colq * 8) * 2);
            xr[u] = ok ? xv : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    auto do_slab = [&](const uint4 (&xr)[SS], const uint4 (&xn)[SS], int sl) {
        unsigned char* slab = s_big + (sl & 1) * 2 * kPlane;
        // The Gram products of the previous slab (complete in LDS since the
        // barrier that ended it) are issued inside this slab's vector work;
        // a change of the running exponent rescales the accumulators after
        // them (they are in the previous slab's units).
        const unsigned char* prev = s_big + ((sl + 1) & 1) * 2 * kPlane;
        float accf = 1.0f;   // rescaling of the accumulators, wave-uniform
        float chsc[8], chzp[8];
        if constexpr (CH) load_chp(chsc, chzp, sl);
        if (slab_ex) {   // wave-uniform
            const uint4 e0 = *reinterpret_cast<const uint4*>(&s_ex[sl & 1][0]);
            const uint4 e1 = *reinterpret_cast<const uint4*>(&s_ex[sl & 1][4]);
            const uint32_t key = __builtin_amdgcn_readfirstlane(
                max(max(max(e0.x, e0.y), max(e0.z, e0.w)), max(max(e1.x, e1.y), max(e1.z, e1.w))));
            const int exs = key == 0u ? kExNone : residual_exponent(h2f(key));
            if (exs < ex) {
                accf = pow2f(2 * (exs - ex));   // >= 2^-80: exact
                ex = exs;
                sx = pow2f(ex);
                rsx = pow2f(-ex);
                m1 = -(sx * rsx);
            }
        }
        uint32_t dm[SS][4], om[SS];
        // ---- outlier mask: dm = x with the outliers set to +0, om bit e set
        // for column 8 colq + e
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            const int row = wr0 + sl * kWaveSlab + u * RPS + rl;
            const bool valid = row < rows;
            const uint32_t t2 = valid ? thr2 : 0x7fff7fffu;
            const uint32_t d[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
            uint32_t bits2 = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const s2v r = __builtin_bit_cast(s2v, t2) - __builtin_bit_cast(s2v, d[i] & 0x7fff7fffu);
                const uint32_t m = __builtin_bit_cast(uint32_t, r >> (s2v){15, 15});
                dm[u][i] = d[i] & ~m;
                bits2 |= m & ((1u << (2 * i)) | (1u << (2 * i + 17)));
            }
            om[u] = (bits2 | (bits2 >> 16)) & 0xffu;
            if (split) {   // wave-uniform: the one block whose ties are split
                // key == tk per 16-bit half: (key ^ tk) - 1 is negative
                // exactly for a zero half (both are 15-bit)
                const uint32_t tk2 = ((uint32_t)tk & 0x7fffu) * 0x10001u;
                uint32_t eq2 = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const s2v z = __builtin_bit_cast(s2v, (d[i] & 0x7fff7fffu) ^ tk2) - (s2v){1, 1};
                    const uint32_t m = __builtin_bit_cast(uint32_t, z >> (s2v){15, 15});
                    eq2 |= m & ((1u << (2 * i)) | (1u << (2 * i + 17)));
                }
                const uint32_t eqm = valid ? (eq2 | (eq2 >> 16)) & 0xffu : 0u;
                if (__ballot(eqm != 0u) != 0ull && ties_seen < take_w) {
                    uint32_t tot;
                    uint32_t r = ties_seen + wave_excl_scan(__builtin_popcount(eqm), lane, &tot);
                    uint32_t tm = 0u, m = eqm;   // ties of this lane taken, column order
                    while (m != 0u && r < take_w) {
                        tm |= m & (0u - m);
                        m &= m - 1u;
                        ++r;
                    }
                    ties_seen += tot;
                    om[u] |= tm;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t clr = (((tm >> (2 * i)) & 1u) ? 0xffffu : 0u) |
                                             (((tm >> (2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
                        dm[u][i] &= ~clr;
                    }
                }
            }
        }
        // ---- CSR: row pointers, then each lane's outliers in column order.
        // One scan serves all SS steps: step u's count sits in bits 16u..16u+15
        // (at most 512 per step).
        if (kk > 0) {
            uint32_t cnt = 0u;
#pragma unroll
            for (int u = 0; u < SS; ++u) cnt |= (uint32_t)__builtin_popcount(om[u]) << (16 * u);
            const uint32_t inc = wave_incl_scan_dpp(cnt);
            const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
            const uint32_t ex_l = inc - cnt;
            uint32_t base = csr;
#pragma unroll
            for (int u = 0; u < SS; ++u) {
                const int row = wr0 + sl * kWaveSlab + u * RPS + rl;
                uint32_t pos = base + ((ex_l >> (16 * u)) & 0xffffu);
                if (row < rows && colq == 0) st_at<int32_t>(rp, (uint32_t)row * 4, (int32_t)pos);
                uint32_t m = om[u];
                const uint4 xw = xr[u];
                // column e of the lane and its fp16 bits (the dword holding it
                // picked with bit selects)
                auto emit = [&](uint32_t e, uint32_t at) {
                    const uint32_t s1 = 0u - ((e >> 1) & 1u), s2 = 0u - ((e >> 2) & 1u);
                    const uint32_t lo2 = xw.x ^ ((xw.x ^ xw.y) & s1);
                    const uint32_t hi2 = xw.z ^ ((xw.z ^ xw.w) & s1);
                    const uint32_t w = lo2 ^ ((lo2 ^ hi2) & s2);
                    if (at < kk) {
                        st_at<uint16_t>(cm, at * 2, (uint16_t)(colq * 8 + e));
                        st_at<uint16_t>(vm, at * 2, (uint16_t)((e & 1u) ? (w >> 16) : w));
                    }
                };
                // a lane rarely holds more than two outliers of a row: the
                // first two without a loop, the rest in one
                if (__ballot(m != 0u) != 0ull) {   // wave-uniform
                    const uint32_t m1 = m & (m - 1u), m2 = m1 & (m1 - 1u);
                    if (m != 0u) emit((uint32_t)__builtin_ctz(m), pos);
                    if (m1 != 0u) emit((uint32_t)__builtin_ctz(m1), pos + 1u);
                    pos += 2u;
                    m = m2;
                    while (m != 0u) {
                        emit((uint32_t)__builtin_ctz(m), pos);
                        m &= m - 1u;
                        ++pos;
                    }
                }
                base += (tot >> (16 * u)) & 0xffffu;
            }
            csr = base;
        } else {
#pragma unroll
            for (int u = 0; u < SS; ++u) {
                const int row = wr0 + sl * kWaveSlab + u * RPS + rl;
                if (row < rows && colq == 0) st_at<int32_t>(rp, (uint32_t)row * 4, 0);
            }
        }
        if (LR && sl > 0) slab_mma<D>(prev, wv, lane, acc);
        if (accf != 1.0f) {   // wave-uniform
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[b] *= accf;
        }
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            const int row = wr0 + sl * kWaveSlab + u * RPS + rl;
            const bool valid = row < rows;
            const uint32_t urow = valid ? (uint32_t)row : 0u;
            // ---- D = X - S, group quantization (in units scaled by 2^ex: every
            // step below is exact under the scaling), R = D - deq.  min and max
            // are taken on the fp16 values (exact), then scaled.
            const h2v a0 = __builtin_bit_cast(h2v, dm[u][0]), a1 = __builtin_bit_cast(h2v, dm[u][1]);
            const h2v a2 = __builtin_bit_cast(h2v, dm[u][2]), a3 = __builtin_bit_cast(h2v, dm[u][3]);
            const h2v hv[4] = {a0, a1, a2, a3};
            float t[8], cf[8], R[8];
            float mn = 0.0f, sc = 0.0f;
            if constexpr (CH) {
                // the column's group minimum and scale, in units of 2^ex; the
                // same rounding and near-tie rule per column
                bool near_tie = false;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sce = chsc[e] * sx;
                    const float inv = fminf(__builtin_amdgcn_rcpf(sce), 3.4028234664e38f);
                    t[e] = fmaf((float)hv[e >> 1][e & 1], sx, -(chzp[e] * sx));
                    cf[e] = rintf(t[e] * inv);
                    R[e] = fmaf(-cf[e], sce, t[e]);
                    near_tie |= fabsf(R[e]) > 0.49999f * sce;
                }
                if (near_tie) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float sce = chsc[e] * sx;
                        cf[e] = sce > 0.0f ? rintf(t[e] / sce) : 0.0f;
                        R[e] = fmaf(-cf[e], sce, t[e]);
                    }
                }
            } else {
            const h2v n2 = __builtin_elementwise_min(__builtin_elementwise_min(a0, a1),
                                                     __builtin_elementwise_min(a2, a3));
            const h2v x2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                     __builtin_elementwise_max(a2, a3));
            mn = (float)__builtin_elementwise_min(n2[0], n2[1]) * sx;
            float mx = (float)__builtin_elementwise_max(x2[0], x2[1]) * sx;
            group_minmax<GL>(mn, mx, gl);
            const float y = mx - mn;
            const float q0 = y * rq;
            // RN(y / qmax); y = +0 gives +0 (every term is +0 or a +0 - 0 sum)
            sc = fmaf(fmaf(-q0, qmax, y), rq, q0);
            // a finite reciprocal also for sc = 0 (then every t is 0 and its
            // code 0); for a tiny sc the near-tie test below sends the group
            // to the exact division
            const float inv = fminf(__builtin_amdgcn_rcpf(sc), 3.4028234664e38f);
            // t * inv is within a few ulp of the correctly rounded quotient, so
            // rint can differ from it only when t / sc is within 1e-5 of a
            // half-integer, that is when |R| > 0.49999 sc
            const float hs = 0.49999f * sc;
            bool near_tie = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                t[e] = fmaf((float)hv[e >> 1][e & 1], sx, -mn);   // = x 2^ex - mn, one rounding
                cf[e] = rintf(t[e] * inv);
                R[e] = fmaf(-cf[e], sc, t[e]);
                near_tie |= fabsf(R[e]) > hs;
            }
            if (near_tie) {
                // rint of the correctly rounded fp32 quotient (as the oracle takes it)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    cf[e] = rintf(t[e] / sc);
                    R[e] = fmaf(-cf[e], sc, t[e]);
                }
            }
            }
            // 0 <= t <= mx - mn, so rint(t / sc) already lies in [0, 2^b - 1]
            uint32_t word = 0;
            if (bits == 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    word = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(cf[2 * i + 1], 16.0f, cf[2 * i]), i, word);
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    word = __builtin_amdgcn_cvt_pk_u8_f32(
                        fmaf(cf[4 * i + 3], 64.0f, fmaf(cf[4 * i + 2], 16.0f, fmaf(cf[4 * i + 1], 4.0f, cf[4 * i]))),
                        i, word);
            }
            // codes, and the group's scale and zero from its first lane
            if (bits == 4) {
                const uint32_t co = valid ? urow * (D / 2) + colq * 4 : kDrop;
                __builtin_amdgcn_raw_buffer_store_b32(word, codes_r, (int)co, 0, 0);
            } else {
                const uint32_t co = valid ? urow * (D / 4) + colq * 2 : kDrop;
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)word, codes_r, (int)co, 0, 0);
            }
            if (!CH) {   // per-channel parameters were written before this kernel
                const uint32_t go = (valid && (colq % gl) == 0) ? (urow * ngr + colq / gl) * 4 : kDrop;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc * rsx), scale_r, (int)go, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, (mn + 0.0f) * rsx), zero_r,
                                                      (int)go, 0, 0);
            }
            if (LR) {
                // fp16 hi (toward zero) + lo of R * 2^ex, row-major into the slab
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const auto h2 = __builtin_amdgcn_cvt_pkrtz(R[2 * i], R[2 * i + 1]);
                    const auto l2 = __builtin_amdgcn_cvt_pkrtz(fmaf((float)h2[0], m1, R[2 * i]),
                                                               fmaf((float)h2[1], m1, R[2 * i + 1]));
                    hw[i] = __builtin_bit_cast(uint32_t, h2);
                    lw[i] = __builtin_bit_cast(uint32_t, l2);
                }
                const int srow = kWaveSlab * wv + u * RPS + rl;
                const int off = srow * (D * 2) + swz_chunk<D>(srow, 2 * colq) * 8;
                *reinterpret_cast<uint4*>(slab + off) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                *reinterpret_cast<uint4*>(slab + kPlane + off) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            }
        }
        if (LR) {
            if (slab_ex && lane == 0) s_ex[(sl + 1) & 1][wv] = wave_max_key<SS>(xn);
            __syncthreads();
        }
    };

    {
        uint4 xa[SS], xb[SS];
        load_slab(xa, 0);
        if (slab_ex) {   // the first slab's bound
            const uint32_t k0 = wave_max_key<SS>(xa);
            if (lane == 0) s_ex[0][wv] = k0;
            __syncthreads();
        }
        for (int sl = 0; sl < nslab; sl += 2) {
            load_slab(xb, sl + 1);
            do_slab(xa, xb, sl);
            if (sl + 1 < nslab) {
                load_slab(xa, sl + 2);
                do_slab(xb, xa, sl + 1);
            }
        }
    }
    if (LR && nslab > 0) slab_mma<D>(s_big + ((nslab - 1) & 1) * 2 * kPlane, wv, lane, acc);
    if (tid == 0) rp[rows] = (int32_t)kk;
    if (!LR) return;

    // ---- C = R^T R (unscaled below) into LDS, both triangles
    __syncthreads();
    float* Cm = reinterpret_cast<float*>(s_big);
    {
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            int I, J;
            if (!gram_block<D>(wv, b, I, J)) continue;   // wave-uniform
            // lane l holds rows 4 (l / 16) + v, column l % 16 of the block
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (lane / 16) + v, n = lane % 16;
                Cm[(16 * I + m) * D + 16 * J + n] = acc[b][v];
                if (I != J) Cm[(16 * J + n) * D + 16 * I + m] = acc[b][v];
            }
        }
    }
    // B0[j][c] = top 24 bits of splitmix64 output j*r + c + 1, times 2^-23, minus 1
    for (int i = tid; i < D * RKX; i += kCompressThreads) {
        const int j = i / RKX, c = i % RKX;
        float v = 0.0f;
        if (c < rank) {
            const uint64_t u = splitmix64(a.seed, (uint64_t)(j * rank + c + 1)) >> 40;
            v = (float)u * 0x1p-23f - 1.0f;
        }
        s_b[i] = v;
    }
    __syncthreads();

    // ---- power steps on C (fp64)
    const double cscale = ldexp(1.0, -2 * ex);
    const int j = tid % D, h = tid / D;   // h < NH: the threads doing the power steps
    constexpr int CPH = D / NH;           // columns of C summed by one thread
    // G = B^T W: LPP lanes per entry (c1 <= c2), each summing every LPP-th j
    constexpr int LPP = NP * 16 <= kCompressThreads ? 16 : 8;
    for (int it = 0; it < a.iters; ++it) {
        const bool last = it == a.iters - 1;
        double wp[RKX];
#pragma unroll
        for (int c = 0; c < RKX; ++c) wp[c] = 0.0;
        if (h < NH) {
            // products summed 8 at a time in fp32 (C and B are fp32), the
            // partial sums accumulated in fp64: one conversion per 8 products
            for (int i0 = 0; i0 < CPH; i0 += 8) {
                float wf[RKX];
#pragma unroll
                for (int c = 0; c < RKX; ++c) wf[c] = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c0 = h * CPH + i0 + i;
                    const float cv = Cm[c0 * D + j];   // C[j][c0], by symmetry
#pragma unroll
                    for (int c = 0; c < RKX; ++c) wf[c] = fmaf(cv, s_b[c0 * RKX + c], wf[c]);
                }
#pragma unroll
                for (int c = 0; c < RKX; ++c) wp[c] += (double)wf[c];
            }
        }
        if (h > 0 && h < NH) {
#pragma unroll
            for (int c = 0; c < RKX; ++c) s_w[((h - 1) * RKX + c) * D + j] = wp[c];
        }
        __syncthreads();
        if (h == 0) {
            for (int hh = 1; hh < NH; ++hh)
#pragma unroll
                for (int c = 0; c < RKX; ++c) wp[c] += s_w[((hh - 1) * RKX + c) * D + j];
#pragma unroll
            for (int c = 0; c < RKX; ++c) wp[c] *= cscale;
        }
        __syncthreads();
        if (h == 0) {
#pragma unroll
            for (int c = 0; c < RKX; ++c) s_w[c * D + j] = wp[c];
        }
        __syncthreads();
        if (tid < NP * LPP) {   // whole aligned groups of LPP lanes
            const int pi = tid / LPP, sub = tid % LPP;
            int c1 = 0, rem = pi;
            while (rem >= RKX - c1) {
                rem -= RKX - c1;
                ++c1;
            }
            const int c2 = c1 + rem;
            double g = 0.0;
#pragma unroll 4
            for (int i = 0; i < D / LPP; ++i) {
                const int jj = sub + LPP * i;
                g += (double)s_b[jj * RKX + c1] * s_w[c2 * D + jj];
            }
            g = row_sum64<LPP>(g);
            if (sub == 0) {
                s_g[c1 * RKX + c2] = g;
                s_g[c2 * RKX + c1] = g;
            }
        }
        __syncthreads();
        if (tid == 0) gram_to_m<RKX>(s_g, s_m);
        __syncthreads();
        if (h == 0) {
            // B' = W M and B_prev M, column by column from the last: M is upper
            // triangular, so column c needs rows 0..c of B_prev, which are
            // still unchanged when column c of B' is written
            float* Bo = o.B + ((size_t)mm * D + j) * rank;
            float* Bf = a.bf + ((size_t)mm * D + j) * RKX;
#pragma unroll
            for (int c = RKX - 1; c >= 0; --c) {
                double x1 = 0.0, x2 = 0.0;
#pragma unroll
                for (int c2 = 0; c2 <= c; ++c2) {
                    x1 += wp[c2] * s_m[c2 * RKX + c];
                    x2 += (double)s_b[j * RKX + c2] * s_m[c2 * RKX + c];
                }
                s_b[j * RKX + c] = (float)x1;
                if (last) {
                    if (c < rank) Bo[c] = (float)x1;
                    Bf[c] = (float)x2;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// A = R Bf (Bf = B_prev M of the last power step), one pass over X and the
// stored codes; independent rows, so many workgroups per matrix.  The outlier
// mask is rebuilt from X with the selection's rule: ties at key T are taken in
// flat order, so rows below r_all take all of them, rows at or above r_none
// none, and only rows in [r_all, r_none) (the one row block whose quota splits
// the ties) look the taken ties up in their CSR entries.
constexpr int kLrSteps = 4;    // 16-row steps per wave

// Ties taken, by flat order: rows [0, r_all) take all, [r_all, r_none) some.
__device__ __forceinline__ void tie_rows(const uint32_t* sel, int rows, int& r_all, int& r_none) {
    const int rw = wave_rows(rows);
    r_all = rows;
    r_none = rows;
#pragma unroll
    for (int b = 0; b < kCompressWaves; ++b) {
        const uint32_t take = sel[kSelTake + b], eq = sel[kSelEq + b];
        if (take < eq && r_all == rows) {
            r_all = min(b * rw, rows);
            r_none = take > 0 ? min((b + 1) * rw, rows) : r_all;
        }
    }
}

template <bool B>
struct BoolTag { static constexpr bool value = B; };

// A = R Bf, 16 token rows per step of a wave.  Lane l holds row l % 16 and
// the CPL = D/4 consecutive columns starting at CPL (l / 16).  At rank <= 4
// (one quantization group per lane) each lane adds R Bf over its columns on
// the VALU (Bf's rows from LDS) and the four lane groups of a row are summed
// with permlane swaps.  Otherwise v_mfma_f32_16x16x4_f32 contracts them: M =
// 16 token rows, N = 16 (the r columns of Bf, zero beyond r), K = 4 per
// instruction; the j-th instruction contracts column CPL q + j of the four
// lane groups q, so CPL instructions cover all D columns and no cross-lane
// sum is needed, and the output lanes n = l % 16 < r hold A[row][n] for the
// rows 4 (l / 16) + 0..3 of the step.  X goes from HBM straight into a
// per-wave LDS tile (row-contiguous load instructions, 16-byte chunks
// XOR-swizzled by row) and is read from there in that layout.
// byte I of x as a float, one instruction (v_cvt_f32_ubyteI)
template <int I>
__device__ __forceinline__ float ubyte_f(uint32_t x) {
    float f;
    if (I == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(x));
    else if (I == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
    else if (I == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(x));
    return f;
}

// BITS4: 4-bit codes (else 2-bit); ONEG: a lane's columns lie in one
// quantization group.  Compile-time, so that each variant gets the registers
// it needs on its own.
template <int D, int RK, bool BITS4, bool ONEG, bool CH = false>
__global__ void __launch_bounds__(kThreads) lowrank_a_kernel(CompressArgs a) {
    constexpr int CPL = D / 4;                // columns per lane
    constexpr int NX = CPL / 8;               // 16-byte chunks of X per lane
    constexpr int ROWS_W = 16 * kLrSteps, ROWS_WG = 4 * ROWS_W;
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int rr = lane & 15, q = lane >> 4;
    const Packed& o = a.out;
    const int rows = o.rows, rank = o.rank;
    constexpr int bits = BITS4 ? 4 : 2;
    const int g = o.group, ngr = D / g;
    const int ngl = g >= CPL ? 1 : CPL / g;   // groups within a lane's columns (<= 4)
    const uint32_t kk = (uint32_t)o.k;
    const int nblk = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = a.m0 + group_id_x() / nblk;
    const int blk = (int)(group_id_x() % nblk);
    const int r0 = blk * ROWS_WG + wv * ROWS_W;
    const int c0 = CPL * q;                   // first column of this lane
    // per-matrix bases; 32-bit offsets below (rows * D * 2 < 2^32)
    const unsigned char* xb = reinterpret_cast<const unsigned char*>(
        mm < a.m_split ? a.x + (size_t)mm * rows * D : a.x2 + (size_t)(mm - a.m_split) * rows * D);
    const unsigned char* cb = o.codes + (size_t)mm * rows * (D * bits / 8);
    const float* scb = o.scale + (size_t)mm * rows * ngr;
    const float* zpb = o.zero + (size_t)mm * rows * ngr;
    // rank <= 4 with one group per lane: A on the VALU (lane (rr, q) sums
    // over its CPL columns, then the four lane groups are added); otherwise on
    // the matrix cores (at rank 8 they do twice the useful work per
    // instruction, and with several groups per lane the compiler would hold
    // all of B's rows in registers)
    constexpr bool VPATH = RK <= 4 && ONEG;
    float Bv[VPATH ? 1 : CPL];                // MFMA B operand: Bf[c0 + j][n = rr]
    // Bf rows, padded to 4 columns, one empty row after every CPL rows: the
    // four lane groups read rows CPL apart at once, which would otherwise
    // fall on the same LDS banks
    __shared__ __attribute__((aligned(16))) float s_bm[VPATH ? (D + D / CPL) * 4 : 4];
    // CH: the per-channel scales and zeros of the token groups of this
    // workgroup's rows (groups of at least 16 tokens: a 16-row step lies in one)
    constexpr int kChG = CH ? ROWS_WG / 16 : 1;
    __shared__ __attribute__((aligned(16))) float s_cs[kChG * D];
    __shared__ __attribute__((aligned(16))) float s_cz[kChG * D];
    const int cg0 = CH ? blk * ROWS_WG / o.group : 0;
    if constexpr (CH) {
        const int cg1 = (min(blk * ROWS_WG + ROWS_WG, rows) - 1) / o.group;
        const float* cs = o.scale + (size_t)mm * (rows / o.group) * D;
        const float* cz = o.zero + (size_t)mm * (rows / o.group) * D;
        for (int i = tid; i < (cg1 - cg0 + 1) * D; i += kThreads) {
            s_cs[i] = cs[(size_t)cg0 * D + i];
            s_cz[i] = cz[(size_t)cg0 * D + i];
        }
        if (!VPATH) __syncthreads();   // the VALU path has a barrier of its own below
    }
    if constexpr (VPATH) {
        if (tid < D) {
            const float* src = a.bf + ((size_t)mm * D + tid) * RK;
            f4v v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (RK == 4) v = *reinterpret_cast<const f4v*>(src);
            else v = f4v{src[0], src[1], 0.0f, 0.0f};
            reinterpret_cast<f4v*>(s_bm)[tid + tid / CPL] = v;
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj)
            Bv[jj] = rr < RK ? a.bf[((size_t)mm * D + c0 + jj) * RK + rr] : 0.0f;
    }

    // outlier rule on keys (|x| bit patterns): key > thrk, thrk = T - 1 in the
    // rows that take all ties at key T, T elsewhere, 0x7fff without outliers;
    // plus, in the one row block whose quota splits the ties, the ties its
    // CSR entries hold
    int thr_all = 0x7fff, thr_none = 0x7fff, tk = -1;
    int r_all = rows, r_none = rows;
    if (kk > 0) {
        const uint32_t* sel = a.sel + (size_t)mm * kSelStride;
        tk = (int)sel[0];
        thr_all = tk - 1;
        thr_none = tk;
        tie_rows(sel, rows, r_all, r_none);
    }
    const bool wave_split = r0 < r_none && r0 + ROWS_W > r_all;   // wave-uniform
    const int32_t* rp = o.row_ptr + (size_t)mm * (rows + 1);
    const uint16_t* cm = o.col + (size_t)mm * kk;
    float* Am = o.A + (size_t)mm * rows * rank;
    float one = 1.0f;   // opaque 1: keeps x - zero a single mixed fma
    asm volatile("" : "+s"(one));

    // per-wave tiles of 16 rows of X, two (steps alternate): [row][chunk ^
    // swizzle(row)], 16-byte chunks.  X goes from HBM straight into a tile
    // (global_load_lds_dwordx4: lane l of a load instruction fills slot l of
    // its 64-slot range, no registers), the next step's while this step
    // computes.
    constexpr int CPR = D / 8;                // chunks per row (16 or 8)
    constexpr int NLD = 16 * CPR / 64;        // load instructions per tile
    __shared__ __attribute__((aligned(16))) uint4 s_x[4][2][16 * CPR];
    auto swz = [](int row, int ch) { return ch ^ (row & (CPR - 1)); };
    auto issue_x = [&](int s, int buf) {
        uint4* t = s_x[wv][buf];
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
            const int slot = 64 * c + lane, trow = slot / CPR;
            const int ch = swz(trow, slot % CPR);   // the chunk stored at this slot
            const uint32_t xr = (uint32_t)min(r0 + s * 16 + trow, rows - 1);   // valid address
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(xb + (xr * D + ch * 8) * 2),
                (__attribute__((address_space(3))) void*)(t + 64 * c), 16, 0, 0);
        }
    };
    struct Buf {
        uint4 cw;
        float sc[4], zp[4];
    };
    auto load = [&](int s) {
        Buf bf;
        const int row = r0 + s * 16 + rr;
        const uint32_t rc = (uint32_t)min(row, rows - 1);   // always a valid address
        constexpr uint32_t cbytes = (uint32_t)(CPL * bits / 8);  // 16, 8 or 4
        const uint32_t coff = rc * (D * bits / 8) + (uint32_t)(c0 * bits / 8);
        if constexpr (cbytes == 16) {
            bf.cw = ld_at<uint4>(cb, coff);
        } else if constexpr (cbytes == 8) {
            const uint2 v = ld_at<uint2>(cb, coff);
            bf.cw = make_uint4(v.x, v.y, 0u, 0u);
        } else {
            bf.cw = make_uint4(ld_at<uint32_t>(cb, coff), 0u, 0u, 0u);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf.sc[t] = 0.0f;
            bf.zp[t] = 0.0f;
            if (!CH && t < ngl) {
                const uint32_t go = (rc * ngr + (c0 + t * g) / g) * 4;
                bf.sc[t] = ld_at<float>(scb, go);
                bf.zp[t] = ld_at<float>(zpb, go);
            }
        }
        return bf;
    };
    auto compute = [&](const uint4 (&xq)[NX], const Buf& bf, int s, auto split_tag) {
        constexpr bool SPLIT = decltype(split_tag)::value;
        const int row = r0 + s * 16 + rr;
        const bool valid = row < rows;
        const int thrk = row < r_all ? thr_all : thr_none;
        const uint32_t t2 = ((uint32_t)thrk & 0xffffu) * 0x10001u;   // thrk in both halves
        // ties of the split block taken by this row: bits of tm (column c0 + j)
        uint32_t tm = 0u;
        if (SPLIT) {
            bool any_eq = false;
#pragma unroll
            for (int c = 0; c < NX; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) any_eq |= (int)(half_of(xq[c], e) & 0x7fffu) == tk;
            any_eq = any_eq && valid && row >= r_all && row < r_none;
            if (__ballot(any_eq) != 0ull && any_eq) {
                const int beg = max(rp[row], 0), end = min(rp[row + 1], (int32_t)kk);
#pragma unroll 1
                for (int i = beg; i < end; ++i) {
                    const int cj = (int)cm[i] - c0;
                    if (cj >= 0 && cj < CPL) tm |= 1u << cj;
                }
            }
        }
        f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        float av[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // VALU path: this lane's partial A row
        const uint32_t cwd[4] = {bf.cw.x, bf.cw.y, bf.cw.z, bf.cw.w};
#pragma unroll
        for (int c = 0; c < NX; ++c) {
            // D = X - S on the fp16 bits: the outliers become +0
            const uint32_t d[4] = {xq[c].x, xq[c].y, xq[c].z, xq[c].w};
            uint32_t dm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const s2v r = __builtin_bit_cast(s2v, t2) - __builtin_bit_cast(s2v, d[i] & 0x7fff7fffu);
                uint32_t m = __builtin_bit_cast(uint32_t, r >> (s2v){15, 15});
                if (SPLIT)
                    m |= (((tm >> (8 * c + 2 * i)) & 1u) ? 0xffffu : 0u) |
                         (((tm >> (8 * c + 2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
                dm[i] = d[i] & ~m;
            }
            float cf[8];
            if (BITS4) {
                const uint32_t lo = cwd[c] & 0x0F0F0F0Fu, hi = (cwd[c] >> 4) & 0x0F0F0F0Fu;
                cf[0] = ubyte_f<0>(lo), cf[2] = ubyte_f<1>(lo), cf[4] = ubyte_f<2>(lo), cf[6] = ubyte_f<3>(lo);
                cf[1] = ubyte_f<0>(hi), cf[3] = ubyte_f<1>(hi), cf[5] = ubyte_f<2>(hi), cf[7] = ubyte_f<3>(hi);
            } else {
                const uint32_t w = cwd[c >> 1] >> (16 * (c & 1));
#pragma unroll
                for (int e = 0; e < 8; ++e) cf[e] = (float)((w >> (2 * e)) & 3u);
            }
            float chs8[8], chz8[8];
            if constexpr (CH) {   // columns c0 + 8 c .. + 7 of this step's token group
                const int gi = (r0 + s * 16) / o.group - cg0;
                const float* ps = s_cs + gi * D + c0 + 8 * c;
                const float* pz = s_cz + gi * D + c0 + 8 * c;
                const float4 s0 = *reinterpret_cast<const float4*>(ps), s1 = *reinterpret_cast<const float4*>(ps + 4);
                const float4 z0 = *reinterpret_cast<const float4*>(pz), z1 = *reinterpret_cast<const float4*>(pz + 4);
                chs8[0] = s0.x, chs8[1] = s0.y, chs8[2] = s0.z, chs8[3] = s0.w;
                chs8[4] = s1.x, chs8[5] = s1.y, chs8[6] = s1.z, chs8[7] = s1.w;
                chz8[0] = z0.x, chz8[1] = z0.y, chz8[2] = z0.z, chz8[3] = z0.w;
                chz8[4] = z1.x, chz8[5] = z1.y, chz8[6] = z1.z, chz8[7] = z1.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = 8 * c + e;
                float scv = bf.sc[0], zpv = bf.zp[0];
                if (CH) {
                    scv = chs8[e];
                    zpv = chz8[e];
                } else if (!ONEG) {   // groups of 8 or 16 columns: group of column jj
                    const int t = jj / (g == 8 ? 8 : 16);
                    scv = t == 0 ? bf.sc[0] : t == 1 ? bf.sc[1] : t == 2 ? bf.sc[2] : bf.sc[3];
                    zpv = t == 0 ? bf.zp[0] : t == 1 ? bf.zp[1] : t == 2 ? bf.zp[2] : bf.zp[3];
                }
                // R = (x or 0) - zero - code * scale; x - zero in one mixed fma
                const float xz = fmaf(h2f(dm[e >> 1] >> (16 * (e & 1))), one, -zpv);
                const float R = fmaf(-cf[e], scv, xz);
                if constexpr (VPATH) {
                    const f4v bm = reinterpret_cast<const f4v*>(s_bm)[c0 + jj + q];
#pragma unroll
                    for (int c2 = 0; c2 < RK; ++c2) av[c2] = fmaf(R, bm[c2], av[c2]);
                } else {
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(R, Bv[jj], acc, 0, 0, 0);
                }
            }
        }
        if constexpr (VPATH) {
            // the row's sums over the four lane groups (lanes rr + 16 q)
#pragma unroll
            for (int c2 = 0; c2 < RK; ++c2) av[c2] = sum_xor32(sum_xor16(av[c2]));
            if (q == 0 && valid) {
                float* dst = Am + (size_t)row * rank;
                if (RK == 4 && rank == 4) {
                    *reinterpret_cast<f4v*>(dst) = f4v{av[0], av[1], av[2], av[3]};
                } else {
#pragma unroll
                    for (int c2 = 0; c2 < RK; ++c2)
                        if (c2 < rank) dst[c2] = av[c2];
                }
            }
        } else if (rr < rank) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int orow = r0 + s * 16 + 4 * q + i;
                if (orow < rows) Am[(size_t)orow * rank + rr] = acc[i];
            }
        }
    };
    // Per step: this step's X from its tile into registers (lane (rr, q) takes
    // row rr, chunks CPL q / 8 .. CPL q / 8 + NX - 1), then the next step's
    // loads are issued, then this step's arithmetic.  The compiler waits for
    // every outstanding load before the first tile read after a tile load,
    // so the next step's loads are issued only after this step's reads; they
    // go to the other tile.
    auto run = [&](auto split_tag) {
        issue_x(0, 0);
        Buf cur = load(0);
#pragma unroll 1
        for (int s = 0; s < kLrSteps; ++s) {
            const uint4* t = s_x[wv][s & 1];
            uint4 xq[NX];
#pragma unroll
            for (int c = 0; c < NX; ++c) xq[c] = t[rr * CPR + swz(rr, (c0 / 8) + c)];
            __builtin_amdgcn_sched_barrier(0);
            Buf nxt = cur;
            if (s + 1 < kLrSteps) {
                issue_x(s + 1, (s + 1) & 1);
                nxt = load(s + 1);
            }
            compute(xq, cur, s, split_tag);
            cur = nxt;
        }
    };
    if (wave_split) run(BoolTag<true>{});
    else run(BoolTag<false>{});
}

// ---------------------------------------------------------------------------
// KIVI keys: scale and zero per channel for each group of `group` tokens of a
// matrix without outliers -- min and max of the group's entries in the
// column, scale = RN((max - min) / (2^b - 1)), zero = min (both +0 when zero),
// as the per-token groups take them.  One workgroup per (matrix, group): 16
// row slots of D/8 lanes, 8 columns per lane, then the slots' results merged.
template <int D>
__global__ void __launch_bounds__(kThreads) channel_params_kernel(CompressArgs a) {
    constexpr int LPR = D / 8, SLOTS = kThreads / LPR;
    __shared__ float s_mn[SLOTS * D];
    __shared__ float s_mx[SLOTS * D];
    const Packed& o = a.out;
    const int tid = thread_id(), colq = tid % LPR, slot = tid / LPR;
    const int g = o.group, ngroups = o.rows / g;
    const int64_t mm = a.m0 + group_id_x() / ngroups;
    const int gi = (int)(group_id_x() % ngroups);
    const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * o.rows * D
                                        : a.x2 + (size_t)(mm - a.m_split) * o.rows * D;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 mn[4], mx[4];
    const bool any = slot < g;   // the slot has at least one row of the group
    for (int row = gi * g + slot; row < (gi + 1) * g; row += SLOTS) {
        const uint4 w = *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8);
        const uint32_t wv4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h2 v = __builtin_bit_cast(h2, wv4[i]);
            if (row == gi * g + slot) {
                mn[i] = v;
                mx[i] = v;
            } else {
                mn[i] = __builtin_elementwise_min(mn[i], v);
                mx[i] = __builtin_elementwise_max(mx[i], v);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s_mn[slot * D + colq * 8 + e] = any ? (float)mn[e >> 1][e & 1] : INFINITY;
        s_mx[slot * D + colq * 8 + e] = any ? (float)mx[e >> 1][e & 1] : -INFINITY;
    }
    __syncthreads();
    if (tid < D) {
        float lo = s_mn[tid], hi = s_mx[tid];
        for (int q = 1; q < SLOTS; ++q) {
            lo = fminf(lo, s_mn[q * D + tid]);
            hi = fmaxf(hi, s_mx[q * D + tid]);
        }
        const float qmax = (float)((1 << o.bits) - 1);
        const float rq = o.bits == 4 ? 0x1.111112p-4f : 0x1.555556p-2f;
        const float y = hi - lo;
        const float q0 = y * rq;
        const float sc = fmaf(fmaf(-q0, qmax, y), rq, q0);   // RN(y / qmax)
        const size_t at = ((size_t)mm * ngroups + gi) * D + tid;
        o.scale[at] = sc + 0.0f;
        o.zero[at] = lo + 0.0f;
    }
}

// ZipCache: per compressed matrix, the channel factors 2^e_j (the smallest
// power of two not below the column's largest |x|; 1 for an all-zero
// column), one workgroup per matrix.
template <int D>
__global__ void __launch_bounds__(kThreads) channel_exponent_kernel(CompressArgs a) {
    constexpr int LPR = D / 8, SLOTS = kThreads / LPR;
    __shared__ uint32_t s_key[SLOTS * D];
    const Packed& o = a.out;
    const int tid = thread_id(), colq = tid % LPR, slot = tid / LPR;
    const int64_t mm = a.m0 + group_id_x();
    const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * o.rows * D
                                        : a.x2 + (size_t)(mm - a.m_split) * o.rows * D;
    typedef unsigned short u2 __attribute__((ext_vector_type(2)));
    u2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    for (int row = slot; row < o.rows; row += SLOTS) {
        const uint4 w = *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8);
        const uint32_t wv4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m[i] = __builtin_elementwise_max(m[i], __builtin_bit_cast(u2, wv4[i] & 0x7fff7fffu));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_key[slot * D + colq * 8 + e] = m[e >> 1][e & 1];
    __syncthreads();
    if (tid < D) {
        uint32_t key = 0;
        for (int q = 0; q < SLOTS; ++q) key = max(key, s_key[q * D + tid]);
        int k = 0;
        if (key != 0) {
            int ex;
            const float f = frexpf((float)__builtin_bit_cast(_Float16, (uint16_t)key), &ex);
            k = f == 0.5f ? ex - 1 : ex;
        }
        o.chan[(size_t)mm * D + tid] = __builtin_bit_cast(float, (uint32_t)(127 + k) << 23);
    }
}

// ZipCache: xt = fl16(x / factor_j), 8 values per thread, grid-stride.
template <int D>
__global__ void __launch_bounds__(kThreads) channel_normalize_kernel(CompressArgs a, uint16_t* xt,
                                                                     int nblocks) {
    const Packed& o = a.out;
    constexpr int LPR = D / 8;
    const size_t per_mat = (size_t)o.rows * LPR;
    const size_t total = (size_t)(a.m1 - a.m0) * per_mat;
    for (size_t i = (size_t)group_id_x() * kThreads + thread_id(); i < total;
         i += (size_t)nblocks * kThreads) {
        const int64_t mm = a.m0 + (int64_t)(i / per_mat);
        const size_t rem = i % per_mat;
        const int colq = (int)(rem % LPR);
        const uint16_t* src = (mm < a.m_split ? a.x + (size_t)mm * o.rows * D
                                              : a.x2 + (size_t)(mm - a.m_split) * o.rows * D) + rem * 8;
        const uint4 w = *reinterpret_cast<const uint4*>(src);
        const float4 f0 = *reinterpret_cast<const float4*>(o.chan + (size_t)mm * D + colq * 8);
        const float4 f1 = *reinterpret_cast<const float4*>(o.chan + (size_t)mm * D + colq * 8 + 4);
        // 1 / 2^e, exact
        const float fi[8] = {1.0f / f0.x, 1.0f / f0.y, 1.0f / f0.z, 1.0f / f0.w,
                             1.0f / f1.x, 1.0f / f1.y, 1.0f / f1.z, 1.0f / f1.w};
        const uint32_t wi[4] = {w.x, w.y, w.z, w.w};
        uint32_t wo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = h2f(wi[q] & 0xffffu) * fi[2 * q];        // exact in fp32
            const float hi = h2f(wi[q] >> 16) * fi[2 * q + 1];
            // one rounding to fp16, to nearest even
            wo[q] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
        }
        *reinterpret_cast<uint4*>(xt + (size_t)mm * o.rows * D + rem * 8) = make_uint4(wo[0], wo[1], wo[2], wo[3]);
    }
}

// Compute units of the current device, cached per device.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D>
constexpr int lowrank_rows_per_wg() { return 4 * 16 * kLrSteps; }

template <int D, int RK>
hipError_t launch_d_rk(const CompressArgs& a, hipStream_t st) {
    const unsigned M = (unsigned)(a.m1 - a.m0);
    if (a.chan_q) {   // KIVI keys (no outliers): the per-channel path
        hipError_t e;
        {
            Timed t(kKCompress, st);
            hipLaunchKernelGGL((compress_kernel<D, RK, D / 8, true>), dim3(M), dim3(kCompressThreads), 0, st, a);
            e = hipGetLastError();
        }
        if constexpr (RK > 0) {
            if (e != hipSuccess) return e;
            constexpr int RPW = lowrank_rows_per_wg<D>();
            const int64_t blocks = (int64_t)M * ((a.out.rows + RPW - 1) / RPW);
            if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
            Timed t(kKLowrankA, st);
            if (a.out.bits == 4)
                hipLaunchKernelGGL((lowrank_a_kernel<D, RK, true, true, true>), dim3((unsigned)blocks),
                                   dim3(kThreads), 0, st, a);
            else
                hipLaunchKernelGGL((lowrank_a_kernel<D, RK, false, true, true>), dim3((unsigned)blocks),
                                   dim3(kThreads), 0, st, a);
            e = hipGetLastError();
        }
        return e;
    }
    if (a.out.k > 0) {   // without outliers the compress kernel bounds R itself
        Timed t(kKSelect, st);
        // 16 waves per matrix when the matrices are too few to give every CU
        // more than two workgroups (their waves are then all a CU has to
        // hide memory latency with), else 8; batches of 2 row steps
        if ((int64_t)M <= 2 * (int64_t)cu_count())
            hipLaunchKernelGGL((select_kernel<D, 2, 1024>), dim3(M), dim3(1024), 0, st, a);
        else
            hipLaunchKernelGGL((select_kernel<D, 2, 512>), dim3(M), dim3(512), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e;
    {
        Timed t(kKCompress, st);
        if (a.out.group == D)
            hipLaunchKernelGGL((compress_kernel<D, RK, D / 8>), dim3(M), dim3(kCompressThreads), 0, st, a);
        else
            hipLaunchKernelGGL((compress_kernel<D, RK, 0>), dim3(M), dim3(kCompressThreads), 0, st, a);
        e = hipGetLastError();
    }
    if constexpr (RK > 0) {
        if (e != hipSuccess) return e;
        constexpr int RPW = lowrank_rows_per_wg<D>();
        const int64_t blocks = (int64_t)M * ((a.out.rows + RPW - 1) / RPW);
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        Timed t(kKLowrankA, st);
        const bool one_group = a.out.group >= D / 4;   // a lane's D/4 columns in one group
        const dim3 grid((unsigned)blocks), wg(kThreads);
        if (a.out.bits == 4) {
            if (one_group) hipLaunchKernelGGL((lowrank_a_kernel<D, RK, true, true>), grid, wg, 0, st, a);
            else hipLaunchKernelGGL((lowrank_a_kernel<D, RK, true, false>), grid, wg, 0, st, a);
        } else {
            if (one_group) hipLaunchKernelGGL((lowrank_a_kernel<D, RK, false, true>), grid, wg, 0, st, a);
            else hipLaunchKernelGGL((lowrank_a_kernel<D, RK, false, false>), grid, wg, 0, st, a);
        }
        e = hipGetLastError();
    }
    return e;
}

template <int D>
hipError_t launch_d(const CompressArgs& a, hipStream_t st) {
    switch (rank_slots(a.out.rank)) {
        case 0: return launch_d_rk<D, 0>(a, st);
        case 2: return launch_d_rk<D, 2>(a, st);
        case 4: return launch_d_rk<D, 4>(a, st);
        default: return launch_d_rk<D, 8>(a, st);
    }
}

}  // namespace

size_t compress_workspace(int64_t M, int d, int rank) {
    // never 0, which the ABI reserves for rejected settings
    const size_t n = align_up((size_t)M * kSelStride * 4) + align_up((size_t)M * d * rank_slots(rank) * 4);
    return n > kAlign ? n : kAlign;
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
    if (a.m1 <= a.m0) return hipSuccess;
    if (a.m1 - a.m0 > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.out.rank > 0 && (a.out.rows < 1 || a.iters < 1)) return hipErrorInvalidValue;
    if (a.chan_q && (a.out.k != 0 || a.out.group < 16 || a.out.rows % a.out.group != 0))
        return hipErrorInvalidValue;
    if (a.out.d == 64) return launch_d<64>(a, st);
    if (a.out.d == 128) return launch_d<128>(a, st);
    return hipErrorInvalidValue;
}

hipError_t launch_channel_params(const CompressArgs& a, hipStream_t st) {
    if (a.m1 <= a.m0) return hipSuccess;
    if (a.out.group < 16 || a.out.rows % a.out.group != 0) return hipErrorInvalidValue;
    const int64_t blocks = (a.m1 - a.m0) * (a.out.rows / a.out.group);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    Timed t(kKChannel, st);
    if (a.out.d == 64)
        hipLaunchKernelGGL((channel_params_kernel<64>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    else if (a.out.d == 128)
        hipLaunchKernelGGL((channel_params_kernel<128>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_channel_normalize(const CompressArgs& a, uint16_t* xt, hipStream_t st) {
    if (a.m1 <= a.m0) return hipSuccess;
    if (a.m1 - a.m0 > 0x7fffffffLL || !a.out.chan) return hipErrorInvalidValue;
    const size_t total = (size_t)(a.m1 - a.m0) * a.out.rows * (a.out.d / 8);
    size_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    Timed t(kKChannel, st);
    if (a.out.d == 64) {
        hipLaunchKernelGGL((channel_exponent_kernel<64>), dim3((unsigned)(a.m1 - a.m0)), dim3(kThreads), 0, st, a);
        hipLaunchKernelGGL((channel_normalize_kernel<64>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a,
                           xt, (int)blocks);
    } else if (a.out.d == 128) {
        hipLaunchKernelGGL((channel_exponent_kernel<128>), dim3((unsigned)(a.m1 - a.m0)), dim3(kThreads), 0, st, a);
        hipLaunchKernelGGL((channel_normalize_kernel<128>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a,
                           xt, (int)blocks);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


}  // namespace gear
