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
//   * A "team" of T workgroups owns one matrix; each workgroup holds its block
//     of rows in VGPRs for the whole pipeline, so X is read from HBM exactly
//     once and the residual R never leaves the register file.  Teams loop over
//     matrices (a persistent, cooperative launch when T > 1).
//   * The team agrees on the outlier threshold with a two-level radix select
//     (1024 coarse bins of |x|>>5, then 32 fine bins) and on each power step
//     with one all-reduce of (W = R^T P, G = P^T P); these are the only
//     cross-workgroup exchanges (plain stores + agent-scope atomics, with a
//     bounded wait that records a failure instead of hanging).
//   * One power step needs one pass over R: P = R B and W = R^T P are formed
//     together, and A = P M, B' = W M with M (r x r, upper triangular) the
//     Gram-Schmidt of P expressed through G.  In exact arithmetic this is the
//     same A, B as modified Gram-Schmidt on P followed by B = R^T A.
//   * The products are bandwidth-shaped (r <= 8 columns): plain fp32 VALU FMAs
//     with a lane owning 8 consecutive columns of a token; a row's dot product
//     is finished with a butterfly over the D/8 lanes of that row.
//   * Quantization is bit-exact IEEE fp32 (correctly rounded division,
//     rint), codes are packed in registers and stored as one 32-bit (4-bit
//     codes) or 16-bit (2-bit codes) word per lane per token: fully coalesced.
#include "gear_internal.h"

namespace gear {
namespace {

constexpr uint32_t kSpinLimit = 1u << 20;
constexpr size_t kTeamHeader = 256;                // barrier counter
constexpr size_t kTeamHist = 2 * 1024 * 4;         // coarse histograms, two parities
constexpr size_t kFineSlot = 64 * 4;               // per-workgroup fine histogram + count
constexpr size_t kTeamZeroBytes = kTeamHeader + kTeamHist;
constexpr size_t kSlotG = 64 * 8;                  // room for the Gram pairs (fp64)

__device__ __forceinline__ float h2f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// All T workgroups of a team reach the barrier before any leaves it.  The
// wait is bounded: on timeout (or once any workgroup has failed) the failure
// word is set and the barrier returns, so every kernel instance terminates.
__device__ void team_barrier(uint32_t* ctr, uint32_t target, uint32_t* err) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    // every thread: later plain loads of the team's data see the released values
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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

template <int LPR>
__device__ __forceinline__ uint32_t row_sum_u32(uint32_t v) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}
template <int LPR>
__device__ __forceinline__ uint32_t row_excl_scan(uint32_t v, int colq) {
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
        uint32_t y = __shfl_up(x, off, LPR);
        if (colq >= off) x += y;
    }
    return x - v;
}

// Exclusive prefix, in local row order, of one count per row.  cnt[s] must be
// valid in the lane with colq == 0 of each row.  Returns the prefix for every
// lane of the row.
template <int RPL, int RPS>
__device__ void rows_excl_scan(const uint32_t (&cnt)[RPL], uint32_t (&base)[RPL],
                               uint32_t* s_rows, uint32_t* s_tmp, int wv, int rl, int colq) {
    constexpr int ROWS_WG = 4 * RPL * RPS;
    constexpr int PER = ROWS_WG >= kThreads ? ROWS_WG / kThreads : 1;
#pragma unroll
    for (int s = 0; s < RPL; ++s)
        if (colq == 0) s_rows[wv * RPL * RPS + s * RPS + rl] = cnt[s];
    __syncthreads();
    uint32_t loc[PER];
    uint32_t sum = 0;
    const int i0 = threadIdx.x * PER;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        loc[q] = (i0 + q < ROWS_WG) ? s_rows[i0 + q] : 0u;
        sum += loc[q];
    }
    uint32_t tot;
    uint32_t ex = block_excl_scan(sum, s_tmp, &tot);
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (i0 + q < ROWS_WG) {
            s_rows[i0 + q] = ex;
            ex += loc[q];
        }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < RPL; ++s) base[s] = s_rows[wv * RPL * RPS + s * RPS + rl];
    __syncthreads();
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + i * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// M (RK x RK, column c = coefficients of A[:,c] in the columns of P) from the
// Gram matrix G = P^T P: Gram-Schmidt carried out on coefficient vectors, with
// inner products taken through G.  A column whose norm after projection is at
// most 1e-6 of its norm before projection (or is zero) becomes zero.
// Run by one thread on LDS arrays (fp64); the loops are kept rolled so the
// kernel's register budget is not spent on this O(RK^3) step.
template <int RK>
__device__ void gram_to_m(const double* G /* RK*RK symmetric */, double* m /* RK*RK: m[c*RK+a] */,
                          double* u /* RK */, double* gu /* RK */, float* Mout) {
#pragma nounroll
    for (int c = 0; c < RK; ++c) {
#pragma nounroll
        for (int a = 0; a < RK; ++a) u[a] = (a == c) ? 1.0 : 0.0;
        const double pre2 = G[c * RK + c];
#pragma nounroll
        for (int i = 0; i < c; ++i) {
            // proj = A_i . (P u) = m_i^T G u
#pragma nounroll
            for (int a = 0; a < RK; ++a) {
                double acc = 0.0;
#pragma nounroll
                for (int b = 0; b < RK; ++b) acc += G[a * RK + b] * u[b];
                gu[a] = acc;
            }
            double proj = 0.0;
#pragma nounroll
            for (int a = 0; a < RK; ++a) proj += m[i * RK + a] * gu[a];
#pragma nounroll
            for (int a = 0; a < RK; ++a) u[a] -= proj * m[i * RK + a];
        }
        double post2 = 0.0;
#pragma nounroll
        for (int a = 0; a < RK; ++a) {
            double acc = 0.0;
#pragma nounroll
            for (int b = 0; b < RK; ++b) acc += G[a * RK + b] * u[b];
            post2 += u[a] * acc;
        }
        const bool dead = !(pre2 > 0.0) || !(post2 > 1e-12 * pre2);
        const double inv = dead ? 0.0 : 1.0 / sqrt(post2);
#pragma nounroll
        for (int a = 0; a < RK; ++a) m[c * RK + a] = u[a] * inv;
    }
#pragma nounroll
    for (int a = 0; a < RK; ++a)
#pragma nounroll
        for (int c = 0; c < RK; ++c) Mout[a * RK + c] = (float)m[c * RK + a];
}

template <int D, int RPL, int RK>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
compress_kernel(CompressArgs a) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPS = 64 / LPR;           // rows per wave per step
    constexpr int ROWS_WAVE = RPL * RPS;
    constexpr int ROWS_WG = 4 * ROWS_WAVE;
    constexpr int RKX = RK > 0 ? RK : 1;
    constexpr int NP = RKX * (RKX + 1) / 2;

    __shared__ uint32_t s_hist[1024];
    __shared__ uint32_t s_fine[kMaxTeam * 33];
    __shared__ uint32_t s_rows[ROWS_WG > kThreads ? ROWS_WG : kThreads];
    __shared__ uint32_t s_tmp[8];
    __shared__ uint32_t s_sel[8];
    __shared__ float s_b0[D * RKX];
    __shared__ float s_w[4 * D * RKX];
    __shared__ float s_p[ROWS_WG * RKX];
    __shared__ double s_g[4 * NP];
    __shared__ double s_gt[RKX * RKX];
    __shared__ double s_mm[RKX * RKX + 2 * RKX];
    __shared__ float s_m[RKX * RKX];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const int T = a.team;
    int team, member;
    if (T == 1) {
        team = blockIdx.x;
        member = 0;
    } else {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        team = (slot / T) * 8 + xcd;
        member = slot % T;
    }
    if (team >= a.num_teams) return;

    const Packed& o = a.out;
    const int rows = o.rows;
    const int bits = o.bits, group = o.group, gl = group / 8;
    const uint32_t kk = (uint32_t)o.k;
    const float qmax = (float)((1 << bits) - 1);
    const int rank = o.rank;

    uint8_t* tb = a.team_ws + (size_t)team * a.team_bytes;
    uint32_t* ctr = reinterpret_cast<uint32_t*>(tb);
    uint32_t* thist = reinterpret_cast<uint32_t*>(tb + kTeamHeader);
    uint32_t* tfine = reinterpret_cast<uint32_t*>(tb + kTeamZeroBytes);
    uint8_t* tslot = tb + kTeamZeroBytes + (size_t)T * kFineSlot;

    // B0, identical for every matrix of the call.
    if (RK > 0) {
        for (int i = tid; i < D * RKX; i += kThreads) {
            const int j = i / RKX, c = i % RKX;
            float v = 0.0f;
            if (c < rank) {
                uint64_t u = splitmix64(a.seed, (uint64_t)(j * rank + c + 1)) >> 40;
                v = (float)u * 0x1p-23f - 1.0f;
            }
            s_b0[i] = v;
        }
    }
    __syncthreads();

    uint32_t epoch = 0;   // team barriers passed
    uint32_t xchg = 0;    // (W, G) exchanges done; slots alternate by its parity
    int iter_m = 0;
    for (int64_t mm = team; mm < o.M; mm += a.num_teams, ++iter_m) {
        const int row0 = member * ROWS_WG;
        const uint16_t* xm = mm < a.m_split ? a.x + (size_t)mm * rows * D
                                             : a.x2 + (size_t)(mm - a.m_split) * rows * D;

        // ---- load this workgroup's rows (each lane: 8 columns x RPL rows)
        uint4 xr[RPL];
        bool valid[RPL];
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const int row = row0 + wv * ROWS_WAVE + s * RPS + rl;
            valid[s] = row < rows;
            xr[s] = valid[s] ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
        }

        // ---- outlier threshold (two-level radix select on |x| bit patterns)
        uint32_t tkey = 0x8000u;   // above every finite key: nothing selected
        uint32_t take_me = 0, eq_me = 0, csr_me = 0;
        if (kk > 0) {
            for (int i = tid; i < 1024; i += kThreads) s_hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                if (!valid[s]) continue;
                const uint32_t w4[4] = {xr[s].x, xr[s].y, xr[s].z, xr[s].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t key = (w4[e >> 1] >> (16 * (e & 1))) & 0x7fffu;
                    atomicAdd(&s_hist[key >> 5], 1u);
                }
            }
            __syncthreads();
            if (T > 1) {
                uint32_t* th = thist + (iter_m & 1) * 1024;
                for (int i = tid; i < 1024; i += kThreads) {
                    const uint32_t v = s_hist[i];
                    if (v) __hip_atomic_fetch_add(th + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                team_barrier(ctr, ++epoch * (uint32_t)T, a.err);
                for (int i = tid; i < 1024; i += kThreads) s_hist[i] = th[i];
                __syncthreads();
            }
            // coarse bin b*: the bin holding the k-th largest key
            {
                const int b0 = (255 - tid) * 4;
                const uint32_t h0 = s_hist[b0], h1 = s_hist[b0 + 1], h2 = s_hist[b0 + 2],
                               h3 = s_hist[b0 + 3];
                uint32_t tot;
                uint32_t cum = block_excl_scan(h0 + h1 + h2 + h3, s_tmp, &tot);
                const uint32_t hh[4] = {h3, h2, h1, h0};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (cum < kk && cum + hh[q] >= kk) {
                        s_sel[0] = (uint32_t)(b0 + 3 - q);
                        s_sel[1] = cum;
                    }
                    cum += hh[q];
                }
            }
            if (tid < 32) s_rows[tid] = 0u;
            if (tid == 32) s_rows[32] = 0u;
            __syncthreads();
            const uint32_t bstar = s_sel[0];
            uint32_t my_above = 0;
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                if (!valid[s]) continue;
                const uint32_t w4[4] = {xr[s].x, xr[s].y, xr[s].z, xr[s].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t key = (w4[e >> 1] >> (16 * (e & 1))) & 0x7fffu;
                    const uint32_t kb = key >> 5;
                    if (kb == bstar) atomicAdd(&s_rows[key & 31u], 1u);
                    my_above += (kb > bstar) ? 1u : 0u;
                }
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) my_above += __shfl_xor(my_above, off, 64);
            if (lane == 0) atomicAdd(&s_rows[32], my_above);
            __syncthreads();
            if (T > 1) {
                uint32_t* fs = tfine + member * 64;
                if (tid < 33) fs[tid] = s_rows[tid];
                team_barrier(ctr, ++epoch * (uint32_t)T, a.err);
                for (int i = tid; i < T * 33; i += kThreads)
                    s_fine[i] = tfine[(i / 33) * 64 + (i % 33)];
                if (member == 0) {
                    uint32_t* th = thist + (iter_m & 1) * 1024;
                    for (int i = tid; i < 1024; i += kThreads)
                        __hip_atomic_store(th + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
                if (tid < 33) s_fine[tid] = s_rows[tid];
            }
            __syncthreads();
            // fine bin f* and the tie quota of each workgroup (wave 0)
            if (wv == 0) {
                // totals over the team, one fine bin per lane (lanes 0..31)
                uint32_t F = 0, above = 0;
                for (int w = 0; w < T; ++w) {
                    if (lane < 32) F += s_fine[w * 33 + lane];
                    above += s_fine[w * 33 + 32];
                }
                const uint32_t needk = kk - above;   // >= 1 by the choice of b*
                // suffix sums over fine bins: lane f gets sum_{f' > f} F[f']
                uint32_t suf = (lane < 32) ? F : 0u;
#pragma unroll
                for (int off = 1; off < 32; off <<= 1) {
                    uint32_t y = __shfl_down(suf, off, 64);
                    if (lane + off < 32) suf += y;
                }
                const uint32_t strictly_above = suf - ((lane < 32) ? F : 0u);
                const bool is_f = lane < 32 && strictly_above < needk && suf >= needk;
                const uint64_t bal = __ballot(is_f);
                const int fstar = bal ? (int)__builtin_ctzll(bal) : 0;
                const uint32_t gt_fine = __shfl(strictly_above, fstar, 64);
                const uint32_t need = needk - gt_fine;   // ties to take, >= 1
                // per workgroup (lane w < T): gt_w, eq_w, then prefixes
                uint32_t eq_w = 0, gt_w = 0;
                if (lane < T) {
                    eq_w = s_fine[lane * 33 + fstar];
                    gt_w = s_fine[lane * 33 + 32];
                    for (int f = fstar + 1; f < 32; ++f) gt_w += s_fine[lane * 33 + f];
                }
                uint32_t ties_before = eq_w;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    uint32_t y = __shfl_up(ties_before, off, 64);
                    if (lane >= off) ties_before += y;
                }
                ties_before -= eq_w;
                const uint32_t take_w = (need > ties_before) ? min(eq_w, need - ties_before) : 0u;
                uint32_t before = gt_w + take_w;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    uint32_t y = __shfl_up(before, off, 64);
                    if (lane >= off) before += y;
                }
                before -= gt_w + take_w;
                if (lane == member) {
                    s_sel[2] = (bstar << 5) | (uint32_t)fstar;
                    s_sel[3] = take_w;
                    s_sel[4] = eq_w;
                    s_sel[5] = before;
                }
            }
            __syncthreads();
            tkey = s_sel[2];
            take_me = s_sel[3];
            eq_me = s_sel[4];
            csr_me = s_sel[5];
        }

        // ---- outlier masks (8 bits per lane and row)
        uint32_t om[RPL];
        uint32_t eqm[RPL];
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            om[s] = 0u;
            eqm[s] = 0u;
            if (!valid[s]) continue;
            const uint32_t w4[4] = {xr[s].x, xr[s].y, xr[s].z, xr[s].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t key = (w4[e >> 1] >> (16 * (e & 1))) & 0x7fffu;
                om[s] |= (key > tkey) ? (1u << e) : 0u;
                eqm[s] |= (key == tkey) ? (1u << e) : 0u;
            }
        }
        if (take_me == eq_me) {
#pragma unroll
            for (int s = 0; s < RPL; ++s) om[s] |= eqm[s];
        } else if (take_me > 0) {
            // rare: the cut falls inside this workgroup's ties -- rank them in
            // flat (row-major) order and take the first take_me
            uint32_t rc[RPL], rb[RPL], lp[RPL];
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const uint32_t c = __builtin_popcount(eqm[s]);
                lp[s] = row_excl_scan<LPR>(c, colq);
                rc[s] = row_sum_u32<LPR>(c);
            }
            rows_excl_scan<RPL, RPS>(rc, rb, s_rows, s_tmp, wv, rl, colq);
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                uint32_t r0 = rb[s] + lp[s];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((eqm[s] >> e) & 1u) {
                        if (r0 < take_me) om[s] |= 1u << e;
                        ++r0;
                    }
                }
            }
        }

        // ---- CSR of S: row_ptr, then (col, val) of every outlier
        int32_t* rp = o.row_ptr + (size_t)mm * (rows + 1);
        if (kk > 0) {
            uint32_t rc[RPL], rb[RPL], lp[RPL];
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const uint32_t c = __builtin_popcount(om[s]);
                lp[s] = row_excl_scan<LPR>(c, colq);
                rc[s] = row_sum_u32<LPR>(c);
            }
            rows_excl_scan<RPL, RPS>(rc, rb, s_rows, s_tmp, wv, rl, colq);
            uint16_t* cm = o.col + (size_t)mm * kk;
            uint16_t* vm = o.val + (size_t)mm * kk;
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                if (!valid[s]) continue;
                const int row = row0 + wv * ROWS_WAVE + s * RPS + rl;
                const uint32_t gpos = csr_me + rb[s];
                if (colq == 0) rp[row] = (int32_t)gpos;
                if (om[s]) {
                    uint32_t pos = gpos + lp[s];
                    const uint32_t w4[4] = {xr[s].x, xr[s].y, xr[s].z, xr[s].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (((om[s] >> e) & 1u) && pos < kk) {
                            cm[pos] = (uint16_t)(colq * 8 + e);
                            vm[pos] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                            ++pos;
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = row0 + wv * ROWS_WAVE + s * RPS + rl;
                if (valid[s] && colq == 0) rp[row] = 0;
            }
        }
        if (member == 0 && tid == 0) rp[rows] = (int32_t)kk;

        // ---- group quantization of D = X - S; residual R kept in registers
        float R[RPL][8];
        const int ngr = D / group;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const uint32_t w4[4] = {xr[s].x, xr[s].y, xr[s].z, xr[s].w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = ((om[s] >> e) & 1u) ? 0.0f : h2f(w4[e >> 1] >> (16 * (e & 1)));
            float mn = v[0], mx = v[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) {
                mn = fminf(mn, v[e]);
                mx = fmaxf(mx, v[e]);
            }
            for (int off = 1; off < gl; off <<= 1) {
                mn = fminf(mn, __shfl_xor(mn, off, 64));
                mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            }
            const float sc = (mx - mn) / qmax;
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = v[e] - mn;
                uint32_t c = 0;
                if (sc != 0.0f) {
                    const float q = rintf(t / sc);
                    c = (uint32_t)fminf(fmaxf(q, 0.0f), qmax);
                }
                word |= c << (e * bits);
                R[s][e] = valid[s] ? fmaf(-(float)c, sc, t) : 0.0f;
            }
            if (valid[s]) {
                const size_t grow = (size_t)mm * rows + row0 + wv * ROWS_WAVE + s * RPS + rl;
                if (bits == 4)
                    reinterpret_cast<uint32_t*>(o.codes)[grow * (D / 8) + colq] = word;
                else
                    reinterpret_cast<uint16_t*>(o.codes)[grow * (D / 8) + colq] = (uint16_t)word;
                if ((colq % gl) == 0) {
                    o.scale[grow * ngr + colq / gl] = sc;
                    o.zero[grow * ngr + colq / gl] = mn;
                }
            }
        }

        // ---- low-rank fit: t power steps, one pass over R each
        if (RK > 0 && rank > 0) {
            float Bm[8][RKX];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int c = 0; c < RKX; ++c) Bm[e][c] = s_b0[(colq * 8 + e) * RKX + c];
            for (int it = 0; it < a.iters; ++it) {
                float W[8][RKX];
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int c = 0; c < RKX; ++c) W[e][c] = 0.0f;
#pragma unroll
                for (int s = 0; s < RPL; ++s) {
                    float p[RKX];
#pragma unroll
                    for (int c = 0; c < RKX; ++c) {
                        float acc = 0.0f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc = fmaf(R[s][e], Bm[e][c], acc);
                        p[c] = acc;
                    }
#pragma unroll
                    for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
                        for (int c = 0; c < RKX; ++c) p[c] += __shfl_xor(p[c], off, 64);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int c = 0; c < RKX; ++c) W[e][c] = fmaf(R[s][e], p[c], W[e][c]);
                    if (colq == 0) {
                        const int lr = wv * ROWS_WAVE + s * RPS + rl;
#pragma unroll
                        for (int c = 0; c < RKX; ++c) s_p[lr * RKX + c] = p[c];
                    }
                }
                // W: reduce over the rows of the wave, then over the 4 waves
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
                        for (int c = 0; c < RKX; ++c)
                            s_w[wv * D * RKX + (colq * 8 + e) * RKX + c] = W[e][c];
                }
                __syncthreads();
                // G = P^T P in fp64 (products of fp32 values are exact in fp64):
                // thread (quarter, pair) sums one pair over a quarter of the rows
                {
                    const int q = tid & 63, quarter = tid >> 6;
                    if (q < NP) {
                        int c1 = 0, rem = q;
                        while (rem >= RKX - c1) {
                            rem -= RKX - c1;
                            ++c1;
                        }
                        const int c2 = c1 + rem;
                        double g = 0.0;
                        for (int lr = quarter; lr < ROWS_WG; lr += 4)
                            g += (double)s_p[lr * RKX + c1] * (double)s_p[lr * RKX + c2];
                        s_g[quarter * NP + q] = g;
                    }
                }
                __syncthreads();
                // this workgroup's partial (W, G); sum over the team
                float* s_wt = s_w;   // reduced W goes to wave slot 0
                double* gsum = s_g;  // reduced G goes to slot 0
                for (int i = tid; i < D * RKX; i += kThreads)
                    s_wt[i] = s_w[i] + s_w[D * RKX + i] + s_w[2 * D * RKX + i] + s_w[3 * D * RKX + i];
                if (tid < NP) gsum[tid] = s_g[tid] + s_g[NP + tid] + s_g[2 * NP + tid] + s_g[3 * NP + tid];
                __syncthreads();
                if (T > 1) {
                    const size_t par = (size_t)(xchg++ & 1u);
                    uint8_t* myslot = tslot + (par * T + member) * a.slot_bytes;
                    double* sg = reinterpret_cast<double*>(myslot);
                    float* sw = reinterpret_cast<float*>(myslot + kSlotG);
                    for (int i = tid; i < D * RKX; i += kThreads) sw[i] = s_wt[i];
                    if (tid < NP) sg[tid] = gsum[tid];
                    team_barrier(ctr, ++epoch * (uint32_t)T, a.err);
                    for (int i = tid; i < D * RKX; i += kThreads) {
                        float acc = 0.0f;
                        for (int w = 0; w < T; ++w) {
                            const uint8_t* sl = tslot + (par * T + w) * a.slot_bytes;
                            acc += reinterpret_cast<const float*>(sl + kSlotG)[i];
                        }
                        s_w[D * RKX + i] = acc;   // team W in wave slot 1
                    }
                    if (tid < NP) {
                        double acc = 0.0;
                        for (int w = 0; w < T; ++w) {
                            const uint8_t* sl = tslot + (par * T + w) * a.slot_bytes;
                            acc += reinterpret_cast<const double*>(sl)[tid];
                        }
                        s_g[NP + tid] = acc;
                    }
                } else {
                    for (int i = tid; i < D * RKX; i += kThreads) s_w[D * RKX + i] = s_wt[i];
                    if (tid < NP) s_g[NP + tid] = gsum[tid];
                }
                __syncthreads();
                if (tid == 0) {
                    int q = 0;
                    for (int c1 = 0; c1 < RKX; ++c1)
                        for (int c2 = c1; c2 < RKX; ++c2) {
                            const double v = s_g[NP + q++];
                            s_gt[c1 * RKX + c2] = v;
                            s_gt[c2 * RKX + c1] = v;
                        }
                    gram_to_m<RKX>(s_gt, s_mm, s_mm + RKX * RKX, s_mm + RKX * RKX + RKX, s_m);
                }
                __syncthreads();
                // B' = W M for this lane's 8 columns
                const float* wt = s_w + D * RKX;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float wrow[RKX];
#pragma unroll
                    for (int c = 0; c < RKX; ++c) wrow[c] = wt[(colq * 8 + e) * RKX + c];
#pragma unroll
                    for (int c = 0; c < RKX; ++c) {
                        float acc = 0.0f;
#pragma unroll
                        for (int c2 = 0; c2 < RKX; ++c2) acc = fmaf(wrow[c2], s_m[c2 * RKX + c], acc);
                        Bm[e][c] = acc;
                    }
                }
                if (it == a.iters - 1) {
                    // A = P M for this workgroup's rows; B from member 0
                    for (int lr = tid; lr < ROWS_WG; lr += kThreads) {
                        const int row = row0 + lr;
                        if (row >= rows) continue;
                        float* Ar = o.A + ((size_t)mm * rows + row) * rank;
                        for (int c = 0; c < rank; ++c) {
                            float acc = 0.0f;
#pragma unroll
                            for (int c2 = 0; c2 < RKX; ++c2) acc = fmaf(s_p[lr * RKX + c2], s_m[c2 * RKX + c], acc);
                            Ar[c] = acc;
                        }
                    }
                    if (member == 0 && wv == 0 && rl == 0) {
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
    }
}

__global__ void zero_team_headers(uint8_t* ws, size_t team_bytes, int num_teams, uint32_t* err) {
    const size_t words = kTeamZeroBytes / 4;
    const size_t total = words * (size_t)num_teams;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / words, w = i % words;
        reinterpret_cast<uint32_t*>(ws + t * team_bytes)[w] = 0u;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0u;
}

template <int D, int RPL, int RK>
hipError_t launch_one(const CompressArgs& a, hipStream_t st) {
    auto kern = compress_kernel<D, RPL, RK>;
    if (a.team == 1) {
        hipLaunchKernelGGL(kern, dim3((unsigned)a.num_teams), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    CompressArgs copy = a;
    void* args[] = {&copy};
    const unsigned grid = (unsigned)(a.num_teams * a.team);
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(grid),
                                      dim3(kThreads), args, 0, st);
}

template <int D, int RPL, int RK>
hipError_t occupancy_one(int* blocks) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks, reinterpret_cast<const void*>(compress_kernel<D, RPL, RK>), kThreads, 0);
}

template <int D, int RK>
hipError_t dispatch_rpl(const CompressShape& cs, const CompressArgs* a, hipStream_t st, int* occ) {
    switch (cs.rpl) {
        case 2: return a ? launch_one<D, 2, RK>(*a, st) : occupancy_one<D, 2, RK>(occ);
        case 4: return a ? launch_one<D, 4, RK>(*a, st) : occupancy_one<D, 4, RK>(occ);
        case 8: return a ? launch_one<D, 8, RK>(*a, st) : occupancy_one<D, 8, RK>(occ);
        default: break;
    }
    if constexpr (RK <= 4) {
        if (cs.rpl == 16) return a ? launch_one<D, 16, RK>(*a, st) : occupancy_one<D, 16, RK>(occ);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t dispatch_rk(const CompressShape& cs, const CompressArgs* a, hipStream_t st, int* occ) {
    switch (cs.rk) {
        case 0: return dispatch_rpl<D, 0>(cs, a, st, occ);
        case 2: return dispatch_rpl<D, 2>(cs, a, st, occ);
        case 4: return dispatch_rpl<D, 4>(cs, a, st, occ);
        case 8: return dispatch_rpl<D, 8>(cs, a, st, occ);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch(const CompressShape& cs, const CompressArgs* a, hipStream_t st, int* occ) {
    if (cs.d == 64) return dispatch_rk<64>(cs, a, st, occ);
    if (cs.d == 128) return dispatch_rk<128>(cs, a, st, occ);
    return hipErrorInvalidValue;
}

}  // namespace

CompressShape choose_compress_shape(int d, int rank, int rows) {
    CompressShape cs;
    cs.d = d;
    cs.rk = rank == 0 ? 0 : rank <= 2 ? 2 : rank <= 4 ? 4 : 8;
    const int max_rpl = cs.rk == 8 ? 8 : 16;
    cs.rpl = max_rpl;
    for (int r = 2; r <= max_rpl; r *= 2) {
        cs.rpl = r;
        if (cs.rows_per_wg() >= rows) break;
    }
    return cs;
}

size_t compress_team_bytes(const CompressShape& cs, int team, size_t* slot_bytes) {
    const int rkx = cs.rk > 0 ? cs.rk : 1;
    const size_t slot = align_up(kSlotG + (size_t)cs.d * rkx * 4);
    if (slot_bytes) *slot_bytes = slot;
    return align_up(kTeamZeroBytes + (size_t)team * kFineSlot + 2 * (size_t)team * slot);
}

hipError_t compress_plan(const CompressShape& cs, int team, int64_t M, int* num_teams) {
    if (team == 1) {
        *num_teams = (int)(M < (int64_t)1 << 30 ? M : (int64_t)1 << 30);
        return hipSuccess;
    }
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = dispatch(cs, nullptr, nullptr, &per_cu);
    if (e != hipSuccess) return e;
    const int resident = per_cu * cus;
    int per_xcd_teams = (resident / 8) / team;   // teams whose members share blockIdx % 8
    if (per_xcd_teams < 1) return hipErrorCooperativeLaunchTooLarge;
    int64_t teams = (int64_t)per_xcd_teams * 8;
    const int64_t need = (M + 7) / 8 * 8;
    if (teams > need) teams = need;
    *num_teams = (int)teams;
    return hipSuccess;
}

hipError_t launch_compress(const CompressShape& cs, const CompressArgs& a, hipStream_t st) {
    if (a.team > 1) {
        hipLaunchKernelGGL(zero_team_headers, dim3(64), dim3(kThreads), 0, st, a.team_ws,
                           a.team_bytes, a.num_teams, a.err);
    } else {
        hipLaunchKernelGGL(zero_team_headers, dim3(1), dim3(64), 0, st, a.team_ws,
                           a.team_bytes, 0, a.err);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return dispatch(cs, &a, st, nullptr);
}

}  // namespace gear
