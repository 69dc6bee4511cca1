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
//   * Pass 1: 1024-bin histogram of |x| >> 5 in LDS -> the coarse bin of the
//     k-th largest magnitude.  Pass 2: per-wave 32-bin histograms inside that
//     bin -> the exact threshold key, the number of ties to take, and every
//     wave's CSR start and tie quota (flat order = wave order, then row, lane).
//   * Pass 3: outlier mask, CSR emit (wave-level prefix sums), bit-exact fp32
//     group quantization (correctly rounded division, rint) with codes packed
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
    double m[RK][RK];
#pragma unroll
    for (int j = 0; j < RK; ++j) {
        const double inv = alive[j] ? 1.0 / c[j][j] : 0.0;
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            if (a > j) {
                m[a][j] = 0.0;
                continue;
            }
            double v = (a == j) ? 1.0 : 0.0;
#pragma unroll
            for (int i = 0; i < j; ++i)
                if (a <= i) v -= m[a][i] * c[i][j];
            m[a][j] = v * inv;
        }
    }
#pragma unroll
    for (int a = 0; a < RK; ++a)
#pragma unroll
        for (int j = 0; j < RK; ++j) Mout[a * RK + j] = (float)m[a][j];
}

template <int RK>
struct PairLanes {
    static constexpr int NP = RK * (RK + 1) / 2;
    // lanes per Gram pair: the largest power of two with NP * LP <= 64
    static constexpr int LP = NP <= 1 ? 64 : NP <= 2 ? 32 : NP <= 4 ? 16 : NP <= 8 ? 8
                            : NP <= 16 ? 4 : NP <= 32 ? 2 : 1;
};

template <int D, int RK, int U>
__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a) {
    constexpr int LPR = D / 8;              // lanes per token row
    constexpr int RPS = 64 / LPR;           // rows per wave per step
    constexpr int RKX = RK > 0 ? RK : 1;
    constexpr int NP = RKX * (RKX + 1) / 2;
    constexpr int LP = PairLanes<RKX>::LP;
    constexpr int RING_STEPS = kRing / RPS;

    __shared__ uint32_t s_hist[1024];
    __shared__ uint32_t s_fine[4 * 33];
    __shared__ uint32_t s_tmp[8];
    __shared__ uint32_t s_sel[4];
    __shared__ uint32_t s_wave[4 * 2];
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

    // ======================= outlier threshold ============================
    uint32_t tkey = 0x8000u;   // above every finite key: nothing selected
    uint32_t take_w = 0, csr_w = 0;
    if (kk > 0) {
        for (int i = tid; i < 1024; i += kThreads) s_hist[i] = 0u;
        if (tid < 4 * 33) s_fine[tid] = 0u;
        __syncthreads();
        // pass 1: coarse histogram
        for (int s0 = 0; s0 < steps; s0 += U) {
            uint4 xr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = wr0 + (s0 + u) * RPS + rl;
                xr[u] = (s0 + u < steps && row < rows)
                            ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = wr0 + (s0 + u) * RPS + rl;
                if (s0 + u < steps && row < rows) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) atomicAdd(&s_hist[(half_of(xr[u], e) & 0x7fffu) >> 5], 1u);
                }
            }
        }
        __syncthreads();
        {   // the coarse bin holding the k-th largest key
            const int b0 = (255 - tid) * 4;
            const uint32_t h0 = s_hist[b0], h1 = s_hist[b0 + 1], h2 = s_hist[b0 + 2],
                           h3 = s_hist[b0 + 3];
            uint32_t tot;
            uint32_t cum = block_excl_scan(h0 + h1 + h2 + h3, s_tmp, &tot);
            const uint32_t hh[4] = {h3, h2, h1, h0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cum < kk && cum + hh[q] >= kk) s_sel[0] = (uint32_t)(b0 + 3 - q);
                cum += hh[q];
            }
        }
        __syncthreads();
        const uint32_t bstar = s_sel[0];
        // pass 2: per-wave fine histograms inside the coarse bin
        uint32_t my_above = 0;
        for (int s0 = 0; s0 < steps; s0 += U) {
            uint4 xr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = wr0 + (s0 + u) * RPS + rl;
                xr[u] = (s0 + u < steps && row < rows)
                            ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = wr0 + (s0 + u) * RPS + rl;
                if (s0 + u < steps && row < rows) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t key = half_of(xr[u], e) & 0x7fffu;
                        const uint32_t kb = key >> 5;
                        if (kb == bstar) atomicAdd(&s_fine[wv * 33 + (key & 31u)], 1u);
                        my_above += (kb > bstar) ? 1u : 0u;
                    }
                }
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) my_above += __shfl_xor(my_above, off, 64);
        if (lane == 0) s_fine[wv * 33 + 32] = my_above;
        __syncthreads();
        if (wv == 0) {
            uint32_t F = 0, above = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (lane < 32) F += s_fine[w * 33 + lane];
                above += s_fine[w * 33 + 32];
            }
            const uint32_t needk = kk - above;   // >= 1 by the choice of the coarse bin
            uint32_t suf = (lane < 32) ? F : 0u;  // lane f: sum of F[f'] for f' >= f
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                const uint32_t y = __shfl_down(suf, off, 64);
                if (lane + off < 32) suf += y;
            }
            const uint32_t strictly_above = suf - ((lane < 32) ? F : 0u);
            const uint64_t bal = __ballot(lane < 32 && strictly_above < needk && suf >= needk);
            const int fstar = bal ? (int)__builtin_ctzll(bal) : 0;
            const uint32_t need = needk - __shfl(strictly_above, fstar, 64);   // ties to take
            uint32_t eq = 0, gt = 0;
            if (lane < 4) {
                eq = s_fine[lane * 33 + fstar];
                gt = s_fine[lane * 33 + 32];
                for (int f = fstar + 1; f < 32; ++f) gt += s_fine[lane * 33 + f];
            }
            uint32_t tt;
            const uint32_t ties_before = wave_excl_scan(eq, lane, &tt);
            const uint32_t take = (need > ties_before) ? min(eq, need - ties_before) : 0u;
            const uint32_t before = wave_excl_scan(gt + take, lane, &tt);
            if (lane < 4) {
                s_wave[lane * 2] = take;
                s_wave[lane * 2 + 1] = before;
            }
            if (lane == 0) s_sel[1] = (bstar << 5) | (uint32_t)fstar;
        }
        __syncthreads();
        tkey = s_sel[1];
        take_w = s_wave[wv * 2];
        csr_w = s_wave[wv * 2 + 1];
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

        for (int s0 = 0; s0 < steps; s0 += U) {
            uint4 xr[U];
            uint32_t cw[U];
            float scl[U], zpt[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = wr0 + (s0 + u) * RPS + rl;
                const bool ok = s0 + u < steps && row < rows;
                const size_t grow = (size_t)mm * rows + (ok ? row : 0);
                xr[u] = ok ? *reinterpret_cast<const uint4*>(xm + (size_t)row * D + colq * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
                cw[u] = 0u;
                scl[u] = 0.0f;
                zpt[u] = 0.0f;
                if (!first && ok) {
                    cw[u] = bits == 4 ? reinterpret_cast<const uint32_t*>(o.codes)[grow * (D / 8) + colq]
                                      : reinterpret_cast<const uint16_t*>(o.codes)[grow * (D / 8) + colq];
                    scl[u] = o.scale[grow * ngr + colq / gl];
                    zpt[u] = o.zero[grow * ngr + colq / gl];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u;
                if (s >= steps) break;   // wave-uniform
                const int row = wr0 + s * RPS + rl;
                const bool valid = row < rows;
                const size_t grow = (size_t)mm * rows + (valid ? row : 0);
                // ---- outlier mask: key > threshold, or a tie within the quota
                uint32_t om = 0u, eqm = 0u;
                if (valid) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t key = half_of(xr[u], e) & 0x7fffu;
                        om |= (key > tkey) ? (1u << e) : 0u;
                        eqm |= (key == tkey) ? (1u << e) : 0u;
                    }
                }
                if (__ballot(eqm != 0u) != 0ull && ties_seen < take_w) {
                    uint32_t tot;
                    const uint32_t c = __builtin_popcount(eqm);
                    uint32_t rank0 = ties_seen + wave_excl_scan(c, lane, &tot);
                    if (ties_seen + tot <= take_w) {
                        om |= eqm;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if ((eqm >> e) & 1u) {
                                if (rank0 < take_w) om |= 1u << e;
                                ++rank0;
                            }
                    }
                    ties_seen += tot;
                }
                // ---- CSR (first pass only)
                if (first && kk > 0) {
                    uint32_t pre = 0, tot = 0;
                    if (__ballot(om != 0u) != 0ull) pre = wave_excl_scan(__builtin_popcount(om), lane, &tot);
                    if (valid && colq == 0) rp[row] = (int32_t)(csr + pre);
                    if (om) {
                        uint32_t pos = csr + pre;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (((om >> e) & 1u) && pos < kk) {
                                cm[pos] = (uint16_t)(colq * 8 + e);
                                vm[pos] = (uint16_t)half_of(xr[u], e);
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
                for (int e = 0; e < 8; ++e) v[e] = ((om >> e) & 1u) ? 0.0f : h2f(half_of(xr[u], e));
                float R[8];
                if (first) {
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
                        if (sc != 0.0f) c = (uint32_t)fminf(fmaxf(rintf(t / sc), 0.0f), qmax);
                        word |= c << (e * bits);
                        R[e] = valid ? fmaf(-(float)c, sc, t) : 0.0f;
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
                        const float t = v[e] - zpt[u];
                        const float c = (float)((cw[u] >> (e * bits)) & cmask);
                        R[e] = valid ? fmaf(-c, scl[u], t) : 0.0f;
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
                    p[c] = acc;
                }
#pragma unroll
                for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
                    for (int c = 0; c < RKX; ++c) p[c] += __shfl_xor(p[c], off, 64);
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
    constexpr int U = RK >= 8 ? 4 : 8;
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
