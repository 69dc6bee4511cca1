// gear_attn.hip -- decode-time reads of the compressed cache.
//
// Decode attention of one query token per sequence straight from the packed
// segments ("GEAR: Efficient KV Cache Compression for LLM Inference", Q4: the
// compressed cache cuts the memory traffic of decoding; Q3 "Streaming
// strategy": recent tokens sit in an fp16 buffer until it fills).  K^ and V^
// are never materialised:
//   q . K^_t = scale_t (q . codes_t) + zero_t (sum of q over the group)
//              + A_t . (B^T q) + sum over token t's outliers of q_j s_tj
//   sum_t p_t V^_t = sum_t p_t (codes_t scale_t + zero_t)
//              + B (sum_t p_t A_t) + sum of p_t s_tj scattered to column j
// One workgroup per (batch, kv-head, 256-token split) serves every query head
// of the GQA group (dequantisation is shared); an exact softmax inside the
// split (scores staged in LDS) and a log-sum-exp merge across splits.
#include <math.h>

#include "gear_internal.h"

namespace gear {
namespace {

constexpr int kTPS = 256;   // tokens per split

__device__ __forceinline__ float h2f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ Packed shifted(const Packed& p, size_t off) {
    Packed q = p;
    q.codes += off;
    q.scale = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(q.scale) + off);
    q.zero = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(q.zero) + off);
    q.row_ptr = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(q.row_ptr) + off);
    q.col = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(q.col) + off);
    q.val = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(q.val) + off);
    q.A = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(q.A) + off);
    q.B = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(q.B) + off);
    return q;
}

// The run of tokens [t, t + len) of one segment matrix, as seen from token t.
struct Piece {
    int kind;          // 0: compressed, 1: fp16 buffer
    Packed p;          // compressed: packed buffer (shifted for fills)
    int64_t mk, mv;    // compressed matrix index of K and of V
    int row0;          // first row inside the matrix (or buffer)
    int len;
};

__device__ Piece find_piece(const AttnArgs& a, int b, int hk, int t, int t_end) {
    Piece pc;
    const int pt = a.prompt.count ? a.prompt.chunks * a.prompt.p.rows : 0;
    const int ft = a.fills.count * a.fills.p.rows;
    if (t < pt) {
        const int rows = a.prompt.p.rows, C = a.prompt.chunks;
        const int chunk = t / rows;
        pc.kind = 0;
        pc.p = a.prompt.p;
        pc.mk = ((int64_t)(0 * a.B + b) * a.Hkv + hk) * C + chunk;
        pc.mv = ((int64_t)(1 * a.B + b) * a.Hkv + hk) * C + chunk;
        pc.row0 = t - chunk * rows;
        pc.len = min(rows - pc.row0, t_end - t);
    } else if (t < pt + ft) {
        const int rows = a.fills.p.rows;
        const int f = (t - pt) / rows;
        pc.kind = 0;
        pc.p = shifted(a.fills.p, (size_t)f * a.fills.stride);
        pc.mk = (int64_t)(0 * a.B + b) * a.Hkv + hk;
        pc.mv = (int64_t)(1 * a.B + b) * a.Hkv + hk;
        pc.row0 = t - pt - f * rows;
        pc.len = min(rows - pc.row0, t_end - t);
    } else {
        pc.kind = 1;
        pc.p = a.prompt.p;
        pc.mk = pc.mv = 0;
        pc.row0 = t - pt - ft;
        pc.len = t_end - t;
    }
    return pc;
}

// Sum over each aligned group of N lanes (N = 8 or 16) with DPP: pairs,
// quads, the mirrored quad, the mirrored half-row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float row_allreduce(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    if (N >= 16) v += dpp<0x140>(v);
    return v;
}

__device__ __forceinline__ float max_xor16(float v) {
    float a, b;
    swap_pair<false>(v, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float v) {
    float a, b;
    swap_pair<true>(v, a, b);
    return fmaxf(a, b);
}
// sum and max over the 64 lanes of the wave, result in every lane
__device__ __forceinline__ float wave_sum(float v) {
    return sum_xor32(sum_xor16(row_allreduce<16>(v)));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return max_xor32(max_xor16(v));
}
// sum over the lanes of the wave with the same lane % LPR (LPR = 8 or 16)
template <int LPR>
__device__ __forceinline__ float sum_rowgroups(float v) {
    if (LPR == 8) v += dpp<0x128>(v);   // row_ror:8 = lane ^ 8 within the row
    return sum_xor32(sum_xor16(v));
}

constexpr int kAttnCsrCap = 2048;   // outliers of one piece staged in LDS
constexpr int kAU = 4;              // token steps per batch of loads

// out[b][hq][:] = merge over the pair's splits of (acc, max, sum), by the
// kThreads threads of a workgroup; the splits are shared out over
// kThreads / D threads per column.  s_m: kThreads / 64 floats, s_num and s_den:
// kThreads floats each (LDS).
template <int D, int G>
__device__ __forceinline__ void merge_head(const AttnArgs& a, int pair, int bh, int h, float* s_m,
                                           float* s_num, float* s_den) {
    constexpr int NQ = kThreads / D;
    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const float* base = a.partial + ((size_t)pair * a.splits * G + h) * (D + 2);
    const size_t stride = (size_t)G * (D + 2);   // between splits
    float m = -INFINITY;
    for (int s = tid; s < a.splits; s += kThreads) {
        const float* part = base + s * stride;
        if (part[D + 1] > 0.0f) m = fmaxf(m, part[D]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) s_m[wv] = m;
    __syncthreads();
    m = s_m[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, s_m[w]);
    const int j = tid % D, q = tid / D;
    float num = 0.0f, den = 0.0f;
    for (int s = q; s < a.splits; s += NQ) {
        const float* part = base + s * stride;
        const float l = part[D + 1];
        if (l > 0.0f) {
            const float w = expf(part[D] - m);
            num = fmaf(w, part[j], num);
            den = fmaf(w, l, den);
        }
    }
    s_num[tid] = num;
    s_den[tid] = den;
    __syncthreads();
    if (q == 0) {
        for (int qq = 1; qq < NQ; ++qq) {
            num += s_num[qq * D + j];
            den += s_den[qq * D + j];
        }
        a.out[(size_t)bh * D + j] = den > 0.0f ? num / den : 0.0f;
    }
}

// One workgroup per (batch, kv-head, split of kTPS tokens).  Each token of a
// compressed piece is read once per phase: 8 codes per lane (D/8 lanes per
// token), the group's scale and zero, the token's A row; the piece's CSR rows
// are staged in LDS first so that the sparse terms need no dependent global
// loads.  Phase 1 writes raw scores to LDS and adds the sparse term per row
// (one thread per token, entries in CSR order); phase 2 folds each token's
// sparse V entries into its dequantised values through a small per-wave LDS
// tile that is scattered, read and cleared again.  When a pair has only one
// split here (fuse_combine), its workgroup then merges all of the pair's
// splits into out itself (no separate combine launch).
template <int D, int G>
__global__ void __launch_bounds__(kThreads) attn_split_kernel(AttnArgs a) {
    constexpr int LPR = D / 8, RPS = 64 / LPR, TILE = 4 * RPS;
    __shared__ float s_q[G * D];
    __shared__ float s_sc[kTPS * G];
    __shared__ float s_qb[G * kMaxRank];
    __shared__ float s_red[4 * G * D];
    __shared__ float s_stat[2 * G];
    __shared__ int32_t s_rp[kTPS + 1];
    __shared__ uint32_t s_cv[kAttnCsrCap];
    __shared__ __attribute__((aligned(16))) float s_tile[4 * RPS * D];
    __shared__ float s_pa[4 * G * kMaxRank];
    __shared__ float s_mg[kThreads / 64 + 2 * kThreads];   // merge scratch (fuse_combine)

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const int nsp = a.splits - a.split0;   // splits [split0, splits) of every (b, kv-head)
    const int pair = (int)(group_id_x() / nsp), split = a.split0 + (int)(group_id_x() % nsp);
    const int b = pair / a.Hkv, hk = pair % a.Hkv;
    const int pt = a.prompt.count ? a.prompt.chunks * a.prompt.p.rows : 0;
    const int N = pt + a.fills.count * a.fills.p.rows + a.buf_len;
    const int t0 = split * a.tokens_per_split;
    const int t1 = min(N, t0 + a.tokens_per_split);

    for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, j = i % D;
        s_q[i] = h2f(a.q[((size_t)b * a.Hq + hk * G + h) * D + j]);
    }
    for (int i = tid; i < 4 * RPS * D; i += kThreads) s_tile[i] = 0.0f;
    __syncthreads();
    float q[G][8], qs[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        qs[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            q[h][e] = s_q[h * D + colq * 8 + e];
            qs[h] += q[h][e];
        }
    }

    // CSR rows [row0, row0 + len) of matrix m of p into s_rp / s_cv; an entry
    // is packed as column (bits 0-6) | row in the piece (bits 7-15) | fp16
    // value (bits 16-31).
    int csr_beg = 0, csr_cnt = 0;
    bool csr_staged = true;
    auto stage_csr = [&](const Packed& p, int64_t m, int row0, int len) {
        __syncthreads();
        const int32_t* rp = p.row_ptr + (size_t)m * (p.rows + 1) + row0;
        for (int i = tid; i <= len; i += kThreads) s_rp[i] = min(max(rp[i], 0), p.k);
        __syncthreads();
        csr_beg = __builtin_amdgcn_readfirstlane(s_rp[0]);
        csr_cnt = max(__builtin_amdgcn_readfirstlane(s_rp[len]) - csr_beg, 0);
        csr_staged = csr_cnt <= kAttnCsrCap;
        if (csr_staged) {
            const uint16_t* cm = p.col + (size_t)m * p.k;
            const uint16_t* vm = p.val + (size_t)m * p.k;
            for (int i = tid; i < len; i += kThreads)
                for (int k = s_rp[i]; k < s_rp[i + 1]; ++k)
                    s_cv[k - csr_beg] = ((uint32_t)cm[k] & (D - 1)) | ((uint32_t)i << 7) |
                                        ((uint32_t)vm[k] << 16);
        }
    };
    // entry k (absolute index) of row `row` of the piece
    auto csr_entry = [&](const Packed& p, int64_t m, int k, int row) -> uint32_t {
        if (csr_staged) return s_cv[k - csr_beg];
        return ((uint32_t)p.col[(size_t)m * p.k + k] & (D - 1)) | ((uint32_t)row << 7) |
               ((uint32_t)p.val[(size_t)m * p.k + k] << 16);
    };

    // ---------------- phase 1: raw scores q . K^_t of the split's tokens
    for (int t = t0; t < t1;) {
        const Piece pc = find_piece(a, b, hk, t, t1);
        const int base = t - t0;
        if (pc.kind == 0) {
            const Packed& p = pc.p;
            const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
            const uint32_t cmask = (1u << bits) - 1u;
            stage_csr(p, pc.mk, pc.row0, pc.len);
            if (r > 0 && wv == 0) {
                // B^T q: one token row of lanes spans all D columns
                for (int c = 0; c < r; ++c) {
                    float part[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = 0.0f;
                    if (rl == 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float bv = p.B[((size_t)pc.mk * D + colq * 8 + e) * r + c];
#pragma unroll
                            for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], bv, part[h]);
                        }
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float v = row_allreduce<LPR>(part[h]);
                        if (lane == 0) s_qb[h * kMaxRank + c] = v;
                    }
                }
            }
            __syncthreads();
            float qbl[G];   // (B^T q)[colq] for colq < r
#pragma unroll
            for (int h = 0; h < G; ++h) qbl[h] = colq < r ? s_qb[h * kMaxRank + colq] : 0.0f;
            const size_t mrow = (size_t)pc.mk * p.rows + pc.row0;
            const int steps = (pc.len + TILE - 1) / TILE;
            uint32_t word[1][kAU];
            float sc[1][kAU], zp[1][kAU], av[1][kAU];   // av: A[t][colq] for colq < r
            // per-piece bases (uniform); lanes use 32-bit offsets and a clamped
            // token (always a valid address), then zero what lies past the piece
            const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
            const float* sbase = p.scale + mrow * ngr;
            const float* zbase = p.zero + mrow * ngr;
            const float* abase = p.A + mrow * r;
            const int acol = min(colq, max(r - 1, 0));
            auto load = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    const bool ok = tok < pc.len;
                    const uint32_t tk = (uint32_t)min(tok, pc.len - 1);
                    const uint32_t w = bits == 4
                        ? ld_at<uint32_t>(cbase, tk * (D / 2) + colq * 4)
                        : (uint32_t)ld_at<uint16_t>(cbase, tk * (D / 4) + colq * 2);
                    const uint32_t go = (tk * ngr + colq / gl) * 4;
                    const float scv = ld_at<float>(sbase, go);
                    const float zpv = ld_at<float>(zbase, go);
                    const float a1 = r > 0 ? ld_at<float>(abase, (tk * r + acol) * 4) : 0.0f;
                    word[bf][u] = ok ? w : 0u;
                    sc[bf][u] = ok ? scv : 0.0f;
                    zp[bf][u] = ok ? zpv : 0.0f;
                    av[bf][u] = (ok && colq < r) ? a1 : 0.0f;
                }
            };
            auto compute = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    float part[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float cf = (float)((word[bf][u] >> (e * bits)) & cmask);
#pragma unroll
                        for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], cf, part[h]);
                    }
                    // + A[t][colq] (B^T q)[colq] in the lanes colq < r, then the row sum
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        part[h] = row_allreduce<LPR>(
                            fmaf(av[bf][u], qbl[h], fmaf(sc[bf][u], part[h], zp[bf][u] * qs[h])));
                    if (tok < pc.len && colq == 0) {
#pragma unroll
                        for (int h = 0; h < G; ++h) s_sc[(base + tok) * G + h] = part[h];
                    }
                }
            };
            for (int s0 = 0; s0 < steps; s0 += kAU) {
                load(0, s0);
                compute(0, s0);
            }
            __syncthreads();
            // sparse term, one thread per token, entries in CSR order
            for (int i = tid; i < pc.len; i += kThreads) {
                float add[G];
#pragma unroll
                for (int h = 0; h < G; ++h) add[h] = 0.0f;
                for (int k = s_rp[i]; k < s_rp[i + 1]; ++k) {
                    const uint32_t cv = csr_entry(p, pc.mk, k, i);
                    const int cj = (int)(cv & (D - 1));
                    const float v = h2f(cv >> 16);
#pragma unroll
                    for (int h = 0; h < G; ++h) add[h] = fmaf(s_q[h * D + cj], v, add[h]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) s_sc[(base + i) * G + h] += add[h];
            }
        } else {
            const uint16_t* kb = a.buf + (((size_t)(0 * a.B + b) * a.Hkv + hk) * a.buf_cap) * D;
            for (int tt = 0; tt < pc.len; tt += TILE) {
                const int tok = tt + wv * RPS + rl;
                const bool valid = tok < pc.len;
                float part[G];
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = 0.0f;
                if (valid) {
                    const uint4 w = *reinterpret_cast<const uint4*>(kb + (size_t)(pc.row0 + tok) * D + colq * 8);
                    const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float kv = h2f(w4[e >> 1] >> (16 * (e & 1)));
#pragma unroll
                        for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], kv, part[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = row_allreduce<LPR>(part[h]);
                if (valid && colq == 0) {
#pragma unroll
                    for (int h = 0; h < G; ++h) s_sc[(base + tok) * G + h] = part[h];
                }
            }
        }
        t += pc.len;
    }
    __syncthreads();

    // ---------------- softmax inside the split (scores scaled here)
    const int n = max(t1 - t0, 0);
    {
        float mx[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = -INFINITY;
        for (int i = tid; i < n; i += kThreads)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float v = a.sm_scale * s_sc[i * G + h];
                s_sc[i * G + h] = v;
                mx[h] = fmaxf(mx[h], v);
            }
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) mx[h] = fmaxf(mx[h], __shfl_xor(mx[h], off, 64));
            if (lane == 0) s_red[wv * G + h] = mx[h];
        }
        __syncthreads();
        if (tid < G) {
            float m = s_red[tid];
            for (int w = 1; w < 4; ++w) m = fmaxf(m, s_red[w * G + tid]);
            s_stat[tid] = m;
        }
        __syncthreads();
        float sm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sm[h] = 0.0f;
        for (int i = tid; i < n; i += kThreads)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pv = expf(s_sc[i * G + h] - s_stat[h]);
                s_sc[i * G + h] = pv;
                sm[h] += pv;
            }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) sm[h] += __shfl_xor(sm[h], off, 64);
            if (lane == 0) s_red[wv * G + h] = sm[h];
        }
        __syncthreads();
        if (tid < G) s_stat[G + tid] = s_red[tid] + s_red[G + tid] + s_red[2 * G + tid] + s_red[3 * G + tid];
        __syncthreads();
    }

    // ---------------- phase 2: probability-weighted sum of V^
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    float* tile = s_tile + wv * RPS * D;
    for (int t = t0; t < t1;) {
        const Piece pc = find_piece(a, b, hk, t, t1);
        const int base = t - t0;
        if (pc.kind == 0) {
            const Packed& p = pc.p;
            const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
            const uint32_t cmask = (1u << bits) - 1u;
            stage_csr(p, pc.mv, pc.row0, pc.len);
            __syncthreads();
            float pa[G];   // sum_t p_t A[t][colq] in the lanes colq < r
#pragma unroll
            for (int h = 0; h < G; ++h) pa[h] = 0.0f;
            const size_t mrow = (size_t)pc.mv * p.rows + pc.row0;
            const int steps = (pc.len + TILE - 1) / TILE;
            uint32_t word[1][kAU];
            float sc[1][kAU], zp[1][kAU], av[1][kAU];
            // per-piece bases (uniform); lanes use 32-bit offsets and a clamped
            // token (always a valid address), then zero what lies past the piece
            const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
            const float* sbase = p.scale + mrow * ngr;
            const float* zbase = p.zero + mrow * ngr;
            const float* abase = p.A + mrow * r;
            const int acol = min(colq, max(r - 1, 0));
            auto load = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    const bool ok = tok < pc.len;
                    const uint32_t tk = (uint32_t)min(tok, pc.len - 1);
                    const uint32_t w = bits == 4
                        ? ld_at<uint32_t>(cbase, tk * (D / 2) + colq * 4)
                        : (uint32_t)ld_at<uint16_t>(cbase, tk * (D / 4) + colq * 2);
                    const uint32_t go = (tk * ngr + colq / gl) * 4;
                    const float scv = ld_at<float>(sbase, go);
                    const float zpv = ld_at<float>(zbase, go);
                    const float a1 = r > 0 ? ld_at<float>(abase, (tk * r + acol) * 4) : 0.0f;
                    word[bf][u] = ok ? w : 0u;
                    sc[bf][u] = ok ? scv : 0.0f;
                    zp[bf][u] = ok ? zpv : 0.0f;
                    av[bf][u] = (ok && colq < r) ? a1 : 0.0f;
                }
            };
            auto compute = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int first = (s0 + u) * TILE + wv * RPS;   // this wave's first token
                    const int tok = first + rl;
                    const bool ok = tok < pc.len;
                    // scatter the sparse entries of the wave's RPS tokens into its
                    // tile, read this lane's 8 values, clear the cells again (LDS
                    // operations of one wave execute in order)
                    const int last = min(first + RPS, pc.len);
                    const int e0 = first < pc.len ? s_rp[first] : 0;
                    const int e1 = first < pc.len ? s_rp[last] : 0;
                    for (int k = e0 + lane; k < e1; k += 64) {
                        int rr = 0;
                        if (!csr_staged)
                            while (rr + 1 < RPS && first + rr + 1 <= last && k >= s_rp[first + rr + 1]) ++rr;
                        const uint32_t cv = csr_entry(p, pc.mv, k, first + rr);
                        tile[(((cv >> 7) & 0x1ffu) - first) * D + (cv & (D - 1))] = h2f(cv >> 16);
                    }
                    __builtin_amdgcn_wave_barrier();
                    const float4 s0v = *reinterpret_cast<const float4*>(tile + rl * D + colq * 8);
                    const float4 s1v = *reinterpret_cast<const float4*>(tile + rl * D + colq * 8 + 4);
                    const float sv[8] = {s0v.x, s0v.y, s0v.z, s0v.w, s1v.x, s1v.y, s1v.z, s1v.w};
                    __builtin_amdgcn_wave_barrier();
                    for (int k = e0 + lane; k < e1; k += 64) {
                        int rr = 0;
                        if (!csr_staged)
                            while (rr + 1 < RPS && first + rr + 1 <= last && k >= s_rp[first + rr + 1]) ++rr;
                        const uint32_t cv = csr_entry(p, pc.mv, k, first + rr);
                        tile[(((cv >> 7) & 0x1ffu) - first) * D + (cv & (D - 1))] = 0.0f;
                    }
                    float pr[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) pr[h] = ok ? s_sc[(base + tok) * G + h] : 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dv = fmaf((float)((word[bf][u] >> (e * bits)) & cmask), sc[bf][u], zp[bf][u]) + sv[e];
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], dv, acc[h][e]);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) pa[h] = fmaf(pr[h], av[bf][u], pa[h]);
                }
            };
            for (int s0 = 0; s0 < steps; s0 += kAU) {
                load(0, s0);
                compute(0, s0);
            }
            // low-rank part of this matrix: acc += B (sum_t p_t A_t), with the
            // sums over the piece's tokens gathered per rank column c = colq
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
                for (int h = 0; h < G; ++h) pa[h] += __shfl_xor(pa[h], off, 64);
            if (rl == 0 && colq < r) {
#pragma unroll
                for (int h = 0; h < G; ++h) s_pa[(wv * G + h) * kMaxRank + colq] = pa[h];
            }
            __syncthreads();
            // the totals are workgroup-wide: one row group adds them
            for (int c = 0; c < (wv == 0 && rl == 0 ? r : 0); ++c) {
                float tot[G];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    tot[h] = s_pa[(0 * G + h) * kMaxRank + c] + s_pa[(1 * G + h) * kMaxRank + c] +
                             s_pa[(2 * G + h) * kMaxRank + c] + s_pa[(3 * G + h) * kMaxRank + c];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float bv = p.B[((size_t)pc.mv * D + colq * 8 + e) * r + c];
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h][e] = fmaf(tot[h], bv, acc[h][e]);
                }
            }
        } else {
            const uint16_t* vb = a.buf + (((size_t)(1 * a.B + b) * a.Hkv + hk) * a.buf_cap) * D;
            for (int tt = 0; tt < pc.len; tt += TILE) {
                const int tok = tt + wv * RPS + rl;
                if (tok >= pc.len) continue;
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pr[h] = s_sc[(base + tok) * G + h];
                const uint4 w = *reinterpret_cast<const uint4*>(vb + (size_t)(pc.row0 + tok) * D + colq * 8);
                const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float vv = h2f(w4[e >> 1] >> (16 * (e & 1)));
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], vv, acc[h][e]);
                }
            }
        }
        t += pc.len;
    }
    // reduce over the row groups of the wave, then over the waves
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
    __syncthreads();
    if (rl == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_red[(wv * G + h) * D + colq * 8 + e] = acc[h][e];
    }
    __syncthreads();
    float* part = a.partial + ((size_t)pair * a.splits + split) * G * (D + 2);
    for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, j = i % D;
        part[h * (D + 2) + j] = s_red[(0 * G + h) * D + j] + s_red[(1 * G + h) * D + j] +
                                s_red[(2 * G + h) * D + j] + s_red[(3 * G + h) * D + j];
    }
    if (tid < G) {
        part[tid * (D + 2) + D] = n > 0 ? s_stat[tid] : -INFINITY;
        part[tid * (D + 2) + D + 1] = n > 0 ? s_stat[G + tid] : 0.0f;
    }
    if (a.fuse_combine) {
        // the pair's only split here: every other split was written by the
        // prompt kernel, launched before on the same stream, and this one's
        // by this workgroup (visible to it after the barrier)
        __syncthreads();
        float* s_m = s_mg;
        float* s_num = s_mg + kThreads / 64;
        float* s_den = s_num + kThreads;
#pragma unroll 1
        for (int h = 0; h < G; ++h) {
            merge_head<D, G>(a, pair, b * a.Hq + hk * G + h, h, s_m, s_num, s_den);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Whole prompt splits: kTPS tokens inside one compressed K matrix and its V
// matrix, at most kFastGroups quantization groups per token.  The same sums
// as attn_split_kernel, organised around a few rounds of loads so that a
// workgroup waits on memory a few times instead of once per batch of tokens:
//   1. q, the K codes (registers), K's scales, zeros and A rows, both
//      matrices' row pointers and both B matrices (LDS);
//   2. issued before the K scores are computed and consumed after: both
//      matrices' CSR entries (a contiguous range, loaded coalesced); V's
//      codes, scales, zeros and A rows are issued after the K scores and
//      consumed after the softmax.
// 8 waves; wave w takes tokens [32 w, 32 w + 32), RPS per step.  The sparse
// V terms p_t s_tj go to per-wave LDS rows (one LDS add per entry and head)
// with one or two query heads per KV head; with more they are folded into
// the dequantised values through a per-wave tile of the step's tokens.
constexpr int kFastCap = 2048;     // outliers of one matrix split staged
constexpr int kFastGroups = 2;     // quantization groups per token staged
constexpr int kFastWaves = 8;
constexpr int kFastThreads = 64 * kFastWaves;

// codes of 8 consecutive columns as floats (code e in bits [BITS e, BITS e + BITS))
template <int BITS>
__device__ __forceinline__ void unpack8(uint32_t w, float (&cf)[8]) {
    if (BITS == 4) {
        // the nibble masks are hidden from the compiler, so that each code is
        // one v_cvt_f32_ubyteN of a masked word (not a field extract + convert)
        uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
        asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cf[2 * i] = (float)((lo >> (8 * i)) & 0xffu);
            cf[2 * i + 1] = (float)((hi >> (8 * i)) & 0xffu);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cf[e] = (float)((w >> (2 * e)) & 3u);
    }
}

// waves per SIMD the registers are budgeted for: 8 at one query head per KV
// head (4 workgroups per CU, within LDS; fits without spills), 4 at four (2
// workgroups per CU; a few VGPRs spill), else 2 (the compiler's choice)
template <int G>
constexpr int prompt_waves() { return G == 1 ? 8 : G == 4 ? 4 : 2; }

template <int D, int G, int BITS>
__global__ void __launch_bounds__(kFastThreads, prompt_waves<G>()) attn_prompt_kernel(AttnArgs a) {
    constexpr int LPR = D / 8, RPS = 64 / LPR, TPW = kTPS / kFastWaves, SPW = TPW / RPS;
    constexpr int CPT = kFastCap / kFastThreads;      // staged CSR entries per thread
    constexpr int ROWB = D * BITS / 8;                 // code bytes per token
    // Sparse V terms.  With up to 2 heads: LDS adds into per-wave rows, a
    // token's even and odd entries on two threads (all 8 waves take part).
    // With 4 or more heads (one LDS add per entry and head) the outliers are
    // folded into the dequantised values instead, through a per-wave fp16
    // tile of the step's RPS tokens.
    constexpr bool VTILE = G >= 4;
    constexpr int VSP = 2;                             // threads per token
    constexpr int kVsRows = 4 * VSP;                   // one row per wave
    constexpr int kTileBytes = RPS * D * 2;            // 1 KB
    constexpr int kVsBytes = VTILE ? kFastWaves * kTileBytes : kVsRows * G * D * 4;
    constexpr int kRedBytes = 4 * G * D * 4;
    constexpr int kCsrBytes = kRedBytes > kFastCap * 4 ? kRedBytes : kFastCap * 4;
    static_assert(kTPS * kFastGroups / 4 <= 128 && kTPS * kMaxRank / 4 <= kFastThreads &&
                  D * kMaxRank / 4 <= kFastThreads, "one float4 per thread stages the side data");
    typedef float f4v __attribute__((ext_vector_type(4)));
    __shared__ float s_q[G * D];
    __shared__ float s_sc[kTPS * G];                   // scores, then probabilities
    __shared__ __attribute__((aligned(16))) float s_gs[kTPS * kFastGroups];
    __shared__ __attribute__((aligned(16))) float s_gz[kTPS * kFastGroups];
    __shared__ __attribute__((aligned(16))) float s_a[kTPS * kMaxRank];
    __shared__ __attribute__((aligned(16))) float s_bkt[kMaxRank * D];   // B_K transposed: [c][j]
    __shared__ __attribute__((aligned(16))) float s_bv[D * kMaxRank];
    __shared__ float s_qb[G * kMaxRank];
    __shared__ int32_t s_rk[kTPS + 1];
    __shared__ int32_t s_rv[kTPS + 1];
    // CSR entries (then the cross-wave sums), sparse V sums
    __shared__ __attribute__((aligned(16))) unsigned char s_big[kCsrBytes + kVsBytes];
    __shared__ float s_wm[4 * G];                      // per-wave max and sum (token waves 0..3)
    __shared__ float s_ws[4 * G];
    __shared__ float s_pa[kFastWaves * G * kMaxRank];
    uint32_t* s_cv = reinterpret_cast<uint32_t*>(s_big);
    float* s_vs = reinterpret_cast<float*>(s_big + kCsrBytes);
    float* s_red = reinterpret_cast<float*>(s_big);

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    // grid (split0, Hkv, B)
    const int split = (int)group_id_x(), hk = (int)group_id_y(), b = (int)group_id_z();
    const int pair = b * a.Hkv + hk;
    const int t0 = split * kTPS;
    const Piece pc = find_piece(a, b, hk, t0, t0 + kTPS);
    const Packed& p = pc.p;
    const int r = p.rank, gl = p.group / 8, ngr = D / p.group;
    const uint32_t kk = (uint32_t)p.k;
    const size_t mrk = (size_t)pc.mk * p.rows + pc.row0, mrv = (size_t)pc.mv * p.rows + pc.row0;
    // this lane's first token; later steps add RPS tokens
    const int tok0 = wv * TPW + rl;
    const uint32_t coff0 = (uint32_t)(tok0 * ROWB + colq * BITS);
    const int gi = colq / gl;

    // ---------------- round 1
    float q[G][8], qs[G];
    {
        const uint16_t* qb = a.q + ((size_t)b * a.Hq + hk * G) * D;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 w = *reinterpret_cast<const uint4*>(qb + h * D + colq * 8);
            const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
            qs[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                q[h][e] = h2f(w4[e >> 1] >> (16 * (e & 1)));
                qs[h] += q[h][e];
            }
        }
        for (int i = tid; i < G * D; i += kFastThreads) s_q[i] = h2f(qb[i]);
    }
    uint32_t wk[SPW];
    const unsigned char* ck = p.codes + mrk * ROWB;
    const unsigned char* cvb = p.codes + mrv * ROWB;
#pragma unroll
    for (int s = 0; s < SPW; ++s)
        wk[s] = BITS == 4 ? ld_at<uint32_t>(ck, coff0 + s * RPS * ROWB)
                          : (uint32_t)ld_at<uint16_t>(ck, coff0 + s * RPS * ROWB);
    // scales and zeros: kTPS * ngr floats each (<= 512: one float4 per thread,
    // threads [0, 128) scales, [128, 256) zeros); A: kTPS * r floats (<= 2048,
    // one float4 per thread)
    const int ng4 = kTPS * ngr / 4, na4 = kTPS * r / 4, nb4 = D * r / 4;
    const f4v z4 = {0.f, 0.f, 0.f, 0.f};
    struct Side {
        f4v gsz, av;
    };
    auto load_side = [&](size_t mrow) {
        const int i = tid & 127;
        const float* src = (tid < 128 ? p.scale : p.zero) + mrow * ngr;
        Side sd;
        sd.gsz = (tid < 256 && i < ng4) ? reinterpret_cast<const f4v*>(src)[i] : z4;
        sd.av = tid < na4 ? reinterpret_cast<const f4v*>(p.A + mrow * r)[tid] : z4;
        return sd;
    };
    auto store_side = [&](const Side sd) {
        const int i = tid & 127;
        if (tid < 256 && i < ng4) reinterpret_cast<f4v*>(tid < 128 ? s_gs : s_gz)[i] = sd.gsz;
        if (tid < na4) reinterpret_cast<f4v*>(s_a)[tid] = sd.av;
    };
    {
        const Side sk = load_side(mrk);
        const int32_t* rpk = p.row_ptr + (size_t)pc.mk * (p.rows + 1) + pc.row0;
        const int32_t* rpv = p.row_ptr + (size_t)pc.mv * (p.rows + 1) + pc.row0;
        // threads [0, kTPS] read K's row pointers, [256, 256 + kTPS] V's
        const int ri = tid & 255;
        const int32_t rp0 = (tid < 256 ? rpk : rpv)[ri];
        const int32_t rp1 = ri == 0 ? (tid < 256 ? rpk : rpv)[kTPS] : 0;
        // B_K transposed: thread i takes element [c = i / D][j = i % D] (r D <= 1024)
        const float* bkm = p.B + (size_t)pc.mk * D * r;
        float bkt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + u * kFastThreads;
            bkt[u] = i < r * D ? bkm[(i % D) * r + i / D] : 0.0f;
        }
        const f4v bv = tid < nb4 ? reinterpret_cast<const f4v*>(p.B + (size_t)pc.mv * D * r)[tid] : z4;
        store_side(sk);
        int32_t* srp = tid < 256 ? s_rk : s_rv;
        srp[ri] = min(max(rp0, 0), (int)kk);
        if (ri == 0) srp[kTPS] = min(max(rp1, 0), (int)kk);
        if (tid < nb4) reinterpret_cast<f4v*>(s_bv)[tid] = bv;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (tid + u * kFastThreads < r * D) s_bkt[tid + u * kFastThreads] = bkt[u];
        for (int i = tid; i < kVsBytes / 16; i += kFastThreads)
            reinterpret_cast<uint4*>(s_vs)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // ---------------- round 2 (issued now, consumed later)
    const int beg_k = s_rk[0], cnt_k = max(s_rk[kTPS] - beg_k, 0);
    const int beg_v = s_rv[0], cnt_v = max(s_rv[kTPS] - beg_v, 0);
    const bool stg_k = cnt_k <= kFastCap, stg_v = cnt_v <= kFastCap;
    const uint16_t* colk = p.col + (size_t)pc.mk * kk;
    const uint16_t* valk = p.val + (size_t)pc.mk * kk;
    const uint16_t* colv = p.col + (size_t)pc.mv * kk;
    const uint16_t* valv = p.val + (size_t)pc.mv * kk;
    uint32_t ek[CPT], ev[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int i = tid + j * kFastThreads;
        ek[j] = (stg_k && i < cnt_k) ? ((uint32_t)colk[beg_k + i] | ((uint32_t)valk[beg_k + i] << 16)) : 0u;
        ev[j] = (stg_v && i < cnt_v) ? ((uint32_t)colv[beg_v + i] | ((uint32_t)valv[beg_v + i] << 16)) : 0u;
    }

    // (B_K^T q)[h][c]: 16 lanes per (h, c), 8 columns each, summed over the
    // lane row
    for (int i = tid; i < G * kMaxRank * 16; i += kFastThreads) {
        const int hc = i / 16, j0 = (i % 16) * (D / 16);
        const int h = hc / kMaxRank, c = hc % kMaxRank;
        float v = 0.0f;
        if (c < r) {
#pragma unroll
            for (int j = 0; j < D / 16; ++j) v = fmaf(s_q[h * D + j0 + j], s_bkt[c * D + j0 + j], v);
        }
        v = row_allreduce<16>(v);
        if ((i % 16) == 0) s_qb[hc] = v;
    }
    __syncthreads();

    // ---------------- phase 1: dense part of q . K^_t
    float qbl[G];   // (B^T q)[colq] in the lanes colq < r
#pragma unroll
    for (int h = 0; h < G; ++h) qbl[h] = colq < r ? s_qb[h * kMaxRank + colq] : 0.0f;
    // side data of token tok0 + s RPS at gidx0 + s gstep (scale, zero) and
    // aidx0 + s astep (A)
    const int gidx0 = tok0 * ngr + gi, gstep = RPS * ngr;
    const int aidx0 = tok0 * r + colq, astep = RPS * r;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int tok = tok0 + s * RPS;
        const float scv = s_gs[gidx0 + s * gstep], zpv = s_gz[gidx0 + s * gstep];
        const float av = colq < r ? s_a[aidx0 + s * astep] : 0.0f;
        float cf[8];
        unpack8<BITS>(wk[s], cf);
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], cf[e], part[h]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float v = row_allreduce<LPR>(fmaf(av, qbl[h], fmaf(scv, part[h], zpv * qs[h])));
            if (colq == 0) s_sc[tok * G + h] = v;
        }
    }
    // K's CSR entries into LDS
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (stg_k && tid + j * kFastThreads < cnt_k) s_cv[tid + j * kFastThreads] = ek[j];
    // V's codes and side data, consumed after the softmax (issued only now,
    // so that they hold no registers during the K phase)
    uint32_t wvv[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
        wvv[s] = BITS == 4 ? ld_at<uint32_t>(cvb, coff0 + s * RPS * ROWB)
                           : (uint32_t)ld_at<uint16_t>(cvb, coff0 + s * RPS * ROWB);
    const Side sv = load_side(mrv);
    __syncthreads();

    // ---------------- sparse part (one thread per token, waves 0..3), softmax
    float pr[G];
    if (tid < kTPS) {
        float add[G];
#pragma unroll
        for (int h = 0; h < G; ++h) add[h] = 0.0f;
        for (int k = s_rk[tid]; k < s_rk[tid + 1]; ++k) {
            const uint32_t e = stg_k ? s_cv[k - beg_k] : ((uint32_t)colk[k] | ((uint32_t)valk[k] << 16));
            const int cj = (int)(e & (D - 1));
            const float v = h2f(e >> 16);
#pragma unroll
            for (int h = 0; h < G; ++h) add[h] = fmaf(s_q[h * D + cj], v, add[h]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            pr[h] = a.sm_scale * (s_sc[tid * G + h] + add[h]);
            const float m = wave_max(pr[h]);
            if (lane == 0) s_wm[wv * G + h] = m;
        }
    }
    // (this barrier also ends the reads of K's CSR entries, whose LDS bytes
    // take V's below)
    __syncthreads();
    if (tid < kTPS) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m = fmaxf(fmaxf(s_wm[h], s_wm[G + h]), fmaxf(s_wm[2 * G + h], s_wm[3 * G + h]));
            pr[h] = expf(pr[h] - m);
            s_sc[tid * G + h] = pr[h];
            const float sm = wave_sum(pr[h]);
            if (lane == 0) s_ws[wv * G + h] = sm;
        }
    }
    // V's side data and CSR entries replace K's
    store_side(sv);
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (stg_v && tid + j * kFastThreads < cnt_v) s_cv[tid + j * kFastThreads] = ev[j];
    __syncthreads();
    // sparse V terms p_t s_tj into the wave's LDS row: entry i (CSR order) of
    // token t by thread t + kTPS (i mod VSP), one LDS add each (a wave's adds
    // execute in program order, rows are per wave, so the sums are
    // deterministic)
    if (!VTILE && tid < kTPS * VSP) {
        const int t = tid & (kTPS - 1), par = tid / kTPS;
        float pt[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pt[h] = par == 0 ? pr[h] : s_sc[t * G + h];
        float* vs = s_vs + wv * G * D;
        for (int k = s_rv[t] + par; k < s_rv[t + 1]; k += VSP) {
            const uint32_t e = stg_v ? s_cv[k - beg_v] : ((uint32_t)colv[k] | ((uint32_t)valv[k] << 16));
            const float v = h2f(e >> 16);
#pragma unroll
            for (int h = 0; h < G; ++h) atomicAdd(&vs[h * D + (e & (D - 1))], pt[h] * v);
        }
    }

    // ---------------- phase 2: sum_t p_t V^_t = sum_t (p_t scale_t) codes_t
    // + sum_t p_t zero_t + sparse + low-rank
    float acc[G][8], pa[G], pz[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        pa[h] = 0.0f;
        pz[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    }
    uint16_t* tile = reinterpret_cast<uint16_t*>(s_big + kCsrBytes) + wv * (kTileBytes / 2);
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int tok = tok0 + s * RPS;
        const float scv = s_gs[gidx0 + s * gstep], zpv = s_gz[gidx0 + s * gstep];
        const float av = colq < r ? s_a[aidx0 + s * astep] : 0.0f;
        float cf[8];
        unpack8<BITS>(wvv[s], cf);
        if constexpr (VTILE) {
            // the V outliers of the wave's RPS tokens of this step into its tile
            // (the LPR lanes of a token take its entries in turn), this lane's 8
            // values read back, its 16 bytes cleared (LDS operations of one wave
            // execute in order; each step's instructions are kept to the step)
            __builtin_amdgcn_sched_barrier(0);
            const int kb = s_rv[tok], ke = s_rv[tok + 1];
            for (int k = kb + colq; k < ke; k += LPR) {
                const uint32_t e = stg_v ? s_cv[k - beg_v] : ((uint32_t)colv[k] | ((uint32_t)valv[k] << 16));
                tile[rl * D + (e & (D - 1))] = (uint16_t)(e >> 16);
            }
            __builtin_amdgcn_wave_barrier();
            uint4* mine = reinterpret_cast<uint4*>(tile + rl * D + colq * 8);
            const uint4 sv4 = *mine;
            *mine = make_uint4(0u, 0u, 0u, 0u);
            __builtin_amdgcn_wave_barrier();
            const uint32_t sw[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
            float dv[8];   // code scale + outlier (a mixed fma), zero added below
#pragma unroll
            for (int e = 0; e < 8; ++e) dv[e] = fmaf(cf[e], scv, h2f(sw[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pp = s_sc[tok * G + h];
                pa[h] = fmaf(pp, av, pa[h]);
                pz[h] = fmaf(pp, zpv, pz[h]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pp, dv[e], acc[h][e]);
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pp = s_sc[tok * G + h];
                pa[h] = fmaf(pp, av, pa[h]);
                pz[h] = fmaf(pp, zpv, pz[h]);
                const float ps = pp * scv;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ps, cf[e], acc[h][e]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += pz[h];
    float* part = a.partial + ((size_t)pair * a.splits + split) * G * (D + 2);
    if (tid < G) {
        part[tid * (D + 2) + D] = fmaxf(fmaxf(s_wm[tid], s_wm[G + tid]), fmaxf(s_wm[2 * G + tid], s_wm[3 * G + tid]));
        part[tid * (D + 2) + D + 1] = s_ws[tid] + s_ws[G + tid] + s_ws[2 * G + tid] + s_ws[3 * G + tid];
    }
    // low-rank part: B_V (sum_t p_t A_t), from the per-rank sums of the waves
#pragma unroll
    for (int h = 0; h < G; ++h) pa[h] = sum_rowgroups<LPR>(pa[h]);
    if (rl == 0 && colq < r) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_pa[(wv * G + h) * kMaxRank + colq] = pa[h];
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = sum_rowgroups<LPR>(acc[h][e]);
    // the final sum for column j of head h: the waves' row sums, the low-rank
    // term and the sparse V sums
    auto emit = [&](const float* rows, int nrows) {
        for (int i = tid; i < G * D; i += kFastThreads) {
            const int h = i / D, j = i % D;
            float lr = 0.0f;
            for (int c = 0; c < r; ++c) {
                float tot = 0.0f;
#pragma unroll
                for (int w = 0; w < kFastWaves; ++w) tot += s_pa[(w * G + h) * kMaxRank + c];
                lr = fmaf(tot, s_bv[j * r + c], lr);
            }
            const float* vs = s_vs + h * D + j;   // row w at vs[w * G * D]
            constexpr int RS = G * D;
            float sp = 0.0f;
            if (!VTILE) sp = (vs[0 * RS] + vs[1 * RS]) + (vs[2 * RS] + vs[3 * RS]);
            if (!VTILE && kVsRows == 8) sp += (vs[4 * RS] + vs[5 * RS]) + (vs[6 * RS] + vs[7 * RS]);
            float dn = 0.0f;
            for (int w = 0; w < nrows; ++w) dn += rows[(w * G + h) * D + j];
            part[h * (D + 2) + j] = dn + lr + sp;
        }
    };
    if constexpr (G == 1) {
        // B_K (read only before the V loop) holds the 8 waves' rows: one
        // barrier, after which the V loop's LDS data is complete
        static_assert(kFastWaves * G * D <= kMaxRank * D, "the wave rows fit where B_K was");
        if (rl == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_bkt[wv * D + colq * 8 + e] = acc[0][e];
        }
        __syncthreads();
        emit(s_bkt, kFastWaves);
    } else {
        // the rows go where the CSR entries were (read in the V loop): waves
        // 4..7 hand theirs to waves 0..3
        __syncthreads();
        if (rl == 0 && wv >= 4) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_red[((wv - 4) * G + h) * D + colq * 8 + e] = acc[h][e];
        }
        __syncthreads();
        if (rl == 0 && wv < 4) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_red[(wv * G + h) * D + colq * 8 + e] += acc[h][e];
        }
        __syncthreads();
        emit(s_red, 4);
    }
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnArgs a) {
    __shared__ float s_m[kThreads / 64];
    __shared__ float s_num[kThreads];
    __shared__ float s_den[kThreads];
    const int bh = (int)group_id_x();                 // b * Hq + hq
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / G, h = hq % G;
    merge_head<D, G>(a, b * a.Hkv + hk, bh, h, s_m, s_num, s_den);
}

// Splits [0, split0) go to attn_prompt_kernel: the prompt's splits when every
// one of them lies inside one compressed chunk and the token's groups fit
// its staging; the rest (fills, the fp16 buffer, other shapes) to
// attn_split_kernel.
template <int D, int G>
hipError_t launch_dg(const AttnArgs& a0, hipStream_t st) {
    AttnArgs a = a0;
    a.split0 = 0;
    if (a.prompt.count == 1 && a.tokens_per_split == kTPS && a.prompt.p.rows % kTPS == 0 &&
        D / a.prompt.p.group <= kFastGroups)
        a.split0 = min(a.splits, a.prompt.chunks * a.prompt.p.rows / kTPS);
    const unsigned pairs = (unsigned)(a.B * a.Hkv);
    // one split of attn_split_kernel per pair and one query head per KV head:
    // that workgroup also merges (with more heads it would merge them one
    // after another, slower than the combine kernel's workgroup per head)
    a.fuse_combine = (G == 1 && a.splits - a.split0 == 1) ? 1 : 0;
    hipError_t e;
    {
        Timed t(kKAttnSplit, st);
        if (a.split0 > 0) {
            const dim3 grid((unsigned)a.split0, (unsigned)a.Hkv, (unsigned)a.B);
            if (a.prompt.p.bits == 4)
                hipLaunchKernelGGL((attn_prompt_kernel<D, G, 4>), grid, dim3(kFastThreads), 0, st, a);
            else
                hipLaunchKernelGGL((attn_prompt_kernel<D, G, 2>), grid, dim3(kFastThreads), 0, st, a);
        }
        if (a.splits > a.split0)
            hipLaunchKernelGGL((attn_split_kernel<D, G>), dim3(pairs * (a.splits - a.split0)), dim3(kThreads),
                               0, st, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.fuse_combine) return e;
    {
        Timed t(kKAttnCombine, st);
        hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3((unsigned)(a.B * a.Hq)), dim3(kThreads), 0, st, a);
        e = hipGetLastError();
    }
    return e;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_dg<D, 1>(a, st);
        case 2: return launch_dg<D, 2>(a, st);
        case 4: return launch_dg<D, 4>(a, st);
        case 8: return launch_dg<D, 8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

__global__ void buffer_append_kernel(const uint16_t* k_new, const uint16_t* v_new, uint16_t* buf,
                                     int B, int H, int d, int cap, int pos, int n_new,
                                     int src_tokens, int src_off, int nblocks) {
    // one thread per 8 fp16 values (16 bytes); a grid-stride loop over nblocks
    // workgroups of kThreads
    const int per_row = d / 8;
    const size_t total = (size_t)2 * B * H * n_new * per_row;
    for (size_t i = (size_t)group_id_x() * kThreads + thread_id(); i < total;
         i += (size_t)nblocks * kThreads) {
        const int c8 = (int)(i % per_row);
        size_t rest = i / per_row;
        const int tok = (int)(rest % n_new);
        rest /= n_new;
        const int h = (int)(rest % H);
        rest /= H;
        const int b = (int)(rest % B);
        const int tensor = (int)(rest / B);
        const uint16_t* src = (tensor == 0 ? k_new : v_new) +
                              (((size_t)b * H + h) * src_tokens + src_off + tok) * d + c8 * 8;
        uint16_t* dst = buf + ((((size_t)tensor * B + b) * H + h) * cap + pos + tok) * d + c8 * 8;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
}

}  // namespace

size_t attn_workspace_bytes(int B, int Hkv, int Hq, int d, int64_t tokens, int* splits,
                            int* tokens_per_split) {
    int64_t s = (tokens + kTPS - 1) / kTPS;
    if (s < 1) s = 1;
    if (splits) *splits = (int)s;
    if (tokens_per_split) *tokens_per_split = kTPS;
    const int G = Hkv > 0 ? Hq / Hkv : 1;
    return align_up((size_t)B * Hkv * s * G * (d + 2) * sizeof(float));
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t st) {
    if (a.B * a.Hq == 0) return hipSuccess;
    if (a.d == 64) return launch_d<64>(a, st);
    if (a.d == 128) return launch_d<128>(a, st);
    return hipErrorInvalidValue;
}

hipError_t launch_buffer_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* buf,
                                int B, int H, int d, int cap, int pos, int n_new,
                                int src_tokens, int src_off, hipStream_t st) {
    const size_t total = (size_t)2 * B * H * n_new * (d / 8);
    if (total == 0) return hipSuccess;
    size_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    Timed t(kKBufferAppend, st);
    hipLaunchKernelGGL(buffer_append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, k_new,
                       v_new, buf, B, H, d, cap, pos, n_new, src_tokens, src_off, (int)blocks);
    return hipGetLastError();
}

}  // namespace gear
