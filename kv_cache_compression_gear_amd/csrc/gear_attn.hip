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

template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads) attn_split_kernel(AttnArgs a) {
    constexpr int LPR = D / 8, RPS = 64 / LPR, TILE = 4 * RPS;
    __shared__ float s_q[G * D];
    __shared__ float s_sc[kTPS * G];
    __shared__ float s_qb[G * kMaxRank];
    __shared__ float s_red[4 * G * D];
    __shared__ float s_stat[2 * G];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const int pair = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
    const int b = pair / a.Hkv, hk = pair % a.Hkv;
    const int pt = a.prompt.count ? a.prompt.chunks * a.prompt.p.rows : 0;
    const int N = pt + a.fills.count * a.fills.p.rows + a.buf_len;
    const int t0 = split * a.tokens_per_split;
    const int t1 = min(N, t0 + a.tokens_per_split);

    for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, j = i % D;
        s_q[i] = h2f(a.q[((size_t)b * a.Hq + hk * G + h) * D + j]);
    }
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

    // ---------------- phase 1: scores of the split's tokens
    for (int t = t0; t < t1;) {
        const Piece pc = find_piece(a, b, hk, t, t1);
        if (pc.kind == 0) {
            const Packed& p = pc.p;
            const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
            const uint32_t cmask = (1u << bits) - 1u;
            // B^T q for this matrix: one row group of wave 0 spans all D columns
            if (r > 0) {
                __syncthreads();
                if (wv == 0) {
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
                            const float v = row_sum<LPR>(part[h]);
                            if (lane == 0) s_qb[h * kMaxRank + c] = v;
                        }
                    }
                }
                __syncthreads();
            }
            const int32_t* rp = p.row_ptr + (size_t)pc.mk * (p.rows + 1);
            const uint16_t* cm = p.col + (size_t)pc.mk * p.k;
            const uint16_t* vm = p.val + (size_t)pc.mk * p.k;
            for (int tt = 0; tt < pc.len; tt += TILE) {
                const int tok = tt + wv * RPS + rl;
                const bool valid = tok < pc.len;
                float part[G];
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = 0.0f;
                const int row = pc.row0 + (valid ? tok : 0);
                const size_t grow = (size_t)pc.mk * p.rows + row;
                if (valid) {
                    uint32_t word;
                    if (bits == 4)
                        word = reinterpret_cast<const uint32_t*>(p.codes)[grow * (D / 8) + colq];
                    else
                        word = reinterpret_cast<const uint16_t*>(p.codes)[grow * (D / 8) + colq];
                    const float sc = p.scale[grow * ngr + colq / gl];
                    const float zp = p.zero[grow * ngr + colq / gl];
                    float dot[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) dot[h] = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float cf = (float)((word >> (e * bits)) & cmask);
#pragma unroll
                        for (int h = 0; h < G; ++h) dot[h] = fmaf(q[h][e], cf, dot[h]);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = fmaf(sc, dot[h], zp * qs[h]);
                    const int beg = max(rp[row], 0), end = min(rp[row + 1], p.k);
                    for (int i = beg; i < end; ++i) {
                        const int cj = cm[i];
                        if ((cj >> 3) == colq) {
                            const float v = h2f(vm[i]);
#pragma unroll
                            for (int h = 0; h < G; ++h) part[h] = fmaf(s_q[h * D + cj], v, part[h]);
                        }
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = row_sum<LPR>(part[h]);
                if (valid && colq == 0) {
                    for (int c = 0; c < r; ++c) {
                        const float av = p.A[grow * r + c];
#pragma unroll
                        for (int h = 0; h < G; ++h) part[h] = fmaf(av, s_qb[h * kMaxRank + c], part[h]);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) s_sc[(t - t0 + tok) * G + h] = a.sm_scale * part[h];
                }
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
                for (int h = 0; h < G; ++h) part[h] = row_sum<LPR>(part[h]);
                if (valid && colq == 0) {
#pragma unroll
                    for (int h = 0; h < G; ++h) s_sc[(t - t0 + tok) * G + h] = a.sm_scale * part[h];
                }
            }
        }
        t += pc.len;
    }
    __syncthreads();

    // ---------------- softmax inside the split
    const int n = max(t1 - t0, 0);
    {
        float mx[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = -INFINITY;
        for (int i = tid; i < n; i += kThreads)
#pragma unroll
            for (int h = 0; h < G; ++h) mx[h] = fmaxf(mx[h], s_sc[i * G + h]);
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
    for (int t = t0; t < t1;) {
        const Piece pc = find_piece(a, b, hk, t, t1);
        if (pc.kind == 0) {
            const Packed& p = pc.p;
            const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
            const uint32_t cmask = (1u << bits) - 1u;
            const int32_t* rp = p.row_ptr + (size_t)pc.mv * (p.rows + 1);
            const uint16_t* cm = p.col + (size_t)pc.mv * p.k;
            const uint16_t* vm = p.val + (size_t)pc.mv * p.k;
            float pa[G][kMaxRank];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int c = 0; c < kMaxRank; ++c) pa[h][c] = 0.0f;
            for (int tt = 0; tt < pc.len; tt += TILE) {
                const int tok = tt + wv * RPS + rl;
                if (tok >= pc.len) continue;
                const int row = pc.row0 + tok;
                const size_t grow = (size_t)pc.mv * p.rows + row;
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pr[h] = s_sc[(t - t0 + tok) * G + h];
                uint32_t word;
                if (bits == 4)
                    word = reinterpret_cast<const uint32_t*>(p.codes)[grow * (D / 8) + colq];
                else
                    word = reinterpret_cast<const uint16_t*>(p.codes)[grow * (D / 8) + colq];
                const float sc = p.scale[grow * ngr + colq / gl];
                const float zp = p.zero[grow * ngr + colq / gl];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dv = fmaf((float)((word >> (e * bits)) & cmask), sc, zp);
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], dv, acc[h][e]);
                }
#pragma unroll
                for (int c = 0; c < kMaxRank; ++c) {
                    if (c < r) {
                        const float av = p.A[grow * r + c];
#pragma unroll
                        for (int h = 0; h < G; ++h) pa[h][c] = fmaf(pr[h], av, pa[h][c]);
                    }
                }
                const int beg = max(rp[row], 0), end = min(rp[row + 1], p.k);
                for (int i = beg; i < end; ++i) {
                    const int cj = cm[i];
                    if ((cj >> 3) == colq) {
                        const float v = h2f(vm[i]);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if ((cj & 7) == e) {
#pragma unroll
                                for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], v, acc[h][e]);
                            }
                    }
                }
            }
            // low-rank part of this matrix: acc += B (sum_t p_t A_t)
#pragma unroll
            for (int c = 0; c < kMaxRank; ++c) {
                if (c < r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float bv = p.B[((size_t)pc.mv * D + colq * 8 + e) * r + c];
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pa[h][c], bv, acc[h][e]);
                    }
                }
            }
        } else {
            const uint16_t* vb = a.buf + (((size_t)(1 * a.B + b) * a.Hkv + hk) * a.buf_cap) * D;
            for (int tt = 0; tt < pc.len; tt += TILE) {
                const int tok = tt + wv * RPS + rl;
                if (tok >= pc.len) continue;
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pr[h] = s_sc[(t - t0 + tok) * G + h];
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
    float* part = a.partial + (size_t)blockIdx.x * G * (D + 2);
    for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, j = i % D;
        part[h * (D + 2) + j] = s_red[(0 * G + h) * D + j] + s_red[(1 * G + h) * D + j] +
                                s_red[(2 * G + h) * D + j] + s_red[(3 * G + h) * D + j];
    }
    if (tid < G) {
        part[tid * (D + 2) + D] = n > 0 ? s_stat[tid] : -INFINITY;
        part[tid * (D + 2) + D + 1] = n > 0 ? s_stat[G + tid] : 0.0f;
    }
}

// out[b][hq][:] = merge over splits of (acc, max, sum).
template <int D, int G>
__global__ void attn_combine_kernel(AttnArgs a) {
    const int bh = blockIdx.x;                 // b * Hq + hq
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / G, h = hq % G;
    const int pair = b * a.Hkv + hk;
    const int j = threadIdx.x;
    float m = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
        const float* part = a.partial + ((size_t)(pair * a.splits + s) * G + h) * (D + 2);
        if (part[D + 1] > 0.0f) m = fmaxf(m, part[D]);
    }
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
        const float* part = a.partial + ((size_t)(pair * a.splits + s) * G + h) * (D + 2);
        if (part[D + 1] > 0.0f) {
            const float w = expf(part[D] - m);
            num = fmaf(w, part[j], num);
            den = fmaf(w, part[D + 1], den);
        }
    }
    a.out[(size_t)bh * D + j] = den > 0.0f ? num / den : 0.0f;
}

template <int D, int G>
hipError_t launch_dg(const AttnArgs& a, hipStream_t st) {
    const unsigned grid = (unsigned)(a.B * a.Hkv * a.splits);
    hipError_t e;
    {
        Timed t(kKAttnSplit, st);
        hipLaunchKernelGGL((attn_split_kernel<D, G>), dim3(grid), dim3(kThreads), 0, st, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    {
        Timed t(kKAttnCombine, st);
        hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3((unsigned)(a.B * a.Hq)), dim3(D), 0, st, a);
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
                                     int src_tokens, int src_off) {
    // one thread per 8 fp16 values (16 bytes)
    const int per_row = d / 8;
    const size_t total = (size_t)2 * B * H * n_new * per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
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
                       v_new, buf, B, H, d, cap, pos, n_new, src_tokens, src_off);
    return hipGetLastError();
}

}  // namespace gear
