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

// Workgroup barrier for LDS traffic only: the wave's LDS operations are
// complete, global loads in flight stay in flight (the compiler waits for
// them where their registers are used).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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

// Folds n split results (max ms, sum ls, numerator vs; ls = 0: left out)
// into a running (m, num, den) under a running maximum: the sums are brought
// to a new maximum once per call, then each result adds exp(ms - m) times its
// own.  Selects, not branches, so that loads feeding it are not waited for in
// a branch.
template <int N>
__device__ __forceinline__ void fold_splits(const float (&ms)[N], const float (&ls)[N], const float (&vs)[N],
                                            float& m, float& num, float& den) {
    float mc = m;
#pragma unroll
    for (int u = 0; u < N; ++u)
        if (ls[u] > 0.0f) mc = fmaxf(mc, ms[u]);
    if (mc > m) {   // (from -inf: times 0)
        const float f = expf(m - mc);
        num *= f;
        den *= f;
        m = mc;
    }
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const bool in = ls[u] > 0.0f;
        const float w = expf((in ? ms[u] : m) - m);
        num = in ? fmaf(w, vs[u], num) : num;
        den = in ? fmaf(w, ls[u], den) : den;
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
// splits into out itself, for all of its query heads (no combine launch; its
// own result is merged from LDS and never written to the workspace).
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
    __shared__ float s_mg[3 * kThreads];   // merge scratch (fuse_combine)
    __shared__ __attribute__((aligned(16))) float s_bm[D * kMaxRank];   // B of the piece's matrix, [j][c]

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const int nsp = a.splits - a.split0;   // splits [split0, splits) of every (b, kv-head)
    const int pair = (int)(group_id_x() / nsp), split = a.split0 + (int)(group_id_x() % nsp);
    const int b = pair / a.Hkv, hk = pair % a.Hkv;
    const int pt = a.prompt.count ? a.prompt.chunks * a.prompt.p.rows : 0;
    const int N = pt + a.fills.count * a.fills.p.rows + a.buf_len;
    const int t0 = split * a.tokens_per_split;
    const int t1 = min(N, t0 + a.tokens_per_split);

    // q of the pair's G heads (contiguous), one load per slot from a clamped
    // index, all in flight together
    constexpr int QPT = (G * D + kThreads - 1) / kThreads;
    const uint16_t* qg = a.q + ((size_t)b * a.Hq + (size_t)hk * G) * D;
    uint16_t qv[QPT];
#pragma unroll
    for (int u = 0; u < QPT; ++u) qv[u] = ld_at<uint16_t>(qg, (uint32_t)min(tid + u * kThreads, G * D - 1) * 2u);

    // With one split here per pair (fuse_combine) this workgroup merges the
    // pair's splits at the end, for all G heads at once: the G D columns
    // (c = h D + j) are taken MW at a time, thread (mc0, mq) taking columns
    // mc0, mc0 + MW, ... of the splits mq, mq + MNQ, ... (MNQ threads per
    // column when G D < kThreads).  The prompt's splits were written by the
    // launch before this one: their first MPF per thread are loaded now and
    // held (loaded in any case, from clamped valid slots, and left out when
    // not needed); this split is merged from LDS.
    constexpr int MC = G * D, MW = MC < kThreads ? MC : kThreads;
    constexpr int MNQ = kThreads / MW, MCPT = MC / MW, MPF = MCPT >= 4 ? 2 : 8;
    static_assert(kThreads % MW == 0 && MC % MW == 0, "thread mapping of the merge");
    const int mc0 = tid % MW, mq = tid / MW;
    const float* mbase = a.partial + (size_t)pair * a.splits * G * (D + 2);
    const size_t mstride = (size_t)G * (D + 2);   // between splits
    int moff[MCPT], mofl[MCPT];
#pragma unroll
    for (int i = 0; i < MCPT; ++i) {
        const int c = mc0 + i * MW, h = c / D;
        moff[i] = h * (D + 2) + c % D;
        mofl[i] = h * (D + 2) + D;
    }
    float pfm[MCPT][MPF], pfl[MCPT][MPF], pfv[MCPT][MPF];
#pragma unroll
    for (int u = 0; u < MPF; ++u) {
        const int sx = mq + u * MNQ;
        const float* part = mbase + (size_t)min(sx, max(split - 1, 0)) * mstride;
#pragma unroll
        for (int i = 0; i < MCPT; ++i) {
            const float2 ml = *reinterpret_cast<const float2*>(part + mofl[i]);
            pfm[i][u] = ml.x;
            pfl[i][u] = sx < split ? ml.y : 0.0f;   // (this split and beyond: left out)
            pfv[i][u] = part[moff[i]];
        }
    }

    // the split's fp16 buffer rows (K and V), their first 4 steps, loaded now
    // too: they depend on nothing (clamped rows: valid addresses also when
    // the split holds no buffer token; then unused)
    constexpr bool kPfBuf = G * D < 512;   // (registers: 4 heads at d = 128 would drop to one wave per SIMD)
    const int bt0 = pt + a.fills.count * a.fills.p.rows;   // first buffer token
    const int brow0 = max(t0, bt0) - bt0, blen = max(t1 - max(t0, bt0), 0);
    // buffer row `row` of K (kv = 0) or V: a token appended by this launch
    // (row new_row) is read from the caller's array instead
    auto brow_src = [&](int kv, int row) -> const uint16_t* {
        const uint16_t* nw = kv == 0 ? a.k_new : a.v_new;
        return row == a.new_row ? nw + ((size_t)b * a.Hkv + hk) * D
                                : a.buf + (((size_t)(kv * a.B + b) * a.Hkv + hk) * a.buf_cap + row) * D;
    };
    uint4 pbk[4], pbv[4];
    if constexpr (kPfBuf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tok = min(u * TILE + wv * RPS + rl, max(blen, 1) - 1);
            const int row = min(brow0 + tok, a.buf_cap - 1);
            pbk[u] = *reinterpret_cast<const uint4*>(brow_src(0, row) + colq * 8);
            pbv[u] = *reinterpret_cast<const uint4*>(brow_src(1, row) + colq * 8);
        }
    }

#pragma unroll
    for (int u = 0; u < QPT; ++u)
        if (tid + u * kThreads < G * D) s_q[tid + u * kThreads] = h2f(qv[u]);
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

    // The LDS staging of one compressed matrix's piece (rows [row0, row0 +
    // len) of matrix m of p): its row pointers into s_rp, its CSR entries (one
    // contiguous range, whose ends are read first, as scalars) into s_cv as
    // column | fp16 value << 16, and B into s_bm padded to kMaxRank columns
    // with zeros.  stage_issue issues every load of it unconditionally, from
    // clamped addresses (a load in a branch is waited for there), into
    // registers; the caller then issues its first tokens' loads, and
    // stage_store waits for the staging loads only (issued first) and stores.
    constexpr int SCPT = kAttnCsrCap / kThreads;                // CSR entries per thread
    constexpr int BPT = (D * kMaxRank + kThreads - 1) / kThreads;   // B slots per thread
    int csr_beg = 0, csr_cnt = 0;
    bool csr_staged = true;
    int32_t st_rp0 = 0, st_rp1 = 0;
    uint16_t st_col[SCPT], st_val[SCPT];
    float st_b[BPT];
    auto stage_issue = [&](const Packed& p, int64_t m, int row0, int len) {
        const int32_t* rp = p.row_ptr + (size_t)m * (p.rows + 1) + row0;
        const int kk = p.k;
        if (row0 == 0 && len == p.rows) {
            // a whole matrix (every fill): its range is [0, k), known without
            // waiting for its row pointers at both ends
            csr_beg = 0;
            csr_cnt = kk;
        } else {
            csr_beg = min(max(rp[0], 0), kk);
            csr_cnt = max(min(max(rp[len], 0), kk) - csr_beg, 0);
        }
        csr_staged = csr_cnt <= kAttnCsrCap;
        st_rp0 = ld_at<int32_t>(rp, (uint32_t)min(tid, len) * 4u);
        st_rp1 = ld_at<int32_t>(rp, (uint32_t)min(tid + kThreads, len) * 4u);
        // (with no outliers the row pointers stand in for the CSR arrays)
        const uint16_t* cm = kk > 0 ? p.col + (size_t)m * kk : reinterpret_cast<const uint16_t*>(rp);
        const uint16_t* vm = kk > 0 ? p.val + (size_t)m * kk : reinterpret_cast<const uint16_t*>(rp);
        // (clamped to the range's last entry: slots past the range re-read it,
        // no further bytes)
        const int elast = min(csr_beg + max(csr_cnt, 1) - 1, max(kk, 1) - 1);
#pragma unroll
        for (int j = 0; j < SCPT; ++j) {
            const uint32_t off = (uint32_t)min(csr_beg + tid + j * kThreads, elast) * 2u;
            st_col[j] = ld_at<uint16_t>(cm, off);
            st_val[j] = ld_at<uint16_t>(vm, off);
        }
        // (with r = 0 the scales stand in for B)
        const int r = p.rank, rl1 = max(r, 1) - 1;
        const float* bsrc = r > 0 ? p.B + (size_t)m * D * r : p.scale;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int i = min(tid + u * kThreads, D * kMaxRank - 1);
            st_b[u] = ld_at<float>(bsrc, (uint32_t)((i / kMaxRank) * r + min(i % kMaxRank, rl1)) * 4u);
        }
    };
    auto stage_store = [&](const Packed& p, int len) {
        __syncthreads();   // the previous piece's reads of the staging arrays
        if (tid <= len) s_rp[tid] = min(max(st_rp0, 0), p.k);
        if (tid + kThreads <= len) s_rp[tid + kThreads] = min(max(st_rp1, 0), p.k);
        if (csr_staged) {
#pragma unroll
            for (int j = 0; j < SCPT; ++j) {
                const int i = tid + j * kThreads;
                if (i < csr_cnt) s_cv[i] = ((uint32_t)st_col[j] & (D - 1)) | ((uint32_t)st_val[j] << 16);
            }
        }
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int i = tid + u * kThreads;
            if (i < D * kMaxRank) s_bm[i] = (i % kMaxRank) < p.rank ? st_b[u] : 0.0f;
        }
        __syncthreads();
    };
    // entry k (absolute index) of the piece: column | fp16 value << 16
    auto csr_entry = [&](const Packed& p, int64_t m, int k) -> uint32_t {
        if (csr_staged) return s_cv[k - csr_beg];
        return ((uint32_t)p.col[(size_t)m * p.k + k] & (D - 1)) | ((uint32_t)p.val[(size_t)m * p.k + k] << 16);
    };

    // ---------------- phase 1: raw scores q . K^_t of the split's tokens
    for (int t = t0; t < t1;) {
        const Piece pc = find_piece(a, b, hk, t, t1);
        const int base = t - t0;
        if (pc.kind == 0) {
            const Packed& p = pc.p;
            const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
            const uint32_t cmask = (1u << bits) - 1u;
            // keys per channel (KIVI), channel factors (ZipCache): uniform
            const bool chk = pc.mk < p.ch_mats;
            float fk[8], qsf[G];   // the key factors of the lane's columns; sum of q fk
#pragma unroll
            for (int e = 0; e < 8; ++e) fk[e] = p.chan ? p.chan[(size_t)pc.mk * D + colq * 8 + e] : 1.0f;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                qsf[h] = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) qsf[h] = fmaf(q[h][e], fk[e], qsf[h]);
            }
            const size_t mrow = (size_t)pc.mk * p.rows + pc.row0;
            const int steps = (pc.len + TILE - 1) / TILE;
            uint32_t word[1][kAU];
            float sc[1][kAU], zp[1][kAU], av[1][kAU];   // av: A[t][colq] for colq < r
            // per-piece bases (uniform); lanes use 32-bit offsets and a clamped
            // token (always a valid address), then zero what lies past the piece
            const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
            const float* sbase = p.scale + mrow * ngr;
            const float* zbase = p.zero + mrow * ngr;
            const float* abase = r > 0 ? p.A + mrow * r : sbase;
            const int acol = min(colq, max(r - 1, 0));
            auto load = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    const bool ok = tok < pc.len;
                    const uint32_t tk = (uint32_t)min(tok, pc.len - 1);
                    // the lane's code word as two 16-bit loads at either width
                    // (no branch on the width: its join would wait for every load)
                    const uint32_t co = bits == 4 ? tk * (D / 2) + colq * 4 : tk * (D / 4) + colq * 2;
                    const uint32_t wlo = ld_at<uint16_t>(cbase, co);
                    const uint32_t whi = ld_at<uint16_t>(cbase, bits == 4 ? co + 2 : co);
                    const uint32_t w = bits == 4 ? wlo | (whi << 16) : wlo;
                    const uint32_t go = (tk * ngr + colq / gl) * 4;
                    const float scv = ld_at<float>(sbase, go);
                    const float zpv = ld_at<float>(zbase, go);
                    const float a1 = ld_at<float>(abase, (r > 0 ? tk * r + acol : 0) * 4);
                    word[bf][u] = ok ? w : 0u;
                    sc[bf][u] = ok ? scv : 0.0f;
                    zp[bf][u] = ok ? zpv : 0.0f;
                    av[bf][u] = (ok && colq < r) ? a1 : 0.0f;
                }
            };
            stage_issue(p, pc.mk, pc.row0, pc.len);
            load(0, 0);
            stage_store(p, pc.len);
            if (r > 0) {
                // B^T q: row group g = wv RPS + rl (one token row of lanes
                // spans all D columns) takes rank column g, all at once (B is
                // zero-padded to kMaxRank columns in LDS)
                static_assert(kThreads / LPR >= kMaxRank, "a row group per rank column");
                const int g = wv * RPS + rl, c = min(g, kMaxRank - 1);
                float part[G];
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float bv = s_bm[(colq * 8 + e) * kMaxRank + c] * fk[e];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], bv, part[h]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float v = row_allreduce<LPR>(part[h]);
                    if (g < r && colq == 0) s_qb[h * kMaxRank + c] = v;
                }
            }
            __syncthreads();
            float qbl[G];   // (B^T q)[colq] for colq < r
#pragma unroll
            for (int h = 0; h < G; ++h) qbl[h] = colq < r ? s_qb[h * kMaxRank + colq] : 0.0f;
            auto compute = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    float part[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = 0.0f;
                    if (chk) {
                        // each column's scale and zero, in the token's group
                        const int tk = min(tok, pc.len - 1);
                        const float* gs = p.scale + ((size_t)pc.mk * (p.rows / p.group) +
                                                     (size_t)(pc.row0 + tk) / p.group) * D + colq * 8;
                        const float* gz = p.zero + (gs - p.scale);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float cf = (float)((word[bf][u] >> (e * bits)) & cmask);
                            const float kv = fmaf(cf, gs[e], gz[e]) * fk[e];
#pragma unroll
                            for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], kv, part[h]);
                        }
#pragma unroll
                        for (int h = 0; h < G; ++h) part[h] = row_allreduce<LPR>(fmaf(av[bf][u], qbl[h], part[h]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float cf = (float)((word[bf][u] >> (e * bits)) & cmask) * fk[e];
#pragma unroll
                            for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], cf, part[h]);
                        }
                        // + A[t][colq] (B^T q)[colq] in the lanes colq < r, then the row sum
#pragma unroll
                        for (int h = 0; h < G; ++h)
                            part[h] = row_allreduce<LPR>(
                                fmaf(av[bf][u], qbl[h], fmaf(sc[bf][u], part[h], zp[bf][u] * qsf[h])));
                    }
                    if (tok < pc.len && colq == 0) {
#pragma unroll
                        for (int h = 0; h < G; ++h) s_sc[(base + tok) * G + h] = part[h];
                    }
                }
            };
            for (int s0 = 0; s0 < steps; s0 += kAU) {
                if (s0 > 0) load(0, s0);
                compute(0, s0);
            }
            __syncthreads();
            // sparse term: four threads per token (every fourth entry, in CSR
            // order), their sums added within the quad
            for (int i0 = 0; i0 < pc.len; i0 += kThreads / 4) {   // (workgroup-uniform)
                const int i = i0 + tid / 4, sub = tid & 3;
                float add[G];
#pragma unroll
                for (int h = 0; h < G; ++h) add[h] = 0.0f;
                if (i < pc.len) {
                    for (int k = s_rp[i] + sub; k < s_rp[i + 1]; k += 4) {
                        const uint32_t cv = csr_entry(p, pc.mk, k);
                        const int cj = (int)(cv & (D - 1));
                        const float v = h2f(cv >> 16) * (p.chan ? p.chan[(size_t)pc.mk * D + cj] : 1.0f);
#pragma unroll
                        for (int h = 0; h < G; ++h) add[h] = fmaf(s_q[h * D + cj], v, add[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    add[h] += dpp<0xB1>(add[h]);   // quad_perm(1,0,3,2)
                    add[h] += dpp<0x4E>(add[h]);   // quad_perm(2,3,0,1)
                }
                if (i < pc.len && sub == 0) {
#pragma unroll
                    for (int h = 0; h < G; ++h) s_sc[(base + i) * G + h] += add[h];
                }
            }
        } else {
            // 4 steps' rows loaded together (clamped rows, unconditional: a
            // load under a divergent condition is waited for at once); the
            // first 4 steps' were loaded at the start.  A token appended by
            // this launch is also written into the buffer here.
            for (int tt0 = 0; tt0 < pc.len; tt0 += 4 * TILE) {
                uint4 wb[4];
                if (kPfBuf && tt0 == 0) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) wb[u] = pbk[u];
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int tok = min(tt0 + u * TILE + wv * RPS + rl, pc.len - 1);
                        wb[u] = *reinterpret_cast<const uint4*>(brow_src(0, pc.row0 + tok) + colq * 8);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tok = tt0 + u * TILE + wv * RPS + rl;
                    if (tok < pc.len && pc.row0 + tok == a.new_row)
                        *reinterpret_cast<uint4*>(a.buf + (((size_t)(0 * a.B + b) * a.Hkv + hk) * a.buf_cap +
                                                           a.new_row) * D + colq * 8) = wb[u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tt = tt0 + u * TILE;
                    if (tt >= pc.len) break;   // workgroup-uniform
                    const int tok = tt + wv * RPS + rl;
                    const bool valid = tok < pc.len;
                    float part[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = 0.0f;
                    const uint32_t w4[4] = {wb[u].x, wb[u].y, wb[u].z, wb[u].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float kv = valid ? h2f(w4[e >> 1] >> (16 * (e & 1))) : 0.0f;
#pragma unroll
                        for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], kv, part[h]);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = row_allreduce<LPR>(part[h]);
                    if (valid && colq == 0) {
#pragma unroll
                        for (int h = 0; h < G; ++h) s_sc[(base + tok) * G + h] = part[h];
                    }
                }
            }
        }
        t += pc.len;
    }
    __syncthreads();

    // ---------------- softmax inside the split (scores scaled here).  The
    // waves' maxima go to s_red[0, 4G) and their sums to s_red[4G, 8G); every
    // thread combines the four maxima itself, so that two barriers suffice
    // (the total sum, in s_stat, is read only after phase 2's barriers).
    const int n = max(t1 - t0, 0);
    {
        float* s_wmax = s_red;
        float* s_wsum = s_red + 4 * G;
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
            mx[h] = wave_max(mx[h]);
            if (lane == 0) s_wmax[wv * G + h] = mx[h];
        }
        __syncthreads();
        auto max4 = [&](int h) {
            return fmaxf(fmaxf(s_wmax[h], s_wmax[G + h]), fmaxf(s_wmax[2 * G + h], s_wmax[3 * G + h]));
        };
        float gm[G], sm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            gm[h] = max4(h);
            sm[h] = 0.0f;
        }
        if (tid < G) s_stat[tid] = max4(tid);
        for (int i = tid; i < n; i += kThreads)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pv = expf(s_sc[i * G + h] - gm[h]);
                s_sc[i * G + h] = pv;
                sm[h] += pv;
            }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sm[h] = wave_sum(sm[h]);
            if (lane == 0) s_wsum[wv * G + h] = sm[h];
        }
        __syncthreads();
        if (tid < G) s_stat[G + tid] = s_wsum[tid] + s_wsum[G + tid] + s_wsum[2 * G + tid] + s_wsum[3 * G + tid];
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
            float fv[8];   // ZipCache: the value matrix's factors of the lane's columns
#pragma unroll
            for (int e = 0; e < 8; ++e) fv[e] = p.chan ? p.chan[(size_t)pc.mv * D + colq * 8 + e] : 1.0f;
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
            const float* abase = r > 0 ? p.A + mrow * r : sbase;
            const int acol = min(colq, max(r - 1, 0));
            auto load = [&](int bf, int s0) {
#pragma unroll
                for (int u = 0; u < kAU; ++u) {
                    const int tok = (s0 + u) * TILE + wv * RPS + rl;
                    const bool ok = tok < pc.len;
                    const uint32_t tk = (uint32_t)min(tok, pc.len - 1);
                    // the lane's code word as two 16-bit loads at either width
                    // (no branch on the width: its join would wait for every load)
                    const uint32_t co = bits == 4 ? tk * (D / 2) + colq * 4 : tk * (D / 4) + colq * 2;
                    const uint32_t wlo = ld_at<uint16_t>(cbase, co);
                    const uint32_t whi = ld_at<uint16_t>(cbase, bits == 4 ? co + 2 : co);
                    const uint32_t w = bits == 4 ? wlo | (whi << 16) : wlo;
                    const uint32_t go = (tk * ngr + colq / gl) * 4;
                    const float scv = ld_at<float>(sbase, go);
                    const float zpv = ld_at<float>(zbase, go);
                    const float a1 = ld_at<float>(abase, (r > 0 ? tk * r + acol : 0) * 4);
                    word[bf][u] = ok ? w : 0u;
                    sc[bf][u] = ok ? scv : 0.0f;
                    zp[bf][u] = ok ? zpv : 0.0f;
                    av[bf][u] = (ok && colq < r) ? a1 : 0.0f;
                }
            };
            stage_issue(p, pc.mv, pc.row0, pc.len);
            load(0, 0);
            stage_store(p, pc.len);
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
                    // the first entries of the step's rows 1 .. RPS - 1 (an entry's
                    // row in the step: how many of them it reaches)
                    int rs[RPS - 1];
#pragma unroll
                    for (int i = 1; i < RPS; ++i) rs[i - 1] = first + i <= last ? s_rp[first + i] : 0x7fffffff;
                    auto row_of = [&](int k) {
                        int rr = 0;
#pragma unroll
                        for (int i = 0; i < RPS - 1; ++i) rr += k >= rs[i] ? 1 : 0;
                        return rr;
                    };
                    // (the lane's first entry is kept for the clearing, which
                    // then reads no entry again; a step rarely has more than
                    // 64 entries)
                    const int k0 = e0 + lane;
                    int cell0 = -1;
                    if (k0 < e1) {
                        const uint32_t cv = csr_entry(p, pc.mv, k0);
                        cell0 = row_of(k0) * D + (int)(cv & (D - 1));
                        tile[cell0] = h2f(cv >> 16);
                    }
                    for (int k = k0 + 64; k < e1; k += 64) {
                        const uint32_t cv = csr_entry(p, pc.mv, k);
                        tile[row_of(k) * D + (cv & (D - 1))] = h2f(cv >> 16);
                    }
                    __builtin_amdgcn_wave_barrier();
                    const float4 s0v = *reinterpret_cast<const float4*>(tile + rl * D + colq * 8);
                    const float4 s1v = *reinterpret_cast<const float4*>(tile + rl * D + colq * 8 + 4);
                    const float sv[8] = {s0v.x, s0v.y, s0v.z, s0v.w, s1v.x, s1v.y, s1v.z, s1v.w};
                    __builtin_amdgcn_wave_barrier();
                    if (cell0 >= 0) tile[cell0] = 0.0f;
                    for (int k = k0 + 64; k < e1; k += 64) {
                        const uint32_t cv = csr_entry(p, pc.mv, k);
                        tile[row_of(k) * D + (cv & (D - 1))] = 0.0f;
                    }
                    float pr[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) pr[h] = ok ? s_sc[(base + tok) * G + h] : 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dv =
                            (fmaf((float)((word[bf][u] >> (e * bits)) & cmask), sc[bf][u], zp[bf][u]) + sv[e]) * fv[e];
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], dv, acc[h][e]);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) pa[h] = fmaf(pr[h], av[bf][u], pa[h]);
                }
            };
            for (int s0 = 0; s0 < steps; s0 += kAU) {
                if (s0 > 0) load(0, s0);
                compute(0, s0);
            }
            // low-rank part of this matrix: acc += B (sum_t p_t A_t), with the
            // sums over the piece's tokens gathered per rank column c = colq
#pragma unroll
            for (int h = 0; h < G; ++h) pa[h] = sum_rowgroups<LPR>(pa[h]);
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
                    const float bv = s_bm[(colq * 8 + e) * kMaxRank + c] * fv[e];
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h][e] = fmaf(tot[h], bv, acc[h][e]);
                }
            }
        } else {
            // 4 steps' rows loaded together, as for K
            for (int tt0 = 0; tt0 < pc.len; tt0 += 4 * TILE) {
                uint4 wb[4];
                if (kPfBuf && tt0 == 0) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) wb[u] = pbv[u];
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int tok = min(tt0 + u * TILE + wv * RPS + rl, pc.len - 1);
                        wb[u] = *reinterpret_cast<const uint4*>(brow_src(1, pc.row0 + tok) + colq * 8);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tok = tt0 + u * TILE + wv * RPS + rl;
                    if (tok < pc.len && pc.row0 + tok == a.new_row)
                        *reinterpret_cast<uint4*>(a.buf + (((size_t)(1 * a.B + b) * a.Hkv + hk) * a.buf_cap +
                                                           a.new_row) * D + colq * 8) = wb[u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // rows past the piece weigh 0 (selects: a branch here
                    // would take the load into it)
                    const int tok = tt0 + u * TILE + wv * RPS + rl;
                    const bool valid = tok < pc.len;
                    const int tc = min(tok, pc.len - 1);
                    float pr[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) pr[h] = valid ? s_sc[(base + tc) * G + h] : 0.0f;
                    const uint32_t w4[4] = {wb[u].x, wb[u].y, wb[u].z, wb[u].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float vv = h2f(w4[e >> 1] >> (16 * (e & 1)));
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[h], vv, acc[h][e]);
                    }
                }
            }
        }
        t += pc.len;
    }
    // reduce over the row groups of the wave (lane swaps, no LDS), then over
    // the waves
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = sum_rowgroups<LPR>(acc[h][e]);
    __syncthreads();
    if (rl == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_red[(wv * G + h) * D + colq * 8 + e] = acc[h][e];
    }
    __syncthreads();
    if (!a.fuse_combine) {
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
        return;
    }
    // ---------------- the pair's merge (this is its only split here): the
    // prefetched prompt splits, any further ones in chunks of 8 loaded
    // together, then this split from LDS (by the threads mq == 0)
    float m[MCPT], num[MCPT], den[MCPT];
#pragma unroll
    for (int i = 0; i < MCPT; ++i) {
        m[i] = -INFINITY;
        num[i] = 0.0f;
        den[i] = 0.0f;
        fold_splits<MPF>(pfm[i], pfl[i], pfv[i], m[i], num[i], den[i]);
    }
    constexpr int CH = 8;
    for (int s0 = mq + MPF * MNQ; s0 < split; s0 += MNQ * CH) {
        float ms[MCPT][CH], ls[MCPT][CH], vs[MCPT][CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int sx = s0 + u * MNQ;
            const float* part = mbase + (size_t)min(sx, split - 1) * mstride;
#pragma unroll
            for (int i = 0; i < MCPT; ++i) {
                const float2 ml = *reinterpret_cast<const float2*>(part + mofl[i]);
                ms[i][u] = ml.x;
                ls[i][u] = sx < split ? ml.y : 0.0f;
                vs[i][u] = part[moff[i]];
            }
        }
#pragma unroll
        for (int i = 0; i < MCPT; ++i) fold_splits<CH>(ms[i], ls[i], vs[i], m[i], num[i], den[i]);
    }
    if (mq == 0 && n > 0) {
#pragma unroll
        for (int i = 0; i < MCPT; ++i) {
            const int c = mc0 + i * MW, h = c / D, j = c % D;
            const float own[1] = {s_red[(0 * G + h) * D + j] + s_red[(1 * G + h) * D + j] +
                                  s_red[(2 * G + h) * D + j] + s_red[(3 * G + h) * D + j]};
            const float om[1] = {s_stat[h]}, ol[1] = {s_stat[G + h]};
            fold_splits<1>(om, ol, own, m[i], num[i], den[i]);
        }
    }
    float* out = a.out + ((size_t)b * a.Hq + (size_t)hk * G) * D;   // the pair's G heads, contiguous
    if constexpr (MNQ == 1) {
#pragma unroll
        for (int i = 0; i < MCPT; ++i) out[mc0 + i * MW] = den[i] > 0.0f ? num[i] / den[i] : 0.0f;
    } else {
        float* s_m = s_mg;
        float* s_num = s_mg + kThreads;
        float* s_den = s_mg + 2 * kThreads;
        s_m[tid] = m[0];
        s_num[tid] = num[0];
        s_den[tid] = den[0];
        __syncthreads();
        if (mq == 0) {
            float M = m[0];
#pragma unroll
            for (int qq = 1; qq < MNQ; ++qq) M = fmaxf(M, s_m[qq * MW + mc0]);
            float tn = 0.0f, td = 0.0f;
#pragma unroll
            for (int qq = 0; qq < MNQ; ++qq) {
                const float mqq = s_m[qq * MW + mc0];
                const float f = mqq > -INFINITY ? expf(mqq - M) : 0.0f;
                tn = fmaf(f, s_num[qq * MW + mc0], tn);
                td = fmaf(f, s_den[qq * MW + mc0], td);
            }
            out[mc0] = td > 0.0f ? tn / td : 0.0f;
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

// QK: the prompt's backbone.  0: GEAR's own; 1: KIVI (keys quantized per
// channel in groups of p.group tokens: the score takes each column's scale and
// zero of the token's group); 2: ZipCache (q is taken times the key matrix's
// channel factors, the output numerators times the value matrix's).
template <int D, int G, int BITS, int QK = 0>
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
        float fk[8];   // ZipCache: the key matrix's channel factors of the lane's columns
#pragma unroll
        for (int e = 0; e < 8; ++e) fk[e] = QK == 2 ? p.chan[(size_t)pc.mk * D + colq * 8 + e] : 1.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 w = *reinterpret_cast<const uint4*>(qb + h * D + colq * 8);
            const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
            qs[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                q[h][e] = h2f(w4[e >> 1] >> (16 * (e & 1))) * fk[e];   // exact (a power of two)
                qs[h] += q[h][e];
            }
        }
        for (int i = tid; i < G * D; i += kFastThreads)
            s_q[i] = h2f(qb[i]) * (QK == 2 ? p.chan[(size_t)pc.mk * D + i % D] : 1.0f);
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
    // (loads from clamped, always valid addresses -- with r = 0 the matrix's
    // scales stand in for A -- selected when stored: a load under a divergent
    // condition would be waited for inside its branch, and the in-order
    // counter would drain every load issued before it)
    auto load_side = [&](size_t mrow, bool scales) {
        const float* src = (tid < 128 ? p.scale : p.zero) + mrow * ngr;
        const f4v* asrc = reinterpret_cast<const f4v*>(r > 0 ? p.A + mrow * r : p.scale + mrow * ngr);
        Side sd;
        const f4v g4 = reinterpret_cast<const f4v*>(src)[min(tid & 127, ng4 - 1)];
        sd.gsz = scales ? g4 : z4;
        sd.av = asrc[min(tid, max(na4, 1) - 1)];
        return sd;
    };
    auto store_side = [&](const Side sd) {
        const int i = tid & 127;
        if (tid < 256 && i < ng4) reinterpret_cast<f4v*>(tid < 128 ? s_gs : s_gz)[i] = sd.gsz;
        if (tid < na4) reinterpret_cast<f4v*>(s_a)[tid] = sd.av;
    };
    {
        const Side sk = load_side(mrk, QK != 1);   // keys per channel: no per-token scales
        const int32_t* rpk = p.row_ptr + (size_t)pc.mk * (p.rows + 1) + pc.row0;
        const int32_t* rpv = p.row_ptr + (size_t)pc.mv * (p.rows + 1) + pc.row0;
        // threads [0, kTPS] read K's row pointers, [256, 256 + kTPS] V's
        const int ri = tid & 255;
        const int32_t rp0 = (tid < 256 ? rpk : rpv)[ri];
        const int32_t rp1 = (tid < 256 ? rpk : rpv)[kTPS];
        // B_K transposed: thread i takes element [c = i / D][j = i % D] (r D <= 1024)
        const float* bkm = r > 0 ? p.B + (size_t)pc.mk * D * r : p.scale + mrk * ngr;
        const f4v* bvm = reinterpret_cast<const f4v*>(r > 0 ? p.B + (size_t)pc.mv * D * r : p.scale + mrv * ngr);
        float bkt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = min(tid + u * kFastThreads, max(r * D, 1) - 1);
            bkt[u] = bkm[(i % D) * r + i / D];
        }
        const f4v bv = bvm[min(tid, max(nb4, 1) - 1)];
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
    // (unconditional loads from clamped indices -- with no outliers the row
    // pointers stand in for the column and value arrays -- all issued before
    // any is combined, so that they make one round trip, not one each)
    const uint16_t* rps = reinterpret_cast<const uint16_t*>(p.row_ptr);
    const uint16_t* colk = kk > 0 ? p.col + (size_t)pc.mk * kk : rps;
    const uint16_t* valk = kk > 0 ? p.val + (size_t)pc.mk * kk : rps;
    const uint16_t* colv = kk > 0 ? p.col + (size_t)pc.mv * kk : rps;
    const uint16_t* valv = kk > 0 ? p.val + (size_t)pc.mv * kk : rps;
    // (each range's loads clamped to its last entry: slots past the range
    // re-read it, no further bytes)
    const int klast = max((int)kk, 1) - 1;
    const int elast_k = min(beg_k + max(cnt_k, 1) - 1, klast), elast_v = min(beg_v + max(cnt_v, 1) - 1, klast);
    // K's entries now (one round trip); V's after the K phase, issued before
    // V's codes and combined after them, so that only they are waited for
    uint32_t ek[CPT], ev[CPT];
    auto load_csr = [&](const uint16_t* colm, const uint16_t* valm, int beg, int elast, uint32_t (&e)[CPT]) {
        uint16_t c[CPT], v[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t off = (uint32_t)min(beg + tid + j * kFastThreads, elast) * 2u;
            c[j] = ld_at<uint16_t>(colm, off);
            v[j] = ld_at<uint16_t>(valm, off);
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) e[j] = (uint32_t)c[j] | ((uint32_t)v[j] << 16);
    };
    load_csr(colk, valk, beg_k, elast_k, ek);

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
        const float av = colq < r ? s_a[aidx0 + s * astep] : 0.0f;
        float cf[8];
        unpack8<BITS>(wk[s], cf);
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = 0.0f;
        if constexpr (QK == 1) {
            // keys per channel: scale and zero of each column, the token's group
            const size_t gb = ((size_t)pc.mk * (p.rows / p.group) + (size_t)(pc.row0 + tok) / p.group) * D +
                              colq * 8;
            float csc[8], czp[8];
            {
                const float4 s0 = *reinterpret_cast<const float4*>(p.scale + gb);
                const float4 s1 = *reinterpret_cast<const float4*>(p.scale + gb + 4);
                const float4 z0 = *reinterpret_cast<const float4*>(p.zero + gb);
                const float4 z1 = *reinterpret_cast<const float4*>(p.zero + gb + 4);
                csc[0] = s0.x, csc[1] = s0.y, csc[2] = s0.z, csc[3] = s0.w;
                csc[4] = s1.x, csc[5] = s1.y, csc[6] = s1.z, csc[7] = s1.w;
                czp[0] = z0.x, czp[1] = z0.y, czp[2] = z0.z, czp[3] = z0.w;
                czp[4] = z1.x, czp[5] = z1.y, czp[6] = z1.z, czp[7] = z1.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = fmaf(q[h][e], fmaf(cf[e], csc[e], czp[e]), part[h]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float v = row_allreduce<LPR>(fmaf(av, qbl[h], part[h]));
                if (colq == 0) s_sc[tok * G + h] = v;
            }
        } else {
            const float scv = s_gs[gidx0 + s * gstep], zpv = s_gz[gidx0 + s * gstep];
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
    }
    // K's CSR entries into LDS
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (stg_k && tid + j * kFastThreads < cnt_k) s_cv[tid + j * kFastThreads] = ek[j];
    // V's CSR entries, codes and side data, consumed after the softmax
    // (issued only now, so that they hold no registers during the K phase)
    uint16_t vcol[CPT], vval[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t off = (uint32_t)min(beg_v + tid + j * kFastThreads, elast_v) * 2u;
        vcol[j] = ld_at<uint16_t>(colv, off);
        vval[j] = ld_at<uint16_t>(valv, off);
    }
    uint32_t wvv[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
        wvv[s] = BITS == 4 ? ld_at<uint32_t>(cvb, coff0 + s * RPS * ROWB)
                           : (uint32_t)ld_at<uint16_t>(cvb, coff0 + s * RPS * ROWB);
    const Side sv = load_side(mrv, true);
#pragma unroll
    for (int j = 0; j < CPT; ++j) ev[j] = (uint32_t)vcol[j] | ((uint32_t)vval[j] << 16);
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
            const float fv = QK == 2 ? p.chan[(size_t)pc.mv * D + j] : 1.0f;   // ZipCache value factor
            part[h * (D + 2) + j] = (dn + lr + sp) * fv;
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

// ---------------------------------------------------------------------------
// Whole prompt splits with G = 2, 4 or 8 query heads per KV head (head_dim
// 128, one or two quantization groups per token, GEAR's own quantizer), with
// the G-head products on the matrix cores.  fp16(q) times a small integer code
// is exact in fp32, so the products are those of the VALU kernels; only the
// order of the fp32 sums differs.
//   K: a wave's 32 tokens in two tiles of 16.  Each lane turns 8 codes of a
//      token into 8 exact fp16 values (byte permutes, minus 1024), and
//      v_mfma_f32_16x16x32_f16 gives q_h . codes_t for all heads (rows of Q,
//      zero past G) and the tile's tokens at once, one accumulator per
//      quantization group; scale, zero, low-rank and sparse terms are added
//      per token as in the VALU kernels.
//   V: per 16-token piece the codes go to the wave's fp16 LDS tile (row per
//      token), transposing reads (ds_read_b64_tr_b16) give the B operands of
//      v_mfma_f32_16x16x16_f16 with A = p_t scale_t (an fp16 hi + lo pair:
//      the product is accurate to ~2^-22); the piece's V outliers are then
//      written into the cleared tile and added the same way with A = p_t.
//      Zero-point and low-rank terms are per-head sums over the tokens.
// 8 waves, one workgroup per (split, KV head, batch); two workgroups per CU.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kMmCap = 1024;        // CSR entries of a matrix split staged in LDS
constexpr bool kUseGqaKernel = true;
constexpr int kMmWaves = 8;
constexpr int kMmThreads = 64 * kMmWaves;

// Position, among the 8 fp16 values codes_f16 makes from one word, of the
// word's e-th code: 4-bit words give the codes in the order 0,2,4,6,1,3,5,7,
// 2-bit (16-bit) words 0,4,1,5,2,6,3,7.
template <int BITS>
__device__ __forceinline__ int code_pos(int e) {
    return BITS == 4 ? ((e & 1) ? 4 + (e >> 1) : (e >> 1)) : (2 * (e & 3) + (e >> 2));
}
template <int BITS>
__device__ __forceinline__ int code_at(int p) {   // inverse of code_pos
    return BITS == 4 ? ((p < 4) ? 2 * p : 2 * (p - 4) + 1) : (4 * (p & 1) + (p >> 1));
}

// 8 codes of a word as 8 exact fp16 values (order: code_pos).  Each byte c
// becomes the fp16 pattern 0x64cc = 1024 + c, and 1024 is subtracted exactly.
template <int BITS>
__device__ __forceinline__ f16x8 codes_f16(uint32_t w) {
    uint32_t u0, u1;
    if (BITS == 4) {
        u0 = w & 0x0F0F0F0Fu;              // codes 0, 2, 4, 6 as bytes
        u1 = (w >> 4) & 0x0F0F0F0Fu;       // codes 1, 3, 5, 7
    } else {
        const uint32_t b0 = w & 0x0303u, b1 = (w >> 2) & 0x0303u;
        const uint32_t b2 = (w >> 4) & 0x0303u, b3 = (w >> 6) & 0x0303u;
        u0 = b0 | (b1 << 16);              // codes 0, 4, 1, 5
        u1 = b2 | (b3 << 16);              // codes 2, 6, 3, 7
    }
    const uint32_t k64 = 0x64646464u;
    const f16x2 m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const f16x2 h0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(k64, u0, 0x04010400u)) + m1024;
    const f16x2 h1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(k64, u0, 0x04030402u)) + m1024;
    const f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(k64, u1, 0x04010400u)) + m1024;
    const f16x2 h3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(k64, u1, 0x04030402u)) + m1024;
    return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// byte offset in the wave's V tile (16 rows of 128 fp16) of the 16-byte chunk
// c of row r, XOR-swizzled so that transposing reads and row writes spread
// over the banks
__device__ __forceinline__ int vtile_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

template <int G, int BITS, int NGR>
__global__ void __launch_bounds__(kMmThreads, NGR == 1 ? 6 : 4) attn_gqa_kernel(AttnArgs a) {
    constexpr int D = 128, TPW = kTPS / kMmWaves;       // 32 tokens per wave
    constexpr int ROWB = D * BITS / 8;                   // code bytes per token
    constexpr int CPT = kMmCap / kMmThreads;             // staged entries per thread
    constexpr int RL = G > 4 ? 32 : 16;                  // lanes holding a tile's results
    typedef float f4v __attribute__((ext_vector_type(4)));
    // LDS.  Until phase 2 the region of the per-wave V tiles (at the end, of
    // the waves' output rows) holds what only the K phase reads (q in fp32,
    // B_K transposed, K's scales, zeros, A rows and CSR entries) and V's A
    // rows (read by the sums that precede the tiles).  A rows and
    // B matrices are padded to kMaxRank with zeros, so that the rank loops
    // run unconditionally over kMaxRank.
    constexpr int kTileBytes = 16 * D * 2;
    constexpr int kVBytes = kMmWaves * kTileBytes > kMmWaves * G * D * 4 ? kMmWaves * kTileBytes
                                                                         : kMmWaves * G * D * 4;
    constexpr int kOffBkt = G * D * 4;
    constexpr int kOffGsk = kOffBkt + kMaxRank * D * 4;
    constexpr int kOffGzk = kOffGsk + kTPS * NGR * 4;
    constexpr int kOffAk = kOffGzk + kTPS * NGR * 4;
    constexpr int kOffCvk = kOffAk + kTPS * kMaxRank * 4;
    constexpr int kOffAv = kOffCvk + kMmCap * 4;   // V's A rows (read before the tiles are written)
    static_assert(kOffAv + kTPS * kMaxRank * 4 <= kVBytes, "the staged data fits the tiles' region");
    __shared__ __attribute__((aligned(16))) unsigned char s_v[kVBytes];
    float* s_q = reinterpret_cast<float*>(s_v);
    float* s_bkt = reinterpret_cast<float*>(s_v + kOffBkt);    // [c][j]
    float* s_gsk = reinterpret_cast<float*>(s_v + kOffGsk);
    float* s_gzk = reinterpret_cast<float*>(s_v + kOffGzk);
    float* s_ak = reinterpret_cast<float*>(s_v + kOffAk);
    uint32_t* s_cvk = reinterpret_cast<uint32_t*>(s_v + kOffCvk);   // column | value << 16
    float* s_a = reinterpret_cast<float*>(s_v + kOffAv);
    __shared__ __attribute__((aligned(16))) uint16_t s_qh[G * D];     // q's fp16 bits
    __shared__ __attribute__((aligned(16))) float s_qb[G * kMaxRank];
    __shared__ float s_qs[G * NGR];                      // sum of q over each group
    __shared__ float s_sc[kTPS * G];                     // scores, then probabilities
    // V's scales, zeros and CSR entries; B_V ([j][c])
    __shared__ __attribute__((aligned(16))) float s_gs[kTPS * NGR];
    __shared__ __attribute__((aligned(16))) float s_gz[kTPS * NGR];
    __shared__ uint32_t s_cv[kMmCap];
    __shared__ __attribute__((aligned(16))) float s_bv[D * kMaxRank];
    __shared__ int32_t s_rk[kTPS + 1];
    __shared__ int32_t s_rv[kTPS + 1];
    __shared__ float s_wm[4 * G];
    __shared__ float s_ws[4 * G];
    __shared__ float s_tm[kMmWaves * G * 16];           // per wave: sum_t p_t [A_t | zero_t | 1]

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int split = (int)group_id_x(), hk = (int)group_id_y(), b = (int)group_id_z();
    const int pair = b * a.Hkv + hk;
    const int t0 = split * kTPS;
    const Piece pc = find_piece(a, b, hk, t0, t0 + kTPS);
    const Packed& p = pc.p;
    const int r = p.rank;
    const uint32_t kk = (uint32_t)p.k;
    const size_t mrk = (size_t)pc.mk * p.rows + pc.row0, mrv = (size_t)pc.mv * p.rows + pc.row0;
    const int li = lane & 15, kb = lane >> 4;           // MFMA lane coordinates

    // ---------------- one round of loads: everything the split reads.  The
    // CSR ranges come from the row pointers at both ends (uniform, read
    // first).  What goes to LDS is issued first and stored at once (one wait,
    // for loads issued together); K's and V's codes stay in registers, V's in
    // flight through the K phase (the barriers wait on LDS only:
    // lds_barrier).  Every load is unconditional, from a clamped (valid)
    // address, and selected where it is stored: a load under a divergent
    // condition is waited for inside its branch, and the in-order counter
    // then drains every load issued before it.  With r = 0 or no outliers
    // the matrix's scales or row pointers stand in for the A, B, column and
    // value arrays (which may then be absent): a valid address whose value
    // is not used.
    static_assert(kTPS == 256 && kTPS * NGR / 4 <= 128 && D <= 128 && G * D <= 2 * kMmThreads,
                  "thread mapping of the staged loads");
    const int32_t* rpk = p.row_ptr + (size_t)pc.mk * (p.rows + 1) + pc.row0;
    const int32_t* rpv = p.row_ptr + (size_t)pc.mv * (p.rows + 1) + pc.row0;
    const int beg_k = min(max(rpk[0], 0), (int)kk);
    const int cnt_k = max(min(max(rpk[kTPS], 0), (int)kk) - beg_k, 0);
    const int beg_v = min(max(rpv[0], 0), (int)kk);
    const int cnt_v = max(min(max(rpv[kTPS], 0), (int)kk) - beg_v, 0);
    const bool stg_k = cnt_k <= kMmCap, stg_v = cnt_v <= kMmCap;
    // (which half, and which quarter below, a thread is in depends on its wave
    // only: read as wave-uniform, so that every base address is scalar and
    // each lane adds a 32-bit offset)
    const int half = __builtin_amdgcn_readfirstlane(tid >> 8);      // 0 stages K's data, 1 V's
    const int qtr = __builtin_amdgcn_readfirstlane((tid >> 7) & 1);
    const int ri = tid & 255;
    const size_t mrow_h = half ? mrv : mrk;
    const int ng4 = kTPS * NGR / 4, rl1 = max(r, 1) - 1;
    // scales (threads [0, 128) of a half) and zeros ([128, 256)): one float4 each
    const float* gsrc = (qtr ? p.zero : p.scale) + mrow_h * NGR;
    const f4v gsz = ld_at<f4v>(gsrc, (uint32_t)min(ri & 127, ng4 - 1) * 16u);
    // row ri of A of the half's matrix
    const float* asrc = r > 0 ? p.A + mrow_h * r : p.scale + mrow_h * NGR;
    float arow[kMaxRank];
#pragma unroll
    for (int c = 0; c < kMaxRank; ++c) arow[c] = ld_at<float>(asrc, (uint32_t)(ri * r + min(c, rl1)) * 4u);
    const uint16_t* qb = a.q + ((size_t)b * a.Hq + hk * G) * D;
    uint16_t qv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) qv[u] = ld_at<uint16_t>(qb, (uint32_t)min(tid + u * kMmThreads, G * D - 1) * 2u);
    // the half's row pointers
    const int32_t* rph = half ? rpv : rpk;
    const int32_t rp0 = ld_at<int32_t>(rph, (uint32_t)ri * 4u);
    const int32_t rp1 = rph[kTPS];
    // row bj of B_K (threads [0, 128)) or of B_V ([128, 256))
    const int bj = tid & 127;
    const float* bsrc = r > 0 ? p.B + (size_t)(qtr ? pc.mv : pc.mk) * D * r : p.scale + mrk * NGR;
    float brow[kMaxRank];
#pragma unroll
    for (int c = 0; c < kMaxRank; ++c) brow[c] = ld_at<float>(bsrc, (uint32_t)(bj * r + min(c, rl1)) * 4u);
    // both matrices' CSR entries of the split (contiguous ranges)
    const uint16_t* rps = reinterpret_cast<const uint16_t*>(rpk);
    const uint16_t* colk = kk > 0 ? p.col + (size_t)pc.mk * kk : rps;
    const uint16_t* valk = kk > 0 ? p.val + (size_t)pc.mk * kk : rps;
    const uint16_t* colv = kk > 0 ? p.col + (size_t)pc.mv * kk : rps;
    const uint16_t* valv = kk > 0 ? p.val + (size_t)pc.mv * kk : rps;
    // (each range's loads clamped to its last entry: slots past the range
    // re-read it, no further bytes)
    const int klast = max((int)kk, 1) - 1;
    const int elast_k = min(beg_k + max(cnt_k, 1) - 1, klast), elast_v = min(beg_v + max(cnt_v, 1) - 1, klast);
    uint16_t ekc[CPT], ekv[CPT], evc[CPT], evv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t ik = (uint32_t)min(beg_k + tid + j * kMmThreads, elast_k) * 2u;
        const uint32_t iv = (uint32_t)min(beg_v + tid + j * kMmThreads, elast_v) * 2u;
        ekc[j] = ld_at<uint16_t>(colk, ik);
        ekv[j] = ld_at<uint16_t>(valk, ik);
        evc[j] = ld_at<uint16_t>(colv, iv);
        evv[j] = ld_at<uint16_t>(valv, iv);
    }
    // K codes of the wave's two tiles: lane (li, kb) takes token li of a tile
    // and, for MFMA m, the 8 columns kcol(m) .. + 7: 32 contiguous columns
    // (one load) with one group per token, 16 in each group with two (the
    // MFMA's reduction order is free, as long as Q's operand follows it)
    auto kcol = [&](int m) { return NGR == 1 ? 32 * kb + 8 * m : 64 * (m >> 1) + 16 * kb + 8 * (m & 1); };
    const unsigned char* ck = p.codes + mrk * ROWB;
    uint32_t wk[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const uint32_t row = (uint32_t)((wv * TPW + tt * 16 + li) * ROWB);
        if (NGR == 1) {
            const uint32_t off = row + (uint32_t)(32 * kb * BITS / 8);
            if (BITS == 4) {
                const uint4 w = ld_at<uint4>(ck, off);
                wk[tt][0] = w.x, wk[tt][1] = w.y, wk[tt][2] = w.z, wk[tt][3] = w.w;
            } else {
                const uint2 w = ld_at<uint2>(ck, off);
                wk[tt][0] = w.x & 0xffffu, wk[tt][1] = w.x >> 16, wk[tt][2] = w.y & 0xffffu, wk[tt][3] = w.y >> 16;
            }
        } else {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const uint32_t off = row + (uint32_t)((64 * g + 16 * kb) * BITS / 8);
                if (BITS == 4) {
                    const uint2 w = ld_at<uint2>(ck, off);
                    wk[tt][2 * g] = w.x, wk[tt][2 * g + 1] = w.y;
                } else {
                    const uint32_t w = ld_at<uint32_t>(ck, off);
                    wk[tt][2 * g] = w & 0xffffu, wk[tt][2 * g + 1] = w >> 16;
                }
            }
        }
    }
    // V's codes: lane (row 4 s + kb of a 16-token piece, columns 8 li .. + 7)
    // of the wave's two pieces
    const unsigned char* cvb = p.codes + mrv * ROWB;
    uint32_t wvv[2][4];
#pragma unroll
    for (int pcs = 0; pcs < 2; ++pcs)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t off = (uint32_t)((wv * TPW + pcs * 16 + 4 * s + kb) * ROWB + li * BITS);
            wvv[pcs][s] = BITS == 4 ? ld_at<uint32_t>(cvb, off) : (uint32_t)ld_at<uint16_t>(cvb, off);
        }
    // into LDS
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (tid + u * kMmThreads < G * D) {
            s_q[tid + u * kMmThreads] = h2f(qv[u]);
            s_qh[tid + u * kMmThreads] = qv[u];
        }
    {
        float* gdst = half ? (qtr ? s_gz : s_gs) : (qtr ? s_gzk : s_gsk);
        if ((ri & 127) < ng4) reinterpret_cast<f4v*>(gdst)[ri & 127] = gsz;
        f4v a0, a1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            a0[c] = c < r ? arow[c] : 0.0f;
            a1[c] = c + 4 < r ? arow[c + 4] : 0.0f;
        }
        float* adst = (half ? s_a : s_ak) + ri * kMaxRank;
        reinterpret_cast<f4v*>(adst)[0] = a0;
        reinterpret_cast<f4v*>(adst)[1] = a1;
        int32_t* srp = half ? s_rv : s_rk;
        srp[ri] = min(max(rp0, 0), (int)kk);
        if (ri == 0) srp[kTPS] = min(max(rp1, 0), (int)kk);
    }
    if (tid < 128) {
#pragma unroll
        for (int c = 0; c < kMaxRank; ++c) s_bkt[c * D + bj] = c < r ? brow[c] : 0.0f;
    } else if (tid < 256) {
        f4v b0, b1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            b0[c] = c < r ? brow[c] : 0.0f;
            b1[c] = c + 4 < r ? brow[c + 4] : 0.0f;
        }
        reinterpret_cast<f4v*>(s_bv + bj * kMaxRank)[0] = b0;
        reinterpret_cast<f4v*>(s_bv + bj * kMaxRank)[1] = b1;
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int i = tid + j * kMmThreads;
        if (stg_k && i < cnt_k) s_cvk[i] = (uint32_t)ekc[j] | ((uint32_t)ekv[j] << 16);
        if (stg_v && i < cnt_v) s_cv[i] = (uint32_t)evc[j] | ((uint32_t)evv[j] << 16);
    }
    lds_barrier();

    // (B_K^T q)[h][c] and the sums of q over each group: 16 lanes per output,
    // D / 16 columns each, summed over the lane row
    for (int i = tid; i < G * kMaxRank * 16; i += kMmThreads) {
        const int hc = i / 16, j0 = (i % 16) * (D / 16);
        const int h = hc / kMaxRank, c = hc % kMaxRank;
        float v = 0.0f;   // (zero past the rank: s_bkt is padded with zeros)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) v = fmaf(s_q[h * D + j0 + j], s_bkt[c * D + j0 + j], v);
        v = row_allreduce<16>(v);
        if ((i % 16) == 0) s_qb[hc] = v;
    }
    for (int i = tid; i < G * NGR * 16; i += kMmThreads) {
        const int hg = i / 16, h = hg / NGR, gi = hg % NGR;
        const int j0 = gi * (D / NGR) + (i % 16) * (D / NGR / 16);
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < D / NGR / 16; ++j) v += s_q[h * D + j0 + j];
        v = row_allreduce<16>(v);
        if ((i % 16) == 0) s_qs[hg] = v;
    }
    // Q operands: row li (head, zero past G), the columns of MFMA m and lane
    // group kb in the order of the code words
    // (q's 8 fp16 values of the columns, one 16-byte read, then their halves
    // rearranged in code_pos order by byte permutes)
    f16x8 qop[4];
    {
        const int qrow = min(li, G - 1);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 w = *reinterpret_cast<const uint4*>(s_qh + qrow * D + kcol(m));
            uint32_t o0, o1, o2, o3;
            if (BITS == 4) {   // values 0, 2, 4, 6, 1, 3, 5, 7
                o0 = __builtin_amdgcn_perm(w.y, w.x, 0x05040100u);
                o1 = __builtin_amdgcn_perm(w.w, w.z, 0x05040100u);
                o2 = __builtin_amdgcn_perm(w.y, w.x, 0x07060302u);
                o3 = __builtin_amdgcn_perm(w.w, w.z, 0x07060302u);
            } else {           // values 0, 4, 1, 5, 2, 6, 3, 7
                o0 = __builtin_amdgcn_perm(w.z, w.x, 0x05040100u);
                o1 = __builtin_amdgcn_perm(w.z, w.x, 0x07060302u);
                o2 = __builtin_amdgcn_perm(w.w, w.y, 0x05040100u);
                o3 = __builtin_amdgcn_perm(w.w, w.y, 0x07060302u);
            }
            const bool on = li < G;   // rows past the heads are zero
            qop[m] = __builtin_bit_cast(f16x8, make_uint4(on ? o0 : 0u, on ? o1 : 0u, on ? o2 : 0u, on ? o3 : 0u));
        }
    }
    lds_barrier();

    // ---------------- phase 1: q . K^_t on the matrix cores
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        f32x4 acc[NGR];
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f16x8 bop = codes_f16<BITS>(wk[tt][m]);
            const int gi = NGR == 1 ? 0 : m / 2;
            acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qop[m], bop, acc[gi], 0, 0, 0);
        }
        // lane (li, kb < RL / 16) holds heads 4 kb + i of token li of the tile
        // (the zero-point, low-rank and sparse terms follow, per token)
        if (lane < RL) {
            const int tok = wv * TPW + tt * 16 + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * kb + i;
                if (h < G) {
                    float v = 0.0f;
#pragma unroll
                    for (int gi = 0; gi < NGR; ++gi) v = fmaf(s_gsk[tok * NGR + gi], acc[gi][i], v);
                    s_sc[tok * G + h] = v;
                }
            }
        }
    }
    lds_barrier();

    // ---------------- rest of the scores, softmax: two threads per token,
    // each with half of the heads (waves 0..3 the first half, 4..7 the other)
    constexpr int GH = G / 2;
    static_assert(G % 2 == 0, "an even number of query heads per KV head");
    const int tt = tid & (kTPS - 1), h0 = half * GH;
    const int wh = wv & 3;                               // wave within the half
    float pr[GH];
    {
        float add[GH];
        // zero-point and low-rank terms (A rows and B_K^T q padded with zeros
        // past the rank)
        const f4v a0 = reinterpret_cast<const f4v*>(s_ak + tt * kMaxRank)[0];
        const f4v a1 = reinterpret_cast<const f4v*>(s_ak + tt * kMaxRank)[1];
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            const int h = h0 + j;
            const f4v q0 = reinterpret_cast<const f4v*>(s_qb + h * kMaxRank)[0];
            const f4v q1 = reinterpret_cast<const f4v*>(s_qb + h * kMaxRank)[1];
            float v = 0.0f;
#pragma unroll
            for (int gi = 0; gi < NGR; ++gi) v = fmaf(s_gzk[tt * NGR + gi], s_qs[h * NGR + gi], v);
#pragma unroll
            for (int c = 0; c < 4; ++c) v = fmaf(a0[c], q0[c], fmaf(a1[c], q1[c], v));
            add[j] = v;
        }
        // the sparse term, entries in CSR order
        for (int k2 = s_rk[tt]; k2 < s_rk[tt + 1]; ++k2) {
            const uint32_t e = stg_k ? s_cvk[k2 - beg_k] : ((uint32_t)colk[k2] | ((uint32_t)valk[k2] << 16));
            const int cj = (int)(e & (D - 1));
            const float v = h2f(e >> 16);
#pragma unroll
            for (int j = 0; j < GH; ++j) add[j] = fmaf(s_q[(h0 + j) * D + cj], v, add[j]);
        }
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            pr[j] = a.sm_scale * (s_sc[tt * G + h0 + j] + add[j]);
            const float m = wave_max(pr[j]);
            if (lane == 0) s_wm[wh * G + h0 + j] = m;
        }
    }
    // (also ends the reads of the K phase's data in the tiles' region)
    lds_barrier();
    // probabilities
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        const int h = h0 + j;
        const float m = fmaxf(fmaxf(s_wm[h], s_wm[G + h]), fmaxf(s_wm[2 * G + h], s_wm[3 * G + h]));
        pr[j] = expf(pr[j] - m);
        s_sc[tt * G + h] = pr[j];
    }
    lds_barrier();
    // sum_t p_t [A_t | zero_t | 1] per head over the wave's 32 tokens, by
    // v_mfma_f32_16x16x4_f32 (M = 16 heads, N = 16 terms, K = 4 tokens; exact
    // fp32 products): lane (li, kb) gives p of head li and term li of token
    // 4 kb + i of each 16-token piece -- A_t[li] (li < 8, zero past the rank),
    // zero_t[li - 8], then 1 (the softmax denominator) -- and receives heads
    // 4 kb + 0..3 of term li.  Before the barrier that hands V's A rows' LDS
    // to the tiles.
    constexpr int kTermOne = kMaxRank + NGR;             // the column of 1
    static_assert(kTermOne < 16, "the terms fit the MFMA's 16 columns");
    {
        f32x4 tacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pcs = 0; pcs < 2; ++pcs)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = wv * TPW + pcs * 16 + 4 * kb + i;
                const float pv = li < G ? s_sc[tok * G + min(li, G - 1)] : 0.0f;
                const float av = s_a[tok * kMaxRank + min(li, kMaxRank - 1)];
                const float zv = s_gz[tok * NGR + min(max(li - kMaxRank, 0), NGR - 1)];
                const float tv = li < kMaxRank ? av : li < kTermOne ? zv : li == kTermOne ? 1.0f : 0.0f;
                tacc = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, tv, tacc, 0, 0, 0);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * kb + i < G && li <= kTermOne) s_tm[(wv * G + 4 * kb + i) * 16 + li] = tacc[i];
    }
    lds_barrier();

    // ---------------- phase 2: sum_t p_t V^_t on the matrix cores
    unsigned char* tile = s_v + wv * kTileBytes;
    f32x4 vacc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) vacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pcs = 0; pcs < 2; ++pcs) {
        const int pb = wv * TPW + pcs * 16;            // the piece's first token
        // the codes as fp16 rows of the tile (row 4 s + kb, 16-byte chunk li)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const f16x8 hv = codes_f16<BITS>(wvv[pcs][s]);
            *reinterpret_cast<f16x8*>(tile + vtile_off(4 * s + kb, li)) = hv;
        }
        // A operands: row li (head), tokens 4 kb + i of the piece
        f16x4 ahi[NGR], alo[NGR], phi, plo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = pb + 4 * kb + i;
            const float pv = li < G ? s_sc[tok * G + li] : 0.0f;
            const _Float16 h0 = (_Float16)pv;
            phi[i] = h0;
            plo[i] = (_Float16)(pv - (float)h0);
#pragma unroll
            for (int gi = 0; gi < NGR; ++gi) {
                const float ps = pv * s_gs[tok * NGR + gi];
                const _Float16 s0 = (_Float16)ps;
                ahi[gi][i] = s0;
                alo[gi][i] = (_Float16)(ps - (float)s0);
            }
        }
        __builtin_amdgcn_wave_barrier();
        // B operands: transposing reads of the tile (column 16 nb + li of rows
        // 4 kb .. 4 kb + 3); lane (li, kb) gives the address of row 4 kb + li / 4,
        // columns 16 nb + 4 (li % 4) .. + 3
        auto bop_at = [&](int nb) {
            const int row = 4 * kb + (li >> 2);
            const int col = 16 * nb + 4 * (li & 3);
            const int off = vtile_off(row, col >> 3) + (col & 7) * 2;
            return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off)));
        };
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int gi = NGR == 1 ? 0 : nb / 4;
            const f16x4 bv = bop_at(nb);
            vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi[gi], bv, vacc[nb], 0, 0, 0);
            vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(alo[gi], bv, vacc[nb], 0, 0, 0);
        }
        // the piece's V outliers: the tile cleared, each token's entries
        // written (lane li < 16 takes token pb + li), then the same products
        // with A = p_t
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s = 0; s < 4; ++s)
            *reinterpret_cast<uint4*>(tile + vtile_off(4 * s + kb, li)) = make_uint4(0u, 0u, 0u, 0u);
        __builtin_amdgcn_wave_barrier();
        const bool any = s_rv[pb + 16] > s_rv[pb];      // wave-uniform
        if (any) {
            {
                // token pb + li's entries, every fourth from the kb-th (columns
                // of a row are distinct: no two lanes write one element)
                const int tk = pb + li;
                for (int k2 = s_rv[tk] + kb; k2 < s_rv[tk + 1]; k2 += 4) {
                    const uint32_t e = stg_v ? s_cv[k2 - beg_v] : ((uint32_t)colv[k2] | ((uint32_t)valv[k2] << 16));
                    const int cj = (int)(e & (D - 1));
                    const int tc = (cj & ~7) | code_pos<BITS>(cj & 7);   // tile column of column cj
                    *reinterpret_cast<uint16_t*>(tile + vtile_off(li, tc >> 3) + (tc & 7) * 2) = (uint16_t)(e >> 16);
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const f16x4 bv = bop_at(nb);
                vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(phi, bv, vacc[nb], 0, 0, 0);
                vacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(plo, bv, vacc[nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    lds_barrier();   // every wave is done with its tile
    // the terms summed over the waves, per head: low-rank into s_qb, zero-point
    // into s_qs (whose K-side values are no longer read), 1 into s_ws
    if (tid < G * 16) {
        const int h = tid / 16, c = tid % 16;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kMmWaves; ++w) v += s_tm[(w * G + h) * 16 + c];
        if (c < kMaxRank) s_qb[h * kMaxRank + c] = v;
        else if (c < kTermOne) s_qs[h * NGR + c - kMaxRank] = v;
        else if (c == kTermOne) s_ws[h] = v;
    }
    // the waves' output rows (heads 4 kb + i, tile column 16 nb + li)
    float* rows = reinterpret_cast<float*>(s_v);
    if (lane < RL) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * kb + i;
                if (h < G) rows[(wv * G + h) * D + 16 * nb + li] = vacc[nb][i];
            }
    }
    __syncthreads();
    float* part = a.partial + ((size_t)pair * a.splits + split) * G * (D + 2);
    if (tid < G) {
        part[tid * (D + 2) + D] = fmaxf(fmaxf(s_wm[tid], s_wm[G + tid]), fmaxf(s_wm[2 * G + tid], s_wm[3 * G + tid]));
        part[tid * (D + 2) + D + 1] = s_ws[tid];
    }
    for (int i = tid; i < G * D; i += kMmThreads) {
        const int h = i / D, j = i % D;
        const int tc = (j & ~7) | code_pos<BITS>(j & 7);   // tile column of column j
        const int gi = NGR == 1 ? 0 : j / (D / NGR);
        float num = 0.0f;
#pragma unroll
        for (int w = 0; w < kMmWaves; ++w) num += rows[(w * G + h) * D + tc];
        float lr = 0.0f;   // (B_V rows padded with zeros past the rank)
        const f4v t0 = reinterpret_cast<const f4v*>(s_qb + h * kMaxRank)[0];
        const f4v t1 = reinterpret_cast<const f4v*>(s_qb + h * kMaxRank)[1];
        const f4v b0 = reinterpret_cast<const f4v*>(s_bv + j * kMaxRank)[0];
        const f4v b1 = reinterpret_cast<const f4v*>(s_bv + j * kMaxRank)[1];
#pragma unroll
        for (int c = 0; c < 4; ++c) lr = fmaf(t0[c], b0[c], fmaf(t1[c], b1[c], lr));
        part[h * (D + 2) + j] = num + s_qs[h * NGR + gi] + lr;
    }
}

// out[b][hq][:] = merge over the splits of (numerators, max, sum): one wave
// per query head, lane l taking columns l D / 64 .. (D / 64 of them).  The
// splits go in chunks of 8, whose (max, sum) pairs and the lane's numerators
// are loaded together and folded into running sums under a running maximum
// (no LDS, no barrier).
template <int D, int G>
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnArgs a) {
    constexpr int CPL = D / 64, CH = 8;
    const int lane = thread_id() & 63;
    const int bh = (int)group_id_x() * (kThreads / 64) + wave_id(thread_id());   // b * Hq + hq
    if (bh >= a.B * a.Hq) return;                     // (whole waves)
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int hk = hq / G, h = hq % G;
    const float* base = a.partial + ((size_t)(b * a.Hkv + hk) * a.splits * G + h) * (D + 2);
    const size_t stride = (size_t)G * (D + 2);        // between splits
    float m = -INFINITY, den = 0.0f, num[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] = 0.0f;
    for (int s0 = 0; s0 < a.splits; s0 += CH) {
        float ms[CH], ls[CH], vs[CH][CPL];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const float* part = base + (size_t)min(s0 + u, a.splits - 1) * stride;
            const float2 ml = *reinterpret_cast<const float2*>(part + D);
            ms[u] = ml.x;
            ls[u] = s0 + u < a.splits ? ml.y : 0.0f;   // past the last split: left out
#pragma unroll
            for (int c = 0; c < CPL; ++c) vs[u][c] = part[lane * CPL + c];
        }
        float mc = m;
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (ls[u] > 0.0f) mc = fmaxf(mc, ms[u]);
        if (mc > m) {   // the running sums to the new maximum (from -inf: times 0)
            const float f = expf(m - mc);
            den *= f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) num[c] *= f;
            m = mc;
        }
        // (selects, not branches: a load sunk into a branch would be waited
        // for there, one split after another)
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const bool in = ls[u] > 0.0f;
            const float w = expf((in ? ms[u] : m) - m);
            den = in ? fmaf(w, ls[u], den) : den;
#pragma unroll
            for (int c = 0; c < CPL; ++c) num[c] = in ? fmaf(w, vs[u][c], num[c]) : num[c];
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.out[(size_t)bh * D + lane * CPL + c] = den > 0.0f ? num[c] / den : 0.0f;
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
    // one split of attn_split_kernel per pair: that workgroup also merges the
    // pair's splits for all of its query heads (no combine launch)
    a.fuse_combine = (a.splits - a.split0 == 1) ? 1 : 0;
    hipError_t e;
    {
        Timed t(kKAttnSplit, st);
        if (a.split0 > 0) {
            const dim3 grid((unsigned)a.split0, (unsigned)a.Hkv, (unsigned)a.B);
            const int qk = a.prompt.p.chan ? 2 : a.prompt.p.ch_mats > 0 ? 1 : 0;
            // several query heads per KV head: the matrix-core kernel
            if constexpr (D == 128 && G >= 2) {
                if (qk == 0 && kUseGqaKernel) {
                    const int ngr = D / a.prompt.p.group;
                    if (a.prompt.p.bits == 4) {
                        if (ngr == 1) hipLaunchKernelGGL((attn_gqa_kernel<G, 4, 1>), grid, dim3(kMmThreads), 0, st, a);
                        else hipLaunchKernelGGL((attn_gqa_kernel<G, 4, 2>), grid, dim3(kMmThreads), 0, st, a);
                    } else {
                        if (ngr == 1) hipLaunchKernelGGL((attn_gqa_kernel<G, 2, 1>), grid, dim3(kMmThreads), 0, st, a);
                        else hipLaunchKernelGGL((attn_gqa_kernel<G, 2, 2>), grid, dim3(kMmThreads), 0, st, a);
                    }
                    goto prompt_done;
                }
            }
            if (a.prompt.p.bits == 4) {
                if (qk == 0) hipLaunchKernelGGL((attn_prompt_kernel<D, G, 4, 0>), grid, dim3(kFastThreads), 0, st, a);
                else if (qk == 1) hipLaunchKernelGGL((attn_prompt_kernel<D, G, 4, 1>), grid, dim3(kFastThreads), 0, st, a);
                else hipLaunchKernelGGL((attn_prompt_kernel<D, G, 4, 2>), grid, dim3(kFastThreads), 0, st, a);
            } else {
                if (qk == 0) hipLaunchKernelGGL((attn_prompt_kernel<D, G, 2, 0>), grid, dim3(kFastThreads), 0, st, a);
                else if (qk == 1) hipLaunchKernelGGL((attn_prompt_kernel<D, G, 2, 1>), grid, dim3(kFastThreads), 0, st, a);
                else hipLaunchKernelGGL((attn_prompt_kernel<D, G, 2, 2>), grid, dim3(kFastThreads), 0, st, a);
            }
        }
    prompt_done:
        if (a.splits > a.split0)
            hipLaunchKernelGGL((attn_split_kernel<D, G>), dim3(pairs * (a.splits - a.split0)), dim3(kThreads),
                               0, st, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.fuse_combine) return e;
    {
        Timed t(kKAttnCombine, st);
        const unsigned heads = (unsigned)(a.B * a.Hq), per = kThreads / 64;
        hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3((heads + per - 1) / per), dim3(kThreads), 0, st, a);
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
