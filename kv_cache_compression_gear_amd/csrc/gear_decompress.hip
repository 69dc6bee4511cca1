// gear_decompress.hip -- reconstruction X^ = deq(Q) + A B^T + S of packed GEAR
// matrices, for the three quantization backbones (GEAR's own, KIVI keys per
// channel, ZipCache's channel factors) ("GEAR: Efficient KV Cache Compression for LLM Inference", Q3: the
// quantized backbone, the low-rank part and the sparse part add up; app.cochat.ai
// "Cites" list, sentence quoted under the Zafrir et al. entry: low-rank for the
// coherent error, sparse for the outliers).
//
// HBM-bound streaming kernels.  A workgroup reconstructs a block of tokens of
// one matrix: every lane -- owning 8 consecutive columns of a token, D/8
// lanes per token -- issues the loads of all its tokens (one 32- or 16-bit
// code word, the group's scale and zero) and the block's row pointers and
// CSR entries before computing, and writes 8 fp16 values as one 16-byte
// store.  Without a low-rank term (decompress_kernel) the block's outliers
// are scattered into a dense fp16 LDS tile and read back as 8 values per
// lane; with one (decompress_mm_kernel) A B^T is taken on the matrix cores
// into an fp32 LDS tile per 16-row step, into which that step's outliers are
// added.
#include "gear_internal.h"

namespace gear {
namespace {

constexpr int kCsrCap = 1024;    // CSR entries of a block staged in LDS
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ uint32_t f2h(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
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

// QM: how the codes were quantized.  0: groups of head_dim columns of a token
// (GEAR's own); 1: groups of p.group tokens of a channel (KIVI keys; scale and
// zero [rows / group][D]); 2: as 0, on a matrix whose channels were divided
// by the factors p.chan (ZipCache), multiplied back here.
// No low-rank term (rank 0).
template <int D, int QM, int BITS>
__global__ void __launch_bounds__(kThreads) decompress_kernel(Packed p, uint16_t* out, int64_t m0) {
    constexpr int kSteps = 8;
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int ROWS_STEP = 4 * RPS;
    constexpr int ROWS_WG = kSteps * ROWS_STEP;
    // S of the block's rows as a dense fp16 tile (the outliers are fp16 values)
    __shared__ __attribute__((aligned(16))) uint16_t s_s[ROWS_WG * D];
    __shared__ int32_t s_rp[ROWS_WG + 1];
    __shared__ uint32_t s_cv[kCsrCap];   // column | fp16 value << 16
    // per-channel scale and zero of the block's token groups (QM 1)
    constexpr int kChG = QM == 1 ? ROWS_WG / 16 : 1;
    __shared__ __attribute__((aligned(16))) float s_cs[kChG * D];
    __shared__ __attribute__((aligned(16))) float s_cz[kChG * D];

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const int rows = p.rows;
    const int blocks_per_mat = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = m0 + group_id_x() / blocks_per_mat;
    const int row0 = (int)(group_id_x() % blocks_per_mat) * ROWS_WG;
    const int nrows = min(ROWS_WG, rows - row0);
    const int gl = p.group / 8, ngr = D / p.group;
    constexpr int bits = BITS;   // (a template parameter: one load per code word)

    // Every load below is unconditional, from a clamped (always valid)
    // address: a load under a divergent condition is waited for inside its
    // branch, and the in-order counter then drains every load issued before
    // it.  The row pointers and the CSR window go first, the tokens' loads
    // after them, so that the LDS staging below waits for the former only.
    //
    // row pointers of the block: nrows + 1 of them, up to 2 * kThreads - 1
    // (ROWS_WG <= 256)
    static_assert(ROWS_WG < 2 * kThreads, "two row pointers per thread at most");
    const int32_t* rp = p.row_ptr + (size_t)mm * (rows + 1) + row0;
    const int32_t rpv0 = rp[min(tid, nrows)];
    const int32_t rpv1 = rp[min(tid + kThreads, nrows)];
    // the block's CSR entries, guessed before the row pointers arrive: a
    // window around the block's share of k at a uniform density, 1.5 times
    // that share plus 128 entries wide (whole multiples of kThreads, at most
    // kCsrCap).  One round of loads instead of two when it covers the block's
    // range; otherwise the entries are loaded again below.  (With no outliers
    // the row pointers stand in for the column and value arrays.)
    const uint16_t* rps = reinterpret_cast<const uint16_t*>(rp);
    const uint16_t* cm = p.k > 0 ? p.col + (size_t)mm * p.k : rps;
    const uint16_t* vm = p.k > 0 ? p.val + (size_t)mm * p.k : rps;
    constexpr int EPT = kCsrCap / kThreads;   // entries per thread, at most
    const int share = (int)((int64_t)nrows * p.k / rows);
    const int wsize = min(kCsrCap, (share * 3 / 2 + 128 + kThreads - 1) / kThreads * kThreads);
    const int guess = (int)((int64_t)row0 * p.k / rows) - (wsize - share) / 2;
    const int wbeg = max(min(guess, p.k - wsize), 0);
    // (slots past the window re-read its last entry: no further bytes)
    const int wlast = min(wbeg + wsize, p.k) - 1 >= 0 ? min(wbeg + wsize, p.k) - 1 : 0;
    uint16_t wcol[EPT], wval[EPT];   // (combined where they are stored)
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const uint32_t off = (uint32_t)min(wbeg + tid + j * kThreads, wlast) * 2u;
        wcol[j] = ld_at<uint16_t>(cm, off);
        wval[j] = ld_at<uint16_t>(vm, off);
    }

    // issue the loads of all the lane's tokens first (clamped rows: always
    // valid addresses)
    const size_t mrow = (size_t)mm * rows + row0;
    const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
    const float* sbase = p.scale + mrow * ngr;
    const float* zbase = p.zero + mrow * ngr;
    uint32_t word[kSteps];
    float sc[kSteps], zp[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        const uint32_t tk = (uint32_t)min(lr, nrows - 1);
        word[s] = bits == 4 ? ld_at<uint32_t>(cbase, tk * (D / 2) + colq * 4)
                            : (uint32_t)ld_at<uint16_t>(cbase, tk * (D / 4) + colq * 2);
        if (QM != 1) {
            const uint32_t go = (tk * ngr + colq / gl) * 4;
            sc[s] = ld_at<float>(sbase, go);
            zp[s] = ld_at<float>(zbase, go);
        }
    }

    {
        uint4* t4 = reinterpret_cast<uint4*>(s_s);
        for (int i = tid; i < ROWS_WG * D / 8; i += kThreads) t4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid <= nrows) s_rp[tid] = min(max(rpv0, 0), p.k);
    if (tid + kThreads <= nrows) s_rp[tid + kThreads] = min(max(rpv1, 0), p.k);
    if constexpr (QM == 1) {
        // the groups the block's rows fall in (group >= 16 tokens, the block
        // starts at a multiple of 16): group gi of the block at s_cs[gi * D]
        const int g = p.group;
        const int gfirst = row0 / g, glast = (row0 + nrows - 1) / g;
        const float* cs = p.scale + (size_t)mm * (rows / g) * D;
        const float* cz = p.zero + (size_t)mm * (rows / g) * D;
        for (int i = tid; i < (glast - gfirst + 1) * D; i += kThreads) {
            s_cs[i] = cs[(size_t)gfirst * D + i];
            s_cz[i] = cz[(size_t)gfirst * D + i];
        }
    }
    __syncthreads();
    // the block's CSR entries: one contiguous range, from the guessed window
    // when it covers the range, else loaded again (coalesced)
    const int beg = s_rp[0], cnt = max(s_rp[nrows] - beg, 0);
    const bool staged = cnt <= kCsrCap;
    if (staged) {
        if (beg >= wbeg && beg + cnt <= wbeg + wsize) {   // workgroup-uniform
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int i = wbeg + tid + j * kThreads - beg;
                if (j * kThreads < wsize && i >= 0 && i < cnt)
                    s_cv[i] = (uint32_t)wcol[j] | ((uint32_t)wval[j] << 16);
            }
        } else {
            // all of the thread's loads in flight at once
            uint32_t ent[EPT];
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int i = tid + j * kThreads;
                ent[j] = i < cnt ? ((uint32_t)cm[beg + i] | ((uint32_t)vm[beg + i] << 16)) : 0u;
            }
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (tid + j * kThreads < cnt) s_cv[tid + j * kThreads] = ent[j];
        }
        __syncthreads();
    }
    // into the dense tile: a row's entries shared out over TPR threads (all
    // waves take part; each (row, column) is written once)
    {
        constexpr int TPR = kThreads / ROWS_WG;
        static_assert(TPR >= 1 && kThreads % ROWS_WG == 0, "threads per row");
        const int i = tid / TPR, par = tid % TPR;
        if (i < nrows) {
            for (int k = s_rp[i] + par; k < s_rp[i + 1]; k += TPR) {
                const uint32_t e = staged ? s_cv[k - beg] : ((uint32_t)cm[k] | ((uint32_t)vm[k] << 16));
                s_s[i * D + (e & (D - 1))] = (uint16_t)(e >> 16);
            }
        }
    }
    float one = 1.0f;   // opaque 1: keeps the outlier add a single mixed fma
    asm volatile("" : "+s"(one));
    float cfac[8];      // QM 2: the channel factors of the lane's columns
    if constexpr (QM == 2) {
        const float4 f0 = *reinterpret_cast<const float4*>(p.chan + (size_t)mm * D + colq * 8);
        const float4 f1 = *reinterpret_cast<const float4*>(p.chan + (size_t)mm * D + colq * 8 + 4);
        cfac[0] = f0.x, cfac[1] = f0.y, cfac[2] = f0.z, cfac[3] = f0.w;
        cfac[4] = f1.x, cfac[5] = f1.y, cfac[6] = f1.z, cfac[7] = f1.w;
    }
    __syncthreads();   // the dense tile is complete

#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        if (s * ROWS_STEP + wv * RPS >= nrows) break;    // wave-uniform
        const uint4 sv = *reinterpret_cast<const uint4*>(s_s + min(lr, ROWS_WG - 1) * D + colq * 8);
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
        float cf[8];
        if (bits == 4) {
            // the 8 nibbles as bytes of two words, each converted in one step
            const uint32_t lo = word[s] & 0x0F0F0F0Fu, hi = (word[s] >> 4) & 0x0F0F0F0Fu;
            cf[0] = ubyte_f<0>(lo), cf[2] = ubyte_f<1>(lo), cf[4] = ubyte_f<2>(lo), cf[6] = ubyte_f<3>(lo);
            cf[1] = ubyte_f<0>(hi), cf[3] = ubyte_f<1>(hi), cf[5] = ubyte_f<2>(hi), cf[7] = ubyte_f<3>(hi);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cf[e] = (float)((word[s] >> (2 * e)) & 3u);
        }
        float x[8];
        float csc[8], czp[8];   // QM 1: this row's group, the lane's columns
        if constexpr (QM == 1) {
            const int gi = (row0 + min(lr, nrows - 1)) / p.group - row0 / p.group;
            const float4 s0 = *reinterpret_cast<const float4*>(s_cs + gi * D + colq * 8);
            const float4 s1 = *reinterpret_cast<const float4*>(s_cs + gi * D + colq * 8 + 4);
            const float4 z0 = *reinterpret_cast<const float4*>(s_cz + gi * D + colq * 8);
            const float4 z1 = *reinterpret_cast<const float4*>(s_cz + gi * D + colq * 8 + 4);
            csc[0] = s0.x, csc[1] = s0.y, csc[2] = s0.z, csc[3] = s0.w;
            csc[4] = s1.x, csc[5] = s1.y, csc[6] = s1.z, csc[7] = s1.w;
            czp[0] = z0.x, czp[1] = z0.y, czp[2] = z0.z, czp[3] = z0.w;
            czp[4] = z1.x, czp[5] = z1.y, czp[6] = z1.z, czp[7] = z1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = QM == 1 ? fmaf(cf[e], csc[e], czp[e]) : fmaf(cf[e], sc[s], zp[s]);
            // + the fp16 outlier value (fp16 operand of a mixed fma)
            x[e] = fmaf(h2f(sw[e >> 1] >> (16 * (e & 1))), one, v);
            if (QM == 2) x[e] *= cfac[e];   // a power of two: exact
        }
        if (lr < nrows) {
            u32x4 o;
            o.x = f2h(x[0]) | (f2h(x[1]) << 16);
            o.y = f2h(x[2]) | (f2h(x[3]) << 16);
            o.z = f2h(x[4]) | (f2h(x[5]) << 16);
            o.w = f2h(x[6]) | (f2h(x[7]) << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (mrow + lr) * D + colq * 8));
        }
    }
}

// With a low-rank term (rank 1..8) the product A·B^T goes to the matrix
// cores.  Per 16-row block and 16 columns, v_mfma_f32_16x16x4_f32 takes B's
// rows (16 columns x 4 rank slots) as its first operand and A's rows as its
// second, so that lane l receives L[row0 + l % 16][16 cb + 4 (l / 16) + i],
// i = 0..3: four consecutive columns of one row, one 16-byte write into the
// step's fp32 LDS tile (rows padded by 4 floats: the 16 rows of a write fall
// on distinct banks).  The step's outliers are added into the tile (each
// (row, column) once: a plain read-add-write), and each lane then reads its
// 8 columns back and adds fma(code, scale, zero).  Rank 8 takes two products
// per block (K = 4 each); ranks below a multiple of 4 meet B's zero padding.
// The loads are issued as in decompress_kernel (row pointers, CSR window and
// B first, then every token's code word, scale, zero and A row).
constexpr int kMmPad = 4;        // floats of padding per tile row
// CSR entries of a (128-row) block staged in LDS: more with rank 8, whose
// 2-bit workload keeps 5 % of the entries
template <int RK>
constexpr int mm_csr_cap() { return RK >= 8 ? 2048 : 1024; }

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, int RK, int QM, int BITS>
__global__ void __launch_bounds__(kThreads) decompress_mm_kernel(Packed p, uint16_t* out, int64_t m0) {
    constexpr int kSteps = 8;
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int ROWS_STEP = 4 * RPS;            // 16 (d = 128) or 32 (d = 64)
    constexpr int ROWS_WG = kSteps * ROWS_STEP;
    constexpr int kMmCsrCap = mm_csr_cap<RK>();
    constexpr int KP = RK <= 4 ? 4 : 8;           // rank slots of the products
    constexpr int NH = KP / 4;                    // products per block
    constexpr int TW = D + kMmPad;                // tile row stride (floats)
    constexpr int CB = D / 16;                    // column blocks
    static_assert(RK > 0 && ROWS_STEP * D == 8 * 256, "8 blocks of 16 x 16 per step, 2 per wave");
    static_assert(ROWS_WG < 2 * kThreads, "two row pointers per thread at most");
    __shared__ __attribute__((aligned(16))) float s_t[2][ROWS_STEP * TW];
    __shared__ __attribute__((aligned(16))) float s_b[D * KP];   // B, [j][c], zero past the rank
    __shared__ int32_t s_rp[ROWS_WG + 1];
    __shared__ uint32_t s_cv[kMmCsrCap];   // column | fp16 value << 16
    constexpr int kChG = QM == 1 ? ROWS_WG / 16 : 1;
    __shared__ __attribute__((aligned(16))) float s_cs[kChG * D];
    __shared__ __attribute__((aligned(16))) float s_cz[kChG * D];

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const int li = lane & 15, kq = lane >> 4;     // MFMA lane coordinates
    const int rows = p.rows;
    const int blocks_per_mat = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = m0 + group_id_x() / blocks_per_mat;
    const int row0 = (int)(group_id_x() % blocks_per_mat) * ROWS_WG;
    const int nrows = min(ROWS_WG, rows - row0);
    const int r = p.rank, gl = p.group / 8, ngr = D / p.group, rl1 = max(r, 1) - 1;
    constexpr int bits = BITS;

    // ---- loads: row pointers, the CSR window and B first (they are staged
    // before the tokens' loads are needed), then the tokens'
    const int32_t* rp = p.row_ptr + (size_t)mm * (rows + 1) + row0;
    const int32_t rpv0 = rp[min(tid, nrows)];
    const int32_t rpv1 = rp[min(tid + kThreads, nrows)];
    const uint16_t* rps = reinterpret_cast<const uint16_t*>(rp);
    const uint16_t* cm = p.k > 0 ? p.col + (size_t)mm * p.k : rps;
    const uint16_t* vm = p.k > 0 ? p.val + (size_t)mm * p.k : rps;
    constexpr int EPT = kMmCsrCap / kThreads;
    const int share = (int)((int64_t)nrows * p.k / rows);
    const int wsize = min(kMmCsrCap, (share * 3 / 2 + 128 + kThreads - 1) / kThreads * kThreads);
    const int guess = (int)((int64_t)row0 * p.k / rows) - (wsize - share) / 2;
    const int wbeg = max(min(guess, p.k - wsize), 0);
    // (slots past the window re-read its last entry: no further bytes)
    const int wlast = max(min(wbeg + wsize, p.k) - 1, 0);
    uint16_t wcol[EPT], wval[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const uint32_t off = (uint32_t)min(wbeg + tid + j * kThreads, wlast) * 2u;
        wcol[j] = ld_at<uint16_t>(cm, off);
        wval[j] = ld_at<uint16_t>(vm, off);
    }
    constexpr int BPT = D * KP / kThreads;   // B slots per thread (2 or 4)
    const float* bsrc = p.B + (size_t)mm * D * r;
    float bv[BPT];
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        const int i = tid + u * kThreads;
        bv[u] = ld_at<float>(bsrc, (uint32_t)((i / KP) * r + min(i % KP, rl1)) * 4u);
    }
    const size_t mrow = (size_t)mm * rows + row0;
    const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
    const float* sbase = p.scale + mrow * ngr;
    const float* zbase = p.zero + mrow * ngr;
    const float* abase = p.A + mrow * r;
    // the wave's blocks: row block rbw of the step, column blocks 2 wv % CB
    // and 2 wv % CB + 1
    const int rbw = (2 * wv) / CB, cb0 = (2 * wv) % CB;
    uint32_t word[kSteps];
    float sc[kSteps], zp[kSteps], ay[kSteps][NH];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        const uint32_t tk = (uint32_t)min(lr, nrows - 1);
        word[s] = bits == 4 ? ld_at<uint32_t>(cbase, tk * (D / 2) + colq * 4)
                            : (uint32_t)ld_at<uint16_t>(cbase, tk * (D / 4) + colq * 2);
        if (QM != 1) {
            const uint32_t go = (tk * ngr + colq / gl) * 4;
            sc[s] = ld_at<float>(sbase, go);
            zp[s] = ld_at<float>(zbase, go);
        }
        // A[row][c] for the products: row rbw 16 + li of the step, slot kq (+ 4 h)
        const uint32_t ar = (uint32_t)min(s * ROWS_STEP + rbw * 16 + li, nrows - 1);
#pragma unroll
        for (int h = 0; h < NH; ++h) ay[s][h] = ld_at<float>(abase, (ar * r + (uint32_t)min(kq + 4 * h, rl1)) * 4u);
    }

    // ---- staging
    if (tid <= nrows) s_rp[tid] = min(max(rpv0, 0), p.k);
    if (tid + kThreads <= nrows) s_rp[tid + kThreads] = min(max(rpv1, 0), p.k);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        const int i = tid + u * kThreads;
        s_b[i] = (i % KP) < r ? bv[u] : 0.0f;
    }
    if constexpr (QM == 1) {
        const int g = p.group;
        const int gfirst = row0 / g, glast = (row0 + nrows - 1) / g;
        const float* cs = p.scale + (size_t)mm * (rows / g) * D;
        const float* cz = p.zero + (size_t)mm * (rows / g) * D;
        for (int i = tid; i < (glast - gfirst + 1) * D; i += kThreads) {
            s_cs[i] = cs[(size_t)gfirst * D + i];
            s_cz[i] = cz[(size_t)gfirst * D + i];
        }
    }
    __syncthreads();
    const int beg = s_rp[0], cnt = max(s_rp[nrows] - beg, 0);
    const bool staged = cnt <= kMmCsrCap;
    if (staged) {
        if (beg >= wbeg && beg + cnt <= wbeg + wsize) {   // workgroup-uniform
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int i = wbeg + tid + j * kThreads - beg;
                if (i >= 0 && i < cnt) s_cv[i] = (uint32_t)wcol[j] | ((uint32_t)wval[j] << 16);
            }
        } else {
            uint32_t ent[EPT];
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int i = tid + j * kThreads;
                ent[j] = i < cnt ? ((uint32_t)cm[beg + i] | ((uint32_t)vm[beg + i] << 16)) : 0u;
            }
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (tid + j * kThreads < cnt) s_cv[tid + j * kThreads] = ent[j];
        }
    }
    // the products' first operands: B's rows 16 cb + li, slot kq (+ 4 h)
    float xb[2][NH];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int h = 0; h < NH; ++h) xb[k][h] = s_b[((cb0 + k) * 16 + li) * KP + kq + 4 * h];
    float cfac[8];   // QM 2: the channel factors of the lane's columns
    if constexpr (QM == 2) {
        const float4 f0 = *reinterpret_cast<const float4*>(p.chan + (size_t)mm * D + colq * 8);
        const float4 f1 = *reinterpret_cast<const float4*>(p.chan + (size_t)mm * D + colq * 8 + 4);
        cfac[0] = f0.x, cfac[1] = f0.y, cfac[2] = f0.z, cfac[3] = f0.w;
        cfac[4] = f1.x, cfac[5] = f1.y, cfac[6] = f1.z, cfac[7] = f1.w;
    }

    constexpr int TPR = kThreads / ROWS_STEP;   // threads per row for the outliers
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s * ROWS_STEP >= nrows) break;   // workgroup-uniform
        // (two tiles: a wave writes step s's while another may still read
        // step s - 1's; step s - 2's readers have all passed step s - 1's
        // barriers)
        float* tl = s_t[s & 1];
        // 1. the wave's two blocks of L
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < NH; ++h) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xb[k][h], ay[s][h], acc, 0, 0, 0);
            *reinterpret_cast<f32x4*>(tl + (rbw * 16 + li) * TW + (cb0 + k) * 16 + 4 * kq) = acc;
        }
        __syncthreads();
        // 2. the step's outliers added into the tile
        {
            const int i = tid / TPR, par = tid % TPR;
            const int row = s * ROWS_STEP + i;
            if (row < nrows) {
                for (int k2 = s_rp[row] + par; k2 < s_rp[row + 1]; k2 += TPR) {
                    const uint32_t e = staged ? s_cv[k2 - beg] : ((uint32_t)cm[k2] | ((uint32_t)vm[k2] << 16));
                    tl[i * TW + (e & (D - 1))] += h2f(e >> 16);
                }
            }
        }
        __syncthreads();
        // 3. the lane's 8 columns: fma(code, scale, zero) + L + S
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        const float4 l0 = *reinterpret_cast<const float4*>(tl + (wv * RPS + rl) * TW + colq * 8);
        const float4 l1 = *reinterpret_cast<const float4*>(tl + (wv * RPS + rl) * TW + colq * 8 + 4);
        const float lt[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        float cf[8];
        if (bits == 4) {
            const uint32_t lo = word[s] & 0x0F0F0F0Fu, hi = (word[s] >> 4) & 0x0F0F0F0Fu;
            cf[0] = ubyte_f<0>(lo), cf[2] = ubyte_f<1>(lo), cf[4] = ubyte_f<2>(lo), cf[6] = ubyte_f<3>(lo);
            cf[1] = ubyte_f<0>(hi), cf[3] = ubyte_f<1>(hi), cf[5] = ubyte_f<2>(hi), cf[7] = ubyte_f<3>(hi);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cf[e] = (float)((word[s] >> (2 * e)) & 3u);
        }
        float csc[8], czp[8];
        if constexpr (QM == 1) {
            const int gi = (row0 + min(lr, nrows - 1)) / p.group - row0 / p.group;
            const float4 s0 = *reinterpret_cast<const float4*>(s_cs + gi * D + colq * 8);
            const float4 s1 = *reinterpret_cast<const float4*>(s_cs + gi * D + colq * 8 + 4);
            const float4 z0 = *reinterpret_cast<const float4*>(s_cz + gi * D + colq * 8);
            const float4 z1 = *reinterpret_cast<const float4*>(s_cz + gi * D + colq * 8 + 4);
            csc[0] = s0.x, csc[1] = s0.y, csc[2] = s0.z, csc[3] = s0.w;
            csc[4] = s1.x, csc[5] = s1.y, csc[6] = s1.z, csc[7] = s1.w;
            czp[0] = z0.x, czp[1] = z0.y, czp[2] = z0.z, czp[3] = z0.w;
            czp[4] = z1.x, czp[5] = z1.y, czp[6] = z1.z, czp[7] = z1.w;
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = QM == 1 ? fmaf(cf[e], csc[e], czp[e]) : fmaf(cf[e], sc[s], zp[s]);
            x[e] = v + lt[e];
            if (QM == 2) x[e] *= cfac[e];   // a power of two: exact
        }
        if (lr < nrows) {
            u32x4 o;
            o.x = f2h(x[0]) | (f2h(x[1]) << 16);
            o.y = f2h(x[2]) | (f2h(x[3]) << 16);
            o.z = f2h(x[4]) | (f2h(x[5]) << 16);
            o.w = f2h(x[6]) | (f2h(x[7]) << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (mrow + lr) * D + colq * 8));
        }
    }
}

template <int D, int RK, int QM>
hipError_t launch_drq(const Packed& p, uint16_t* out, int64_t m0, int64_t m1, hipStream_t st) {
    if constexpr (RK > 0) {
        constexpr int ROWS_WG = 8 * 4 * (64 / (D / 8));
        const int64_t blocks = (m1 - m0) * ((p.rows + ROWS_WG - 1) / ROWS_WG);
        if (blocks <= 0) return hipSuccess;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        Timed t(kKDecompress, st);
        if (p.bits == 4)
            hipLaunchKernelGGL((decompress_mm_kernel<D, RK, QM, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                               p, out, m0);
        else
            hipLaunchKernelGGL((decompress_mm_kernel<D, RK, QM, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                               p, out, m0);
        return hipGetLastError();
    } else {
        constexpr int ROWS_WG = 8 * 4 * (64 / (D / 8));
        const int64_t blocks = (m1 - m0) * ((p.rows + ROWS_WG - 1) / ROWS_WG);
        if (blocks <= 0) return hipSuccess;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        Timed t(kKDecompress, st);
        if (p.bits == 4)
            hipLaunchKernelGGL((decompress_kernel<D, QM, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p,
                               out, m0);
        else
            hipLaunchKernelGGL((decompress_kernel<D, QM, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p,
                               out, m0);
        return hipGetLastError();
    }
}

template <int D, int RK>
hipError_t launch_dr(const Packed& p, uint16_t* out, hipStream_t st) {
    if (p.chan) return launch_drq<D, RK, 2>(p, out, 0, p.M, st);
    hipError_t e = hipSuccess;
    if (p.ch_mats > 0) e = launch_drq<D, RK, 1>(p, out, 0, p.ch_mats, st);
    if (e == hipSuccess && p.ch_mats < p.M) e = launch_drq<D, RK, 0>(p, out, p.ch_mats, p.M, st);
    return e;
}

template <int D>
hipError_t launch_d(const Packed& p, uint16_t* out, hipStream_t st) {
    switch (rank_slots(p.rank)) {
        case 0: return launch_dr<D, 0>(p, out, st);
        case 2: return launch_dr<D, 2>(p, out, st);
        case 4: return launch_dr<D, 4>(p, out, st);
        default: return launch_dr<D, 8>(p, out, st);
    }
}

}  // namespace

hipError_t launch_decompress(const Packed& p, uint16_t* out, hipStream_t st) {
    if (p.d == 64) return launch_d<64>(p, out, st);
    if (p.d == 128) return launch_d<128>(p, out, st);
    return hipErrorInvalidValue;
}

}  // namespace gear
