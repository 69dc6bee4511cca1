// gear_decompress.hip -- reconstruction X^ = deq(Q) + A B^T + S of packed GEAR
// matrices ("GEAR: Efficient KV Cache Compression for LLM Inference", Q3: the
// quantized backbone, the low-rank part and the sparse part add up; app.cochat.ai
// "Cites" list, sentence quoted under the Zafrir et al. entry: low-rank for the
// coherent error, sparse for the outliers).
//
// HBM-bound streaming kernel.  A workgroup reconstructs a block of tokens of
// one matrix: every lane
// -- owning 8 consecutive columns of a token, D/8 lanes per token -- issues the
// loads of all its tokens (one 32- or 16-bit code word, the group's scale and
// zero, the token's A row) and the block's row pointers before computing.
// The block's CSR entries (one contiguous range) are then loaded coalesced
// into LDS and written into a dense fp16 LDS tile (each row's entries shared
// out over kThreads / rows threads), read back as 8 values per lane; each lane
// writes 8 fp16 values as one 16-byte store.
#include "gear_internal.h"

namespace gear {
namespace {

// token rows per lane: 8, or 4 with rank 8 (the A rows of all steps are held
// in registers)
constexpr int steps_for(int rk) { return rk >= 8 ? 4 : 8; }
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

template <int D, int RK>
__global__ void __launch_bounds__(kThreads) decompress_kernel(Packed p, uint16_t* out) {
    constexpr int kSteps = steps_for(RK);
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int ROWS_STEP = 4 * RPS;
    constexpr int ROWS_WG = kSteps * ROWS_STEP;
    constexpr int RKX = RK > 0 ? RK : 1;
    // B as [e][colq][c]: lane colq reads B[colq * 8 + e][0..RKX) contiguously
    __shared__ __attribute__((aligned(16))) float s_b[D * RKX];
    // S of the block's rows as a dense fp16 tile (the outliers are fp16 values)
    __shared__ __attribute__((aligned(16))) uint16_t s_s[ROWS_WG * D];
    __shared__ int32_t s_rp[ROWS_WG + 1];
    __shared__ uint32_t s_cv[kCsrCap];   // column | fp16 value << 16

    const int tid = thread_id(), lane = tid & 63, wv = wave_id(tid);
    const int colq = lane % LPR, rl = lane / LPR;
    const int rows = p.rows;
    const int blocks_per_mat = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = group_id_x() / blocks_per_mat;
    const int row0 = (int)(group_id_x() % blocks_per_mat) * ROWS_WG;
    const int nrows = min(ROWS_WG, rows - row0);
    const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;

    // issue the loads of all the lane's tokens first (clamped rows: always
    // valid addresses)
    const size_t mrow = (size_t)mm * rows + row0;
    const unsigned char* cbase = p.codes + mrow * (D * bits / 8);
    const float* sbase = p.scale + mrow * ngr;
    const float* zbase = p.zero + mrow * ngr;
    const float* abase = p.A + mrow * r;
    uint32_t word[kSteps];
    float sc[kSteps], zp[kSteps], ar[kSteps][RKX];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        const uint32_t tk = (uint32_t)min(lr, nrows - 1);
        word[s] = bits == 4 ? ld_at<uint32_t>(cbase, tk * (D / 2) + colq * 4)
                            : (uint32_t)ld_at<uint16_t>(cbase, tk * (D / 4) + colq * 2);
        const uint32_t go = (tk * ngr + colq / gl) * 4;
        sc[s] = ld_at<float>(sbase, go);
        zp[s] = ld_at<float>(zbase, go);
        if (RK > 0 && r == RK) {            // the A row as one or two vector loads
            if (RK >= 4) {
#pragma unroll
                for (int c4 = 0; c4 < RKX / 4; ++c4) {
                    const float4 a4 = ld_at<float4>(abase, (tk * RK + 4 * c4) * 4);
                    ar[s][(4 * c4) % RKX] = a4.x;
                    ar[s][(4 * c4 + 1) % RKX] = a4.y;
                    ar[s][(4 * c4 + 2) % RKX] = a4.z;
                    ar[s][(4 * c4 + 3) % RKX] = a4.w;
                }
            } else {
                const float2 a2 = ld_at<float2>(abase, tk * RK * 4);
                ar[s][0] = a2.x;
                ar[s][1 % RKX] = a2.y;
            }
        } else {
#pragma unroll
            for (int c = 0; c < RKX; ++c) ar[s][c] = (RK > 0 && c < r) ? ld_at<float>(abase, (tk * r + c) * 4) : 0.0f;
        }
    }

    // row pointers of the block (with the loads above), S tile cleared, B
    // nrows + 1 pointers, up to 2 * kThreads - 1 of them (ROWS_WG <= 256)
    static_assert(ROWS_WG < 2 * kThreads, "two row pointers per thread at most");
    const int32_t* rp = p.row_ptr + (size_t)mm * (rows + 1) + row0;
    const int32_t rpv0 = tid <= nrows ? rp[tid] : 0;
    const int32_t rpv1 = tid + kThreads <= nrows ? rp[tid + kThreads] : 0;
    // the block's CSR entries, guessed before the row pointers arrive: a
    // window around the block's share of k at a uniform density, 1.5 times
    // that share plus 128 entries wide (whole multiples of kThreads, at most
    // kCsrCap).  One round of loads instead of two when it covers the block's
    // range; otherwise the entries are loaded again below.
    const uint16_t* cm = p.col + (size_t)mm * p.k;
    const uint16_t* vm = p.val + (size_t)mm * p.k;
    constexpr int EPT = kCsrCap / kThreads;   // entries per thread, at most
    const int share = (int)((int64_t)nrows * p.k / rows);
    const int wsize = min(kCsrCap, (share * 3 / 2 + 128 + kThreads - 1) / kThreads * kThreads);
    const int guess = (int)((int64_t)row0 * p.k / rows) - (wsize - share) / 2;
    const int wbeg = max(min(guess, p.k - wsize), 0);
    uint32_t went[EPT] = {};
    if (p.k > 0) {   // workgroup-uniform; indices clamped to valid entries
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (j * kThreads >= wsize) break;   // workgroup-uniform
            const int ic = min(wbeg + tid + j * kThreads, p.k - 1);
            went[j] = (uint32_t)cm[ic] | ((uint32_t)vm[ic] << 16);
        }
    }
    {
        uint4* t4 = reinterpret_cast<uint4*>(s_s);
        for (int i = tid; i < ROWS_WG * D / 8; i += kThreads) t4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (RK > 0)
        for (int i = tid; i < D * RKX; i += kThreads) {
            const int j = i / RKX, c = i % RKX;
            s_b[((j % 8) * LPR + j / 8) * RKX + c] = c < r ? p.B[((size_t)mm * D + j) * r + c] : 0.0f;
        }
    if (tid <= nrows) s_rp[tid] = min(max(rpv0, 0), p.k);
    if (tid + kThreads <= nrows) s_rp[tid + kThreads] = min(max(rpv1, 0), p.k);
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
                if (j * kThreads < wsize && i >= 0 && i < cnt) s_cv[i] = went[j];
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
    float Bm[8][RKX];
    float one = 1.0f;   // opaque 1: keeps the outlier add a single mixed fma
    asm volatile("" : "+s"(one));
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < RKX; ++c) Bm[e][c] = RK > 0 ? s_b[(e * LPR + colq) * RKX + c] : 0.0f;

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
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = fmaf(cf[e], sc[s], zp[s]);
#pragma unroll
            for (int c = 0; c < RKX; ++c) v = fmaf(ar[s][c], Bm[e][c], v);
            // + the fp16 outlier value (fp16 operand of a mixed fma)
            x[e] = fmaf(h2f(sw[e >> 1] >> (16 * (e & 1))), one, v);
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

template <int D, int RK>
hipError_t launch_dr(const Packed& p, uint16_t* out, hipStream_t st) {
    constexpr int ROWS_WG = steps_for(RK) * 4 * (64 / (D / 8));
    const int64_t blocks = p.M * ((p.rows + ROWS_WG - 1) / ROWS_WG);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    Timed t(kKDecompress, st);
    hipLaunchKernelGGL((decompress_kernel<D, RK>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, out);
    return hipGetLastError();
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
