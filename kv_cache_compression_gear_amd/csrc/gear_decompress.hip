// gear_decompress.hip -- reconstruction X^ = deq(Q) + A B^T + S of packed GEAR
// matrices ("GEAR: Efficient KV Cache Compression for LLM Inference", Q3: the
// quantized backbone, the low-rank part and the sparse part add up; app.cochat.ai
// "Cites" list, sentence quoted under the Zafrir et al. entry: low-rank for the
// coherent error, sparse for the outliers).
//
// HBM-bound streaming kernel.  A workgroup reconstructs a block of tokens of
// one matrix: it first stages the block's slice of row_ptr and its outliers
// (contiguous in the CSR arrays) in LDS with coalesced loads, then every lane
// -- owning 8 consecutive columns of a token, D/8 lanes per token -- issues the
// loads of all its tokens (one 32- or 16-bit code word, the group's scale and
// zero, the token's A row) before computing, adds its outliers from LDS, and
// writes 8 fp16 values as one 16-byte store.
#include "gear_internal.h"

namespace gear {
namespace {

constexpr int kSteps = 8;        // token rows per lane
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCsrCap = 4096;    // outliers a block stages in LDS

__device__ __forceinline__ float h2f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ uint32_t f2h(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int D, int RK>
__global__ void __launch_bounds__(kThreads) decompress_kernel(Packed p, uint16_t* out) {
    constexpr int LPR = D / 8, RPS = 64 / LPR;
    constexpr int ROWS_STEP = 4 * RPS;
    constexpr int ROWS_WG = kSteps * ROWS_STEP;
    constexpr int RKX = RK > 0 ? RK : 1;
    __shared__ int32_t s_rp[ROWS_WG + 1];
    __shared__ uint32_t s_cv[kCsrCap];       // col | (fp16 value << 16)
    __shared__ float s_b[D * RKX];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const int rows = p.rows;
    const int blocks_per_mat = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = blockIdx.x / blocks_per_mat;
    const int row0 = (int)(blockIdx.x % blocks_per_mat) * ROWS_WG;
    const int nrows = min(ROWS_WG, rows - row0);
    const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
    const uint32_t cmask = (1u << bits) - 1u;

    const int32_t* rp = p.row_ptr + (size_t)mm * (rows + 1) + row0;
    const uint16_t* cm = p.col + (size_t)mm * p.k;
    const uint16_t* vm = p.val + (size_t)mm * p.k;
    for (int i = tid; i <= nrows; i += kThreads) s_rp[i] = min(max(rp[i], 0), p.k);
    if (RK > 0)
        for (int i = tid; i < D * RKX; i += kThreads) {
            const int j = i / RKX, c = i % RKX;
            s_b[i] = c < r ? p.B[((size_t)mm * D + j) * r + c] : 0.0f;
        }
    __syncthreads();
    const int beg = s_rp[0], cnt = max(s_rp[nrows] - beg, 0);
    const bool staged = cnt <= kCsrCap;
    if (staged)
        for (int i = tid; i < cnt; i += kThreads)
            s_cv[i] = (uint32_t)cm[beg + i] | ((uint32_t)vm[beg + i] << 16);

    // all loads of the lane's tokens first
    uint32_t word[kSteps];
    float sc[kSteps], zp[kSteps], ar[kSteps][RKX];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        const bool ok = lr < nrows;
        const size_t grow = (size_t)mm * rows + row0 + (ok ? lr : 0);
        word[s] = 0u;
        sc[s] = zp[s] = 0.0f;
        if (ok) {
            word[s] = bits == 4 ? reinterpret_cast<const uint32_t*>(p.codes)[grow * (D / 8) + colq]
                                : reinterpret_cast<const uint16_t*>(p.codes)[grow * (D / 8) + colq];
            sc[s] = p.scale[grow * ngr + colq / gl];
            zp[s] = p.zero[grow * ngr + colq / gl];
        }
#pragma unroll
        for (int c = 0; c < RKX; ++c) ar[s][c] = (RK > 0 && ok && c < r) ? p.A[grow * r + c] : 0.0f;
    }
    float Bm[8][RKX];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < RKX; ++c) Bm[e][c] = RK > 0 ? s_b[(colq * 8 + e) * RKX + c] : 0.0f;

#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int lr = s * ROWS_STEP + wv * RPS + rl;
        if (lr >= nrows) continue;
        const size_t grow = (size_t)mm * rows + row0 + lr;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = fmaf((float)((word[s] >> (e * bits)) & cmask), sc[s], zp[s]);
#pragma unroll
            for (int c = 0; c < RKX; ++c) v = fmaf(ar[s][c], Bm[e][c], v);
            x[e] = v;
        }
        const int lo = max(s_rp[lr] - beg, 0), hi = min(s_rp[lr + 1] - beg, cnt);
        for (int i = lo; i < hi; ++i) {
            const uint32_t cv = staged ? s_cv[i]
                                       : ((uint32_t)cm[beg + i] | ((uint32_t)vm[beg + i] << 16));
            const int cj = (int)(cv & 0xffffu);
            if ((cj >> 3) == colq) {
                const float v = h2f(cv >> 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] += ((cj & 7) == e) ? v : 0.0f;
            }
        }
        u32x4 o;
        o.x = f2h(x[0]) | (f2h(x[1]) << 16);
        o.y = f2h(x[2]) | (f2h(x[3]) << 16);
        o.z = f2h(x[4]) | (f2h(x[5]) << 16);
        o.w = f2h(x[6]) | (f2h(x[7]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + grow * D + colq * 8));
    }
}

template <int D>
hipError_t launch_d(const Packed& p, uint16_t* out, hipStream_t st) {
    constexpr int ROWS_WG = kSteps * 4 * (64 / (D / 8));
    const int64_t blocks = p.M * ((p.rows + ROWS_WG - 1) / ROWS_WG);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    Timed t(kKDecompress, st);
    switch (rank_slots(p.rank)) {
        case 0: hipLaunchKernelGGL((decompress_kernel<D, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, out); break;
        case 2: hipLaunchKernelGGL((decompress_kernel<D, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, out); break;
        case 4: hipLaunchKernelGGL((decompress_kernel<D, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, out); break;
        default: hipLaunchKernelGGL((decompress_kernel<D, 8>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, out); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decompress(const Packed& p, uint16_t* out, hipStream_t st) {
    if (p.d == 64) return launch_d<64>(p, out, st);
    if (p.d == 128) return launch_d<128>(p, out, st);
    return hipErrorInvalidValue;
}

}  // namespace gear
