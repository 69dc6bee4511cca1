// gear_decompress.hip -- reconstruction X^ = deq(Q) + A B^T + S of packed GEAR
// matrices ("GEAR: Efficient KV Cache Compression for LLM Inference", Q3: the
// quantized backbone, the low-rank part and the sparse part add up; app.cochat.ai
// "Cites" list, sentence quoted under the Zafrir et al. entry: low-rank for the
// coherent error, sparse for the outliers).
//
// HBM-bound streaming kernel: a lane owns 8 consecutive columns of a token
// (D/8 lanes per token), reads that token's packed codes as one 32- or 16-bit
// word, the group's scale/zero, the token's A row, and the token's CSR
// entries, and writes 8 fp16 values as one 16-byte store.  B (D x r) for the
// lane's columns stays in registers for all the workgroup's tokens.
#include "gear_internal.h"

namespace gear {
namespace {

constexpr int kStepsPerWG = 8;

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
    constexpr int ROWS_WG = kStepsPerWG * ROWS_STEP;
    constexpr int RKX = RK > 0 ? RK : 1;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int colq = lane % LPR, rl = lane / LPR;
    const int rows = p.rows;
    const int blocks_per_mat = (rows + ROWS_WG - 1) / ROWS_WG;
    const int64_t mm = blockIdx.x / blocks_per_mat;
    const int row0 = (int)(blockIdx.x % blocks_per_mat) * ROWS_WG;
    const int r = p.rank, bits = p.bits, gl = p.group / 8, ngr = D / p.group;
    const uint32_t cmask = (1u << bits) - 1u;

    float Bm[8][RKX];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < RKX; ++c)
            Bm[e][c] = (RK > 0 && c < r) ? p.B[((size_t)mm * D + colq * 8 + e) * r + c] : 0.0f;

    const int32_t* rp = p.row_ptr + (size_t)mm * (rows + 1);
    const uint16_t* cm = p.col + (size_t)mm * p.k;
    const uint16_t* vm = p.val + (size_t)mm * p.k;
#pragma unroll 2
    for (int s = 0; s < kStepsPerWG; ++s) {
        const int row = row0 + s * ROWS_STEP + wv * RPS + rl;
        if (row >= rows) continue;
        const size_t grow = (size_t)mm * rows + row;
        uint32_t word;
        if (bits == 4)
            word = reinterpret_cast<const uint32_t*>(p.codes)[grow * (D / 8) + colq];
        else
            word = reinterpret_cast<const uint16_t*>(p.codes)[grow * (D / 8) + colq];
        const float sc = p.scale[grow * ngr + colq / gl];
        const float zp = p.zero[grow * ngr + colq / gl];
        float ar[RKX];
#pragma unroll
        for (int c = 0; c < RKX; ++c) ar[c] = (RK > 0 && c < r) ? p.A[grow * r + c] : 0.0f;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = fmaf((float)((word >> (e * bits)) & cmask), sc, zp);
#pragma unroll
            for (int c = 0; c < RKX; ++c) v = fmaf(ar[c], Bm[e][c], v);
            x[e] = v;
        }
        const int beg = max(rp[row], 0), end = min(rp[row + 1], p.k);
        for (int i = beg; i < end; ++i) {
            const int cj = cm[i];
            if ((cj >> 3) == colq) {
                const float v = h2f(vm[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] += ((cj & 7) == e) ? v : 0.0f;
            }
        }
        uint4 o;
        o.x = f2h(x[0]) | (f2h(x[1]) << 16);
        o.y = f2h(x[2]) | (f2h(x[3]) << 16);
        o.z = f2h(x[4]) | (f2h(x[5]) << 16);
        o.w = f2h(x[6]) | (f2h(x[7]) << 16);
        *reinterpret_cast<uint4*>(out + grow * D + colq * 8) = o;
    }
}

template <int D>
hipError_t launch_d(const Packed& p, uint16_t* out, hipStream_t st) {
    constexpr int ROWS_WG = kStepsPerWG * 4 * (64 / (D / 8));
    const int64_t blocks = p.M * ((p.rows + ROWS_WG - 1) / ROWS_WG);
    if (blocks <= 0) return hipSuccess;
    const int rk = p.rank == 0 ? 0 : p.rank <= 2 ? 2 : p.rank <= 4 ? 4 : 8;
    switch (rk) {
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
