// gear_internal.h -- declarations shared by the HIP sources of libgear.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gear.h"

namespace gear {

constexpr int kThreads = 256;        // every kernel here runs 4 waves of 64
constexpr int kMaxRank = 8;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// Work-item and workgroup ids read from the hardware registers.  In a file
// built with IEEE mode off, the device library's id functions (built with it
// on) are not inlined: as calls they return the ids in vector registers, and
// everything derived from a workgroup id (base addresses, per-block
// parameters) would then be held and computed per lane.
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ uint32_t group_id_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ uint32_t group_id_y() { return __builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ uint32_t group_id_z() { return __builtin_amdgcn_workgroup_id_z(); }
// wave index within the workgroup, known to the compiler as wave-uniform
__device__ __forceinline__ int wave_id(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// Lanes l ^ 16 and l ^ 32 through the gfx950 permlane swaps (no LDS): each
// swap leaves a lane's own value in one result and its partner's in the
// other, so op(first, second) is the same in both partners.  Both results
// are pinned as integers before they are read as floats: reading them as
// floats directly, this compiler takes the first result for both.
template <bool S32>
__device__ __forceinline__ void swap_pair(float v, float& a, float& b) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    uint32_t x, y;
    if (S32) {
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        x = p[0];
        y = p[1];
    } else {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x = p[0];
        y = p[1];
    }
    asm("" : "+v"(x), "+v"(y));
    a = __builtin_bit_cast(float, x);
    b = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float sum_xor16(float v) {
    float a, b;
    swap_pair<false>(v, a, b);
    return a + b;
}
__device__ __forceinline__ float sum_xor32(float v) {
    float a, b;
    swap_pair<true>(v, a, b);
    return a + b;
}

// Loads and stores at a 32-bit byte offset from a (workgroup-uniform) base, so
// that the address is formed as base + zero-extended offset in one step (the
// scalar-base addressing form), not with 64-bit vector arithmetic.
template <typename T>
__device__ __forceinline__ T ld_at(const void* base, uint32_t byte_off) {
    return *reinterpret_cast<const T*>(static_cast<const unsigned char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ void st_at(void* base, uint32_t byte_off, T v) {
    *reinterpret_cast<T*>(static_cast<unsigned char*>(base) + byte_off) = v;
}

// Opt-in per-kernel timing (gear_timing_enable): a Timed object brackets one
// launch with HIP events on its stream while timing is on; a no-op otherwise.
enum KernelId {
    kKSelect, kKCompress, kKLowrankA, kKDecompress, kKAttnSplit, kKAttnCombine,
    kKBufferAppend, kKChannel, kKernelCount
};
bool timing_on();
hipEvent_t timing_begin(hipStream_t st);                    // nullptr on failure
void timing_end(KernelId k, hipEvent_t start, hipStream_t st);
struct Timed {
    KernelId k;
    hipStream_t st;
    hipEvent_t start;
    Timed(KernelId k_, hipStream_t st_)
        : k(k_), st(st_), start(timing_on() ? timing_begin(st_) : nullptr) {}
    ~Timed() {
        if (start) timing_end(k, start, st);
    }
    Timed(const Timed&) = delete;
    Timed& operator=(const Timed&) = delete;
};

// Resolved packed layout, with device pointers of one buffer.
struct Packed {
    int64_t M;         // compressed matrices
    int32_t rows;      // tokens per compressed matrix
    int32_t d, bits, group, rank, k;
    int64_t ch_mats;   // matrices [0, ch_mats) are quantized per channel (KIVI
                       // keys: scale / zero [rows / group][d]); the rest per token
    uint8_t* codes;
    float* scale;
    float* zero;
    int32_t* row_ptr;
    uint16_t* col;
    uint16_t* val;     // fp16 bits
    float* A;
    float* B;
    float* chan;       // ZipCache channel factors [M][d], else nullptr
};

// ---- compress -------------------------------------------------------------
struct CompressArgs {
    const uint16_t* x;     // matrices [0, m_split): [m][rows][d] fp16 bits
    const uint16_t* x2;    // matrices [m_split, M) (a second tensor)
    int64_t m_split;
    int64_t m0, m1;        // this launch compresses matrices [m0, m1)
    int32_t chan_q;        // 1: quantize per channel (groups of out.group tokens)
    Packed out;
    int32_t iters;
    uint64_t seed;
    uint32_t* sel;         // workspace [M][kSelStride]: outlier threshold, per-block quotas
    float* bf;             // workspace [M][d][rank_slots(rank)]: maps R to A
};
// Selection results per matrix: [0] threshold key T, then per row block b
// (= wave of the compress kernel): [kSelTake + b] ties at T it takes,
// [kSelCsr + b] its first CSR position, [kSelEq + b] ties at T it holds;
// [kSelBound] a key bounding |x| over the non-outliers.
constexpr int kCompressWaves = 8;    // waves (row blocks) per compressed matrix
constexpr int kSelTake = 1, kSelCsr = 9, kSelEq = 17, kSelBound = 25;
constexpr int kSelStride = 32;
// Rank rounded up to the register tile the kernels are compiled for.
inline int rank_slots(int r) { return r == 0 ? 0 : r <= 2 ? 2 : r <= 4 ? 4 : 8; }
// Rows of a matrix owned by each of the kCompressWaves waves of a compress
// workgroup (a multiple of 8: every wave adds whole 8-row slices to the
// 64-row MFMA slabs).  The selection and the A-projection kernels use the
// same split to find which wave's tie quota a row falls under.
__host__ __device__ inline int wave_rows(int rows) {
    return ((rows + kCompressWaves - 1) / kCompressWaves + 7) / 8 * 8;
}
size_t compress_workspace(int64_t M, int d, int rank);
// Compress matrices [a.m0, a.m1) of a.out.
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);
// Per-channel scale and zero of matrices [a.m0, a.m1) (KIVI keys without
// outliers): groups of out.group tokens of each channel.
hipError_t launch_channel_params(const CompressArgs& a, hipStream_t st);
// ZipCache: channel factors 2^e_j of every matrix into out.chan, then the
// normalized stack fl16(x 2^-e_j) into xt ([M][rows][d], contiguous).
hipError_t launch_channel_normalize(const CompressArgs& a, uint16_t* xt, hipStream_t st);

// ---- decompress -----------------------------------------------------------
hipError_t launch_decompress(const Packed& p, uint16_t* out, hipStream_t st);

// ---- streaming cache kernels ---------------------------------------------
// Copy n_new tokens per (tensor, b, h) into the fp16 buffer at position pos.
hipError_t launch_buffer_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* buf,
                                int B, int H, int d, int cap, int pos, int n_new,
                                int src_tokens, int src_off, hipStream_t st);

// One compressed segment kind as seen by decode attention.
struct AttnSeg {
    Packed p;              // matrices ordered (tensor, b, h, chunk)
    int32_t chunks;        // chunks per (tensor, b, h)
    int32_t count;         // number of such packed buffers laid out back to back
    size_t stride;         // bytes between consecutive buffers (count > 1)
};

struct AttnArgs {
    int B, Hkv, Hq, d;
    float sm_scale;
    const uint16_t* q;     // [B][Hq][d]
    float* out;            // [B][Hq][d]
    AttnSeg prompt;        // prompt.count is 0 or 1
    AttnSeg fills;         // fills.count = number of fills
    uint16_t* buf;         // [2][B][Hkv][cap][d] (written only at row new_row)
    int32_t buf_cap, buf_len;
    float* partial;        // workspace: [B*Hkv][splits][G][d + 2]
    int32_t splits;
    int32_t tokens_per_split;
    int32_t split0;        // splits [0, split0) are whole prompt splits (fast kernel)
    int32_t fuse_combine;  // 1: the one split of attn_split_kernel per pair also merges
    // one appended token per (b, kv-head), [B][Hkv][d] each, that the split
    // holding buffer row new_row reads from here and writes into the buffer
    // (new_row < 0: none; buf_len counts it)
    const uint16_t* k_new;
    const uint16_t* v_new;
    int32_t new_row;
};
size_t attn_workspace_bytes(int B, int Hkv, int Hq, int d, int64_t tokens, int* splits,
                            int* tokens_per_split);
hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t st);

}  // namespace gear
