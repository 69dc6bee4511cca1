/*
 * gear.h -- C ABI of libgear.so: GEAR KV-cache compression on one AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources: the GEAR pages -- "GEAR: Efficient KV Cache
 * Compression for LLM Inference", allpcb.com Q&A, section Q3 "How does the
 * paper solve the problem?"; and the app.cochat.ai page for "GEAR: An
 * Efficient KV Cache Compression Recipe for Near-Lossless Generative
 * Inference of LLM", whose "Cites" list quotes the paper's Method sentences):
 * each per-head K or V matrix X (tokens x head_dim, fp16) is split into
 *   S  -- the k = floor(s * n * d) largest-magnitude entries, kept exactly
 *         ("in full precision with a sparse matrix S = Filter_s(X)"),
 *   Q  -- b-bit uniform codes of D = X - S with a scale and zero-point per
 *         group of g consecutive head_dim columns of one token,
 *   L  -- a rank-r fit A B^T of the residual R = D - deq(Q), obtained by t
 *         power-iteration (PowerSGD) steps from a fixed start B0,
 * and read back as X^ = deq(Q) + L + S.  New decode tokens go to a small fp16
 * buffer that is compressed when it fills (Q3, "Streaming strategy").
 *
 * Conventions for every call:
 *   - Pointers named *_f16 / *_f32 / packed / workspace / arena are DEVICE
 *     pointers, 256-byte aligned (torch allocations are).  `stream` is a
 *     hipStream_t (NULL = the default stream).  Every call is asynchronous on
 *     `stream`: none allocates, frees or synchronises device memory (the
 *     opt-in kernel timing below records HIP events, and reading it waits
 *     for them).
 *   - The caller owns all device memory.  The library owns only the host-side
 *     gear_cache object.
 *   - Every check (null or misaligned pointers, shapes, parameters, workspace
 *     and arena sizes, cache capacity) runs on the host before any launch.  A
 *     status other than GEAR_OK and GEAR_ERR_HIP means nothing was enqueued
 *     and no cache state changed; gear_last_error() then holds a message
 *     (thread-local).
 *   - GEAR_ERR_HIP reports a failed kernel launch.  The launches of the same
 *     call that came before it stay enqueued, so the outputs of that call are
 *     undefined.  A cache whose call returned GEAR_ERR_HIP is marked failed:
 *     every later call on it (load_prompt, append, decode_attn) returns
 *     GEAR_ERR_INVALID_ARG without enqueuing anything, and the only use left
 *     is gear_cache_destroy.  Device faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this ABI.
 *   - Calls on distinct caches may run from different threads; one cache is
 *     not thread-safe.
 *
 * Limits of this implementation: head_dim 64 or 128; bits 2 or 4; group in
 * {8,16,32,64,128} dividing head_dim (KIVI keys: 16..128 dividing the tokens
 * per matrix); rank <= 8 (and <= tokens per matrix); power_iters >= 1 when
 * rank > 0 and <= 64.
 */
#ifndef GEAR_H
#define GEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEAR_OK = 0,
    GEAR_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad shape or setting */
    GEAR_ERR_UNSUPPORTED = 2,  /* valid GEAR setting outside this library's limits */
    GEAR_ERR_CAPACITY = 3,     /* cache arena or token capacity exhausted */
    GEAR_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
    GEAR_ERR_WORKSPACE = 5     /* workspace too small */
} gear_status;

/*
 * Quantization backbone (the Q step; outliers and the low-rank fit are the
 * same for all):
 *   GEAR_QUANT_GROUP     GEAR's own: groups of `group` consecutive head_dim
 *                        columns of one token, for keys and values.
 *   GEAR_QUANT_KIVI      KIVI's (app.cochat.ai GEAR page, "Cites" list, the
 *                        KIVI entry, and the "Cited by" quote that KIVI
 *                        quantizes keys per channel and values per token):
 *                        keys in groups of `group` consecutive tokens of one
 *                        channel, values as GEAR_QUANT_GROUP.  Keys need
 *                        outlier_ppm = 0 in this library (GEAR-L with a KIVI
 *                        backbone) and tokens per matrix divisible by group.
 *   GEAR_QUANT_ZIPCACHE  ZipCache's channel-separable tokenwise quantization
 *                        ("ZipCache: Accurate and Efficient KV Cache
 *                        Quantization with Salient Token Identification",
 *                        abstract): channel j is divided by 2^e_j, the
 *                        smallest power of two not below its largest |x|
 *                        (e_j = 0 for an all-zero channel; the normalized
 *                        entries rounded to fp16, to nearest even), GEAR runs
 *                        on the normalized matrix with one group per token
 *                        (group must equal head_dim), and the reconstruction
 *                        multiplies channel j back by 2^e_j.  The factors are
 *                        stored in the packed `chan` section.
 */
typedef enum { GEAR_QUANT_GROUP = 0, GEAR_QUANT_KIVI = 1, GEAR_QUANT_ZIPCACHE = 2 } gear_quant;

/* GEAR settings.  Outlier share s = outlier_ppm / 1e6; k = floor(n*d*s). */
typedef struct {
    int32_t bits;          /* b: 2 or 4 */
    int32_t group;         /* g: columns per quantization group, divides head_dim */
    int32_t outlier_ppm;   /* s in parts per million, 0..1000000 */
    int32_t rank;          /* r: 0 (no low-rank term) .. 8 */
    int32_t power_iters;   /* t: power-iteration steps, >= 1 if rank > 0 */
    int32_t chunk_tokens;  /* 0: each matrix is fitted whole; else each run of
                              chunk_tokens tokens is its own matrix (must divide
                              n_tokens) */
    uint64_t seed;         /* B0[j][c] = top 24 bits of splitmix64 output
                              (j*r + c + 1) from state `seed`, * 2^-23 - 1 */
    int32_t quant;         /* gear_quant */
    int32_t reserved;      /* must be 0 */
} gear_params;

/* What the matrices of a stack hold (only the KIVI backbone treats keys and
   values differently). */
typedef enum {
    GEAR_ROLE_KEYS = 0,
    GEAR_ROLE_VALUES = 1,
    GEAR_ROLE_KEYS_THEN_VALUES = 2   /* num_mats even: the first half keys, the
                                        second half values (a cache segment) */
} gear_role;

/* A stack of num_mats matrices, each n_tokens x head_dim fp16, row-major,
   contiguous: element (m, t, j) at ((m * n_tokens + t) * head_dim + j). */
typedef struct {
    int64_t num_mats;
    int32_t n_tokens;
    int32_t head_dim;
    int32_t role;          /* gear_role */
    int32_t reserved;      /* must be 0 */
} gear_shape;

/*
 * Packed form of a compressed stack.  One buffer; M = num_mats * chunks
 * compressed matrices of `rows` tokens each (chunk c of matrix m is compressed
 * matrix m * chunks + c).  Sections, each 256-byte aligned, at these offsets:
 *   codes   u8  [M][rows][head_dim*bits/8]  code of column j of a token at
 *                                           byte j*bits/8, bit (j*bits)%8,
 *                                           least significant bits first
 *   scale   f32 [M][rows][head_dim/group]   (KIVI keys: [M][rows/group][head_dim])
 *   zero    f32 [M][rows][head_dim/group]   (= group minimum; layout as scale)
 *   row_ptr i32 [M][rows+1]                 CSR of S, offsets into col/val of
 *                                           the same matrix; row_ptr[0] = 0,
 *                                           row_ptr[rows] = k
 *   col     u16 [M][k]                      ascending within a token
 *   val     f16 [M][k]                      the original entries, exact
 *   A       f32 [M][rows][rank]
 *   B       f32 [M][head_dim][rank]         L = A B^T
 *   chan    f32 [M][head_dim]               ZipCache: channel factors 2^e_j
 *                                           (empty for the other backbones)
 * With ZipCache, codes, scales, zeros, outlier values, A and B describe the
 * normalized matrix.  Offsets are relative to the buffer start; the buffer
 * holds no pointers, so it may be copied or saved as plain bytes.
 */
typedef struct {
    int64_t num_compressed;  /* M */
    int32_t rows;            /* tokens per compressed matrix */
    int32_t k;               /* outliers per compressed matrix */
    size_t off_codes, off_scale, off_zero, off_row_ptr, off_col, off_val, off_a, off_b, off_chan;
    size_t total_bytes;
} gear_layout;

/* Fills *out; GEAR_ERR_INVALID_ARG / GEAR_ERR_UNSUPPORTED for bad settings. */
gear_status gear_packed_layout(const gear_params* p, const gear_shape* s, gear_layout* out);

/* Bytes of the packed buffer; 0 if the settings are rejected. */
size_t gear_packed_bytes(const gear_params* p, const gear_shape* s);

/* Bytes of device workspace gear_compress needs; 0 if rejected (ZipCache
   adds room for the normalized copy of the stack). */
size_t gear_compress_workspace_bytes(const gear_params* p, const gear_shape* s);

/*
 * Compress: x_f16 (the stack described by s) -> packed (gear_packed_bytes).
 * Runs the outlier filter, group quantization and the low-rank fit of every
 * matrix.  workspace: >= gear_compress_workspace_bytes, contents need not be
 * initialised (it carries per-matrix results between the call's kernels:
 * 128 bytes of outlier-selection results and up to head_dim x 8 floats of the
 * low-rank fit per compressed matrix); it must not be shared by calls that may run
 * concurrently.  Every entry of x_f16 must be finite: NaN or infinity is not
 * detected, and the packed result for such input is unspecified.
 */
gear_status gear_compress(const gear_params* p, const gear_shape* s, const void* x_f16,
                          void* packed, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Compress without any workspace or allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same inputs, outputs and results as
 * gear_compress; the per-call scratch (the workspace of gear_compress) is a
 * static device array of GEAR_NOALLOC_SCRATCH_BYTES that each GPU holds for
 * the life of the process.  GEAR_ERR_WORKSPACE (nothing enqueued) when
 * gear_compress_workspace_bytes(p, s) exceeds it.  The first call on a device
 * looks up the array's address there (GEAR_ERR_HIP if that fails).  All calls
 * on one GPU share its array: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  No
 * part of the array needs clearing between calls.
 */
#define GEAR_NOALLOC_SCRATCH_BYTES (16u << 20)
gear_status gear_compress_noalloc(const gear_params* p, const gear_shape* s, const void* x_f16,
                                  void* packed, void* stream);

/*
 * Decompress: packed -> out_f16 (the stack described by s), each entry
 * fl16(code*scale + zero + (A B^T)[t][j] + S[t][j]) with round to nearest even.
 * Source: the app.cochat.ai GEAR page, "Cites" list, the Background sentence
 * quoted under the PowerSGD entry (the composite approximation: a low-rank
 * term for the coherent part of the quantization error plus a sparse term for
 * the individual outliers, both on top of the dequantized matrix), and the
 * allpcb Q&A, Q3 (the three components combined).  packed must be
 * 256-byte aligned and hold the layout of (p, s); out_f16 16-byte aligned,
 * num_mats * n_tokens * head_dim fp16 values.  Nothing is read outside the
 * packed layout, nothing is written outside out_f16.
 */
gear_status gear_decompress(const gear_params* p, const gear_shape* s, const void* packed,
                            void* out_f16, void* stream);

/* ------------------------------------------------------------------------ */
/* Streaming cache of one attention layer                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    gear_params prompt;       /* settings for the prompt (chunk_tokens allowed) */
    gear_params fill;         /* settings for each full buffer (chunk_tokens ignored);
                                 same backbone (quant) as the prompt.  With the
                                 KIVI backbone buf_tokens must be a multiple of
                                 the key group: the buffer holds whole groups */
    int32_t batch;            /* B */
    int32_t kv_heads;         /* Hkv */
    int32_t head_dim;         /* d */
    int32_t prompt_tokens;    /* tokens compressed by gear_cache_load_prompt (may be 0) */
    int32_t buf_tokens;       /* n_b: fp16 buffer length; a full buffer is compressed */
    int32_t max_new_tokens;   /* capacity for gear_append_tokens, summed over calls */
} gear_cache_config;

typedef struct gear_cache gear_cache;   /* opaque host object: offsets and counters */

typedef struct {
    int64_t tokens;           /* tokens a query sees: prompt + appended */
    int32_t buf_len;          /* tokens now in the fp16 buffer */
    int32_t num_fills;        /* compressed buffer segments so far */
    const void* prompt_packed;  /* packed prompt: matrices K[b][h] then V[b][h] */
    const void* fill_packed;    /* packed fill f at fill_packed + f * fill_stride */
    size_t fill_stride;
    const void* buffer_f16;     /* [2][B][Hkv][buf_tokens][d], K then V */
} gear_cache_info;

/* Bytes of the caller-owned device arena the cache lives in; 0 if rejected. */
size_t gear_cache_arena_bytes(const gear_cache_config* c);

/* Bytes of workspace needed by load_prompt / append / decode_attn with
   q_heads query heads; 0 if rejected. */
size_t gear_cache_workspace_bytes(const gear_cache_config* c, int32_t q_heads);

/* Creates the host object over `arena` (>= gear_cache_arena_bytes).  Nothing
   is launched; the cache starts empty (no prompt, empty buffer). */
gear_status gear_cache_create(const gear_cache_config* c, void* arena, size_t arena_bytes,
                              gear_cache** out);
void gear_cache_destroy(gear_cache* cache);

/* Compresses the prompt: k_f16, v_f16 are [B][Hkv][prompt_tokens][d].  Only
   valid on a cache with no tokens yet.  Entries must be finite (as for
   gear_compress). */
gear_status gear_cache_load_prompt(gear_cache* cache, const void* k_f16, const void* v_f16,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Appends n_new tokens per sequence: k_new_f16, v_new_f16 are
 * [B][Hkv][n_new][d].  Tokens go to the buffer in order; every time the
 * buffer holds buf_tokens tokens it is compressed (fill settings) into a new
 * segment and emptied, before the next token is placed.  Entries must be
 * finite (as for gear_compress).
 * GEAR_ERR_CAPACITY if the total would exceed max_new_tokens.
 */
gear_status gear_append_tokens(gear_cache* cache, const void* k_new_f16, const void* v_new_f16,
                               int32_t n_new, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Decode attention of one query token per sequence over everything cached
 * (prompt segments, fill segments, buffer), no mask.  Source: the allpcb
 * Q&A, Q1 and Q4 (decoding is bound by reading the KV cache; the compressed
 * cache cuts that traffic and raises decode throughput), and Q3 "Streaming
 * strategy" (the most recent tokens are read from the small fp16 buffer).
 * K^ and V^ are never formed in memory: the scores and the weighted sum are
 * taken over codes, scales, zeros, A, B and the outliers directly.
 *   out[b][h] = sum_t softmax_t(sm_scale * q[b][h] . K^_t) V^_t
 * with K^, V^ of KV head floor(h * Hkv / q_heads).  q_f16 is [B][q_heads][d],
 * out_f32 is [B][q_heads][d]; both 16-byte aligned.  q_heads / Hkv must be 1,
 * 2, 4 or 8.  With no cached tokens the output is zero.  q_f16 must be finite
 * (NaN or infinity is not detected; the output for it is unspecified).
 * workspace: >= gear_cache_workspace_bytes(config, q_heads), 256-byte aligned
 * (split partials); it must not be shared by calls that may run concurrently.
 */
gear_status gear_decode_attn(const gear_cache* cache, const void* q_f16, int32_t q_heads,
                             float sm_scale, float* out_f32, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * One decode step of the streaming cache in one call: appends one token per
 * sequence (k_new_f16, v_new_f16: [B][Hkv][d], 16-byte aligned) and then
 * takes decode attention as gear_decode_attn, with the same results, cache
 * contents and errors as gear_append_tokens(..., 1, ...) followed by
 * gear_decode_attn (source: the allpcb Q&A, Q3 "Streaming strategy" -- new
 * tokens go to the fp16 buffer, which is compressed when full -- and Q4 --
 * decode attention reads the compressed cache).  The token is written into
 * the buffer by the attention launch itself, which reads it from k_new_f16 /
 * v_new_f16 (one launch fewer per step); when it fills the buffer, the two
 * calls are made one after the other (the buffer's compression lies between
 * them).  workspace as for both calls (gear_cache_workspace_bytes).  On
 * GEAR_ERR_HIP from a launch the cache is marked failed (every later call on
 * it is refused with GEAR_ERR_INVALID_ARG), as for gear_append_tokens.
 */
gear_status gear_append_decode_attn(gear_cache* cache, const void* k_new_f16, const void* v_new_f16,
                                    const void* q_f16, int32_t q_heads, float sm_scale, float* out_f32,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Current counters and section pointers (host call, nothing launched). */
gear_status gear_cache_get_info(const gear_cache* cache, gear_cache_info* out);

/*
 * Kernel timing with HIP events, for profiling; off by default.  While it is
 * on, every kernel launch of the library is bracketed by two events recorded
 * on the launch stream.  gear_timing_enable(1) starts a new measurement (0
 * stops it and drops what was recorded).  gear_timing_read() waits for the
 * recorded events and returns, for the kernel named `kernel` -- one of
 * "select", "compress", "lowrank_a", "decompress", "attn_split",
 * "attn_combine", "buffer_append" -- the launches and their summed duration
 * in milliseconds since the measurement started ("attn_combine" has none when
 * the split kernel merges the splits itself).  It blocks; host-thread-safe.
 */
gear_status gear_timing_enable(int on);
gear_status gear_timing_read(const char* kernel, int64_t* launches, double* total_ms);

/* Status name, and the detail of this thread's last non-OK status. */
const char* gear_status_str(gear_status s);
const char* gear_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GEAR_H */
