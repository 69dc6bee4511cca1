// gear_api.hip -- the C ABI of libgear.so: validation, packed layouts, the
// streaming cache's host bookkeeping, and kernel launches.  Every check runs
// before any launch; a non-OK status other than GEAR_ERR_HIP leaves device
// memory and cache state untouched.  A failed launch inside a cache call
// marks that cache failed (later calls on it are refused).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "gear_internal.h"

using namespace gear;

namespace {

thread_local std::string g_last_error;

gear_status fail(gear_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gear_status hip_fail(hipError_t e, const char* what) {
    return fail(GEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

gear_status failed_cache() {
    return fail(GEAR_ERR_INVALID_ARG,
                "an earlier kernel launch on this cache failed; destroy the cache");
}

// Checks GEAR settings for matrices of `rows` tokens and head_dim d.
gear_status check_params(const gear_params* p, int64_t rows, int d) {
    if (!p) return fail(GEAR_ERR_INVALID_ARG, "params is NULL");
    if (p->bits != 2 && p->bits != 4)
        return fail(p->bits > 0 && p->bits <= 8 ? GEAR_ERR_UNSUPPORTED : GEAR_ERR_INVALID_ARG,
                    "bits must be 2 or 4 (got %d)", p->bits);
    if (d != 64 && d != 128)
        return fail(d > 0 ? GEAR_ERR_UNSUPPORTED : GEAR_ERR_INVALID_ARG,
                    "head_dim must be 64 or 128 (got %d)", d);
    if (p->group <= 0 || d % p->group != 0)
        return fail(GEAR_ERR_INVALID_ARG, "group %d does not divide head_dim %d", p->group, d);
    if (p->group % 8 != 0 || (p->group & (p->group - 1)) != 0)
        return fail(GEAR_ERR_UNSUPPORTED, "group must be one of 8,16,32,64,128 (got %d)", p->group);
    if (p->outlier_ppm < 0 || p->outlier_ppm > 1000000)
        return fail(GEAR_ERR_INVALID_ARG, "outlier_ppm %d outside 0..1000000", p->outlier_ppm);
    if (p->rank < 0) return fail(GEAR_ERR_INVALID_ARG, "rank %d < 0", p->rank);
    if (p->rank > kMaxRank) return fail(GEAR_ERR_UNSUPPORTED, "rank %d > %d", p->rank, kMaxRank);
    if (p->rank > 0 && (p->power_iters < 1 || p->power_iters > 64))
        return fail(GEAR_ERR_INVALID_ARG, "power_iters must be 1..64 when rank > 0 (got %d)",
                    p->power_iters);
    if (p->power_iters < 0) return fail(GEAR_ERR_INVALID_ARG, "power_iters < 0");
    if (p->chunk_tokens < 0) return fail(GEAR_ERR_INVALID_ARG, "chunk_tokens < 0");
    if (rows < 1) return fail(GEAR_ERR_INVALID_ARG, "tokens per matrix must be >= 1");
    if (p->chunk_tokens > 0 && rows % p->chunk_tokens != 0)
        return fail(GEAR_ERR_INVALID_ARG, "chunk_tokens %d does not divide n_tokens %lld",
                    p->chunk_tokens, (long long)rows);
    const int64_t mrows = p->chunk_tokens > 0 ? p->chunk_tokens : rows;
    if (p->rank > mrows)
        return fail(GEAR_ERR_INVALID_ARG, "rank %d exceeds tokens per matrix %lld", p->rank,
                    (long long)mrows);
    if (mrows > (1 << 24))
        return fail(GEAR_ERR_UNSUPPORTED, "%lld tokens per matrix is above this library's limit of %d",
                    (long long)mrows, 1 << 24);
    if (p->reserved != 0) return fail(GEAR_ERR_INVALID_ARG, "params.reserved must be 0");
    if (p->quant < GEAR_QUANT_GROUP || p->quant > GEAR_QUANT_ZIPCACHE)
        return fail(GEAR_ERR_INVALID_ARG, "unknown quantization backbone %d", p->quant);
    if (p->quant == GEAR_QUANT_ZIPCACHE && p->group != d)
        return fail(GEAR_ERR_INVALID_ARG,
                    "ZipCache quantizes tokenwise: group must equal head_dim (%d, got %d)", d, p->group);
    return GEAR_OK;
}

// Keys quantized per channel (KIVI backbone): the extra conditions.
gear_status check_channel_keys(const gear_params* p, int64_t mrows) {
    if (p->group < 16)
        return fail(GEAR_ERR_UNSUPPORTED, "KIVI key groups must be 16..128 tokens (got %d)", p->group);
    if (mrows % p->group != 0)
        return fail(GEAR_ERR_INVALID_ARG, "KIVI keys: %lld tokens per matrix is not a multiple of the group %d",
                    (long long)mrows, p->group);
    if (p->outlier_ppm != 0)
        return fail(GEAR_ERR_UNSUPPORTED,
                    "KIVI keys are supported without outliers only (outlier_ppm = 0: GEAR-L)");
    return GEAR_OK;
}

// Leading matrices of a stack quantized per channel.
int64_t channel_mats(const gear_params* p, int64_t M, int role) {
    if (p->quant != GEAR_QUANT_KIVI) return 0;
    return role == GEAR_ROLE_KEYS ? M : role == GEAR_ROLE_KEYS_THEN_VALUES ? M / 2 : 0;
}

gear_status compute_layout(const gear_params* p, const gear_shape* s, gear_layout* L) {
    if (!s) return fail(GEAR_ERR_INVALID_ARG, "shape is NULL");
    if (s->num_mats < 0) return fail(GEAR_ERR_INVALID_ARG, "num_mats < 0");
    gear_status st = check_params(p, s->n_tokens, s->head_dim);
    if (st != GEAR_OK) return st;
    if (s->reserved != 0) return fail(GEAR_ERR_INVALID_ARG, "shape.reserved must be 0");
    if (s->role < GEAR_ROLE_KEYS || s->role > GEAR_ROLE_KEYS_THEN_VALUES)
        return fail(GEAR_ERR_INVALID_ARG, "unknown role %d", s->role);
    if (s->role == GEAR_ROLE_KEYS_THEN_VALUES && s->num_mats % 2 != 0)
        return fail(GEAR_ERR_INVALID_ARG, "a keys-then-values stack needs an even num_mats");
    const int64_t rows = p->chunk_tokens > 0 ? p->chunk_tokens : s->n_tokens;
    if (channel_mats(p, s->num_mats, s->role) > 0) {
        st = check_channel_keys(p, rows);
        if (st != GEAR_OK) return st;
    }
    const int64_t M = s->num_mats * (s->n_tokens / rows);
    const int64_t d = s->head_dim;
    const int64_t k = rows * d * (int64_t)p->outlier_ppm / 1000000;
    L->num_compressed = M;
    L->rows = (int32_t)rows;
    L->k = (int32_t)k;
    size_t off = 0;
    L->off_codes = off; off = align_up(off + (size_t)(M * rows * d * p->bits / 8));
    L->off_scale = off; off = align_up(off + (size_t)(M * rows * (d / p->group)) * 4);
    L->off_zero = off; off = align_up(off + (size_t)(M * rows * (d / p->group)) * 4);
    L->off_row_ptr = off; off = align_up(off + (size_t)(M * (rows + 1)) * 4);
    L->off_col = off; off = align_up(off + (size_t)(M * k) * 2);
    L->off_val = off; off = align_up(off + (size_t)(M * k) * 2);
    L->off_a = off; off = align_up(off + (size_t)(M * rows * p->rank) * 4);
    L->off_b = off; off = align_up(off + (size_t)(M * d * p->rank) * 4);
    L->off_chan = off; off = align_up(off + (p->quant == GEAR_QUANT_ZIPCACHE ? (size_t)(M * d) * 4 : 0));
    L->total_bytes = off;
    return GEAR_OK;
}

Packed make_packed(const gear_params* p, const gear_layout& L, int d, void* base, int role) {
    uint8_t* b = static_cast<uint8_t*>(base);
    Packed k;
    k.M = L.num_compressed;
    k.ch_mats = channel_mats(p, L.num_compressed, role);
    k.chan = p->quant == GEAR_QUANT_ZIPCACHE ? reinterpret_cast<float*>(b + L.off_chan) : nullptr;
    k.rows = L.rows;
    k.d = d;
    k.bits = p->bits;
    k.group = p->group;
    k.rank = p->rank;
    k.k = L.k;
    k.codes = b + L.off_codes;
    k.scale = reinterpret_cast<float*>(b + L.off_scale);
    k.zero = reinterpret_cast<float*>(b + L.off_zero);
    k.row_ptr = reinterpret_cast<int32_t*>(b + L.off_row_ptr);
    k.col = reinterpret_cast<uint16_t*>(b + L.off_col);
    k.val = reinterpret_cast<uint16_t*>(b + L.off_val);
    k.A = reinterpret_cast<float*>(b + L.off_a);
    k.B = reinterpret_cast<float*>(b + L.off_b);
    return k;
}

struct CompressPlan {
    size_t ws_bytes;
};

// The compress workspace: selection results and the projection for A, then
// (ZipCache) the normalized copy of the stack.
CompressPlan plan_compress(const gear_params* p, const gear_layout& L, int d) {
    size_t n = compress_workspace(L.num_compressed, d, p->rank);
    if (p->quant == GEAR_QUANT_ZIPCACHE)
        n = align_up(n) + align_up((size_t)L.num_compressed * L.rows * d * 2);
    return CompressPlan{n};
}

// Compress matrices [0, m_split) from x and [m_split, M) from x2; role as in
// gear_shape (which matrices are keys).
gear_status run_compress(const gear_params* p, const gear_layout& L, int d, const void* x,
                         const void* x2, int64_t m_split, int role, void* packed, void* ws,
                         size_t ws_bytes, hipStream_t st) {
    const CompressPlan pl = plan_compress(p, L, d);
    if (ws_bytes < pl.ws_bytes)
        return fail(GEAR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, pl.ws_bytes);
    if (L.num_compressed == 0) return GEAR_OK;
    CompressArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.x2 = static_cast<const uint16_t*>(x2);
    a.m_split = m_split;
    a.m0 = 0;
    a.m1 = L.num_compressed;
    a.chan_q = 0;
    a.out = make_packed(p, L, d, packed, role);
    a.iters = p->power_iters;
    a.seed = p->seed;
    a.sel = static_cast<uint32_t*>(ws);
    const size_t base_ws = align_up(compress_workspace(L.num_compressed, d, p->rank));
    a.bf = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                    align_up((size_t)L.num_compressed * kSelStride * 4));
    hipError_t e = hipSuccess;
    if (p->quant == GEAR_QUANT_ZIPCACHE) {
        // channel factors, then the normalized stack, which the GEAR steps read
        uint16_t* xt = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + base_ws);
        e = launch_channel_normalize(a, xt, st);
        if (e != hipSuccess) return hip_fail(e, "channel normalization launch");
        a.x = a.x2 = xt;
        a.m_split = L.num_compressed;
    }
    const int64_t kc = a.out.ch_mats;
    if (kc > 0) {   // KIVI keys: per-channel parameters, then the compression
        CompressArgs ak = a;
        ak.m1 = kc;
        ak.chan_q = 1;
        e = launch_channel_params(ak, st);
        if (e == hipSuccess) e = launch_compress(ak, st);
        if (e != hipSuccess) return hip_fail(e, "compress launch (keys per channel)");
        a.m0 = kc;
    }
    if (a.m0 < a.m1) e = launch_compress(a, st);
    if (e != hipSuccess) return hip_fail(e, "compress launch");
    return GEAR_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of gear_compress_noalloc: the per-matrix selection results
// and the d x r projection that gear_compress keeps in the caller's
// workspace.  Each GPU holds its own copy for the life of the process.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and is what the kernels get.
static __device__ __align__(256) unsigned char scratch[GEAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up on its first use.
gear_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GEAR_ERR_UNSUPPORTED, "device %d is beyond this library's %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
        if (!ptr || !aligned(ptr, kAlign))
            return fail(GEAR_ERR_HIP, "static scratch at an unexpected address %p", ptr);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GEAR_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Kernel timing

namespace {

const char* const kKernelNames[kKernelCount] = {
    "select", "compress", "lowrank_a", "decompress", "attn_split", "attn_combine", "buffer_append",
    "channel"};

struct TimingRec {
    KernelId k;
    hipEvent_t start, stop;
};

std::atomic<bool> g_timing{false};
std::mutex g_timing_mu;
std::vector<TimingRec> g_pending;
int64_t g_launches[kKernelCount];
double g_total_ms[kKernelCount];

void timing_drop_locked() {
    for (const TimingRec& r : g_pending) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_pending.clear();
    for (int i = 0; i < kKernelCount; ++i) {
        g_launches[i] = 0;
        g_total_ms[i] = 0.0;
    }
}

}  // namespace

namespace gear {

bool timing_on() { return g_timing.load(std::memory_order_relaxed); }

hipEvent_t timing_begin(hipStream_t st) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    if (hipEventRecord(e, st) != hipSuccess) {
        (void)hipEventDestroy(e);
        return nullptr;
    }
    return e;
}

void timing_end(KernelId k, hipEvent_t start, hipStream_t st) {
    hipEvent_t e = timing_begin(st);
    if (!e) {
        (void)hipEventDestroy(start);
        return;
    }
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_pending.push_back(TimingRec{k, start, e});
}

}  // namespace gear

// ---------------------------------------------------------------------------

struct gear_cache {
    gear_cache_config cfg;
    uint8_t* arena;
    gear_layout prompt_layout, fill_layout;
    size_t off_prompt, off_fills, off_buf, fill_stride;
    int max_fills;
    bool prompt_loaded;
    int64_t appended;
    int buf_len;
    int num_fills;
    bool failed;   // a launch of a cache call failed: the device state is unknown
};

namespace {

gear_status cache_layouts(const gear_cache_config* c, gear_layout* pl, gear_layout* fl,
                          size_t* off_fills, size_t* off_buf, size_t* total, int* max_fills) {
    if (!c) return fail(GEAR_ERR_INVALID_ARG, "config is NULL");
    if (c->batch < 1 || c->kv_heads < 1)
        return fail(GEAR_ERR_INVALID_ARG, "batch and kv_heads must be >= 1");
    if (c->prompt_tokens < 0 || c->max_new_tokens < 0 || c->buf_tokens < 1)
        return fail(GEAR_ERR_INVALID_ARG, "bad token counts");
    const int64_t mats = 2LL * c->batch * c->kv_heads;
    size_t off = 0;
    if (c->prompt_tokens > 0) {
        gear_shape s{mats, c->prompt_tokens, c->head_dim, GEAR_ROLE_KEYS_THEN_VALUES, 0};
        gear_status st = compute_layout(&c->prompt, &s, pl);
        if (st != GEAR_OK) return st;
        off = pl->total_bytes;
    } else {
        *pl = gear_layout{};
    }
    gear_params fp = c->fill;
    fp.chunk_tokens = 0;
    if (c->prompt_tokens > 0 && fp.quant != c->prompt.quant)
        return fail(GEAR_ERR_INVALID_ARG, "prompt and fill settings must use the same backbone");
    if (fp.quant == GEAR_QUANT_KIVI && c->buf_tokens % fp.group != 0)
        return fail(GEAR_ERR_INVALID_ARG,
                    "KIVI backbone: the buffer (%d tokens) must hold whole key groups of %d tokens",
                    c->buf_tokens, fp.group);
    gear_shape fs{mats, c->buf_tokens, c->head_dim, GEAR_ROLE_KEYS_THEN_VALUES, 0};
    gear_status st = compute_layout(&fp, &fs, fl);
    if (st != GEAR_OK) return st;
    *max_fills = c->max_new_tokens / c->buf_tokens;
    *off_fills = off;
    off += (size_t)*max_fills * fl->total_bytes;
    *off_buf = off;
    off = align_up(off + (size_t)mats * c->buf_tokens * c->head_dim * 2);
    *total = off;
    return GEAR_OK;
}

}  // namespace

extern "C" {

const char* gear_status_str(gear_status s) {
    // read as an int: a C caller may pass any int, and in C++ a value outside
    // the enumerators' range may not be loaded as the enum type
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case GEAR_OK: return "GEAR_OK";
        case GEAR_ERR_INVALID_ARG: return "GEAR_ERR_INVALID_ARG";
        case GEAR_ERR_UNSUPPORTED: return "GEAR_ERR_UNSUPPORTED";
        case GEAR_ERR_CAPACITY: return "GEAR_ERR_CAPACITY";
        case GEAR_ERR_HIP: return "GEAR_ERR_HIP";
        case GEAR_ERR_WORKSPACE: return "GEAR_ERR_WORKSPACE";
    }
    return "GEAR_ERR_UNKNOWN";
}

const char* gear_last_error(void) { return g_last_error.c_str(); }

gear_status gear_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    timing_drop_locked();
    g_timing.store(on != 0, std::memory_order_relaxed);
    return GEAR_OK;
}

gear_status gear_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return fail(GEAR_ERR_INVALID_ARG, "NULL argument");
    int id = -1;
    for (int i = 0; i < kKernelCount; ++i)
        if (std::string(kernel) == kKernelNames[i]) id = i;
    if (id < 0) return fail(GEAR_ERR_INVALID_ARG, "unknown kernel name '%s'", kernel);
    std::lock_guard<std::mutex> lk(g_timing_mu);
    for (const TimingRec& r : g_pending) {
        hipError_t e = hipEventSynchronize(r.stop);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "kernel timing event");
        g_launches[r.k] += 1;
        g_total_ms[r.k] += ms;
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_pending.clear();
    *launches = g_launches[id];
    *total_ms = g_total_ms[id];
    return GEAR_OK;
}

gear_status gear_packed_layout(const gear_params* p, const gear_shape* s, gear_layout* out) {
    if (!out) return fail(GEAR_ERR_INVALID_ARG, "out is NULL");
    gear_layout L;
    gear_status st = compute_layout(p, s, &L);
    if (st == GEAR_OK) *out = L;
    return st;
}

size_t gear_packed_bytes(const gear_params* p, const gear_shape* s) {
    gear_layout L;
    return compute_layout(p, s, &L) == GEAR_OK ? L.total_bytes : 0;
}

size_t gear_compress_workspace_bytes(const gear_params* p, const gear_shape* s) {
    gear_layout L;
    if (compute_layout(p, s, &L) != GEAR_OK) return 0;
    return plan_compress(p, L, s->head_dim).ws_bytes;
}

gear_status gear_compress(const gear_params* p, const gear_shape* s, const void* x_f16,
                          void* packed, void* workspace, size_t workspace_bytes, void* stream) {
    gear_layout L;
    gear_status st = compute_layout(p, s, &L);
    if (st != GEAR_OK) return st;
    if (L.num_compressed > 0 && (!x_f16 || !packed || !workspace))
        return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(x_f16, 16) || !aligned(packed, kAlign) || !aligned(workspace, kAlign))
        return fail(GEAR_ERR_INVALID_ARG, "x_f16 must be 16-byte, packed/workspace 256-byte aligned");
    const int64_t all = s->num_mats * (s->n_tokens / L.rows);
    return run_compress(p, L, s->head_dim, x_f16, x_f16, all, s->role, packed, workspace,
                        workspace_bytes, static_cast<hipStream_t>(stream));
}

gear_status gear_compress_noalloc(const gear_params* p, const gear_shape* s, const void* x_f16,
                                  void* packed, void* stream) {
    gear_layout L;
    gear_status st = compute_layout(p, s, &L);
    if (st != GEAR_OK) return st;
    if (L.num_compressed > 0 && (!x_f16 || !packed))
        return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(x_f16, 16) || !aligned(packed, kAlign))
        return fail(GEAR_ERR_INVALID_ARG, "x_f16 must be 16-byte, packed 256-byte aligned");
    const size_t need = plan_compress(p, L, s->head_dim).ws_bytes;
    if (need > (size_t)GEAR_NOALLOC_SCRATCH_BYTES)
        return fail(GEAR_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use gear_compress with a workspace, or fewer matrices per call)",
                    need, (size_t)GEAR_NOALLOC_SCRATCH_BYTES);
    if (L.num_compressed == 0) return GEAR_OK;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != GEAR_OK) return st;
    const int64_t all = s->num_mats * (s->n_tokens / L.rows);
    return run_compress(p, L, s->head_dim, x_f16, x_f16, all, s->role, packed, ws,
                        (size_t)GEAR_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

gear_status gear_decompress(const gear_params* p, const gear_shape* s, const void* packed,
                            void* out_f16, void* stream) {
    gear_layout L;
    gear_status st = compute_layout(p, s, &L);
    if (st != GEAR_OK) return st;
    if (L.num_compressed > 0 && (!packed || !out_f16))
        return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(packed, kAlign) || !aligned(out_f16, 16))
        return fail(GEAR_ERR_INVALID_ARG, "packed must be 256-byte, out_f16 16-byte aligned");
    Packed k = make_packed(p, L, s->head_dim, const_cast<void*>(packed), s->role);
    hipError_t e = launch_decompress(k, static_cast<uint16_t*>(out_f16), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decompress launch");
    return GEAR_OK;
}

size_t gear_cache_arena_bytes(const gear_cache_config* c) {
    gear_layout pl, fl;
    size_t of, ob, total;
    int mf;
    return cache_layouts(c, &pl, &fl, &of, &ob, &total, &mf) == GEAR_OK ? total : 0;
}

size_t gear_cache_workspace_bytes(const gear_cache_config* c, int32_t q_heads) {
    gear_layout pl, fl;
    size_t of, ob, total;
    int mf;
    if (cache_layouts(c, &pl, &fl, &of, &ob, &total, &mf) != GEAR_OK) return 0;
    if (q_heads < c->kv_heads || q_heads % c->kv_heads != 0) {
        fail(GEAR_ERR_INVALID_ARG, "q_heads must be a multiple of kv_heads");
        return 0;
    }
    size_t ws = 0;
    if (c->prompt_tokens > 0) ws = plan_compress(&c->prompt, pl, c->head_dim).ws_bytes;
    gear_params fp = c->fill;
    fp.chunk_tokens = 0;
    const size_t wf = plan_compress(&fp, fl, c->head_dim).ws_bytes;
    if (wf > ws) ws = wf;
    const size_t wa = attn_workspace_bytes(c->batch, c->kv_heads, q_heads, c->head_dim,
                                           (int64_t)c->prompt_tokens + c->max_new_tokens, nullptr,
                                           nullptr);
    return ws > wa ? ws : wa;
}

gear_status gear_cache_create(const gear_cache_config* c, void* arena, size_t arena_bytes,
                              gear_cache** out) {
    if (!out) return fail(GEAR_ERR_INVALID_ARG, "out is NULL");
    gear_layout pl, fl;
    size_t of, ob, total;
    int mf;
    gear_status st = cache_layouts(c, &pl, &fl, &of, &ob, &total, &mf);
    if (st != GEAR_OK) return st;
    if (!arena || !aligned(arena, kAlign))
        return fail(GEAR_ERR_INVALID_ARG, "arena must be a 256-byte aligned device pointer");
    if (arena_bytes < total)
        return fail(GEAR_ERR_CAPACITY, "arena of %zu bytes is smaller than the %zu needed",
                    arena_bytes, total);
    gear_cache* g = new (std::nothrow) gear_cache;
    if (!g) return fail(GEAR_ERR_INVALID_ARG, "out of host memory");
    g->cfg = *c;
    g->cfg.fill.chunk_tokens = 0;
    g->arena = static_cast<uint8_t*>(arena);
    g->prompt_layout = pl;
    g->fill_layout = fl;
    g->off_prompt = 0;
    g->off_fills = of;
    g->off_buf = ob;
    g->fill_stride = fl.total_bytes;
    g->max_fills = mf;
    g->prompt_loaded = false;
    g->appended = 0;
    g->buf_len = 0;
    g->num_fills = 0;
    g->failed = false;
    *out = g;
    return GEAR_OK;
}

void gear_cache_destroy(gear_cache* cache) { delete cache; }

gear_status gear_cache_load_prompt(gear_cache* g, const void* k_f16, const void* v_f16,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (!g) return fail(GEAR_ERR_INVALID_ARG, "cache is NULL");
    if (g->failed) return failed_cache();
    const gear_cache_config& c = g->cfg;
    if (g->prompt_loaded || g->appended > 0)
        return fail(GEAR_ERR_INVALID_ARG, "the prompt can only be loaded into an empty cache");
    if (c.prompt_tokens == 0) {
        g->prompt_loaded = true;
        return GEAR_OK;
    }
    if (!k_f16 || !v_f16 || !workspace)
        return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(k_f16, 16) || !aligned(v_f16, 16) || !aligned(workspace, kAlign))
        return fail(GEAR_ERR_INVALID_ARG, "k/v must be 16-byte, workspace 256-byte aligned");
    const int64_t half = (int64_t)c.batch * c.kv_heads * (c.prompt_tokens / g->prompt_layout.rows);
    gear_status st = run_compress(&c.prompt, g->prompt_layout, c.head_dim, k_f16, v_f16, half,
                                  GEAR_ROLE_KEYS_THEN_VALUES, g->arena + g->off_prompt, workspace,
                                  workspace_bytes, static_cast<hipStream_t>(stream));
    if (st == GEAR_OK) g->prompt_loaded = true;
    if (st == GEAR_ERR_HIP) g->failed = true;
    return st;
}

gear_status gear_append_tokens(gear_cache* g, const void* k_new_f16, const void* v_new_f16,
                               int32_t n_new, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!g) return fail(GEAR_ERR_INVALID_ARG, "cache is NULL");
    if (g->failed) return failed_cache();
    const gear_cache_config& c = g->cfg;
    if (n_new < 0) return fail(GEAR_ERR_INVALID_ARG, "n_new < 0");
    if (n_new == 0) return GEAR_OK;
    if (c.prompt_tokens > 0 && !g->prompt_loaded)
        return fail(GEAR_ERR_INVALID_ARG, "load the prompt before appending tokens");
    if (g->appended + n_new > c.max_new_tokens)
        return fail(GEAR_ERR_CAPACITY, "appending %d tokens exceeds max_new_tokens %d (have %lld)",
                    n_new, c.max_new_tokens, (long long)g->appended);
    if (!k_new_f16 || !v_new_f16) return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(k_new_f16, 16) || !aligned(v_new_f16, 16))
        return fail(GEAR_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
    const int fills_needed = (g->buf_len + n_new) / c.buf_tokens;
    if (fills_needed > 0) {
        const CompressPlan pl = plan_compress(&c.fill, g->fill_layout, c.head_dim);
        if (!workspace || !aligned(workspace, kAlign))
            return fail(GEAR_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
        if (workspace_bytes < pl.ws_bytes)
            return fail(GEAR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                        workspace_bytes, pl.ws_bytes);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t* buf = reinterpret_cast<uint16_t*>(g->arena + g->off_buf);
    const int64_t mats_half = (int64_t)c.batch * c.kv_heads;
    int done = 0;
    while (done < n_new) {
        const int take = (n_new - done < c.buf_tokens - g->buf_len) ? n_new - done
                                                                     : c.buf_tokens - g->buf_len;
        hipError_t e = launch_buffer_append(static_cast<const uint16_t*>(k_new_f16),
                                            static_cast<const uint16_t*>(v_new_f16), buf, c.batch,
                                            c.kv_heads, c.head_dim, c.buf_tokens, g->buf_len, take,
                                            n_new, done, st);
        if (e != hipSuccess) {
            g->failed = true;
            return hip_fail(e, "buffer append launch");
        }
        g->buf_len += take;
        g->appended += take;
        done += take;
        if (g->buf_len == c.buf_tokens) {
            uint8_t* dst = g->arena + g->off_fills + (size_t)g->num_fills * g->fill_stride;
            gear_status s2 = run_compress(&c.fill, g->fill_layout, c.head_dim, buf, buf, 2 * mats_half,
                                          GEAR_ROLE_KEYS_THEN_VALUES, dst, workspace, workspace_bytes, st);
            if (s2 != GEAR_OK) {   // checked above: only a failed launch gets here
                g->failed = true;
                return s2;
            }
            g->num_fills += 1;
            g->buf_len = 0;
        }
    }
    return GEAR_OK;
}

namespace {

// Validates a decode-attention call and fills its arguments; `extra` tokens
// (appended by the same launch) are counted as cached already.
gear_status attn_args(const gear_cache* g, const void* q_f16, int32_t q_heads, float sm_scale,
                      float* out_f32, void* workspace, size_t workspace_bytes, int extra, AttnArgs* pa) {
    const gear_cache_config& c = g->cfg;
    if (q_heads < c.kv_heads || q_heads % c.kv_heads != 0)
        return fail(GEAR_ERR_INVALID_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads,
                    c.kv_heads);
    const int G = q_heads / c.kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(GEAR_ERR_UNSUPPORTED, "q_heads / kv_heads must be 1, 2, 4 or 8 (got %d)", G);
    if (!q_f16 || !out_f32 || !workspace) return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(q_f16, 16) || !aligned(out_f32, 16) || !aligned(workspace, kAlign))
        return fail(GEAR_ERR_INVALID_ARG,
                    "q_f16 and out_f32 must be 16-byte, workspace 256-byte aligned");
    if (c.prompt_tokens > 0 && !g->prompt_loaded)
        return fail(GEAR_ERR_INVALID_ARG, "load the prompt before decoding");
    const int64_t tokens = (int64_t)(c.prompt_tokens) + g->appended + extra;
    AttnArgs a{};
    const size_t need = attn_workspace_bytes(c.batch, c.kv_heads, q_heads, c.head_dim, tokens,
                                             &a.splits, &a.tokens_per_split);
    if (workspace_bytes < need)
        return fail(GEAR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    workspace_bytes, need);
    a.B = c.batch;
    a.Hkv = c.kv_heads;
    a.Hq = q_heads;
    a.d = c.head_dim;
    a.sm_scale = sm_scale;
    a.q = static_cast<const uint16_t*>(q_f16);
    a.out = out_f32;
    a.prompt.count = c.prompt_tokens > 0 ? 1 : 0;
    a.prompt.chunks = c.prompt_tokens > 0 ? c.prompt_tokens / g->prompt_layout.rows : 0;
    a.prompt.stride = 0;
    const int kv = GEAR_ROLE_KEYS_THEN_VALUES;
    if (c.prompt_tokens > 0)
        a.prompt.p = make_packed(&c.prompt, g->prompt_layout, c.head_dim, g->arena + g->off_prompt, kv);
    else
        a.prompt.p = make_packed(&c.fill, g->fill_layout, c.head_dim, g->arena + g->off_fills, kv);
    a.fills.p = make_packed(&c.fill, g->fill_layout, c.head_dim, g->arena + g->off_fills, kv);
    a.fills.chunks = 1;
    a.fills.count = g->num_fills;
    a.fills.stride = g->fill_stride;
    a.buf = reinterpret_cast<uint16_t*>(g->arena + g->off_buf);
    a.buf_cap = c.buf_tokens;
    a.buf_len = g->buf_len + extra;
    a.partial = static_cast<float*>(workspace);
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.new_row = -1;
    *pa = a;
    return GEAR_OK;
}

}  // namespace

gear_status gear_decode_attn(const gear_cache* g, const void* q_f16, int32_t q_heads,
                             float sm_scale, float* out_f32, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!g) return fail(GEAR_ERR_INVALID_ARG, "cache is NULL");
    if (g->failed) return failed_cache();
    AttnArgs a;
    const gear_status s = attn_args(g, q_f16, q_heads, sm_scale, out_f32, workspace, workspace_bytes, 0, &a);
    if (s != GEAR_OK) return s;
    hipError_t e = launch_decode_attn(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
    return GEAR_OK;
}

gear_status gear_append_decode_attn(gear_cache* g, const void* k_new_f16, const void* v_new_f16,
                                    const void* q_f16, int32_t q_heads, float sm_scale, float* out_f32,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!g) return fail(GEAR_ERR_INVALID_ARG, "cache is NULL");
    if (g->failed) return failed_cache();
    const gear_cache_config& c = g->cfg;
    // a token that fills the buffer: its compression runs between the two
    if (g->buf_len + 1 >= c.buf_tokens) {
        const gear_status s = gear_append_tokens(g, k_new_f16, v_new_f16, 1, workspace, workspace_bytes, stream);
        if (s != GEAR_OK) return s;
        return gear_decode_attn(g, q_f16, q_heads, sm_scale, out_f32, workspace, workspace_bytes, stream);
    }
    // the checks of gear_append_tokens for one token, then those of decoding
    if (c.prompt_tokens > 0 && !g->prompt_loaded)
        return fail(GEAR_ERR_INVALID_ARG, "load the prompt before appending tokens");
    if (g->appended + 1 > c.max_new_tokens)
        return fail(GEAR_ERR_CAPACITY, "appending 1 token exceeds max_new_tokens %d (have %lld)",
                    c.max_new_tokens, (long long)g->appended);
    if (!k_new_f16 || !v_new_f16) return fail(GEAR_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(k_new_f16, 16) || !aligned(v_new_f16, 16))
        return fail(GEAR_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
    AttnArgs a;
    const gear_status s = attn_args(g, q_f16, q_heads, sm_scale, out_f32, workspace, workspace_bytes, 1, &a);
    if (s != GEAR_OK) return s;
    a.k_new = static_cast<const uint16_t*>(k_new_f16);
    a.v_new = static_cast<const uint16_t*>(v_new_f16);
    a.new_row = g->buf_len;
    hipError_t e = launch_decode_attn(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        // the token may or may not have reached the buffer: the cache is no
        // longer usable (as after a failed append)
        g->failed = true;
        return hip_fail(e, "append + decode attention launch");
    }
    g->buf_len += 1;
    g->appended += 1;
    return GEAR_OK;
}

gear_status gear_cache_get_info(const gear_cache* g, gear_cache_info* out) {
    if (!g || !out) return fail(GEAR_ERR_INVALID_ARG, "NULL argument");
    out->tokens = (int64_t)g->cfg.prompt_tokens + g->appended;
    out->buf_len = g->buf_len;
    out->num_fills = g->num_fills;
    out->prompt_packed = g->arena + g->off_prompt;
    out->fill_packed = g->arena + g->off_fills;
    out->fill_stride = g->fill_stride;
    out->buffer_f16 = g->arena + g->off_buf;
    return GEAR_OK;
}

}  // extern "C"
