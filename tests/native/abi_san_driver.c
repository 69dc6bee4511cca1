/*
 * Driver for an AddressSanitizer + UndefinedBehaviorSanitizer build of the
 * host side of libgear.so (test infrastructure, no GPU): layouts, parameter
 * validation, workspace and arena sizing, the streaming cache's bookkeeping
 * and its refusals, status strings and the timing registry.  Device pointers
 * are fake: every call here must be refused on the host before any launch,
 * except the one append whose launch fails because no GPU is present (which
 * also exercises the failed-cache state).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gear.h"

#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            printf("FAILED line %d: %s (%s)\n", __LINE__, #cond,        \
                   gear_last_error());                                 \
            return 1;                                                  \
        }                                                              \
    } while (0)

static gear_params P(int bits, int group, int ppm, int rank, int iters, int chunk)
{
    gear_params p;
    memset(&p, 0, sizeof p);
    p.bits = bits;
    p.group = group;
    p.outlier_ppm = ppm;
    p.rank = rank;
    p.power_iters = iters;
    p.chunk_tokens = chunk;
    p.seed = 0;
    return p;
}

int main(int argc, char** argv)
{
    setvbuf(stdout, NULL, _IONBF, 0);
    const int no_gpu = argc > 1 && strcmp(argv[1], "--no-gpu") == 0;
    void* fake = (void*)(uintptr_t)0x20000000u;
    /* layouts over a grid of valid and invalid settings */
    const int bits[] = {0, 2, 3, 4, 8};
    const int groups[] = {4, 8, 16, 48, 64, 128, 256};
    const int ranks[] = {-1, 0, 1, 4, 8, 9};
    const int dims[] = {0, 64, 96, 128};
    const int ns[] = {0, 1, 4, 37, 64, 4096, 1 << 25};
    int ok = 0, rejected = 0;
    for (unsigned a = 0; a < sizeof bits / sizeof *bits; ++a)
        for (unsigned b = 0; b < sizeof groups / sizeof *groups; ++b)
            for (unsigned c = 0; c < sizeof ranks / sizeof *ranks; ++c)
                for (unsigned e = 0; e < sizeof dims / sizeof *dims; ++e)
                    for (unsigned f = 0; f < sizeof ns / sizeof *ns; ++f) {
                        gear_params p = P(bits[a], groups[b], 20000, ranks[c], 3, 0);
                        gear_shape s = {3, ns[f], dims[e]};
                        gear_layout L;
                        const gear_status st = gear_packed_layout(&p, &s, &L);
                        const size_t nb = gear_packed_bytes(&p, &s);
                        const size_t ws = gear_compress_workspace_bytes(&p, &s);
                        if (st == GEAR_OK) {
                            ++ok;
                            EXPECT(nb == L.total_bytes && nb % 256 == 0 && ws >= 256);
                            EXPECT(L.off_b + (size_t)L.num_compressed * s.head_dim * p.rank * 4 <= nb);
                        } else {
                            ++rejected;
                            EXPECT(nb == 0 && ws == 0 && strlen(gear_last_error()) > 0);
                            EXPECT(gear_compress(&p, &s, fake, fake, fake, 1 << 20, NULL) == st);
                        }
                    }
    EXPECT(ok > 0 && rejected > 0);
    {
        gear_params p = P(4, 128, 20000, 4, 3, 0);
        gear_shape s = {2, 128, 128};
        EXPECT(gear_compress(NULL, &s, fake, fake, fake, 1 << 20, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_compress(&p, NULL, fake, fake, fake, 1 << 20, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_compress(&p, &s, NULL, fake, fake, 1 << 20, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_compress(&p, &s, (char*)fake + 8, fake, fake, 1 << 20, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_compress(&p, &s, fake, fake, fake, 0, NULL) == GEAR_ERR_WORKSPACE);
        EXPECT(gear_decompress(&p, &s, NULL, fake, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_decompress(&p, &s, (char*)fake + 16, fake, NULL) == GEAR_ERR_INVALID_ARG);
        gear_shape e = {0, 128, 128};   /* an empty stack launches nothing */
        EXPECT(gear_compress(&p, &e, NULL, NULL, NULL, 0, NULL) == GEAR_ERR_INVALID_ARG ||
               gear_compress(&p, &e, fake, fake, fake, 1 << 20, NULL) == GEAR_OK);
    }
    /* caches: sizing, capacity, refusals, info, destroy */
    for (int pt = 0; pt <= 2048; pt += 2048) {
        gear_cache_config c;
        memset(&c, 0, sizeof c);
        c.prompt = P(4, 128, 20000, 4, 3, pt ? 512 : 0);
        c.fill = P(4, 128, 20000, 2, 3, 0);
        c.batch = 3;
        c.kv_heads = 2;
        c.head_dim = 128;
        c.prompt_tokens = pt;
        c.buf_tokens = 64;
        c.max_new_tokens = 200;
        const size_t n = gear_cache_arena_bytes(&c);
        EXPECT(n > 0 && gear_cache_workspace_bytes(&c, 8) > 0 && gear_cache_workspace_bytes(&c, 3) == 0);
        gear_cache* h = NULL;
        EXPECT(gear_cache_create(&c, fake, n - 1, &h) == GEAR_ERR_CAPACITY);
        EXPECT(gear_cache_create(&c, (char*)fake + 16, n, &h) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_cache_create(&c, fake, n, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_cache_create(&c, fake, n, &h) == GEAR_OK && h != NULL);
        gear_cache_info inf;
        EXPECT(gear_cache_get_info(h, &inf) == GEAR_OK && inf.tokens == pt && inf.buf_len == 0);
        EXPECT(gear_append_tokens(h, fake, fake, 201, fake, 1 << 30, NULL) ==
               (pt > 0 ? GEAR_ERR_INVALID_ARG : GEAR_ERR_CAPACITY));
        EXPECT(gear_append_tokens(h, fake, fake, -1, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_append_tokens(h, fake, fake, 0, fake, 1 << 30, NULL) == GEAR_OK);
        EXPECT(gear_decode_attn(h, fake, 3, 0.1f, fake, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_decode_attn(h, fake, 32, 0.1f, fake, fake, 1 << 30, NULL) == GEAR_ERR_UNSUPPORTED);
        EXPECT(gear_decode_attn(h, (char*)fake + 2, 4, 0.1f, fake, fake, 1 << 30, NULL) ==
               GEAR_ERR_INVALID_ARG);
        EXPECT(gear_append_decode_attn(h, NULL, fake, fake, 4, 0.1f, fake, fake, 1 << 30, NULL) ==
               GEAR_ERR_INVALID_ARG);
        EXPECT(gear_append_decode_attn(h, fake, fake, fake, 32, 0.1f, fake, fake, 1 << 30, NULL) ==
               (pt > 0 ? GEAR_ERR_INVALID_ARG : GEAR_ERR_UNSUPPORTED));
        EXPECT(gear_append_decode_attn(h, fake, fake, fake, 4, 0.1f, fake, fake, 16, NULL) ==
               (pt > 0 ? GEAR_ERR_INVALID_ARG : GEAR_ERR_WORKSPACE));
        if (pt > 0) {
            EXPECT(gear_decode_attn(h, fake, 4, 0.1f, fake, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
            EXPECT(gear_append_tokens(h, fake, fake, 1, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
            EXPECT(gear_cache_load_prompt(h, NULL, fake, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
            EXPECT(gear_cache_load_prompt(h, fake, fake, fake, 16, NULL) == GEAR_ERR_WORKSPACE);
        } else if (no_gpu) {
            /* the buffer-append launch fails without a GPU: the cache is failed */
            EXPECT(gear_append_tokens(h, fake, fake, 1, fake, 1 << 30, NULL) == GEAR_ERR_HIP);
            EXPECT(gear_append_tokens(h, fake, fake, 1, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
            EXPECT(gear_decode_attn(h, fake, 4, 0.1f, fake, fake, 1 << 30, NULL) == GEAR_ERR_INVALID_ARG);
        }
        gear_cache_destroy(h);
    }
    gear_cache_destroy(NULL);
    for (int s = -1; s <= 6; ++s) EXPECT(strlen(gear_status_str((gear_status)s)) > 0);
    {
        int64_t n = -1;
        double ms = -1.0;
        EXPECT(gear_timing_enable(1) == GEAR_OK);
        EXPECT(gear_timing_read("compress", &n, &ms) == GEAR_OK && n == 0 && ms == 0.0);
        EXPECT(gear_timing_read("nope", &n, &ms) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_timing_read(NULL, &n, &ms) == GEAR_ERR_INVALID_ARG);
        EXPECT(gear_timing_enable(0) == GEAR_OK);
    }
    printf("host library sanitizer run: ok\n");
    return 0;
}
