/*
 * Driver for an AddressSanitizer + UndefinedBehaviorSanitizer build of the
 * CPU oracle (test infrastructure): runs every oracle step on small seeded
 * inputs, including the degenerate settings (k = 0, k = n*d, r = 0, full
 * rank, constant and zero matrices), so that any out-of-bounds access,
 * use of freed memory, signed overflow or misaligned access aborts.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half_to_double(uint16_t h);
int64_t orc_num_outliers(int64_t n, int64_t d, int32_t ppm);
void orc_select_outliers(const uint16_t *x, int64_t n, int64_t d, int64_t k, uint8_t *mask);
void orc_mgs(double *P, int64_t n, int r);
void orc_compress_matrix(const uint16_t *x, int64_t n, int64_t d, int bits, int group,
                         int32_t ppm, int r, int iters, uint64_t seed, uint8_t *packed,
                         float *scale, float *zero, int32_t *row_ptr, uint16_t *col,
                         uint16_t *val, double *A, double *B, double *L, double *xhat);
void orc_attention(const double *K, const double *V, int64_t ntok, int64_t d,
                   const double *q, double scale, double *out);
void orc_compress_matrix_mode(const uint16_t *x, int64_t n, int64_t d, int bits, int group,
                              int mode, int32_t ppm, int r, int iters, uint64_t seed,
                              uint8_t *packed, float *scale, float *zero, int32_t *row_ptr,
                              uint16_t *col, uint16_t *val, double *A, double *B, double *L,
                              double *xhat);
void orc_channel_exponents(const uint16_t *x, int64_t n, int64_t d, int32_t *e);
uint16_t orc_double_to_half(double v);
void orc_channel_normalize(const uint16_t *x, int64_t n, int64_t d, const int32_t *e,
                           uint16_t *xt);

static uint64_t rng_state = 88172645463325252ull;
static uint64_t next_u64(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

/* a finite fp16 bit pattern of moderate magnitude (exponent field 5..24) */
static uint16_t rand_half(void)
{
    uint64_t u = next_u64();
    uint16_t e = (uint16_t)(5 + (u % 20));
    return (uint16_t)(((u >> 8) & 0x8000u) | (e << 10) | ((u >> 20) & 0x3ffu));
}

static int run_case(int64_t n, int64_t d, int bits, int group, int32_t ppm, int r, int iters,
                    int fill, int mode)
{
    const int64_t k = orc_num_outliers(n, d, ppm);
    uint16_t *x = malloc(sizeof(uint16_t) * n * d);
    for (int64_t i = 0; i < n * d; ++i)
        x[i] = fill == 0 ? rand_half() : fill == 1 ? 0u : 0x3e00u /* 1.5 */;
    uint8_t *packed = malloc(n * d * bits / 8);
    float *scale = malloc(sizeof(float) * n * (d / group));
    float *zero = malloc(sizeof(float) * n * (d / group));
    int32_t *row_ptr = malloc(sizeof(int32_t) * (n + 1));
    uint16_t *col = malloc(sizeof(uint16_t) * (k > 0 ? k : 1));
    uint16_t *val = malloc(sizeof(uint16_t) * (k > 0 ? k : 1));
    double *A = malloc(sizeof(double) * n * (r > 0 ? r : 1));
    double *B = malloc(sizeof(double) * d * (r > 0 ? r : 1));
    double *L = malloc(sizeof(double) * n * d);
    double *xhat = malloc(sizeof(double) * n * d);
    orc_compress_matrix_mode(x, n, d, bits, group, mode, ppm, r, iters, 7, packed, scale, zero,
                             row_ptr, col, val, A, B, L, xhat);
    int bad = row_ptr[n] != (int32_t)k;
    if (mode == 0) {   /* the ZipCache steps on the same input */
        int32_t *e = malloc(sizeof(int32_t) * d);
        uint16_t *xt = malloc(sizeof(uint16_t) * n * d);
        orc_channel_exponents(x, n, d, e);
        orc_channel_normalize(x, n, d, e, xt);
        for (int64_t i = 0; i < n * d; ++i) bad |= (xt[i] & 0x7fffu) > 0x3c00u;   /* |x~| <= 1 */
        free(e);
        free(xt);
    }
    for (int64_t i = 0; i < n * d; ++i) bad |= !isfinite(xhat[i]);
    free(x); free(packed); free(scale); free(zero); free(row_ptr); free(col); free(val);
    free(A); free(B); free(L); free(xhat);
    return bad;
}

int main(void)
{
    int bad = 0;
    for (uint32_t h = 0; h < 0x7c00u; h += 7) bad |= !isfinite(orc_half_to_double((uint16_t)h));
    bad |= run_case(256, 64, 4, 64, 20000, 4, 3, 0, 0);
    bad |= run_case(37, 64, 2, 16, 30000, 1, 1, 0, 0);
    bad |= run_case(100, 128, 4, 32, 20000, 3, 2, 0, 0);
    bad |= run_case(64, 128, 2, 8, 1000000, 2, 2, 0, 0);    /* every entry an outlier */
    bad |= run_case(64, 64, 4, 64, 0, 0, 0, 0, 0);          /* plain quantization */
    bad |= run_case(16, 8 * 8, 4, 8, 50000, 8, 4, 0, 0);
    bad |= run_case(8, 64, 4, 64, 20000, 8, 2, 0, 0);       /* r = n (full rank) */
    bad |= run_case(32, 64, 4, 32, 20000, 4, 3, 1, 0);      /* zero matrix */
    bad |= run_case(32, 64, 2, 64, 20000, 4, 3, 2, 0);      /* constant matrix */
    bad |= run_case(128, 64, 4, 32, 20000, 4, 3, 0, 1);     /* per-channel (KIVI keys) */
    bad |= run_case(64, 128, 2, 64, 0, 2, 2, 0, 1);
    for (double v = 1e-9; v < 1e6; v *= 1.37) bad |= orc_double_to_half(v) == 0x7e00u;
    {
        double P[12] = {1, 2, 3, 2, 4, 6, 0, 0, 0, 1, 0, 1};   /* dependent and zero columns */
        orc_mgs(P, 4, 3);
        uint16_t x[6] = {0x3c00, 0xc200, 0x4200, 0x4000, 0x0000, 0x8000};
        uint8_t mask[6];
        orc_select_outliers(x, 3, 2, 6, mask);
        orc_select_outliers(x, 3, 2, 0, mask);
        double K[3 * 4] = {0}, V[3 * 4] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12}, q[4] = {1, 0, 0, 0};
        double out[4];
        orc_attention(K, V, 3, 4, q, 0.5, out);
        bad |= fabs(out[0] - 5.0) > 1e-12;
        orc_attention(K, V, 0, 4, q, 0.5, out);
    }
    printf(bad ? "oracle sanitizer run: FAILED\n" : "oracle sanitizer run: ok\n");
    return bad;
}
