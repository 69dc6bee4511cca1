/*
 * gear_oracle.c -- plain, slow CPU oracle for the GEAR KV-cache compression path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) shares no code, header, table or helper with this file.
 *
 * Sources (web pages about GEAR, arXiv 2403.05527):
 *   [QA]    "GEAR: Efficient KV Cache Compression for LLM Inference" (allpcb.com
 *           Q&A summary), section "Q3: How does the paper solve the problem?"
 *   [CITES] "GEAR: An Efficient KV Cache Compression Recipe for Near-Lossless
 *           Generative Inference of LLM" (app.cochat.ai page), "Cites" list:
 *           sentences of the paper quoted under each cited work, tagged with
 *           the paper section they come from.
 *
 * What each step computes is stated next to it.  Where the pages leave a step
 * open, the reading taken is named in the comment ("reading: ...").
 *
 * Precision: the quantizer runs in IEEE fp32 (round to nearest even, correctly
 * rounded division), because its integer codes must be reproducible; all else
 * is fp64.  Build with -ffp-contract=off so no multiply-add is fused.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle's fp32 steps need float expressions evaluated in float"
#endif

/* ------------------------------------------------------------------------ */
/* fp16 helpers (exact)                                                      */
/* ------------------------------------------------------------------------ */

/* Exact value of an IEEE binary16 bit pattern. */
double orc_half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Step 1: the outlier filter S = Filter_s(X)                                */
/* ------------------------------------------------------------------------ */
/*
 * [CITES] (sentence quoted under the SqueezeLLM entry, paper Background/
 * Method): the largest-magnitude entries are kept "in full precision with a
 * sparse matrix S = Filter_s(X)"; the definition after "where" is lost on the
 * page.  [QA] Q3: a sparse matrix stores and corrects high-magnitude outliers.
 * [CITES] (ZeroQuant entry, Method): s is fixed at 2%.
 *
 * reading: k = floor(n*d*s) entries of largest |x| over the whole matrix,
 * both signs; ties broken by the lower flat index t*d+j, so the set is unique.
 */

/* k = floor(n*d*ppm / 1e6), integer arithmetic. */
int64_t orc_num_outliers(int64_t n, int64_t d, int32_t ppm)
{
    return (n * d * (int64_t)ppm) / 1000000;
}

typedef struct {
    uint16_t mag; /* |x| as the fp16 bit pattern without its sign bit */
    int64_t idx;  /* flat index t*d + j */
} orc_entry;

/* Order: larger magnitude first, then lower flat index first. */
static int orc_entry_cmp(const void *a, const void *b)
{
    const orc_entry *x = (const orc_entry *)a, *y = (const orc_entry *)b;
    if (x->mag != y->mag)
        return x->mag > y->mag ? -1 : 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * mask[t*d+j] = 1 for the k selected entries, 0 otherwise.  For finite fp16
 * values the bit pattern with the sign cleared orders exactly like |x|.
 */
void orc_select_outliers(const uint16_t *x, int64_t n, int64_t d, int64_t k,
                         uint8_t *mask)
{
    int64_t nd = n * d;
    memset(mask, 0, (size_t)nd);
    if (k <= 0)
        return;
    orc_entry *e = (orc_entry *)malloc(sizeof(orc_entry) * (size_t)nd);
    for (int64_t i = 0; i < nd; ++i) {
        e[i].mag = (uint16_t)(x[i] & 0x7fff);
        e[i].idx = i;
    }
    qsort(e, (size_t)nd, sizeof(orc_entry), orc_entry_cmp);
    for (int64_t i = 0; i < k && i < nd; ++i)
        mask[e[i].idx] = 1;
    free(e);
}

/*
 * CSR form of S: row_ptr[n+1], col[k], val[k] (the original fp16 bits, so the
 * stored value is exact -- [CITES] "in full precision").  Columns ascend
 * within a row.
 */
void orc_build_csr(const uint16_t *x, const uint8_t *mask, int64_t n, int64_t d,
                   int32_t *row_ptr, uint16_t *col, uint16_t *val)
{
    int64_t pos = 0;
    for (int64_t t = 0; t < n; ++t) {
        row_ptr[t] = (int32_t)pos;
        for (int64_t j = 0; j < d; ++j) {
            if (mask[t * d + j]) {
                col[pos] = (uint16_t)j;
                val[pos] = x[t * d + j];
                ++pos;
            }
        }
    }
    row_ptr[n] = (int32_t)pos;
}

/* ------------------------------------------------------------------------ */
/* Step 2: group-wise uniform quantization of the extracted matrix           */
/* ------------------------------------------------------------------------ */
/*
 * [CITES] (SqueezeLLM entry): "we perform the quantization on the extracted
 * matrix", i.e. on D = X - S.  [QA] Q3: ultra-low precision, e.g. 4-bit.
 * [CITES] (Jacob et al. / KVQuant entries, Method): group-wise quantization;
 * (FlexGen entry, Method): per-token quantization with fine-grained grouping.
 *
 * readings: groups are g consecutive columns of one token row; the zeros left
 * at outlier positions take part in min/max; zero-point = group min (fp32),
 * scale = (max-min)/(2^b-1) (fp32); code = clamp(rne((D-min)/scale)); a
 * constant group has scale 0 and all codes 0.
 */
void orc_quantize(const float *D, int64_t n, int64_t d, int bits, int group,
                  uint8_t *code, float *scale, float *zero)
{
    const int qmax = (1 << bits) - 1;
    const int64_t ng = d / group;
    for (int64_t t = 0; t < n; ++t) {
        for (int64_t gi = 0; gi < ng; ++gi) {
            const float *v = D + t * d + gi * group;
            float mn = v[0], mx = v[0];
            for (int j = 1; j < group; ++j) {
                if (v[j] < mn) mn = v[j];
                if (v[j] > mx) mx = v[j];
            }
            float diff = mx - mn;                 /* fp32, rounded */
            float s = diff / (float)qmax;         /* fp32, correctly rounded */
            /* a zero scale or zero-point is stored as +0: with -0 and +0 in
               one group the scan order would otherwise pick the sign */
            scale[t * ng + gi] = s + 0.0f;
            zero[t * ng + gi] = mn + 0.0f;
            for (int j = 0; j < group; ++j) {
                int c = 0;
                if (s != 0.0f) {
                    float q = (v[j] - mn) / s;    /* two fp32 roundings */
                    float r = rintf(q);           /* round half to even */
                    if (r < 0.0f) r = 0.0f;
                    if (r > (float)qmax) r = (float)qmax;
                    c = (int)r;
                }
                code[t * d + gi * group + j] = (uint8_t)c;
            }
        }
    }
}

/*
 * Packing (this library's storage format): the b-bit code of column j of row
 * t sits in byte t*(d*b/8) + floor(j*b/8) at bit offset (j*b) mod 8, least
 * significant bits first.
 */
void orc_pack_codes(const uint8_t *code, int64_t n, int64_t d, int bits,
                    uint8_t *packed)
{
    const int64_t row_bytes = d * bits / 8;
    memset(packed, 0, (size_t)(n * row_bytes));
    for (int64_t t = 0; t < n; ++t)
        for (int64_t j = 0; j < d; ++j)
            packed[t * row_bytes + (j * bits) / 8] |=
                (uint8_t)(code[t * d + j] << ((j * bits) % 8));
}

/* deq = code*scale + zero, in fp64. */
void orc_dequantize(const uint8_t *code, const float *scale, const float *zero,
                    int64_t n, int64_t d, int group, double *deq)
{
    const int64_t ng = d / group;
    for (int64_t t = 0; t < n; ++t)
        for (int64_t j = 0; j < d; ++j) {
            int64_t gi = t * ng + j / group;
            deq[t * d + j] = (double)code[t * d + j] * (double)scale[gi] + (double)zero[gi];
        }
}

/*
 * KIVI-style key quantization ([CITES], the KIVI entry and the sentence quoted
 * under it, Method: when GEAR is combined with KIVI the streaming buffer must
 * hold at least one group; the "Cited by" quote of the same page: KIVI
 * quantizes keys per channel and values per token).
 *
 * reading: a group is `group` consecutive tokens of one channel (column j);
 * min, max, scale, zero-point, rounding and clamping exactly as in
 * orc_quantize.  scale and zero are laid out [n/group][d] (group index, then
 * channel); n must be a multiple of group.
 */
void orc_quantize_channel(const float *D, int64_t n, int64_t d, int bits, int group,
                          uint8_t *code, float *scale, float *zero)
{
    const int qmax = (1 << bits) - 1;
    for (int64_t gi = 0; gi < n / group; ++gi) {
        for (int64_t j = 0; j < d; ++j) {
            const float *v = D + gi * group * d + j;   /* v[i * d]: token gi*group + i */
            float mn = v[0], mx = v[0];
            for (int i = 1; i < group; ++i) {
                if (v[i * d] < mn) mn = v[i * d];
                if (v[i * d] > mx) mx = v[i * d];
            }
            float diff = mx - mn;
            float sc = diff / (float)qmax;
            scale[gi * d + j] = sc + 0.0f;
            zero[gi * d + j] = mn + 0.0f;
            for (int i = 0; i < group; ++i) {
                int c = 0;
                if (sc != 0.0f) {
                    float q = (v[i * d] - mn) / sc;
                    float r = rintf(q);
                    if (r < 0.0f) r = 0.0f;
                    if (r > (float)qmax) r = (float)qmax;
                    c = (int)r;
                }
                code[(gi * group + i) * d + j] = (uint8_t)c;
            }
        }
    }
}

/* deq = code*scale + zero for the per-channel layout, in fp64. */
void orc_dequantize_channel(const uint8_t *code, const float *scale, const float *zero,
                            int64_t n, int64_t d, int group, double *deq)
{
    for (int64_t t = 0; t < n; ++t)
        for (int64_t j = 0; j < d; ++j) {
            int64_t gi = (t / group) * d + j;
            deq[t * d + j] = (double)code[t * d + j] * (double)scale[gi] + (double)zero[gi];
        }
}

/*
 * ZipCache's channel-separable tokenwise quantization ("ZipCache: Accurate and
 * Efficient KV Cache Quantization with Salient Token Identification",
 * abstract): the channel dimension is separated out of the quantization
 * parameters, which are then per token.
 *
 * reading: channel j of X is divided by a power of two 2^e_j, the smallest one
 * not below the channel's largest |x| (e_j = 0 for an all-zero channel), so
 * that the normalized entries lie in [-1, 1] and the division is exact up to
 * fp16 rounding of subnormal results; GEAR (outliers, quantization with one
 * group per token, low-rank fit) then runs on the normalized matrix, and the
 * reconstruction multiplies channel j back by 2^e_j.
 */

/* e_j for every channel of x (n x d fp16 bits). */
void orc_channel_exponents(const uint16_t *x, int64_t n, int64_t d, int32_t *e)
{
    for (int64_t j = 0; j < d; ++j) {
        double m = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double v = fabs(orc_half_to_double(x[t * d + j]));
            if (v > m) m = v;
        }
        int32_t k = 0;
        if (m > 0.0) {
            int ex;
            double f = frexp(m, &ex);          /* m = f 2^ex, f in [0.5, 1) */
            k = (f == 0.5) ? ex - 1 : ex;      /* smallest k with 2^k >= m */
        }
        e[j] = k;
    }
}

/* The binary16 bit pattern nearest to a finite double (ties to even),
 * subnormals included; values beyond the largest finite half become
 * infinity. */
uint16_t orc_double_to_half(double v)
{
    uint16_t sign = (uint16_t)(signbit(v) ? 0x8000u : 0u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                    /* a in [2^(ex-1), 2^ex) */
    int e = ex - 1;                   /* unbiased exponent of a */
    if (e < -14) e = -14;             /* subnormal range: fixed quantum 2^-24 */
    double q = ldexp(1.0, e - 10);    /* spacing of halves around a */
    double m = a / q;                 /* exact: a scaled by a power of two */
    double r = nearbyint(m);          /* ties to even (default rounding mode) */
    double h = r * q;
    if (h >= 65520.0)                 /* rounds above the largest finite half */
        return (uint16_t)(sign | 0x7c00u);
    /* h = r 2^(e-10) with r <= 2048: encode */
    if (h < ldexp(1.0, -14))          /* subnormal (or rounded up to the min normal) */
        return (uint16_t)(sign | (uint16_t)(h / ldexp(1.0, -24)));
    int hex;
    double hf = frexp(h, &hex);       /* h = hf 2^hex, hf in [0.5, 1) */
    uint16_t mant = (uint16_t)((hf * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((hex - 1 + 15) << 10) | mant);
}

/* xt = fl16(x * 2^-e_j), channel by channel. */
void orc_channel_normalize(const uint16_t *x, int64_t n, int64_t d, const int32_t *e,
                           uint16_t *xt)
{
    for (int64_t t = 0; t < n; ++t)
        for (int64_t j = 0; j < d; ++j)
            xt[t * d + j] = orc_double_to_half(ldexp(orc_half_to_double(x[t * d + j]), -e[j]));
}

/* ------------------------------------------------------------------------ */
/* Step 3: low-rank approximation of the quantization residual               */
/* ------------------------------------------------------------------------ */
/*
 * [QA] Q3: a low-rank matrix approximates the residual error of quantization,
 * "implemented via singular value decomposition".  [CITES] (PowerSGD entry):
 * the paper cites PowerSGD's power-iteration scheme.  [CITES] (ZeroQuant
 * entry, Method): rank 4 for prefill inputs, rank 2 per group of new tokens.
 *
 * reading: a fixed number t of PowerSGD steps from a deterministic start B0:
 *     P = R B;  A = orthonormalise(P) (modified Gram-Schmidt);  B = R^T A,
 * and L = A B^T = A A^T R.  A column whose norm after projection is <= 1e-6
 * times its norm before projection (or is zero) is set to zero.
 */

/* splitmix64 (Steele, Lea and Flood 2014; Vigna's reference formulation):
 * output number i (i >= 1) of the generator whose state starts at `seed`. */
uint64_t orc_splitmix64(uint64_t seed, uint64_t i)
{
    uint64_t z = seed + i * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* B0[j][c] = u24 * 2^-23 - 1, u24 = top 24 bits of output (j*r + c + 1). */
void orc_init_b0(int64_t d, int r, uint64_t seed, double *B0)
{
    for (int64_t j = 0; j < d; ++j)
        for (int c = 0; c < r; ++c) {
            uint64_t u = orc_splitmix64(seed, (uint64_t)(j * r + c + 1)) >> 40;
            B0[j * r + c] = ldexp((double)u, -23) - 1.0;
        }
}

/* Modified Gram-Schmidt on the r columns of P (n x r, row-major), in place. */
void orc_mgs(double *P, int64_t n, int r)
{
    for (int c = 0; c < r; ++c) {
        double pre = 0.0;
        for (int64_t t = 0; t < n; ++t)
            pre += P[t * r + c] * P[t * r + c];
        pre = sqrt(pre);
        for (int i = 0; i < c; ++i) {
            double dot = 0.0;
            for (int64_t t = 0; t < n; ++t)
                dot += P[t * r + i] * P[t * r + c];
            for (int64_t t = 0; t < n; ++t)
                P[t * r + c] -= dot * P[t * r + i];
        }
        double post = 0.0;
        for (int64_t t = 0; t < n; ++t)
            post += P[t * r + c] * P[t * r + c];
        post = sqrt(post);
        int dead = (pre == 0.0) || (post <= 1e-6 * pre);
        for (int64_t t = 0; t < n; ++t)
            P[t * r + c] = dead ? 0.0 : P[t * r + c] / post;
    }
}

/*
 * R: n x d; B0: d x r.  Outputs A (n x r) and B (d x r), row-major, after
 * `iters` steps.  With r == 0 nothing is written.
 */
void orc_power_iteration(const double *R, int64_t n, int64_t d, int r, int iters,
                         const double *B0, double *A, double *B)
{
    if (r <= 0)
        return;
    memcpy(B, B0, sizeof(double) * (size_t)(d * r));
    for (int it = 0; it < iters; ++it) {
        for (int64_t t = 0; t < n; ++t)            /* P = R B */
            for (int c = 0; c < r; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < d; ++j)
                    acc += R[t * d + j] * B[j * r + c];
                A[t * r + c] = acc;
            }
        orc_mgs(A, n, r);                          /* A = orth(P) */
        for (int64_t j = 0; j < d; ++j)            /* B = R^T A */
            for (int c = 0; c < r; ++c) {
                double acc = 0.0;
                for (int64_t t = 0; t < n; ++t)
                    acc += R[t * d + j] * A[t * r + c];
                B[j * r + c] = acc;
            }
    }
}

/* L = A B^T (n x d). */
void orc_low_rank_product(const double *A, const double *B, int64_t n, int64_t d,
                          int r, double *L)
{
    for (int64_t t = 0; t < n; ++t)
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int c = 0; c < r; ++c)
                acc += A[t * r + c] * B[j * r + c];
            L[t * d + j] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* The whole compression of one matrix, and its reconstruction               */
/* ------------------------------------------------------------------------ */
/*
 * [QA] Q3 and [CITES] (Zafrir et al. entry, Background): X is approximated by
 * the composite D^ + L + S -- quantized backbone, low-rank part, sparse part.
 *
 * Inputs: x (n x d fp16 bits), bits, group, ppm, r, iters, seed.
 * Outputs (any may be NULL except where noted):
 *   packed   n*d*bits/8 bytes            codes, packed as in orc_pack_codes
 *   scale    n*(d/group) floats          zero  n*(d/group) floats
 *   row_ptr  n+1;  col, val  k entries   (k = orc_num_outliers)
 *   A        n*r doubles;  B  d*r doubles
 *   L        n*d doubles (the low-rank term)
 *   xhat     n*d doubles (D^ + L + S, the reconstruction)
 */
/* mode 0: groups of `group` columns of a token (scale/zero [n][d/group]);
 * mode 1: groups of `group` tokens of a channel (KIVI keys; scale/zero
 * [n/group][d]).  Both hold n*d/group parameters. */
void orc_compress_matrix_mode(const uint16_t *x, int64_t n, int64_t d, int bits,
                              int group, int mode, int32_t ppm, int r, int iters,
                              uint64_t seed, uint8_t *packed, float *scale,
                              float *zero, int32_t *row_ptr, uint16_t *col,
                              uint16_t *val, double *A, double *B, double *L,
                              double *xhat)
{
    const int64_t nd = n * d, ng = d / group;
    const int64_t k = orc_num_outliers(n, d, ppm);
    uint8_t *mask = (uint8_t *)malloc((size_t)nd);
    float *Dm = (float *)malloc(sizeof(float) * (size_t)nd);
    uint8_t *code = (uint8_t *)malloc((size_t)nd);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(n * ng));
    float *zr = (float *)malloc(sizeof(float) * (size_t)(n * ng));
    double *deq = (double *)malloc(sizeof(double) * (size_t)nd);
    double *R = (double *)malloc(sizeof(double) * (size_t)nd);
    double *Lw = (double *)calloc((size_t)nd, sizeof(double));
    double *Aw = (double *)malloc(sizeof(double) * (size_t)(n * (r > 0 ? r : 1)));
    double *Bw = (double *)malloc(sizeof(double) * (size_t)(d * (r > 0 ? r : 1)));
    double *B0 = (double *)malloc(sizeof(double) * (size_t)(d * (r > 0 ? r : 1)));

    /* S = Filter_s(X); D = X with the S positions set to zero. */
    orc_select_outliers(x, n, d, k, mask);
    for (int64_t i = 0; i < nd; ++i)
        Dm[i] = mask[i] ? 0.0f : (float)orc_half_to_double(x[i]);

    /* Q = quantize(D); D^ = deq(Q). */
    if (mode == 1) {
        orc_quantize_channel(Dm, n, d, bits, group, code, sc, zr);
        orc_dequantize_channel(code, sc, zr, n, d, group, deq);
    } else {
        orc_quantize(Dm, n, d, bits, group, code, sc, zr);
        orc_dequantize(code, sc, zr, n, d, group, deq);
    }

    /* R = X - S - D^ = D - D^; L = rank-r fit of R. */
    for (int64_t i = 0; i < nd; ++i)
        R[i] = (double)Dm[i] - deq[i];
    if (r > 0) {
        orc_init_b0(d, r, seed, B0);
        orc_power_iteration(R, n, d, r, iters, B0, Aw, Bw);
        orc_low_rank_product(Aw, Bw, n, d, r, Lw);
    }

    if (packed) orc_pack_codes(code, n, d, bits, packed);
    if (scale) memcpy(scale, sc, sizeof(float) * (size_t)(n * ng));
    if (zero) memcpy(zero, zr, sizeof(float) * (size_t)(n * ng));
    if (row_ptr && col && val) orc_build_csr(x, mask, n, d, row_ptr, col, val);
    if (A && r > 0) memcpy(A, Aw, sizeof(double) * (size_t)(n * r));
    if (B && r > 0) memcpy(B, Bw, sizeof(double) * (size_t)(d * r));
    if (L) memcpy(L, Lw, sizeof(double) * (size_t)nd);
    if (xhat)
        for (int64_t i = 0; i < nd; ++i)   /* S is added, not substituted */
            xhat[i] = deq[i] + Lw[i] + (mask[i] ? orc_half_to_double(x[i]) : 0.0);

    free(mask); free(Dm); free(code); free(sc); free(zr); free(deq);
    free(R); free(Lw); free(Aw); free(Bw); free(B0);
}

/* GEAR's own quantizer (groups along head_dim). */
void orc_compress_matrix(const uint16_t *x, int64_t n, int64_t d, int bits,
                         int group, int32_t ppm, int r, int iters, uint64_t seed,
                         uint8_t *packed, float *scale, float *zero,
                         int32_t *row_ptr, uint16_t *col, uint16_t *val,
                         double *A, double *B, double *L, double *xhat)
{
    orc_compress_matrix_mode(x, n, d, bits, group, 0, ppm, r, iters, seed, packed, scale,
                             zero, row_ptr, col, val, A, B, L, xhat);
}

/* ------------------------------------------------------------------------ */
/* Decode-time read: one query against a reconstructed K^/V^                 */
/* ------------------------------------------------------------------------ */
/*
 * [QA] Q4 (system performance): the compressed cache is read back at decode
 * time.  Scaled dot-product attention of one query over ntok cached tokens:
 *     s_t = scale * q . K^_t;  p = softmax(s);  out = sum_t p_t V^_t.
 * reading: no mask; fp64 throughout.
 */
void orc_attention(const double *K, const double *V, int64_t ntok, int64_t d,
                   const double *q, double scale, double *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
    double mx = -INFINITY;
    for (int64_t t = 0; t < ntok; ++t) {
        double acc = 0.0;
        for (int64_t j = 0; j < d; ++j)
            acc += q[j] * K[t * d + j];
        s[t] = scale * acc;
        if (s[t] > mx) mx = s[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < ntok; ++t) {
        s[t] = exp(s[t] - mx);
        sum += s[t];
    }
    for (int64_t j = 0; j < d; ++j)
        out[j] = 0.0;
    for (int64_t t = 0; t < ntok; ++t)
        for (int64_t j = 0; j < d; ++j)
            out[j] += (s[t] / sum) * V[t * d + j];
    free(s);
}
