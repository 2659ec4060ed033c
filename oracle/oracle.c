/*
 * oracle.c -- plain, slow CPU reference for the quantized dense projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no source
 * with the HIP library (no headers, helpers, tables or constants).
 *
 * What it computes is taken from the five documentation pages on the method
 * (cited by page file name and item).  Where the pages leave a rule open the
 * reading taken is stated next to the code:
 *   - absmax scaling: int8 scale = amax/127, row FP8 scale = amax/448,
 *     NVFP4 sub-block scale = E4M3(amax / (6 * scale2));
 *   - every rounding onto a code grid is round-to-nearest, ties to the even
 *     code; E4M3 saturates at +-448, E2M1 at +-6, int8 at +-127;
 *   - the element is divided by the *stored* scale with one IEEE binary32
 *     division, then rounded onto the grid;
 *   - the sign of a value that rounds to zero is kept (E4M3 0x80, E2M1 0x8);
 *   - a block (or row) whose scale is 0 gets scale 0 and all-+0 codes.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * that each "fl(.)" below is one binary32 operation rounded to nearest even.
 * Integer block sums are exact in int64; float sums are carried in binary64.
 *
 * Parity status: every function here is pinned by the CPU tests (decode
 * tables, hand-worked blocks, brute force on tiny shapes, library cross
 * checks and the pages' invariants).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Codecs                                                              */
/* ------------------------------------------------------------------ */

/* E2M1 (OCP MX FP4): 1 sign bit, 2 exponent bits, 1 mantissa bit.  The
 * magnitudes of codes 0..7 are the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t c)
{
    double v = E2M1_GRID[c & 7];
    return (c & 8) ? -v : v;
}

/* E4M3 (OCP E4M3FN): bias 7, no infinities, S.1111.111 is NaN, max 448. */
double oracle_e4m3_decode(uint8_t c)
{
    int e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);           /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);    /* normal */
    return (c & 0x80) ? -v : v;
}

/* Nearest point of a sorted magnitude grid g[0..n-1] (g[0] = 0) to a >= 0.
 * Ties go to the even index, which for both FP formats here is the code
 * with an even mantissa LSB.  Values beyond the last point saturate. */
static int nearest_index(const double *g, int n, double a)
{
    int lo = 0;
    if (a >= g[n - 1])
        return n - 1;
    /* largest index with g[lo] <= a (binary search over the sorted grid) */
    int hi = n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - g[lo], dhi = g[lo + 1] - a;   /* exact in binary64 */
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

uint8_t oracle_e2m1_encode(float y)
{
    double a = fabs((double)y);
    int i = nearest_index(E2M1_GRID, 8, a);       /* |y| >= 6 -> 7 (6.0) */
    return (uint8_t)(i | (signbit(y) ? 8 : 0));
}

static double E4M3_GRID[127];   /* magnitudes of codes 0x00..0x7E */

/* Filled once when the library is loaded, before any parallel region. */
__attribute__((constructor)) static void e4m3_grid_init(void)
{
    for (int c = 0; c < 127; ++c)
        E4M3_GRID[c] = oracle_e4m3_decode((uint8_t)c);
}

uint8_t oracle_e4m3_encode(float y)
{
    double a = fabs((double)y);
    /* |y| >= 448 saturates to 0x7E (this covers the (448, 464) band that
     * rounds to 448 anyway and everything that would reach the NaN slot). */
    int i = nearest_index(E4M3_GRID, 127, a);
    return (uint8_t)(i | (signbit(y) ? 0x80 : 0));
}

int8_t oracle_int8_encode(float y)
{
    double r = nearbyint((double)y);    /* round half to even */
    if (r > 127.0)
        r = 127.0;
    if (r < -127.0)
        r = -127.0;
    return (int8_t)r;
}

/* The three encoders above over an array (one code per byte; E2M1 codes in
 * the low nibble), for checks that sweep many values at once. */
void oracle_encode_array(int kind, const float *y, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = kind == 0 ? oracle_e4m3_encode(y[i])
               : kind == 1 ? oracle_e2m1_encode(y[i])
                           : (uint8_t)oracle_int8_encode(y[i]);
}

float oracle_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary64 value to the nearest bfloat16 (ties to even), once. */
uint16_t oracle_bf16_from_double(double x)
{
    if (isnan(x))
        return 0x7FC0;
    int sign = signbit(x) ? 1 : 0;
    double a = fabs(x);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                     /* a = f * 2^e, f in [0.5, 1) */
        int q = e - 8;                    /* bf16 keeps 8 significant bits */
        if (q < -133)
            q = -133;                     /* subnormal spacing 2^-133 */
        r = ldexp(nearbyint(ldexp(a, -q)), q);
        if (r >= 0x1p128)
            r = INFINITY;
    }
    float f = (float)r;                   /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u >> 16) | (sign ? 0x8000u : 0u));
}

/* One binary32 division, as the f32 division instruction of the host. */
static float fdiv32(float x, float y)
{
    volatile float r = x / y;
    return r;
}

/* ------------------------------------------------------------------ */
/* Quantizers                                                          */
/* ------------------------------------------------------------------ */

/* Absmax int8 quantisation of one block of n f32 values (shared by the
 * activation requant and the weight requant below, both per 32). */
static void int8_block(const float *v, int n, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    float s = fdiv32(amax, 127.0f);
    *scale = s;
    for (int i = 0; i < n; ++i)
        q[i] = (s == 0.0f) ? 0 : oracle_int8_encode(fdiv32(v[i], s));
}

/* gemm_dense_int8.rs, int8_gemm_faith2_prefill, step (a): BF16 activations
 * [m,k] -> int8 [m,k] plus one F32 scale per 32 elements [m,k/32]. */
void oracle_requant_a_bf16_int8(const uint16_t *a, int8_t *q, float *scale,
                                int64_t m, int64_t k)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i)
                v[i] = oracle_bf16_to_float(a[r * k + b * 32 + i]);
            int8_block(v, 32, q + r * k + b * 32, scale + r * nb + b);
        }
    }
}

/* gemm_dense_int8.rs, requant_w_nvfp4_int8: packed E2M1 [n,k/2] (low nibble
 * = even k), E4M3 sub-block scales [n,k/16] and the per-tensor scale2 are
 * dequantised (value = e2m1 * e4m3 * scale2, the first product exact, one
 * f32 rounding for the second), then two 16-element sub-blocks are re-blocked
 * into one 32-element int8 block with an F32 absmax scale. */
void oracle_requant_w_nvfp4_int8(const uint8_t *packed, const uint8_t *sc16,
                                 float scale2, int8_t *q, float *scale,
                                 int64_t n, int64_t k)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i) {
                int64_t kk = b * 32 + i;
                uint8_t byte = packed[r * (k / 2) + kk / 2];
                uint8_t code = (kk % 2 == 0) ? (byte & 15) : (byte >> 4);
                double p = oracle_e2m1_decode(code) *
                           oracle_e4m3_decode(sc16[r * (k / 16) + kk / 16]);
                v[i] = (float)p * scale2;   /* p is exact in f32 */
            }
            int8_block(v, 32, q + r * k + b * 32, scale + r * nb + b);
        }
    }
}

/* gemm_fp4.rs, quantize_bf16_to_nvfp4: BF16 [rows,k] -> packed E2M1
 * [rows,k/2] plus one E4M3 scale per 16 elements [rows,k/16].  The scale
 * maps the block absmax onto the largest E2M1 magnitude (6) after the
 * per-tensor scale2 is taken out: sb = E4M3(amax / (6*scale2)); elements
 * are divided by the decoded scale d = e4m3(sb)*scale2 and rounded to E2M1. */
void oracle_quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed,
                                uint8_t *sc16, float scale2,
                                int64_t rows, int64_t k)
{
    int64_t nb = k / 16;
    float six_s2 = 6.0f * scale2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float v[16];
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                v[i] = oracle_bf16_to_float(x[r * k + b * 16 + i]);
                if (fabsf(v[i]) > amax)
                    amax = fabsf(v[i]);
            }
            uint8_t sb = oracle_e4m3_encode(fdiv32(amax, six_s2));
            float d = (float)oracle_e4m3_decode(sb) * scale2;
            sc16[r * nb + b] = sb;
            uint8_t codes[16];
            for (int i = 0; i < 16; ++i)
                codes[i] = (d == 0.0f) ? 0 : oracle_e2m1_encode(fdiv32(v[i], d));
            for (int i = 0; i < 8; ++i)
                packed[r * (k / 2) + b * 8 + i] =
                    (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

/* dispatch_proj_rowwise.rs, quant_rowwise_fp8 (and quantize_fns.rs,
 * quantize_to_fp8): each row of a BF16 [rows,k] matrix -> E4M3 codes plus
 * one F32 scale per row, s = amax/448. */
static void rowwise_fp8_row(const float *v, int64_t k, uint8_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < k; ++i)
        if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    float s = fdiv32(amax, 448.0f);
    *s_out = s;
    for (int64_t i = 0; i < k; ++i)
        q[i] = (s == 0.0f) ? 0 : oracle_e4m3_encode(fdiv32(v[i], s));
}

void oracle_quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *scale,
                              int64_t rows, int64_t k)
{
#pragma omp parallel
    {
        float *v = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t i = 0; i < k; ++i)
                v[i] = oracle_bf16_to_float(x[r * k + i]);
            rowwise_fp8_row(v, k, q + r * k, scale + r);
        }
        free(v);
    }
}

/* dispatch_proj_rowwise.rs, requant_weight_rowwise_fp8_cached: a
 * block-scaled FP8 weight (E4M3 [n,k] with an F32 grid [n/128,k/128]) goes
 * block-FP8 -> BF16 -> row-wise FP8.  The BF16 intermediate is normative:
 * y = bf16(fl(e4m3(w) * S[n/128][k/128])), then the row quantiser above runs
 * on y.  The per-row passthrough of that page is pointer logic and lives in
 * the tests, not here. */
void oracle_requant_w_blockfp8_rowwise(const uint8_t *w, const float *grid,
                                       uint8_t *q, float *scale,
                                       int64_t n, int64_t k)
{
    int64_t sk = k / 128;
#pragma omp parallel
    {
        float *v = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < n; ++r) {
            for (int64_t i = 0; i < k; ++i) {
                float p = (float)oracle_e4m3_decode(w[r * k + i]) *
                          grid[(r / 128) * sk + i / 128];
                v[i] = oracle_bf16_to_float(oracle_bf16_from_double((double)p));
            }
            rowwise_fp8_row(v, k, q + r * k, scale + r);
        }
        free(v);
    }
}

/* ------------------------------------------------------------------ */
/* Contractions (outputs rounded to BF16 once, from binary64)          */
/* ------------------------------------------------------------------ */

/* gemm_dense_int8.rs, int8_gemm_faith2: exact int32 partial sum of every
 * 32-element K block, P[m][n][b] = sum_{k in b} a[m,k] * w[n,k]. */
void oracle_int8_block_partials(const int8_t *a, const int8_t *w, int32_t *p,
                                int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t b = 0; b < nb; ++b) {
                int64_t acc = 0;
                for (int64_t t = b * 32; t < b * 32 + 32; ++t)
                    acc += (int64_t)a[i * k + t] * (int64_t)w[j * k + t];
                p[(i * n + j) * nb + b] = (int32_t)acc;
            }
}

/* C[m,n] = bf16( sum_b a_scale[m,b] * w_scale[n,b] * P_b[m,n] ). */
void oracle_int8_gemm_blockscaled(const int8_t *a, const int8_t *w,
                                  const float *as, const float *ws,
                                  uint16_t *out, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double c = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int64_t pb = 0;
                for (int64_t t = b * 32; t < b * 32 + 32; ++t)
                    pb += (int64_t)a[i * k + t] * (int64_t)w[j * k + t];
                c += (double)pb * ((double)as[i * nb + b] * (double)ws[j * nb + b]);
            }
            out[i * n + j] = oracle_bf16_from_double(c);
        }
}

/* gemm_fp4.rs, w4a4_gemm: NVFP4 x NVFP4 with 16-element blocks,
 * C = bf16(scaleA2 * scaleW2 * sum_b e4m3(sa[m,b]) * e4m3(sw[n,b]) * P_b),
 * P_b = sum_{k in b} e2m1(a[m,k]) * e2m1(w[n,k]) (exact). */
void oracle_w4a4_gemm(const uint8_t *ap, const uint8_t *asc,
                      const uint8_t *wp, const uint8_t *wsc, uint16_t *out,
                      float scale_a2, float scale_w2,
                      int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / 16;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double c = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                double pb = 0.0;
                for (int64_t t = b * 16; t < b * 16 + 16; ++t) {
                    uint8_t ab = ap[i * (k / 2) + t / 2], wb = wp[j * (k / 2) + t / 2];
                    uint8_t ac = (t % 2 == 0) ? (ab & 15) : (ab >> 4);
                    uint8_t wc = (t % 2 == 0) ? (wb & 15) : (wb >> 4);
                    pb += oracle_e2m1_decode(ac) * oracle_e2m1_decode(wc);
                }
                c += oracle_e4m3_decode(asc[i * nb + b]) *
                     oracle_e4m3_decode(wsc[j * nb + b]) * pb;
            }
            out[i * n + j] = oracle_bf16_from_double((double)scale_a2 * (double)scale_w2 * c);
        }
}

/* fp8_gemv_batch.rs, fp8_gemv_rowscale_batch{8,16}_rt2: BF16 x [m,k] times
 * an E4M3 weight [n,k] with a per-row F32 scale applied at write-out,
 * C[m,n] = bf16(s[n] * sum_k x[m,k] * e4m3(w[n,k])). */
void oracle_fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                              const float *rs, uint16_t *out,
                              int64_t m, int64_t n, int64_t k)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < m; ++i) {
            double c = 0.0;
            for (int64_t t = 0; t < k; ++t)
                c += (double)oracle_bf16_to_float(x[i * k + t]) *
                     oracle_e4m3_decode(w[j * k + t]);
            out[i * n + j] = oracle_bf16_from_double((double)rs[j] * c);
        }
}

/* fp8_gemv_batch.rs, w8a16_gemv / w8a16_gemv_batch2 / w8a16_gemv_batch4: BF16
 * x [m,k] times a block-scaled E4M3 weight [n,k] whose F32 scale grid s
 * [n/128, k/128] holds one scale per 128 x 128 block:
 *   C[i,j] = bf16( sum_t x[i,t] * e4m3(w[j,t]) * s[j/128, t/128] ).
 * Each product is exact in binary64 (8 + 4 + 24 significant bits), so only
 * the sum and the final BF16 rounding round. */
void oracle_fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                                const float *s, uint16_t *out,
                                int64_t m, int64_t n, int64_t k)
{
    const int64_t kb = k / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < m; ++i) {
            const float *srow = s + (j / 128) * kb;
            double c = 0.0;
            for (int64_t t = 0; t < k; ++t)
                c += (double)oracle_bf16_to_float(x[i * k + t]) *
                     oracle_e4m3_decode(w[j * k + t]) * (double)srow[t / 128];
            out[i * n + j] = oracle_bf16_from_double(c);
        }
}

/* fp8_gemv_batch.rs names w4a16_gemv_batch8_rt2 as the NVFP4-weight twin of
 * the row-scaled FP8 GEMV.  BF16 x [m,k] times an NVFP4 weight: E2M1 codes
 * packed [n,k/2] (element 2j in the low nibble of byte j), an E4M3 scale per
 * 16 elements [n,k/16] and the per-tensor F32 scale2 (value = e2m1 * e4m3 *
 * scale2, as for gemm_fp4.rs, quantize_bf16_to_nvfp4):
 *   C[i,j] = bf16( scale2 * sum_t x[i,t] * e2m1(w[j,t]) * e4m3(s[j,t/16]) ).
 * Each product is exact in binary64 (8 + 2 + 4 significant bits); the sum
 * and the final scale2 product are binary64, and BF16 rounding happens once. */
void oracle_w4a16_gemv(const uint16_t *x, const uint8_t *wp, const uint8_t *ws,
                       float scale2, uint16_t *out,
                       int64_t m, int64_t n, int64_t k)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < m; ++i) {
            double c = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                uint8_t b = wp[j * (k / 2) + t / 2];
                uint8_t code = (t % 2 == 0) ? (uint8_t)(b & 15) : (uint8_t)(b >> 4);
                c += (double)oracle_bf16_to_float(x[i * k + t]) *
                     oracle_e2m1_decode(code) *
                     oracle_e4m3_decode(ws[j * (k / 16) + t / 16]);
            }
            out[i * n + j] = oracle_bf16_from_double((double)scale2 * c);
        }
}

/* dispatch_proj_rowwise.rs, cublas_fp8_rowwise_proj (the row-wise FP8 GEMM
 * it ends in): C = bf16(sa[m] * sw[n] * sum_k e4m3(a[m,k]) * e4m3(w[n,k])). */
void oracle_fp8_gemm_rowscale(const uint8_t *a, const float *sa,
                              const uint8_t *w, const float *sw, uint16_t *out,
                              int64_t m, int64_t n, int64_t k)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double c = 0.0;
            for (int64_t t = 0; t < k; ++t)
                c += oracle_e4m3_decode(a[i * k + t]) * oracle_e4m3_decode(w[j * k + t]);
            out[i * n + j] = oracle_bf16_from_double((double)sa[i] * (double)sw[j] * c);
        }
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int oracle_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
    return t;
}
