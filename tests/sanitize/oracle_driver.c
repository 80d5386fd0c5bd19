/* Drives the CPU oracle (oracle/mx_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point on small seeded inputs,
 * ragged shapes, every code of every format, special values and the
 * argument checks.  Built and run by tests/test_sanitize_host.py; exits
 * non-zero (or the sanitizers abort) on any finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mx_oracle_decode(int fmt, const uint8_t *packed, int64_t rows, int64_t K, double *out);
int mx_oracle_decode_scale(const uint8_t *codes, int64_t n, double *out);
int mx_oracle_gemm(int fmt, const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb,
                   int64_t M, int64_t N, int64_t K, double *c, double *s);
int mx_oracle_gemm_at(int fmt, const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb,
                      int64_t M, int64_t N, int64_t K, const int64_t *ms, const int64_t *ns, int64_t n,
                      double *c, double *s);
int mx_oracle_round_bf16(const double *x, int64_t n, uint16_t *out);
int mx_oracle_round_f16(const double *x, int64_t n, uint16_t *out);
int mx_oracle_quantize(int fmt, const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales);

static uint64_t state = 88172645463325252ull;
static uint32_t rnd(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)state;
}

#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                  \
        }                                                              \
    } while (0)

static int gemm_case(int fmt, int64_t M, int64_t N, int64_t K)
{
    const int64_t rb = fmt ? K / 2 : K;
    /* exact-size heap buffers, so any overrun is caught */
    uint8_t *a = malloc((size_t)(M * rb)), *b = malloc((size_t)(N * rb));
    uint8_t *sa = malloc((size_t)(M * K / 32)), *sb = malloc((size_t)(N * K / 32));
    double *c = malloc(sizeof(double) * (size_t)(M * N)), *s = malloc(sizeof(double) * (size_t)(M * N));
    for (int64_t i = 0; i < M * rb; ++i) a[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < N * rb; ++i) b[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < M * K / 32; ++i) sa[i] = (uint8_t)(rnd() % 256);   /* includes 0xFF (NaN) */
    for (int64_t i = 0; i < N * K / 32; ++i) sb[i] = (uint8_t)(rnd() % 256);
    CHECK(mx_oracle_gemm(fmt, a, b, sa, sb, M, N, K, c, s) == 0);
    int64_t ms[5] = {0, M - 1, 0, M - 1, M / 2}, ns[5] = {0, 0, N - 1, N - 1, N / 2};
    double c2[5], s2[5];
    CHECK(mx_oracle_gemm_at(fmt, a, b, sa, sb, M, N, K, ms, ns, 5, c2, s2) == 0);
    for (int i = 0; i < 5; ++i) {
        const double v = c[ms[i] * N + ns[i]];
        CHECK((isnan(v) && isnan(c2[i])) || v == c2[i]);
    }
    uint16_t *r = malloc(sizeof(uint16_t) * (size_t)(M * N));
    CHECK(mx_oracle_round_bf16(c, M * N, r) == 0);
    CHECK(mx_oracle_round_f16(c, M * N, r) == 0);
    double *d = malloc(sizeof(double) * (size_t)(M * K));
    CHECK(mx_oracle_decode(fmt, a, M, K, d) == 0);
    free(a); free(b); free(sa); free(sb); free(c); free(s); free(r); free(d);
    return 0;
}

int main(void)
{
    /* every E8M0 code and every element code, by decode */
    uint8_t codes[256];
    double vals[512];
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    CHECK(mx_oracle_decode_scale(codes, 256, vals) == 0);
    CHECK(mx_oracle_decode(0, codes, 1, 256, vals) == 0);
    CHECK(mx_oracle_decode(1, codes, 1, 512, vals) == 0);
    /* GEMMs of both formats on ragged shapes (one row, one column, K = 128 .. 640) */
    const int64_t shapes[][3] = {{1, 1, 128}, {3, 5, 256}, {17, 9, 384}, {2, 33, 640}};
    for (int f = 0; f < 2; ++f)
        for (int i = 0; i < 4; ++i)
            if (gemm_case(f, shapes[i][0], shapes[i][1], shapes[i][2]))
                return 1;
    /* rounding of special values */
    const double sp[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e300, -1e-300, 65519.0, 65520.0, 3.4e38, 1e-45};
    uint16_t out[11];
    CHECK(mx_oracle_round_bf16(sp, 11, out) == 0);
    CHECK(mx_oracle_round_f16(sp, 11, out) == 0);
    /* quantizer over every BF16 bit pattern (as rows of 32), both formats */
    const int64_t rows = 65536 / 32;
    uint16_t *x = malloc(sizeof(uint16_t) * 65536);
    for (int i = 0; i < 65536; ++i) x[i] = (uint16_t)i;
    uint8_t *qc = malloc(65536), *qs = malloc((size_t)rows);
    CHECK(mx_oracle_quantize(0, x, rows, 32, qc, qs) == 0);
    CHECK(mx_oracle_quantize(1, x, rows, 32, qc, qs) == 0);
    /* argument checks */
    CHECK(mx_oracle_gemm(0, codes, codes, codes, codes, 1, 1, 100, vals, vals) != 0);
    CHECK(mx_oracle_gemm(2, codes, codes, codes, codes, 1, 1, 128, vals, vals) != 0);
    CHECK(mx_oracle_quantize(0, x, 1, 33, qc, qs) != 0);
    free(x); free(qc); free(qs);
    puts("oracle sanitizer run ok");
    return 0;
}
