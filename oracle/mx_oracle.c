/*
 * mx_oracle.c -- plain, slow, obviously-correct CPU oracle for the NT MX
 * block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, loads or calls it, and the two share no code, tables or headers.
 *
 * What it computes (the plain definition, written out):
 *
 *   C[m,n] = sum_{kb=0}^{K/32-1}  2^(sa[m,kb]-127) * 2^(sb[n,kb]-127)
 *                                 * sum_{j=0}^{31} dec(A[m,32kb+j]) * dec(B[n,32kb+j])
 *
 * Sources on the pages:
 *  - "PyTorch 接上 FlyDSL" (5ulink.com), section "支持边界" (support matrix),
 *    row "MXFP 缩放 GEMM": F.scaled_mm over MXFP8 / MXFP4 inputs, A row-major,
 *    B column-major (NT), K a multiple of 128.
 *  - same page, paragraph under the support matrix: one E8M0 scale per 32
 *    values (BlockWise1x32), FP32 accumulation, FP16/BF16 output.
 * The element encodings (E2M1 for MXFP4, E4M3 "FN" for MXFP8, E8M0 for the
 * scale) are not spelled out on the pages; they follow the public OCP
 * Microscaling Formats (MX) v1.0 specification.
 *
 * Everything is computed in double.  A block sum of 32 element products is
 * exact in double (E4M3 products have at most 8 significant bits and lie in
 * [2^-18, 2^18), so 32 of them fit in 42 bits), and a scale factor is an
 * exact power of two, so the only rounding is in the sum over blocks.
 *
 * Layouts (the ABI reading of "A row-major, B column-major"):
 *   A: FP8 [M][K] bytes; FP4 [M][K/2] bytes, element k in byte k/2,
 *      low nibble when k is even, high nibble when k is odd.
 *   B: the same with N rows (B is K x N column-major, i.e. [N][K]).
 *   sa: [M][K/32] E8M0 bytes; sb: [N][K/32] E8M0 bytes, row-major.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define MXO_FMT_FP8 0
#define MXO_FMT_FP4 1

static double tab_e2m1[16];
static double tab_e4m3[256];
static double tab_e8m0[256];
static int tables_ready = 0;

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa.  Exponent field 0 is subnormal: value = m * 2^-1.  Otherwise
 * value = (1 + m/2) * 2^(e-1).  No Inf, no NaN. */
static double e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3 "FN" (OCP MX v1.0 FP8 E4M3): bit 7 sign, bits 6..3 exponent (bias 7),
 * bits 2..0 mantissa.  Exponent 0 is subnormal: (m/8) * 2^-6.  Otherwise
 * (1 + m/8) * 2^(e-7).  S.1111.111 is NaN; there is no infinity, so the
 * largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX v1.0 shared scale): unsigned 8-bit exponent, bias 127,
 * value 2^(e-127); 0xFF is NaN; there is no zero and no sign. */
static double e8m0_value(int code)
{
    if (code == 255)
        return NAN;
    return ldexp(1.0, code - 127);
}

static void build_tables(void)
{
    if (tables_ready)
        return;
    for (int c = 0; c < 16; ++c)
        tab_e2m1[c] = e2m1_value(c);
    for (int c = 0; c < 256; ++c) {
        tab_e4m3[c] = e4m3_value(c);
        tab_e8m0[c] = e8m0_value(c);
    }
    tables_ready = 1;
}

/* Element k of packed row r (row length K elements). */
static double element(int fmt, const uint8_t *base, int64_t r, int64_t K, int64_t k)
{
    if (fmt == MXO_FMT_FP8)
        return tab_e4m3[base[r * K + k]];
    uint8_t byte = base[r * (K / 2) + k / 2];
    int code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return tab_e2m1[code];
}

/* Decode a packed operand into doubles: out[r*K + k] = dec(element k of row r).
 * Exposed so the tests can pin the tables against independent decoders. */
int mx_oracle_decode(int fmt, const uint8_t *packed, int64_t rows, int64_t K, double *out)
{
    if ((fmt != MXO_FMT_FP8 && fmt != MXO_FMT_FP4) || rows < 0 || K < 0)
        return -1;
    build_tables();
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = element(fmt, packed, r, K, k);
    return 0;
}

/* Decode E8M0 bytes to doubles. */
int mx_oracle_decode_scale(const uint8_t *codes, int64_t n, double *out)
{
    build_tables();
    for (int64_t i = 0; i < n; ++i)
        out[i] = tab_e8m0[codes[i]];
    return 0;
}

/* One output element: the exact-block, double-accumulated definition.
 * Also returns S = sum_k |a_k b_k| including the scales. */
static void one_element(int fmt, const uint8_t *a, const uint8_t *b,
                        const uint8_t *sa, const uint8_t *sb,
                        int64_t K, int64_t m, int64_t n, double *c, double *s)
{
    int64_t nblk = K / 32;
    double acc = 0.0, absacc = 0.0;
    for (int64_t kb = 0; kb < nblk; ++kb) {
        double blk = 0.0, absblk = 0.0;
        for (int64_t j = 0; j < 32; ++j) {
            int64_t k = 32 * kb + j;
            double p = element(fmt, a, m, K, k) * element(fmt, b, n, K, k);
            blk += p;
            absblk += fabs(p);
        }
        double f = tab_e8m0[sa[m * nblk + kb]] * tab_e8m0[sb[n * nblk + kb]];
        acc += f * blk;
        absacc += f * absblk;
    }
    *c = acc;
    *s = absacc;
}

static int check_args(int fmt, int64_t M, int64_t N, int64_t K)
{
    if (fmt != MXO_FMT_FP8 && fmt != MXO_FMT_FP4)
        return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0)
        return -2;
    return 0;
}

/* Full GEMM: c[m*N+n] and s[m*N+n] for every output element.
 * s may be NULL.  Threads split the (m, n) pairs; every element keeps the
 * same block order, so the result does not depend on the thread count. */
int mx_oracle_gemm(int fmt, const uint8_t *a, const uint8_t *b,
                   const uint8_t *sa, const uint8_t *sb,
                   int64_t M, int64_t N, int64_t K, double *c, double *s)
{
    int rc = check_args(fmt, M, N, K);
    if (rc)
        return rc;
    build_tables();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double cv, sv;
            one_element(fmt, a, b, sa, sb, K, m, n, &cv, &sv);
            c[m * N + n] = cv;
            if (s)
                s[m * N + n] = sv;
        }
    return 0;
}

/* Selected elements only: (ms[i], ns[i]) for i < count. */
int mx_oracle_gemm_at(int fmt, const uint8_t *a, const uint8_t *b,
                      const uint8_t *sa, const uint8_t *sb,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t *ms, const int64_t *ns, int64_t count,
                      double *c, double *s)
{
    int rc = check_args(fmt, M, N, K);
    if (rc)
        return rc;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -3;
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double cv, sv;
        one_element(fmt, a, b, sa, sb, K, ms[i], ns[i], &cv, &sv);
        c[i] = cv;
        if (s)
            s[i] = sv;
    }
    return 0;
}

/* Round a double directly to a 16-bit float with round-to-nearest-even, so
 * there is no intermediate rounding to float.  `mbits` is the number of
 * stored mantissa bits, `emin` the exponent of the smallest normal, `emax`
 * the exponent of the largest finite binade, `ebias` the exponent bias.
 * Results below the smallest normal are rounded on the subnormal grid;
 * results that round to 2^(emax+1) or beyond become infinity; NaN becomes
 * the canonical quiet NaN (sign clear). */
static uint16_t round_to_half_format(double x, int mbits, int emin, int emax, int ebias,
                                     uint16_t qnan)
{
    if (isnan(x))
        return qnan;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    uint16_t inf = (uint16_t)(((2 * ebias + 1) << mbits) & 0x7FFF);
    if (isinf(ax))
        return sign | inf;
    if (ax == 0.0)
        return sign;
    int e2;
    frexp(ax, &e2);            /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;            /* floor(log2(ax)) */
    if (e < emin)
        e = emin;              /* subnormal grid has the quantum of the smallest binade */
    double quantum = ldexp(1.0, e - mbits);
    double q = nearbyint(ax / quantum);   /* exact division; default mode = nearest-even */
    double r = q * quantum;
    if (r >= ldexp(1.0, emax + 1))
        return sign | inf;
    /* r is exactly representable: encode it. */
    if (r < ldexp(1.0, emin)) {
        uint16_t mant = (uint16_t)(r / ldexp(1.0, emin - mbits));
        return sign | mant;
    }
    frexp(r, &e2);
    e = e2 - 1;
    uint16_t mant = (uint16_t)(r / ldexp(1.0, e - mbits) - ldexp(1.0, mbits));
    uint16_t expf = (uint16_t)(e + ebias);
    return sign | (uint16_t)(expf << mbits) | mant;
}

/* BF16: 8 exponent bits (bias 127), 7 mantissa bits. */
int mx_oracle_round_bf16(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_to_half_format(x[i], 7, -126, 127, 127, 0x7FC0u);
    return 0;
}

/* FP16: 5 exponent bits (bias 15), 10 mantissa bits. */
int mx_oracle_round_f16(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_to_half_format(x[i], 10, -14, 15, 15, 0x7E00u);
    return 0;
}

/* ------------------------------------------------------------------------
 * MX quantization: BF16 rows -> element codes + one E8M0 scale per 32
 * consecutive K values (the step before the GEMM; "PyTorch 接上 FlyDSL",
 * 5ulink.com, paragraph under the support matrix: BlockWise1x32 E8M0
 * scales).  The conversion rule is not spelled out on the pages; this
 * follows the OCP MX v1.0 conversion (shared exponent from the block's
 * largest magnitude, elements rounded to nearest even and saturated):
 *
 *   1. decode the 32 BF16 values of the block to double;
 *   2. a block holding a NaN or an infinity gets scale code 0xFF (NaN) and
 *      element codes 0;
 *   3. amax = max |x|; scale code s = floor(log2 amax) - emax + 127 clamped
 *      to [0, 254], emax = 2 (E2M1) or 8 (E4M3); an all-zero block gets 0;
 *   4. each element: v = |x| / 2^(s-127), replaced by the representable
 *      magnitude nearest to v (searched over every non-NaN code), ties to
 *      the code with an even last bit (= even mantissa); magnitudes beyond
 *      the largest code take the largest code (saturation); the sign bit is
 *      the sign bit of x;
 *   5. FP4 codes are packed two per byte, even k in the low nibble.
 * ------------------------------------------------------------------------ */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* nearest non-negative code to v >= 0; ties to the even code */
static int nearest_code(int fmt, double v)
{
    int best = 0, ncodes = (fmt == MXO_FMT_FP4) ? 8 : 128;
    double bestd = INFINITY;
    for (int c = 0; c < ncodes; ++c) {
        double q = (fmt == MXO_FMT_FP4) ? tab_e2m1[c] : tab_e4m3[c];
        if (isnan(q))
            continue;
        double d = fabs(v - q);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

int mx_oracle_quantize(int fmt, const uint16_t *x, int64_t rows, int64_t K,
                       uint8_t *codes, uint8_t *scales)
{
    if ((fmt != MXO_FMT_FP4 && fmt != MXO_FMT_FP8) || rows < 0 || K <= 0 || K % 32)
        return -1;
    build_tables();
    const int emax = (fmt == MXO_FMT_FP4) ? 2 : 8;
    const int sbit = (fmt == MXO_FMT_FP4) ? 8 : 128;
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *xb = x + r * K + 32 * b;
            double val[32];
            int special = 0;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                val[j] = bf16_value(xb[j]);
                if (isnan(val[j]) || isinf(val[j]))
                    special = 1;
                else if (fabs(val[j]) > amax)
                    amax = fabs(val[j]);
            }
            int s, q[32];
            if (special) {
                s = 255;
                for (int j = 0; j < 32; ++j)
                    q[j] = 0;
            } else {
                if (amax == 0.0) {
                    s = 0;
                } else {
                    int ex;
                    frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1) */
                    s = (ex - 1) - emax + 127;
                    if (s < 0) s = 0;
                    if (s > 254) s = 254;
                }
                for (int j = 0; j < 32; ++j) {
                    double v = ldexp(fabs(val[j]), 127 - s);
                    q[j] = nearest_code(fmt, v) | (signbit(val[j]) ? sbit : 0);
                }
            }
            scales[r * nb + b] = (uint8_t)s;
            if (fmt == MXO_FMT_FP4) {
                uint8_t *cb = codes + r * (K / 2) + 16 * b;
                for (int j = 0; j < 16; ++j)
                    cb[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
            } else {
                uint8_t *cb = codes + r * K + 32 * b;
                for (int j = 0; j < 32; ++j)
                    cb[j] = (uint8_t)q[j];
            }
        }
    }
    return 0;
}

int mx_oracle_abi_version(void) { return 1; }
