/*
 * mxq_oracle.c -- plain CPU oracle for the MXFP8 and per-token NVFP4 quantizers.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is loaded by the test suite, by the
 * smoke check and by the benchmark's CPU-baseline leg, and by nothing else.  It
 * shares no source, header, table or helper with the GPU library; the GPU path
 * never calls it.
 *
 * What it computes (the precision contract of the page "Miles: end-to-end MXFP8
 * and per-token NVFP4 RL on Blackwell"):
 *
 *   MXFP8 (MXFP8 format paragraph): runs of 32 consecutive values share one
 *     power-of-two E8M0 scale; the scale is rounded up so that the largest
 *     magnitude of the run is not clipped; elements are E4M3 codes.  Both a
 *     rowwise 1x32 copy and a columnwise 32x1 copy are made, each from the
 *     full-precision input (MXFP8 recipe paragraph on backward activations).
 *   NVFP4 (NVFP4 format paragraph): E2M1 codes, one E4M3 scale per 16 values
 *     rounded to the nearest E4M3 value, and one FP32 scale over a larger scope.
 *     The scope is one token row for activations (per-token activation scale
 *     paragraph), the gate/up pair of one expert for SwiGLU weights (gate/up
 *     paragraph), or one tensor otherwise.
 *   Dequant (dequantized backward paragraph): BF16 values of the exact
 *     low-precision operands.
 *
 * Readings taken where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   - E4M3 is the variant without infinities: largest finite value 448, codes
 *     0x7F/0xFF are NaN and never produced.  E2M1 magnitudes are
 *     {0, .5, 1, 1.5, 2, 3, 4, 6}.  E8M0 byte b means 2^(b-127).
 *   - Every narrowing conversion picks the nearest value of the target format;
 *     an exact tie goes to the code whose last bit is 0; magnitudes beyond the
 *     largest finite value give that value; the code keeps the input's sign
 *     (so a negative value that rounds to zero gives a negative-zero code).
 *   - MXFP8 scale exponent: the smallest e >= -127 with amax <= 448 * 2^e.
 *   - NVFP4 FP32 scale s = fp32(amax_scope / 2688) (2688 = 6 * 448): one IEEE
 *     binary32 division.  s is the decode multiplier (page "Using Quantization
 *     in RL", the paragraph on scales: value = code * scale).
 *     Block scale b = nearest E4M3 value to amax_block / (6 s); element code
 *     = nearest E2M1 value to x / (dec(b) s).  Both are rounded once, from the
 *     exact quotient.  If dec(b) == 0 the block's codes are 0x0.
 *   - Dequant: the exact product of the stored values, rounded once to BF16
 *     (nearest, ties to even), saturating at the largest finite BF16.
 *
 * How it stays exact: no quotient is ever formed.  To find the value v of a
 * format nearest to a / D (a >= 0, D > 0), the oracle walks the sorted table of
 * the format's non-negative values and compares 2a with (v[k] + v[k+1]) * D.
 * Every such product is exact in binary64: v[k] + v[k+1] has at most 5
 * significant bits, D is a power of two, 6 * s (26 bits) or dec(b) * s (28
 * bits), so the product has at most 33 significant bits, far inside the 53 of
 * binary64 and far from its exponent limits.  Comparing exact numbers decides
 * "nearer", "farther" and "tie" exactly.
 *
 * Loops are plain; rows are spread over OpenMP threads, nothing else.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* BF16: sign | 8-bit exponent (bias 127) | 7-bit mantissa, with subnormals
 * (table of formats on the page "Training Quality").  Inf/NaN are outside the
 * contract; they decode to +-inf / NaN here. */
double oracle_bf16_value(uint16_t b)
{
    int sign = b >> 15;
    int E = (b >> 7) & 0xFF;
    int m = b & 0x7F;
    double mag;
    if (E == 0xFF)
        mag = (m == 0) ? INFINITY : NAN;
    else if (E == 0)
        mag = ldexp((double)m, -133);            /* m/128 * 2^-126 */
    else
        mag = ldexp((double)(128 + m), E - 134); /* (1 + m/128) * 2^(E-127) */
    return sign ? -mag : mag;
}

/* E4M3: sign | 4-bit exponent (bias 7) | 3-bit mantissa. */
double oracle_e4m3_value(uint8_t c)
{
    int sign = c >> 7;
    int E = (c >> 3) & 0xF;
    int m = c & 7;
    double mag;
    if (E == 0xF && m == 7)
        return NAN;                              /* 0x7F / 0xFF */
    if (E == 0)
        mag = ldexp((double)m, -9);              /* m/8 * 2^-6 */
    else
        mag = ldexp((double)(8 + m), E - 10);    /* (1 + m/8) * 2^(E-7) */
    return sign ? -mag : mag;
}

/* E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa, in the low nibble. */
double oracle_e2m1_value(uint8_t c)
{
    int sign = (c >> 3) & 1;
    int E = (c >> 1) & 3;
    int m = c & 1;
    double mag;
    if (E == 0)
        mag = 0.5 * m;
    else
        mag = ldexp((double)(2 + m), E - 2);     /* (1 + m/2) * 2^(E-1) */
    return sign ? -mag : mag;
}

/* E8M0: unsigned exponent, value 2^(b-127); 0xFF is NaN. */
double oracle_e8m0_value(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Non-negative values of E4M3 (codes 0x00..0x7E) and E2M1 (codes 0..7), in
 * code order, which is increasing value order. */
static double E4M3_TABLE[127];
static double E2M1_TABLE[8];

/* Filled once when the library is loaded, before any thread reads them. */
__attribute__((constructor)) static void make_tables(void)
{
    for (int c = 0; c < 127; c++)
        E4M3_TABLE[c] = oracle_e4m3_value((uint8_t)c);
    for (int c = 0; c < 8; c++)
        E2M1_TABLE[c] = oracle_e2m1_value((uint8_t)c);
}

/* Index k of the table value nearest to a / D (a >= 0, D > 0): ties go to the
 * even index, and anything beyond the last value gives the last index.  Exact:
 * see the header. */
static int nearest_index(const double *v, int n, double a, double D)
{
    int k = 0;
    while (k + 1 < n) {
        double twice_mid = (v[k] + v[k + 1]) * D;
        double twice_a = 2.0 * a;
        if (twice_a < twice_mid)
            break;                               /* v[k] is nearer */
        if (twice_a == twice_mid) {              /* exact tie */
            if (k % 2 == 1)
                k++;
            break;
        }
        k++;
    }
    return k;
}

/* E4M3 code of x / D, nearest-even, saturating, sign of x kept. */
uint8_t oracle_e4m3_nearest(double x, double D)
{
    int k = nearest_index(E4M3_TABLE, 127, fabs(x), D);
    return (uint8_t)(k | (signbit(x) ? 0x80 : 0));
}

/* E2M1 code of x / D, nearest-even, saturating, sign of x kept. */
uint8_t oracle_e2m1_nearest(double x, double D)
{
    int k = nearest_index(E2M1_TABLE, 8, fabs(x), D);
    return (uint8_t)(k | (signbit(x) ? 0x8 : 0));
}

/* MXFP8 scale byte for a block whose largest magnitude is A: the smallest
 * e in [-127, 127] with A <= 448 * 2^e, stored as e + 127. */
int oracle_e8m0_byte(double A)
{
    for (int e = -127; e <= 127; e++)
        if (A <= ldexp(448.0, e))
            return e + 127;
    return 254;
}

/* The OCP MX rule, a variant the library offers for comparison (it can
 * clip): the shared exponent is floor(log2 A) minus the largest exponent of
 * the element format (8 for E4M3, whose largest value is 1.75 * 2^8),
 * clamped to [-127, 127]; A = 0 gives -127.  Stored as e + 127. */
int oracle_e8m0_byte_ocp(double A)
{
    if (A == 0.0)
        return 0;
    int ex;
    frexp(A, &ex);                          /* A = f * 2^ex, f in [.5, 1) */
    int e = (ex - 1) - 8;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e + 127;
}

static int scale_byte(double A, int ocp)
{
    return ocp ? oracle_e8m0_byte_ocp(A) : oracle_e8m0_byte(A);
}

/* NVFP4 FP32 scale of a scope whose largest magnitude is A (A is a BF16 value,
 * hence exact in binary32): one IEEE binary32 division. */
float oracle_nvfp4_scale(double A)
{
    float a = (float)A;
    float divisor = 2688.0f;
    return a / divisor;
}

/* Nearest BF16 to an exact value y, ties to even, |y| >= max finite gives the
 * max finite, sign kept.  The nearest point of the grid of spacing
 * 2^(e-7) (e = exponent of |y|, at least -126) is found with nearbyint, which
 * rounds half to even; scaling by powers of two is exact. */
uint16_t oracle_bf16_round_sat(double y)
{
    if (isnan(y))
        return 0x7FC0;
    const double BF16_MAX = ldexp(255.0, 120);
    double a = fabs(y);
    uint16_t mag;
    if (a >= BF16_MAX) {
        mag = 0x7F7F;
    } else if (a == 0.0) {
        mag = 0;
    } else {
        int ex;
        frexp(a, &ex);                           /* a = f * 2^ex, f in [.5, 1) */
        int e = ex - 1;
        if (e < -126)
            e = -126;
        double n = nearbyint(ldexp(a, 7 - e));   /* a / 2^(e-7), exact scaling */
        double r = ldexp(n, e - 7);              /* a BF16 value, <= BF16_MAX */
        float rf = (float)r;                     /* exact: r is a BF16 value */
        uint32_t bits;
        memcpy(&bits, &rf, sizeof bits);
        mag = (uint16_t)(bits >> 16);
    }
    return (uint16_t)(mag | (signbit(y) ? 0x8000 : 0));
}

/* ------------------------------------------------------------------------ */
/* MXFP8                                                                     */
/* ------------------------------------------------------------------------ */

/* Rowwise copy: X[rows][cols], cols % 32 == 0.  codes[rows][cols],
 * scales[rows][cols/32]. */
void oracle_mxfp8_rowwise_rule(const uint16_t *x, int64_t rows, int64_t cols,
                               uint8_t *codes, uint8_t *scales, int ocp)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        for (int64_t j = 0; j < nb; j++) {
            double A = 0.0;
            for (int64_t k = 0; k < 32; k++) {
                double a = fabs(oracle_bf16_value(x[i * cols + j * 32 + k]));
                if (a > A)
                    A = a;
            }
            int byte = scale_byte(A, ocp);
            double D = ldexp(1.0, byte - 127);
            scales[i * nb + j] = (uint8_t)byte;
            for (int64_t k = 0; k < 32; k++) {
                int64_t idx = i * cols + j * 32 + k;
                codes[idx] = oracle_e4m3_nearest(oracle_bf16_value(x[idx]), D);
            }
        }
    }
}

void oracle_mxfp8_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                          uint8_t *codes, uint8_t *scales)
{
    oracle_mxfp8_rowwise_rule(x, rows, cols, codes, scales, 0);
}

/* Columnwise blocks over the rows [r0, r1) of X (r1 - r0 <= 32; a short block
 * takes its largest magnitude over the rows that exist).  Writes codes at the
 * same [row][col] index as X and one scale row scales_row[cols]. */
static void colwise_block_rows(const uint16_t *x, int64_t cols, int64_t r0,
                               int64_t r1, uint8_t *codes, uint8_t *scales_row, int ocp)
{
    for (int64_t j = 0; j < cols; j++) {
        double A = 0.0;
        for (int64_t r = r0; r < r1; r++) {
            double a = fabs(oracle_bf16_value(x[r * cols + j]));
            if (a > A)
                A = a;
        }
        int byte = scale_byte(A, ocp);
        double D = ldexp(1.0, byte - 127);
        scales_row[j] = (uint8_t)byte;
        for (int64_t r = r0; r < r1; r++)
            codes[r * cols + j] =
                oracle_e4m3_nearest(oracle_bf16_value(x[r * cols + j]), D);
    }
}

/* Columnwise copy: rows % 32 == 0.  codes[rows][cols], scales[rows/32][cols]. */
void oracle_mxfp8_colwise_rule(const uint16_t *x, int64_t rows, int64_t cols,
                               uint8_t *codes, uint8_t *scales, int ocp)
{
    int64_t nt = rows / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nt; t++)
        colwise_block_rows(x, cols, 32 * t, 32 * t + 32, codes, scales + t * cols, ocp);
}

void oracle_mxfp8_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                          uint8_t *codes, uint8_t *scales)
{
    oracle_mxfp8_colwise_rule(x, rows, cols, codes, scales, 0);
}

/* Columnwise copy over ragged segments: segment e is rows [off[e], off[e+1]).
 * Its blocks start at off[e]; its last block covers the rows that remain.
 * Segment e's scale rows start at P[e] = sum over f < e of ceil(n_f / 32);
 * P is written to scale_offsets[0..n_groups]. */
void oracle_mxfp8_colwise_grouped(const uint16_t *x, int64_t cols,
                                  const int64_t *off, int64_t n_groups,
                                  uint8_t *codes, uint8_t *scales,
                                  int64_t *scale_offsets)
{
    int64_t p = 0;
    for (int64_t e = 0; e < n_groups; e++) {
        scale_offsets[e] = p;
        p += (off[e + 1] - off[e] + 31) / 32;
    }
    scale_offsets[n_groups] = p;
    for (int64_t e = 0; e < n_groups; e++) {
        int64_t n = off[e + 1] - off[e];
        int64_t nt = (n + 31) / 32;
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < nt; t++) {
            int64_t r0 = off[e] + 32 * t;
            int64_t r1 = r0 + 32 < off[e + 1] ? r0 + 32 : off[e + 1];
            colwise_block_rows(x, cols, r0, r1, codes,
                               scales + (scale_offsets[e] + t) * cols, 0);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* NVFP4                                                                     */
/* ------------------------------------------------------------------------ */

/* One row of cols values (cols % 16 == 0) under the FP32 scale s:
 * codes[cols/2] (even element in the low nibble), block_scales[cols/16]. */
static void nvfp4_row(const uint16_t *x, int64_t cols, float s, uint8_t *codes,
                      uint8_t *block_scales)
{
    double sd = (double)s;
    for (int64_t j = 0; j < cols / 16; j++) {
        double A = 0.0;
        for (int64_t k = 0; k < 16; k++) {
            double a = fabs(oracle_bf16_value(x[j * 16 + k]));
            if (a > A)
                A = a;
        }
        uint8_t b = 0;
        if (sd > 0.0)
            b = oracle_e4m3_nearest(A, 6.0 * sd);  /* A >= 0: positive code */
        block_scales[j] = b;
        double d = oracle_e4m3_value(b);
        for (int64_t k = 0; k < 16; k += 2) {
            uint8_t c[2];
            for (int h = 0; h < 2; h++) {
                double v = oracle_bf16_value(x[j * 16 + k + h]);
                c[h] = (d > 0.0) ? oracle_e2m1_nearest(v, d * sd) : 0;
            }
            codes[(j * 16 + k) / 2] = (uint8_t)(c[0] | (c[1] << 4));
        }
    }
}

static double row_amax(const uint16_t *x, int64_t n)
{
    double A = 0.0;
    for (int64_t k = 0; k < n; k++) {
        double a = fabs(oracle_bf16_value(x[k]));
        if (a > A)
            A = a;
    }
    return A;
}

/* Per-token NVFP4: each row is its own scope.  codes[rows][cols/2],
 * block_scales[rows][cols/16], token_scales[rows]. */
void oracle_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols,
                            uint8_t *codes, uint8_t *block_scales,
                            float *token_scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < rows; t++) {
        float s = oracle_nvfp4_scale(row_amax(x + t * cols, cols));
        token_scales[t] = s;
        nvfp4_row(x + t * cols, cols, s, codes + t * (cols / 2),
                  block_scales + t * (cols / 16));
    }
}

/* NVFP4 of a whole tensor X[rows][cols] under a given FP32 scale s. */
void oracle_nvfp4_with_scale(const uint16_t *x, int64_t rows, int64_t cols,
                             float s, uint8_t *codes, uint8_t *block_scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < rows; t++)
        nvfp4_row(x + t * cols, cols, s, codes + t * (cols / 2),
                  block_scales + t * (cols / 16));
}

/* Weight export: for each expert e, one FP32 scale over gate[e] and up[e]
 * together (or over gate[e] alone when up is NULL), then both tensors are
 * quantized under it.  gate, up: [n_experts][rows][cols]. */
void oracle_nvfp4_gateup_pair(const uint16_t *gate, const uint16_t *up,
                              int64_t n_experts, int64_t rows, int64_t cols,
                              uint8_t *gate_codes, uint8_t *gate_block_scales,
                              uint8_t *up_codes, uint8_t *up_block_scales,
                              float *scope_scales)
{
    int64_t n = rows * cols;
    for (int64_t e = 0; e < n_experts; e++) {
        double A = row_amax(gate + e * n, n);
        if (up) {
            double Au = row_amax(up + e * n, n);
            if (Au > A)
                A = Au;
        }
        float s = oracle_nvfp4_scale(A);
        scope_scales[e] = s;
        oracle_nvfp4_with_scale(gate + e * n, rows, cols, s, gate_codes + e * n / 2,
                                gate_block_scales + e * n / 16);
        if (up)
            oracle_nvfp4_with_scale(up + e * n, rows, cols, s, up_codes + e * n / 2,
                                    up_block_scales + e * n / 16);
    }
}

/* ------------------------------------------------------------------------ */
/* Dequant                                                                   */
/* ------------------------------------------------------------------------ */

/* MXFP8 rowwise copy -> BF16: y = RN_bf16(dec(c) * 2^(b-127)). */
void oracle_dequant_mxfp8_rowwise(const uint8_t *codes, const uint8_t *scales,
                                  int64_t rows, int64_t cols, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++)
        for (int64_t k = 0; k < cols; k++) {
            double y = oracle_e4m3_value(codes[i * cols + k]) *
                       oracle_e8m0_value(scales[i * (cols / 32) + k / 32]);
            out[i * cols + k] = oracle_bf16_round_sat(y);
        }
}

/* MXFP8 columnwise copy -> BF16 (rows % 32 == 0). */
void oracle_dequant_mxfp8_colwise(const uint8_t *codes, const uint8_t *scales,
                                  int64_t rows, int64_t cols, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++)
        for (int64_t k = 0; k < cols; k++) {
            double y = oracle_e4m3_value(codes[i * cols + k]) *
                       oracle_e8m0_value(scales[(i / 32) * cols + k]);
            out[i * cols + k] = oracle_bf16_round_sat(y);
        }
}

/* NVFP4 -> BF16: y = RN_bf16(dec(c) * dec(b) * s), with s = fp32_scales[i /
 * rows_per_scale] for row i (1 = per token, rows = one scale per tensor). */
void oracle_dequant_nvfp4(const uint8_t *codes, const uint8_t *block_scales,
                          const float *fp32_scales, int64_t rows_per_scale,
                          int64_t rows, int64_t cols, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        double s = (double)fp32_scales[i / rows_per_scale];
        for (int64_t k = 0; k < cols; k++) {
            uint8_t byte = codes[i * (cols / 2) + k / 2];
            uint8_t c = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double y = oracle_e2m1_value(c) *
                       oracle_e4m3_value(block_scales[i * (cols / 16) + k / 16]) * s;
            out[i * cols + k] = oracle_bf16_round_sat(y);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Element-wise entry points for the exhaustive checks                       */
/* ------------------------------------------------------------------------ */

void oracle_e4m3_nearest_many(const double *x, const double *D, int64_t n,
                              uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_nearest(x[i], D[i]);
}

void oracle_e2m1_nearest_many(const double *x, const double *D, int64_t n,
                              uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e2m1_nearest(x[i], D[i]);
}

void oracle_e8m0_byte_many(const double *A, int64_t n, int32_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e8m0_byte(A[i]);
}

void oracle_nvfp4_scale_many(const double *A, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_nvfp4_scale(A[i]);
}

void oracle_bf16_round_sat_many(const double *y, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_round_sat(y[i]);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
