/*
 * mxq.h -- C ABI of libmxq: bit-exact MXFP8 and per-token NVFP4 quantizers
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are the precision contract that training forward and
 * rollout share, as described on the page "Miles: end-to-end MXFP8 and
 * per-token NVFP4 RL on Blackwell" (aioga.com news page, English text):
 * its MXFP8 format and MXFP8 recipe paragraphs, its NVFP4 format paragraph,
 * its per-token activation scale paragraphs, its gate/up pairing paragraph
 * and its dequantized-backward paragraph.  Each entry point below names the
 * passage it implements.
 *
 * ---------------------------------------------------------------------------
 * Formats (readings where the pages only name the format):
 *   BF16   input/output, passed as uint16_t bit patterns.
 *   E4M3   1-4-3 float without infinities: largest finite 448 (0x7E), NaN
 *          0x7F/0xFF (never produced), subnormals down to 2^-9.
 *   E8M0   unsigned byte b meaning 2^(b-127); 0xFF (NaN) is never produced.
 *   E2M1   1-2-1 float in a nibble: magnitudes {0,.5,1,1.5,2,3,4,6}, bit 3 is
 *          the sign.  Two per byte, the even element in the low nibble.
 *   FP32   IEEE binary32.
 *
 * Arithmetic (the same for every entry point):
 *   - Every narrowing conversion rounds to the nearest value of the target
 *     format, an exact tie going to the even code; magnitudes at or above the
 *     largest finite value give that value; the sign is kept (a negative input
 *     that rounds to zero gives a negative-zero code).  Every result is
 *     rounded once, from the exact value.
 *   - MXFP8: per block of 32 values, e = the smallest integer >= -127 with
 *     amax <= 448 * 2^e (so the block maximum is never clipped); scale byte
 *     e + 127; code = E4M3(x / 2^e).  An all-zero block gets byte 0x00.
 *   - NVFP4: s = fp32(amax_scope / 2688) (one IEEE binary32 division; 2688 =
 *     6 * 448); s is the decode multiplier.  Per block of 16 values: block
 *     scale b = E4M3(amax_block / (6 s)); element code c = E2M1(x / (dec(b) s)).
 *     If dec(b) == 0 (which includes s == 0) the block's codes are 0x0.
 *   - Dequant: BF16(dec(code) * dec(scale) [* s]) rounded once from the exact
 *     product, ties to even, saturating at the largest finite BF16 (0x7F7F).
 *   - NaN and Inf inputs are outside the contract.
 *
 * Layouts: plain row-major, no padding, no swizzle.  X is [rows][cols] with
 * cols the contiguous (contraction) dimension.
 *
 * Conventions for every entry point:
 *   - Every array is device memory of the current HIP device, allocated and
 *     owned by the caller.  The library allocates no device memory and keeps
 *     no state between calls beyond a per-process cache of each kernel's
 *     occupancy.  Inputs are never modified.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue their kernels and return; results are valid once the
 *     stream has been synchronized.  Calls on one stream are ordered.
 *   - A return value other than MXQ_OK means nothing was launched and nothing
 *     was written.  All validation happens on the host before any launch:
 *     null pointers, sizes, divisibility, 16-byte alignment of every array
 *     that the kernels access with vector loads or stores, pointers that are
 *     not device memory of the current device, arrays whose extent runs past
 *     the end of their device allocation (the allocation the runtime knows:
 *     a tensor carved from a caching allocator's segment is checked against
 *     the segment), and overlapping ranges between any input and any output
 *     or between two outputs.  A failed launch returns MXQ_ERR_LAUNCH; faults
 *     on the device surface at synchronization.
 *   - Sizes are int64_t; element counts up to 2^62 are supported.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raised whenever an entry point is added or changes (2: the caller-amax
 * export variant, the copy floor, the grouped GEMMs, the grouped
 * weight-gradient pair and the grouped rowwise + transposed quantize). */
#define MXQ_VERSION 2

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_NULL = 1,      /* a required pointer is NULL                      */
    MXQ_ERR_SIZE = 2,      /* a size is <= 0 (or n_groups < 1), or beyond a   */
                           /* limit stated below                              */
    MXQ_ERR_SHAPE = 3,     /* cols (or rows) not divisible as required        */
    MXQ_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                */
    MXQ_ERR_ALIAS = 5,     /* an output overlaps an input or another output   */
    MXQ_ERR_OFFSETS = 6,   /* inconsistent optional-output combination        */
    MXQ_ERR_DEVICE = 7,    /* not device memory of the current device         */
    MXQ_ERR_LAUNCH = 8,    /* the kernel launch failed                        */
    MXQ_ERR_ARG = 9        /* an enum argument has an unknown value           */
} mxq_status;

/*
 * Size limits common to the entry points (MXQ_ERR_SIZE beyond them).  Each
 * launch is one grid of at most 2^32 - 1 work-items, so:
 *   - per-token NVFP4 calls take rows (tokens) below 2^26 (one 64-lane
 *     workgroup per row);
 *   - MXFP8 quantize calls take at most 2^26 - 9 tiles of 32 rows x 128
 *     columns: ceil(rows / 32) * ceil(cols / 128), where grouped and
 *     dispatch calls with a columnwise copy count total_rows / 32 + n_groups
 *     row tiles;
 *   - GEMMs take at most 2^24 - 9 output tiles: ceil(M/256) * ceil(N/256);
 *   - the weight export takes n_experts below 2^26 and at most 2^26 - 1
 *     amax chunks: ceil(elements per scope / 4096) * n_experts.
 * Dequant walks its grid in strides and has no grid limit of its own.
 */

typedef enum {
    MXQ_FMT_MXFP8_ROW = 1,     /* MXFP8 rowwise 1x32 copy                    */
    MXQ_FMT_MXFP8_COL = 2,     /* MXFP8 columnwise 32x1 copy                 */
    MXQ_FMT_MXFP8_ROWCOL = 3,  /* both MXFP8 copies from one read            */
    MXQ_FMT_NVFP4 = 4          /* NVFP4 with a per-token FP32 scale          */
} mxq_format;

typedef enum {
    MXQ_OUT_F32 = 0,           /* GEMM result as fp32                        */
    MXQ_OUT_BF16 = 1           /* GEMM result rounded to BF16, nearest-even  */
} mxq_out_dtype;

/*
 * MXFP8 quantize, rowwise and columnwise copies from one read of X.
 * Implements the MXFP8 format paragraph (32 E4M3 values per E8M0 scale, scale
 * rounded up so the block maximum is not clipped) and the MXFP8 recipe
 * paragraph (rowwise 1x32 and columnwise 32x1 copies, each quantized from the
 * full-precision data, both made during one quantization).
 *
 *   x          [rows][cols] BF16, 16-byte aligned.
 *   row_codes  [rows][cols] E4M3; row_codes[i][k] is x[i][k]'s code under the
 *              scale of its rowwise block k/32.
 *   row_scales [rows][cols/32] E8M0.
 *   col_codes  [rows][cols] E4M3, same index as x; col_codes[i][k] is
 *              x[i][k]'s code under the scale of its columnwise block i/32.
 *   col_scales [rows/32][cols] E8M0.
 *   Pass both row pointers NULL to skip the rowwise copy, both col pointers
 *   NULL to skip the columnwise copy (not both copies); one NULL of a pair is
 *   MXQ_ERR_OFFSETS.  Requires cols % 32 == 0, and rows % 32 == 0 when the
 *   columnwise copy is requested.  Code arrays must be 16-byte aligned.
 *   cols must not exceed 2^26, and the tile count is limited as stated above
 *   (MXQ_ERR_SIZE otherwise).
 */
int mxq_mxfp8_quantize_rowcol(const uint16_t *x, int64_t rows, int64_t cols,
                              uint8_t *row_codes, uint8_t *row_scales,
                              uint8_t *col_codes, uint8_t *col_scales,
                              void *stream);

/*
 * Comparison variant, not the contract: both MXFP8 copies under the OCP MX
 * scale rule, shared exponent floor(log2 amax) - 8 (E4M3's largest
 * exponent), elements the nearest E4M3 of x / 2^e saturated at 448.  Unlike
 * the contract's rounded-up scale (the MXFP8 format paragraph: the block
 * maximum is not clipped) this clips every block whose amax mantissa exceeds
 * 1.75; the call exists to measure that.  Arguments, layouts and errors as
 * mxq_mxfp8_quantize_rowcol.
 */
int mxq_mxfp8_quantize_ocp_floor(const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *row_codes, uint8_t *row_scales, uint8_t *col_codes,
                                 uint8_t *col_scales, void *stream);

/*
 * Layout variant: both MXFP8 copies from one read, the columnwise one stored
 * transposed, codes [cols][rows] and scales [cols][rows/32] (the same bytes as
 * mxq_mxfp8_quantize_rowcol's columnwise copy, permuted).  Each 32x1 block
 * then lies along a row, so a GEMM contracting over the rows (the weight
 * gradient of the MXFP8 recipe's backward) reads it K-contiguous, as
 * mxq_mxfp8_gemm requires.
 *   col_codes_t, col_scales_t required (16-byte aligned codes); row_codes and
 *   row_scales both or neither; rows % 32 == 0, cols % 32 == 0; MXFP8 tile
 *   limit as above.
 */
int mxq_mxfp8_quantize_rowcol_t(const uint16_t *x, int64_t rows, int64_t cols,
                                uint8_t *row_codes, uint8_t *row_scales, uint8_t *col_codes_t,
                                uint8_t *col_scales_t, void *stream);

/*
 * NVFP4 quantize with one online FP32 scale per token (row), in one call that
 * returns the packed codes, the E4M3 block scales and the per-token scales.
 * Implements the NVFP4 format paragraph (E2M1 codes, one E4M3 scale per 16
 * values rounded to the nearest E4M3 value, one FP32 scale over a larger
 * scope) and the per-token activation paragraphs (the scope is one token; the
 * scale is computed inside the quantization call, with no separate pass).
 *
 *   x            [rows][cols] BF16, 16-byte aligned; cols % 16 == 0.
 *   codes        [rows][cols/2] packed E2M1, 16-byte aligned.
 *   block_scales [rows][cols/16] E4M3.
 *   token_scales [rows] FP32: s_t = fp32(amax_t / 2688), the decode multiplier.
 *   rows must be below 2^26 (MXQ_ERR_SIZE otherwise).
 */
int mxq_nvfp4_quantize_per_token(const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *codes, uint8_t *block_scales,
                                 float *token_scales, void *stream);

/*
 * Opt-in approximate variant, not the contract (the exactness paragraph makes
 * approximation opt-in): per-token NVFP4 as mxq_nvfp4_quantize_per_token, but
 * the block scale and each code come from one conversion of a
 * reciprocal-multiply, with no exactness fix-up.  The FP32 token scale is
 * exact.  A block scale or code can differ from the exact one only where the
 * exact quotient lies within about 2^-21 (relative) of a rounding midpoint,
 * and then it is the other neighbour.  cols <= 4096 (MXQ_ERR_SIZE); other
 * arguments and errors as mxq_nvfp4_quantize_per_token.
 */
int mxq_nvfp4_quantize_per_token_approx(const uint16_t *x, int64_t rows, int64_t cols,
                                        uint8_t *codes, uint8_t *block_scales,
                                        float *token_scales, void *stream);

/*
 * NVFP4 weight export with one FP32 scale per scope.  Implements the gate/up
 * pairing paragraph: a SwiGLU expert's gate and up projections are quantized
 * together under one shared FP32 scale (the scope is gate[e] together with
 * up[e]); with up == NULL each gate[e] is its own scope (e.g. a down
 * projection).  Blocks of 16 run along each tensor's last dimension, the
 * contraction axis (the paragraph on one-dimensional blocks and contraction
 * axes).  The scope's amax is reduced over every element of the scope before
 * any code is produced.
 *
 *   gate, up             [n_experts][rows][cols] BF16, 16-byte aligned;
 *                        cols % 16 == 0.
 *   gate_codes, up_codes [n_experts][rows][cols/2], 16-byte aligned.
 *   gate_block_scales, up_block_scales  [n_experts][rows][cols/16].
 *   scope_scales         [n_experts] FP32: s_e = fp32(amax_e / 2688).
 *   gate_codes also serves the call as scratch for per-chunk partial maxima
 *   (written before, and overwritten by, the codes).
 *   up, up_codes and up_block_scales must be all NULL or all non-NULL.
 *   n_experts * rows * cols must be below 2^36, and the export limits above
 *   hold (MXQ_ERR_SIZE otherwise).
 */
int mxq_nvfp4_quantize_gateup_pair(const uint16_t *gate, const uint16_t *up,
                                   int64_t n_experts, int64_t rows, int64_t cols,
                                   uint8_t *gate_codes, uint8_t *gate_block_scales,
                                   uint8_t *up_codes, uint8_t *up_block_scales,
                                   float *scope_scales, void *stream);

/*
 * The weight export of mxq_nvfp4_quantize_gateup_pair with each scope's amax
 * supplied by the caller, which skips the export's first read of the weights
 * (the amax pass).  The gate/up pairing paragraph fixes the scope and its one
 * FP32 scale; whoever last wrote the weights (for instance the optimizer step)
 * can reduce the scope amax on the way and hand it over here.
 *
 *   scope_amax  [n_experts] BF16 bit patterns (device memory, 2-byte
 *               aligned): A_e, the largest magnitude in scope e (the sign bit
 *               is ignored).  s_e = fp32(A_e / 2688) is written to
 *               scope_scales and every tensor of the scope is quantized
 *               under it.
 *   Every other argument, layout, alignment and limit as
 *   mxq_nvfp4_quantize_gateup_pair.  With A_e the true amax of scope e the
 *   bytes equal that call's; with any other A_e they are the scope quantized
 *   under s_e (codes saturate where A_e is too small).
 */
int mxq_nvfp4_quantize_gateup_pair_amax(const uint16_t *gate, const uint16_t *up,
                                        const uint16_t *scope_amax, int64_t n_experts,
                                        int64_t rows, int64_t cols, uint8_t *gate_codes,
                                        uint8_t *gate_block_scales, uint8_t *up_codes,
                                        uint8_t *up_block_scales, float *scope_scales,
                                        void *stream);

/*
 * Dequantize to BF16: the exact low-precision operands made by the calls
 * above, decoded and rounded once to BF16.  Implements the dequantized-
 * backward paragraph (backward GEMMs consume BF16 dequantizations of the exact
 * forward operands).
 *
 *   fmt == MXQ_FMT_MXFP8_ROW: codes [rows][cols], scales [rows][cols/32];
 *          cols % 32 == 0.
 *   fmt == MXQ_FMT_MXFP8_COL: codes [rows][cols], scales [rows/32][cols];
 *          rows % 32 == 0, cols % 32 == 0.
 *   fmt == MXQ_FMT_NVFP4: codes [rows][cols/2], scales [rows][cols/16] (E4M3),
 *          fp32_scales[i / rows_per_fp32_scale] is row i's FP32 scale
 *          (1 = per token, rows = one per tensor, R = one per R-row expert);
 *          cols % 16 == 0, rows_per_fp32_scale >= 1.
 *   fp32_scales and rows_per_fp32_scale are ignored for MXFP8 (may be NULL/0).
 *   out [rows][cols] BF16, 16-byte aligned.
 *   rows * cols must be below 2^36 (MXQ_ERR_SIZE otherwise).
 */
int mxq_dequantize_bf16(int fmt, const uint8_t *codes, const uint8_t *scales,
                        const float *fp32_scales, int64_t rows_per_fp32_scale,
                        int64_t rows, int64_t cols, uint16_t *out, void *stream);

/*
 * Quantize and dequantize in one pass: the rowwise MXFP8 or per-token NVFP4
 * quantization of x together with its BF16 dequantization, written from
 * registers, so the dequantized-backward mode (backward GEMMs consume BF16
 * dequantizations of the exact forward operands: the dequantized-backward
 * paragraph) needs no second pass over the codes.  Byte-identical to the
 * quantize call followed by mxq_dequantize_bf16 on its outputs.
 *
 *   fmt == MXQ_FMT_MXFP8_ROW: codes [rows][cols] (16-byte aligned), scales
 *          [rows][cols/32] as mxq_mxfp8_quantize_rowcol's rowwise copy;
 *          token_scales must be NULL; cols % 32 == 0, cols <= 2^26, MXFP8
 *          tile limit as above.
 *   fmt == MXQ_FMT_NVFP4: codes [rows][cols/2] (16-byte aligned), scales
 *          [rows][cols/16], token_scales [rows] as
 *          mxq_nvfp4_quantize_per_token; cols % 16 == 0, rows < 2^26.
 *   out  [rows][cols] BF16, 16-byte aligned, required.
 *   codes and scales must be both NULL or both non-NULL (NULL: not stored,
 *   only the dequantized copy is written); NVFP4 token_scales may be NULL
 *   (not stored).  A mismatched pair, or token_scales with MXFP8, gives
 *   MXQ_ERR_OFFSETS.
 */
int mxq_quantize_dequant_bf16(int fmt, const uint16_t *x, int64_t rows, int64_t cols,
                              uint8_t *codes, uint8_t *scales, float *token_scales,
                              uint16_t *out, void *stream);

/*
 * Block-scaled GEMM on MXFP8 operands: C = A x B^T with
 *   C[m][n] = sum_k dec(a[m][k]) 2^(sa[m][k/32] - 127) dec(b[n][k]) 2^(sb[n][k/32] - 127),
 * the forward GEMM that consumes the rowwise copies made by
 * mxq_mxfp8_quantize_rowcol (activations [M][K], weights [N][K], both
 * K-contiguous; the MXFP8 format and recipe paragraphs).  Products are
 * exact; each matrix instruction sums its 64 products to about 12 bits of
 * their magnitude sum and the instructions' results are accumulated in
 * fp32, so C differs from the exact sum by at most (2^-10 + K 2^-24)
 * sum_k |a b| (plus one BF16 rounding, nearest-even, for MXQ_OUT_BF16).
 *
 *   a  [M][K] E4M3 codes, 16-byte aligned;  a_scales [M][K/32] E8M0, 4-byte aligned.
 *   b  [N][K] E4M3 codes, 16-byte aligned;  b_scales [N][K/32] E8M0, 4-byte aligned.
 *   c  [M][N] fp32 or BF16 (out_dtype), row-major.
 *   K % 128 == 0 (MXQ_ERR_SHAPE) and K <= 2^23 (MXQ_ERR_SIZE); any M, N >= 1
 *   within the GEMM tile limit above.
 */
int mxq_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                   const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                   void *c, void *stream);

/*
 * Grouped (per-expert) MXFP8 GEMM, the MoE expert layer fed by the grouped
 * quantizer: for every expert e and every row r of its segment
 * seg_offsets[e] <= r < seg_offsets[e+1],
 *   C[r][n] = sum_k dec(a[r][k]) 2^(sa[r][k/32] - 127) dec(b_e[n][k]) 2^(sb_e[n][k/32] - 127),
 * the product of the expert-sorted rowwise copy (the grouped MXFP8
 * quantize's row_codes / row_scales; the expert layers that the MXFP8
 * recipe paragraph of "Miles: end-to-end MXFP8 and per-token NVFP4 RL on
 * Blackwell" runs) with expert e's weight.  Same accumulation and bound as
 * mxq_mxfp8_gemm.
 *
 *   a  [total_rows][K] E4M3 codes, 16-byte aligned; a_scales [total_rows][K/32] E8M0.
 *   b  [n_groups][N][K] E4M3 codes, 16-byte aligned; b_scales [n_groups][N][K/32] E8M0.
 *   seg_offsets  [n_groups + 1] int64, device memory, 0 = o_0 <= ... <= o_G = total_rows.
 *   c  [total_rows][N] fp32 or BF16 (out_dtype), row-major; rows outside every
 *      segment are not written.
 *   K % 128 == 0 (MXQ_ERR_SHAPE); K <= 2^23, n_groups >= 1 and
 *   (ceil(total_rows / 256) + n_groups) * ceil(N / 256) within the GEMM tile
 *   limit above (MXQ_ERR_SIZE).  The offsets are device data the host cannot
 *   check: each segment is clamped into [0, total_rows), so malformed
 *   offsets give meaningless rows, never an access out of bounds.
 */
int mxq_mxfp8_grouped_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                           const uint8_t *b_scales, const int64_t *seg_offsets, int64_t n_groups,
                           int64_t total_rows, int64_t N, int64_t K, int out_dtype, void *c,
                           void *stream);

/*
 * Block-scaled GEMM on NVFP4 operands: C = A x B^T with
 *   C[m][n] = sa[m / rows_per_a_scale] sb[n / rows_per_b_scale]
 *             sum_k dec(a[m][k]) dec(ba[m][k/16]) dec(b[n][k]) dec(bb[n][k/16]),
 * the forward GEMM of the per-token NVFP4 recipe (activations with one FP32
 * scale per token, rows_per_a_scale = 1; weights with one FP32 scale per
 * tensor or expert, rows_per_b_scale = its rows): the NVFP4 format and
 * per-token activation scale paragraphs.  Each dec(code) dec(block scale) is
 * exactly an FP16 value; the sum is accumulated in fp32 by the FP16 matrix
 * instructions and the FP32 scales are applied to it as
 * fp32(fp32(sum * sa) * sb), then rounded to BF16 (nearest-even) for
 * MXQ_OUT_BF16.
 *
 *   a  [M][K/2] packed E2M1 (even element in the low nibble), 16-byte aligned;
 *   a_block_scales [M][K/16] E4M3, 4-byte aligned;  a_scales FP32, one per
 *   rows_per_a_scale rows.  b, b_block_scales, b_scales likewise for [N][K].
 *   c  [M][N] fp32 or BF16 (out_dtype).
 *   K % 64 == 0 (MXQ_ERR_SHAPE) and K <= 2^23 (MXQ_ERR_SIZE); any M, N >= 1
 *   within the GEMM tile limit above;
 *   rows_per_a_scale, rows_per_b_scale >= 1.
 */
int mxq_nvfp4_gemm(const uint8_t *a, const uint8_t *a_block_scales, const float *a_scales,
                   int64_t rows_per_a_scale, const uint8_t *b, const uint8_t *b_block_scales,
                   const float *b_scales, int64_t rows_per_b_scale, int64_t M, int64_t N,
                   int64_t K, int out_dtype, void *c, void *stream);

/*
 * Grouped columnwise MXFP8 copy in the layout of the expert layer's weight
 * gradient (the columnwise copy of the MXFP8 recipe paragraph of "Miles:
 * end-to-end MXFP8 and per-token NVFP4 RL on Blackwell", which feeds the
 * backward GEMMs): the same 32x1 blocks as mxq_grouped_quantize's
 * columnwise copy (32-row blocks from each segment's first row, a partial
 * tail block per segment), stored transposed so that each segment's rows
 * are contiguous, with every segment padded to a multiple of 128 rows by
 * zero blocks (code 0, scale byte 0):
 *   codes_t[c][32 P[e] + i] = code of x[o_e + i][c] for i < n_e, 0 up to the padding;
 *   scales_t[c][P[e] + j] = E8M0 byte of block j of segment e in column c.
 *
 *   x  [total_rows][cols] BF16 (expert-sorted), 16-byte aligned; cols % 32 == 0.
 *   seg_offsets  [n_groups + 1] int64, device memory, as for mxq_grouped_quantize.
 *   codes_t [cols][pitch], 16-byte aligned, and scales_t [cols][pitch / 32],
 *      4-byte aligned, pitch = 128 * ceil(total_rows / 128) + 128 * n_groups;
 *      columns past the last segment's padding are not written.
 *   block_offsets [n_groups + 1] int64 (written): P[e], segment e's first
 *      32-row block in the padded layout (P[0] = 0).
 *   n_groups <= 2^40; malformed offsets are clamped as in mxq_grouped_quantize.
 */
int mxq_mxfp8_grouped_colwise_t(const uint16_t *x, int64_t total_rows, int64_t cols,
                                const int64_t *seg_offsets, int64_t n_groups, uint8_t *codes_t,
                                uint8_t *scales_t, int64_t *block_offsets, void *stream);

/*
 * Both MXFP8 copies the expert layer's backward needs from one read of its
 * input (dY): the rowwise 1x32 copy, as mxq_grouped_quantize writes it
 * (feeding the data gradient through mxq_mxfp8_grouped_gemm), and the
 * columnwise copy of mxq_mxfp8_grouped_colwise_t (feeding
 * mxq_mxfp8_grouped_wgrad), each block quantized independently from x as
 * the MXFP8 recipe paragraph of "Miles: end-to-end MXFP8 and per-token NVFP4
 * RL on Blackwell" states.  The bytes equal those two calls'.
 *
 *   row_codes [total_rows][cols], 16-byte aligned; row_scales [total_rows][cols / 32].
 *      Rows in no segment are not written.
 *   The other arguments as for mxq_mxfp8_grouped_colwise_t.
 */
int mxq_mxfp8_grouped_quantize_rowcol_t(const uint16_t *x, int64_t total_rows, int64_t cols,
                                        const int64_t *seg_offsets, int64_t n_groups,
                                        uint8_t *row_codes, uint8_t *row_scales,
                                        uint8_t *codes_t, uint8_t *scales_t,
                                        int64_t *block_offsets, void *stream);

/*
 * The expert layer's MXFP8 weight gradient: for every expert e,
 *   C_e[m][n] = sum over k in [32 P[e], 32 P[e+1]) of dec(a[m][k]) 2^(sa[m][k/32] - 127)
 *               dec(b[n][k]) 2^(sb[n][k/32] - 127),
 * a contraction over the segment's rows, with a and b two copies made by
 * mxq_mxfp8_grouped_colwise_t over the same segments (a from dY [rows][M],
 * b from X [rows][N]: C_e = dW_e = dY_e^T X_e) and P their block_offsets.
 * Padding blocks hold zeros and add nothing.  Same accumulation and bound
 * as mxq_mxfp8_gemm, with K the segment's rows.
 *
 *   a [M][pitch], a_scales [M][pitch / 32]; b [N][pitch], b_scales [N][pitch / 32].
 *   block_offsets [n_groups + 1] int64, device memory.
 *   c [n_groups][M][N] fp32 or BF16 (out_dtype); an expert with no rows gets zeros.
 *   pitch % 128 == 0 (MXQ_ERR_SHAPE), pitch <= 2^23 and n_groups * ceil(M / 256) *
 *   ceil(N / 256) within the GEMM tile limit (MXQ_ERR_SIZE).  Malformed
 *   offsets are clamped into [0, pitch) and cut to whole 128-column steps.
 */
int mxq_mxfp8_grouped_wgrad(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                            const uint8_t *b_scales, const int64_t *block_offsets,
                            int64_t n_groups, int64_t M, int64_t N, int64_t pitch, int out_dtype,
                            void *c, void *stream);

/*
 * Grouped (per-expert) NVFP4 GEMM, the MoE expert layer on per-token NVFP4
 * rows (the rollout forward of the NVFP4 format and per-token
 * activation-scale paragraphs of "Miles: end-to-end MXFP8 and per-token
 * NVFP4 RL on Blackwell"): for every expert e and every row r of its
 * segment seg_offsets[e] <= r < seg_offsets[e+1],
 *   C[r][n] = fp32(fp32(S * a_scales[r]) * b_scales[e]),
 *   S = sum_k dec(a[r][k]) dec(ab[r][k/16]) dec(b_e[n][k]) dec(bb_e[n][k/16]),
 * the expert-sorted rows as the grouped NVFP4 quantize writes them (codes,
 * E4M3 block scales, one FP32 scale per row) times expert e's weight as the
 * export writes it (one FP32 scope scale per expert).  Same accumulation and
 * bound as mxq_nvfp4_gemm.
 *
 *   a  [total_rows][K/2] E2M1 codes, 16-byte aligned; a_block_scales [total_rows][K/16]
 *      E4M3, 4-byte aligned; a_scales [total_rows] fp32.
 *   b  [n_groups][N][K/2], 16-byte aligned; b_block_scales [n_groups][N][K/16], 4-byte
 *      aligned; b_scales [n_groups] fp32.
 *   seg_offsets  [n_groups + 1] int64, device memory, as for mxq_mxfp8_grouped_gemm.
 *   c  [total_rows][N] fp32 or BF16 (out_dtype); rows outside every segment are not written.
 *   K % 64 == 0 (MXQ_ERR_SHAPE); the size limits and the treatment of malformed offsets
 *   are those of mxq_mxfp8_grouped_gemm.
 */
int mxq_nvfp4_grouped_gemm(const uint8_t *a, const uint8_t *a_block_scales, const float *a_scales,
                           const uint8_t *b, const uint8_t *b_block_scales, const float *b_scales,
                           const int64_t *seg_offsets, int64_t n_groups, int64_t total_rows,
                           int64_t N, int64_t K, int out_dtype, void *c, void *stream);

/*
 * Outputs of the grouped call.  MXFP8 uses the first five fields, NVFP4 the
 * last three; the others are ignored.
 *   row_codes, row_scales  as mxq_mxfp8_quantize_rowcol over all total_rows.
 *   col_codes   [total_rows][cols], same index as x.
 *   col_scales  room for total_rows/32 + n_groups rows of cols bytes; segment
 *               e's blocks of 32 rows start at its first row, its last block
 *               covers the rows that remain (amax over existing rows), and its
 *               scale rows start at P[e] = sum_{f<e} ceil(n_f / 32).
 *   col_scale_offsets [n_groups + 1] int64, written by the call: P[0..G].
 *   codes, block_scales, token_scales  as mxq_nvfp4_quantize_per_token.
 */
typedef struct {
    uint8_t *row_codes;
    uint8_t *row_scales;
    uint8_t *col_codes;
    uint8_t *col_scales;
    int64_t *col_scale_offsets;
    uint8_t *codes;
    uint8_t *block_scales;
    float *token_scales;
} mxq_grouped_out;

/*
 * Grouped quantize over ragged MoE expert segments: x holds the rows of all
 * experts, sorted by expert; segment e is rows [seg_offsets[e],
 * seg_offsets[e+1]).  Rowwise MXFP8 and per-token NVFP4 outputs do not depend
 * on the segments (per-token scales make every row independent of the others:
 * the batch-invariance argument of the per-token paragraphs); columnwise MXFP8
 * blocks restart at each segment.  Implements the MXFP8 and NVFP4 passages
 * above for the MoE expert path.
 *
 *   fmt           MXQ_FMT_MXFP8_ROWCOL or MXQ_FMT_NVFP4.
 *   x             [total_rows][cols] BF16, 16-byte aligned.
 *   seg_offsets   device int64 [n_groups + 1], 0 = o_0 <= ... <= o_G =
 *                 total_rows (read on the device; not validated on the host).
 *   out           host pointer to the output struct (device arrays inside).
 *   For NVFP4, total_rows must be below 2^26; for MXFP8, cols must not exceed
 *   2^26 and the tile limit above holds (MXQ_ERR_SIZE otherwise).
 */
int mxq_grouped_quantize(int fmt, const uint16_t *x, int64_t total_rows,
                         int64_t cols, const int64_t *seg_offsets,
                         int64_t n_groups, const mxq_grouped_out *out,
                         void *stream);

/*
 * Grouped quantize fused with MoE dispatch: reads the unpermuted tokens
 * instead of a gathered copy.  Row r of the expert-sorted layout is token
 * row_tokens[r] of x; copy c of token t is row token_rows[t * top_k + c].
 * The outputs are byte-identical to mxq_grouped_quantize on the gathered
 * tensor x[row_tokens[r]] (same segments, same fields).  NVFP4 quantizes
 * each token once and writes it to its top_k rows: per-token outputs do not
 * depend on the rest of the batch (the batch-invariance argument of the
 * per-token activation paragraphs of the page "Miles: end-to-end MXFP8 and
 * per-token NVFP4 RL on Blackwell"); MXFP8 columnwise blocks need the rows
 * in segment order, so the tiles gather their rows through row_tokens.
 *
 *   fmt           MXQ_FMT_MXFP8_ROWCOL or MXQ_FMT_NVFP4.
 *   x             [n_tokens][cols] BF16, 16-byte aligned.
 *   token_rows    device int64 [n_tokens][top_k] (NVFP4; ignored for MXFP8).
 *                 An entry outside [0, total_rows) is skipped (a dropped
 *                 copy); a row that no entry names is left unwritten.
 *   row_tokens    device int64 [total_rows] (MXFP8; ignored for NVFP4).
 *                 Entries are clamped into [0, n_tokens).
 *   seg_offsets   as mxq_grouped_quantize (MXFP8 columnwise only; may be
 *                 NULL when only the rowwise copy is requested, and for
 *                 NVFP4).
 *   out           as mxq_grouped_quantize, over total_rows rows.
 * The maps are device data, not validated on the host: when they are not
 * inverse to each other the outputs are unspecified bytes, but no access
 * leaves the arrays.  For NVFP4, n_tokens must be below 2^26; for MXFP8 the
 * tile limit above holds.
 */
int mxq_grouped_quantize_dispatch(int fmt, const uint16_t *x, int64_t n_tokens,
                                  int64_t cols, int64_t top_k,
                                  const int64_t *token_rows,
                                  const int64_t *row_tokens, int64_t total_rows,
                                  const int64_t *seg_offsets, int64_t n_groups,
                                  const mxq_grouped_out *out, void *stream);

/*
 * Measurement reference, not an operation of the pages: reads src_bytes of
 * src and writes dst_bytes of dst with no arithmetic beyond an XOR fold, in
 * the quantizers' launch style (one-shot grid, 16-byte coalesced accesses).
 * Timed on a workload's read and write byte counts it gives the floor that
 * any kernel moving exactly those bytes meets on the device, against which
 * the quantizers' times are reported beside the HBM peak.
 *   With n_r = src_bytes / 16 and n_w = dst_bytes / 16 chunks of 16 bytes:
 *   n_r >= n_w: dst chunk j = XOR of src chunks j + i n_w (every i with
 *               j + i n_w < n_r);
 *   n_r <  n_w: dst chunk j = src chunk floor(j m / 2^32), where
 *               m = floor(n_r 2^32 / n_w).
 *   src, dst device memory of the current device, 16-byte aligned, not
 *   overlapping; src_bytes and dst_bytes positive multiples of 16
 *   (MXQ_ERR_SHAPE) of at most 2^35 (MXQ_ERR_SIZE).
 */
int mxq_copy_floor(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                   void *stream);

/* A static, human-readable message for a status code. */
const char *mxq_status_string(int status);

/* MXQ_VERSION of the built library. */
int mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
