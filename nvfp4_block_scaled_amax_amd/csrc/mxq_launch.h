// mxq_launch.h -- internal launchers behind the C ABI (mxq_api.cpp).  Each
// launcher enqueues on `stream` and returns the launch status; arguments have
// been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Grid limits.  A dispatch packet holds the grid size in work-items as a
// 32-bit field per dimension, and every launcher here uses a one-dimensional
// grid, so a launch has at most 2^32 - 1 work-items.  The C entry points
// check the limits below before anything is launched.
constexpr int64_t MAX_GRID_ITEMS = 0xFFFFFFFF;

// Rows (tokens) of the per-token NVFP4 launches: one 64-lane workgroup per
// row.  (The split path uses two wavefronts per row, on grids of at most a
// few tens of thousands of rows.)
constexpr int64_t MAX_TOKEN_ROWS = MAX_GRID_ITEMS / 64;

// 32 x 128 tiles of the MXFP8 tile launches: one wavefront per tile, in
// workgroups of up to 8 wavefronts (the last workgroup rounded up).
constexpr int64_t MAX_MXFP8_TILES = MAX_GRID_ITEMS / 64 - 8;
inline int64_t mxfp8_tiles(int64_t row_tiles, int64_t cols)
{
    return row_tiles * ((cols + 127) / 128);
}

// 256 x 256 output tiles of the GEMM launches: one 256-thread workgroup per
// tile, the count rounded up to a multiple of 8 (one share per XCD).
constexpr int64_t MAX_GEMM_TILES = MAX_GRID_ITEMS / 256 - 8;

// Row pitch of the grouped transposed columnwise copy: every segment's
// rows rounded up to a multiple of 128 fit in it.
inline int64_t grouped_colt_pitch(int64_t rows, int64_t n_groups)
{
    return (rows + 127) / 128 * 128 + 128 * n_groups;
}

// 256-row tiles the grouped GEMM launches for: every segment's rows in
// 256-row tiles, at most one partial tile per segment.
inline int64_t grouped_gemm_mtiles(int64_t rows, int64_t n_groups)
{
    return (rows + 255) / 256 + n_groups;
}

// Workgroups (64 lanes each) of the export's amax pass over n_experts scopes
// of n_per elements per tensor (two tensors when `pair`).
int64_t scoped_amax_workgroups(int64_t n_experts, int64_t n_per, bool pair);
constexpr int64_t MAX_SCOPED_AMAX_WORKGROUPS = MAX_GRID_ITEMS / 64;

// Workgroups of `kernel` (launched with `block_threads` threads) that the
// current device holds at once: compute units x the occupancy the runtime
// reports for the kernel's register and LDS use.  Cached per kernel and
// device; grid-stride kernels size their grids from it.
int64_t resident_workgroups(const void *kernel, int block_threads);

// row_tokens != nullptr (dispatch): row r is row row_tokens[r] of x.
hipError_t launch_mxfp8_dense(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *row_codes,
                              uint8_t *row_scales, uint8_t *col_codes, uint8_t *col_scales,
                              const int64_t *row_tokens, int64_t n_tokens, hipStream_t stream);

// Writes P (col_scale_offsets) and quantizes; at most `max_tiles` column
// blocks (the capacity of col_scales) are written whatever the offsets say.
// row_tokens != nullptr (dispatch): row r of the grouped layout is row
// row_tokens[r] of x (x has n_tokens rows; entries are clamped into range).
hipError_t launch_mxfp8_grouped(const uint16_t *x, int64_t total_rows, int64_t cols,
                                const int64_t *seg_offsets, int64_t n_groups, uint8_t *row_codes,
                                uint8_t *row_scales, uint8_t *col_codes, uint8_t *col_scales,
                                int64_t *col_scale_offsets, const int64_t *row_tokens,
                                int64_t n_tokens, hipStream_t stream);

// Both MXFP8 copies under the OCP MX scale rule (floor(log2 amax) - 8,
// saturating), a comparison variant; arguments as launch_mxfp8_dense.
hipError_t launch_mxfp8_ocp_floor(const uint16_t *x, int64_t rows, int64_t cols,
                                  uint8_t *row_codes, uint8_t *row_scales, uint8_t *col_codes,
                                  uint8_t *col_scales, hipStream_t stream);

// Both MXFP8 copies with the columnwise one transposed: codes [cols][rows],
// scales [cols][rows/32] (rows % 32 == 0); row_codes/row_scales may be null.
hipError_t launch_mxfp8_colt(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *row_codes,
                             uint8_t *row_scales, uint8_t *col_codes_t, uint8_t *col_scales_t,
                             hipStream_t stream);

// Rowwise MXFP8 and its BF16 dequantization in one pass; rc/rs may be null
// (only the dequantized copy is stored).
hipError_t launch_mxfp8_row_qdq(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *row_codes,
                                uint8_t *row_scales, uint16_t *dq, hipStream_t stream);

// Per-token NVFP4 and its BF16 dequantization in one pass; codes/block_scales
// and token_scales may be null (not stored).
hipError_t launch_nvfp4_qdq(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                            uint8_t *block_scales, float *token_scales, uint16_t *dq,
                            hipStream_t stream);

// Approximate per-token NVFP4 (opt-in variant, cols <= 4096): one
// reciprocal-multiply and one conversion per block scale and per code.
hipError_t launch_nvfp4_approx(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                               uint8_t *block_scales, float *token_scales, hipStream_t stream);

hipError_t launch_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                  uint8_t *block_scales, float *token_scales, hipStream_t stream);

// Quantizes each token once and writes it to rows token_rows[t * top_k + c]
// (c < top_k) of the outputs; rows outside [0, out_rows) are skipped.
hipError_t launch_nvfp4_dispatch(const uint16_t *x, int64_t n_tokens, int64_t cols,
                                 const int64_t *token_rows, int64_t top_k, int64_t out_rows,
                                 uint8_t *codes, uint8_t *block_scales, float *token_scales,
                                 hipStream_t stream);

hipError_t launch_nvfp4_scoped(const uint16_t *gate, const uint16_t *up, int64_t n_experts,
                               int64_t rows, int64_t cols, uint8_t *gate_codes,
                               uint8_t *gate_block_scales, uint8_t *up_codes,
                               uint8_t *up_block_scales, float *scope_scales, hipStream_t stream);

// The export's code pass alone, under s_e = fp32(A_e / 2688) from scope
// amaxes the caller supplies (BF16 bits, [n_experts]).
hipError_t launch_nvfp4_scoped_amax(const uint16_t *gate, const uint16_t *up,
                                    const uint16_t *scope_amax, int64_t n_experts, int64_t rows,
                                    int64_t cols, uint8_t *gate_codes, uint8_t *gate_block_scales,
                                    uint8_t *up_codes, uint8_t *up_block_scales,
                                    float *scope_scales, hipStream_t stream);

hipError_t launch_dequant_mxfp8(bool col, const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream);

hipError_t launch_dequant_nvfp4(const uint8_t *codes, const uint8_t *block_scales,
                                const float *fp32_scales, int64_t rows_per_scale, int64_t rows,
                                int64_t cols, uint16_t *out, hipStream_t stream);

// C[M][N] = A (MXFP8 [M][K], scales [M][K/32]) x B (MXFP8 [N][K], scales
// [N][K/32])^T, fp32 accumulation, fp32 or BF16 result; K % 128 == 0.
hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                             const uint8_t *b_scales, int64_t M, int64_t N, int64_t K,
                             bool bf16_out, void *c, hipStream_t stream);

// Grouped columnwise copy, transposed and padded: codes [cols][pitch] and
// scales [cols][pitch / 32] (pitch = grouped_colt_pitch), segment e's
// blocks from block P[e] (P [G+1], written), each segment rounded up to 128
// rows with zero blocks; with rc != nullptr also the rowwise copy (rc
// [rows][cols], rs [rows][cols / 32]) from the same read.
hipError_t launch_mxfp8_grouped_colt(const uint16_t *x, int64_t total_rows, int64_t cols,
                                     const int64_t *off, int64_t n_groups, uint8_t *rc,
                                     uint8_t *rs, uint8_t *cct, uint8_t *cst, int64_t *P,
                                     hipStream_t stream);

// Grouped weight gradient: C_e[M][N] = A[:, 32 P[e] .. 32 P[e+1]) x
// B[:, same]^T for every expert e, A [M][ld] and B [N][ld] in the grouped
// transposed padded layout (ld % 128 == 0); C [G][M][N].
hipError_t launch_mxfp8_grouped_wgrad(const uint8_t *a, const uint8_t *a_scales,
                                      const uint8_t *b, const uint8_t *b_scales,
                                      const int64_t *block_offsets, int64_t n_groups, int64_t M,
                                      int64_t N, int64_t ld, bool bf16_out, void *c,
                                      hipStream_t stream);

// Grouped: C[r][N] = A[r] (MXFP8 rows of segment e) x B_e^T for every r in
// segment e = seg_offsets[e] .. seg_offsets[e+1] (device data); B [G][N][K],
// scales [G][N][K/32]; K % 128 == 0.
hipError_t launch_mxfp8_grouped_gemm(const uint8_t *a, const uint8_t *a_scales,
                                     const uint8_t *b, const uint8_t *b_scales,
                                     const int64_t *seg_offsets, int64_t n_groups, int64_t rows,
                                     int64_t N, int64_t K, bool bf16_out, void *c,
                                     hipStream_t stream);

// Grouped: C[r][N] = sa[r] sb[e] x A[r] (NVFP4 rows of segment e: codes
// [R][K/2], E4M3 block scales [R][K/16], FP32 sa [R]) x B_e^T (codes
// [G][N][K/2], block scales [G][N][K/16], one FP32 sb[e] per expert);
// K % 64 == 0.
hipError_t launch_nvfp4_grouped_gemm(const uint8_t *a, const uint8_t *a_block_scales,
                                     const float *a_scales, const uint8_t *b,
                                     const uint8_t *b_block_scales, const float *b_scales,
                                     const int64_t *seg_offsets, int64_t n_groups, int64_t rows,
                                     int64_t N, int64_t K, bool bf16_out, void *c,
                                     hipStream_t stream);

// C[M][N] = sa[m / rows_per_a] sb[n / rows_per_b] x A (NVFP4 [M][K/2], E4M3
// block scales [M][K/16]) x B (NVFP4 [N][K/2], [N][K/16])^T; K % 64 == 0.
hipError_t launch_nvfp4_gemm(const uint8_t *a, const uint8_t *a_block_scales,
                             const float *a_scales, int64_t rows_per_a, const uint8_t *b,
                             const uint8_t *b_block_scales, const float *b_scales,
                             int64_t rows_per_b, int64_t M, int64_t N, int64_t K, bool bf16_out,
                             void *c, hipStream_t stream);

// Reads src_bytes and writes dst_bytes (both multiples of 16, at most 2^35)
// with an XOR fold or spread and no other arithmetic: the measurement
// reference of mxq_copy_floor.
hipError_t launch_copy_floor(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                             hipStream_t stream);

}  // namespace mxq
