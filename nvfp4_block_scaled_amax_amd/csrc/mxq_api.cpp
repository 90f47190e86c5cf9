// mxq_api.cpp -- the C ABI of libmxq (declared in include/mxq.h): host-side
// validation, then the launch.  Nothing here allocates device memory.
#include "mxq.h"

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "mxq_launch.h"

namespace {

// One array argument: its extent in bytes, required alignment, and whether
// the call writes it.
struct Buf {
    const void *p;
    int64_t bytes;
    int align;
    bool output;
};

constexpr int64_t MAX_ELEMS = (int64_t)1 << 62;
// GEMM tiles address their 256 rows with 32-bit offsets.
constexpr int64_t MAX_GEMM_K = (int64_t)1 << 23;
constexpr int64_t MAX_GRID_ROWS = mxq::MAX_TOKEN_ROWS;   // per-token NVFP4: one workgroup per row
constexpr int64_t MAX_BLOCKS = 0xFFFFFFFF;        // 16-element blocks indexed in 32 bits
constexpr int64_t MAX_MXFP8_COLS = (int64_t)1 << 26;  // 32-row tile offsets fit 32 bits
constexpr int64_t MAX_COPY_FLOOR_BYTES = (int64_t)1 << 35;

bool size_ok(int64_t a, int64_t b)
{
    return a > 0 && b > 0 && a <= MAX_ELEMS / b;
}

// The MXFP8 tile launches over `row_tiles` 32-row tiles of `cols` columns
// fit one grid.
bool mxfp8_grid_ok(int64_t row_tiles, int64_t cols)
{
    return row_tiles <= MAX_ELEMS / cols && mxq::mxfp8_tiles(row_tiles, cols) <= mxq::MAX_MXFP8_TILES;
}

// One allocation of the current device: [base, base + size).
struct Range {
    uintptr_t base;
    uint64_t size;
};

bool inside(const Buf &b, const Range &r)
{
    const uintptr_t p = (uintptr_t)b.p;
    return p >= r.base && (uint64_t)(p - r.base) + (uint64_t)b.bytes <= r.size;
}

// Device memory of the current device, and [p, p + bytes) inside one
// allocation, whose range is returned in *r.
int check_device(const Buf &b, int device, Range *r)
{
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, b.p) != hipSuccess) {
        (void)hipGetLastError();
        return MXQ_ERR_DEVICE;
    }
    if (attr.type != hipMemoryTypeDevice || attr.device != device)
        return MXQ_ERR_DEVICE;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(b.p)) != hipSuccess) {
        (void)hipGetLastError();
        return MXQ_ERR_DEVICE;
    }
    *r = Range{(uintptr_t)base, (uint64_t)size};
    if (!inside(b, *r))
        return MXQ_ERR_DEVICE;
    return MXQ_OK;
}

bool overlaps(const Buf &a, const Buf &b)
{
    const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
    const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
    return a0 < b1 && b0 < a1;
}

// Alignment, device residency and extent of every buffer, then pairwise
// overlap between any output and any other buffer.
int check_bufs(const Buf *bufs, int n)
{
    for (int i = 0; i < n; i++)
        if (((uintptr_t)bufs[i].p) % (uintptr_t)bufs[i].align != 0)
            return MXQ_ERR_ALIGN;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return MXQ_ERR_DEVICE;
    }
    // A buffer inside an allocation already queried in this call (same
    // device, device memory) needs no runtime query of its own: each query
    // costs about 0.4 us of host time, which bounds back-to-back launches
    // of small kernels.
    Range seen[16];
    int n_seen = 0;
    for (int i = 0; i < n; i++) {
        bool known = false;
        for (int k = 0; k < n_seen && !known; k++)
            known = inside(bufs[i], seen[k]);
        if (known)
            continue;
        Range r{0, 0};
        const int st = check_device(bufs[i], device, &r);
        if (st != MXQ_OK)
            return st;
        if (n_seen < 16)
            seen[n_seen++] = r;
    }
    for (int i = 0; i < n; i++)
        for (int j = i + 1; j < n; j++)
            if ((bufs[i].output || bufs[j].output) && overlaps(bufs[i], bufs[j]))
                return MXQ_ERR_ALIAS;
    return MXQ_OK;
}

int launched(hipError_t e)
{
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int mxq_version(void)
{
    return MXQ_VERSION;
}

const char *mxq_status_string(int status)
{
    switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SIZE: return "a size is not positive (or too large), or n_groups < 1";
    case MXQ_ERR_SHAPE: return "rows/cols not divisible as the format requires";
    case MXQ_ERR_ALIGN: return "a pointer is not aligned as required (16 bytes for vector-accessed arrays)";
    case MXQ_ERR_ALIAS: return "an output overlaps an input or another output";
    case MXQ_ERR_OFFSETS: return "inconsistent combination of optional outputs";
    case MXQ_ERR_DEVICE: return "an array is not device memory of the current device, or extends past the end of its allocation";
    case MXQ_ERR_LAUNCH: return "kernel launch failed";
    case MXQ_ERR_ARG: return "unknown format argument";
    default: return "unknown status";
    }
}

int mxq_mxfp8_quantize_rowcol(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *row_codes,
                              uint8_t *row_scales, uint8_t *col_codes, uint8_t *col_scales,
                              void *stream)
{
    if (!x)
        return MXQ_ERR_NULL;
    if ((row_codes == nullptr) != (row_scales == nullptr) ||
        (col_codes == nullptr) != (col_scales == nullptr) || (!row_codes && !col_codes))
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols) || cols > MAX_MXFP8_COLS || !mxfp8_grid_ok((rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0 || (col_codes && rows % 32 != 0))
        return MXQ_ERR_SHAPE;
    const int64_t n = rows * cols;
    Buf b[5];
    int k = 0;
    b[k++] = {x, 2 * n, 16, false};
    if (row_codes) {
        b[k++] = {row_codes, n, 16, true};
        b[k++] = {row_scales, n / 32, 1, true};
    }
    if (col_codes) {
        b[k++] = {col_codes, n, 16, true};
        b[k++] = {col_scales, n / 32, 8, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_dense(x, rows, cols, row_codes, row_scales, col_codes,
                                            col_scales, nullptr, 0, (hipStream_t)stream));
}

int mxq_mxfp8_quantize_ocp_floor(const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *row_codes, uint8_t *row_scales, uint8_t *col_codes,
                                 uint8_t *col_scales, void *stream)
{
    if (!x)
        return MXQ_ERR_NULL;
    if ((row_codes == nullptr) != (row_scales == nullptr) ||
        (col_codes == nullptr) != (col_scales == nullptr) || (!row_codes && !col_codes))
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols) || cols > MAX_MXFP8_COLS || !mxfp8_grid_ok((rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0 || (col_codes && rows % 32 != 0))
        return MXQ_ERR_SHAPE;
    const int64_t n = rows * cols;
    Buf b[5];
    int k = 0;
    b[k++] = {x, 2 * n, 16, false};
    if (row_codes) {
        b[k++] = {row_codes, n, 16, true};
        b[k++] = {row_scales, n / 32, 1, true};
    }
    if (col_codes) {
        b[k++] = {col_codes, n, 16, true};
        b[k++] = {col_scales, n / 32, 8, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_ocp_floor(x, rows, cols, row_codes, row_scales, col_codes,
                                                col_scales, (hipStream_t)stream));
}

int mxq_mxfp8_quantize_rowcol_t(const uint16_t *x, int64_t rows, int64_t cols,
                                uint8_t *row_codes, uint8_t *row_scales, uint8_t *col_codes_t,
                                uint8_t *col_scales_t, void *stream)
{
    if (!x || !col_codes_t || !col_scales_t)
        return MXQ_ERR_NULL;
    if ((row_codes == nullptr) != (row_scales == nullptr))
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols) || cols > MAX_MXFP8_COLS || !mxfp8_grid_ok((rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0 || rows % 32 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = rows * cols;
    Buf b[5];
    int k = 0;
    b[k++] = {x, 2 * n, 16, false};
    b[k++] = {col_codes_t, n, 16, true};
    b[k++] = {col_scales_t, n / 32, 1, true};
    if (row_codes) {
        b[k++] = {row_codes, n, 16, true};
        b[k++] = {row_scales, n / 32, 1, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_colt(x, rows, cols, row_codes, row_scales, col_codes_t,
                                           col_scales_t, (hipStream_t)stream));
}

int mxq_nvfp4_quantize_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                 uint8_t *block_scales, float *token_scales, void *stream)
{
    if (!x || !codes || !block_scales || !token_scales)
        return MXQ_ERR_NULL;
    if (!size_ok(rows, cols) || rows > MAX_GRID_ROWS)
        return MXQ_ERR_SIZE;
    if (cols % 16 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = rows * cols;
    const Buf b[4] = {{x, 2 * n, 16, false},
                      {codes, n / 2, 16, true},
                      {block_scales, n / 16, 1, true},
                      {token_scales, 4 * rows, 4, true}};
    const int st = check_bufs(b, 4);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_per_token(x, rows, cols, codes, block_scales, token_scales,
                                                (hipStream_t)stream));
}

int mxq_nvfp4_quantize_per_token_approx(const uint16_t *x, int64_t rows, int64_t cols,
                                        uint8_t *codes, uint8_t *block_scales,
                                        float *token_scales, void *stream)
{
    if (!x || !codes || !block_scales || !token_scales)
        return MXQ_ERR_NULL;
    if (!size_ok(rows, cols) || rows > MAX_GRID_ROWS || cols > 4096)
        return MXQ_ERR_SIZE;
    if (cols % 16 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = rows * cols;
    const Buf b[4] = {{x, 2 * n, 16, false},
                      {codes, n / 2, 16, true},
                      {block_scales, n / 16, 1, true},
                      {token_scales, 4 * rows, 4, true}};
    const int st = check_bufs(b, 4);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_approx(x, rows, cols, codes, block_scales, token_scales,
                                             (hipStream_t)stream));
}

int mxq_nvfp4_quantize_gateup_pair(const uint16_t *gate, const uint16_t *up, int64_t n_experts,
                                   int64_t rows, int64_t cols, uint8_t *gate_codes,
                                   uint8_t *gate_block_scales, uint8_t *up_codes,
                                   uint8_t *up_block_scales, float *scope_scales, void *stream)
{
    if (!gate || !gate_codes || !gate_block_scales || !scope_scales)
        return MXQ_ERR_NULL;
    const bool has_up = up != nullptr;
    if ((up_codes != nullptr) != has_up || (up_block_scales != nullptr) != has_up)
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols) || n_experts <= 0 || !size_ok(n_experts, rows * cols))
        return MXQ_ERR_SIZE;
    if (cols % 16 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = n_experts * rows * cols;
    if (n / 16 > MAX_BLOCKS || n_experts > mxq::MAX_GRID_ITEMS / 64 ||
        mxq::scoped_amax_workgroups(n_experts, rows * cols, has_up) >
            mxq::MAX_SCOPED_AMAX_WORKGROUPS)
        return MXQ_ERR_SIZE;
    Buf b[7];
    int k = 0;
    b[k++] = {gate, 2 * n, 16, false};
    b[k++] = {gate_codes, n / 2, 16, true};
    b[k++] = {gate_block_scales, n / 16, 1, true};
    b[k++] = {scope_scales, 4 * n_experts, 4, true};
    if (has_up) {
        b[k++] = {up, 2 * n, 16, false};
        b[k++] = {up_codes, n / 2, 16, true};
        b[k++] = {up_block_scales, n / 16, 1, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_scoped(gate, up, n_experts, rows, cols, gate_codes,
                                             gate_block_scales, up_codes, up_block_scales,
                                             scope_scales, (hipStream_t)stream));
}

int mxq_nvfp4_quantize_gateup_pair_amax(const uint16_t *gate, const uint16_t *up,
                                        const uint16_t *scope_amax, int64_t n_experts,
                                        int64_t rows, int64_t cols, uint8_t *gate_codes,
                                        uint8_t *gate_block_scales, uint8_t *up_codes,
                                        uint8_t *up_block_scales, float *scope_scales,
                                        void *stream)
{
    if (!gate || !scope_amax || !gate_codes || !gate_block_scales || !scope_scales)
        return MXQ_ERR_NULL;
    const bool has_up = up != nullptr;
    if ((up_codes != nullptr) != has_up || (up_block_scales != nullptr) != has_up)
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols) || n_experts <= 0 || !size_ok(n_experts, rows * cols))
        return MXQ_ERR_SIZE;
    if (cols % 16 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = n_experts * rows * cols;
    if (n / 16 > MAX_BLOCKS || n_experts > mxq::MAX_GRID_ITEMS / 64)
        return MXQ_ERR_SIZE;
    Buf b[8];
    int k = 0;
    b[k++] = {gate, 2 * n, 16, false};
    b[k++] = {scope_amax, 2 * n_experts, 2, false};
    b[k++] = {gate_codes, n / 2, 16, true};
    b[k++] = {gate_block_scales, n / 16, 1, true};
    b[k++] = {scope_scales, 4 * n_experts, 4, true};
    if (has_up) {
        b[k++] = {up, 2 * n, 16, false};
        b[k++] = {up_codes, n / 2, 16, true};
        b[k++] = {up_block_scales, n / 16, 1, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_scoped_amax(gate, up, scope_amax, n_experts, rows, cols,
                                                  gate_codes, gate_block_scales, up_codes,
                                                  up_block_scales, scope_scales,
                                                  (hipStream_t)stream));
}

int mxq_dequantize_bf16(int fmt, const uint8_t *codes, const uint8_t *scales,
                        const float *fp32_scales, int64_t rows_per_fp32_scale, int64_t rows,
                        int64_t cols, uint16_t *out, void *stream)
{
    if (fmt != MXQ_FMT_MXFP8_ROW && fmt != MXQ_FMT_MXFP8_COL && fmt != MXQ_FMT_NVFP4)
        return MXQ_ERR_ARG;
    if (!codes || !scales || !out || (fmt == MXQ_FMT_NVFP4 && !fp32_scales))
        return MXQ_ERR_NULL;
    if (!size_ok(rows, cols) || (fmt == MXQ_FMT_NVFP4 && rows_per_fp32_scale < 1))
        return MXQ_ERR_SIZE;
    const int64_t n = rows * cols;
    if (n / 16 > MAX_BLOCKS)
        return MXQ_ERR_SIZE;
    if (fmt == MXQ_FMT_NVFP4) {
        if (cols % 16 != 0)
            return MXQ_ERR_SHAPE;
        const int64_t n_scales = (rows + rows_per_fp32_scale - 1) / rows_per_fp32_scale;
        const Buf b[4] = {{codes, n / 2, 8, false},
                          {scales, n / 16, 1, false},
                          {fp32_scales, 4 * n_scales, 4, false},
                          {out, 2 * n, 16, true}};
        const int st = check_bufs(b, 4);
        if (st != MXQ_OK)
            return st;
        return launched(mxq::launch_dequant_nvfp4(codes, scales, fp32_scales, rows_per_fp32_scale,
                                                  rows, cols, out, (hipStream_t)stream));
    }
    const bool col = fmt == MXQ_FMT_MXFP8_COL;
    if (cols % 32 != 0 || (col && rows % 32 != 0))
        return MXQ_ERR_SHAPE;
    const Buf b[3] = {{codes, n, 16, false}, {scales, n / 32, col ? 16 : 1, false},
                      {out, 2 * n, 16, true}};
    const int st = check_bufs(b, 3);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_dequant_mxfp8(col, codes, scales, rows, cols, out,
                                              (hipStream_t)stream));
}

int mxq_quantize_dequant_bf16(int fmt, const uint16_t *x, int64_t rows, int64_t cols,
                              uint8_t *codes, uint8_t *scales, float *token_scales,
                              uint16_t *out, void *stream)
{
    if (fmt != MXQ_FMT_MXFP8_ROW && fmt != MXQ_FMT_NVFP4)
        return MXQ_ERR_ARG;
    if (!x || !out)
        return MXQ_ERR_NULL;
    if ((codes == nullptr) != (scales == nullptr) ||
        (fmt == MXQ_FMT_MXFP8_ROW && token_scales != nullptr))
        return MXQ_ERR_OFFSETS;
    if (!size_ok(rows, cols))
        return MXQ_ERR_SIZE;
    const int64_t n = rows * cols;
    Buf b[5];
    int k = 0;
    b[k++] = {x, 2 * n, 16, false};
    b[k++] = {out, 2 * n, 16, true};
    if (fmt == MXQ_FMT_NVFP4) {
        if (rows > MAX_GRID_ROWS)
            return MXQ_ERR_SIZE;
        if (cols % 16 != 0)
            return MXQ_ERR_SHAPE;
        if (codes) {
            b[k++] = {codes, n / 2, 16, true};
            b[k++] = {scales, n / 16, 1, true};
        }
        if (token_scales)
            b[k++] = {token_scales, 4 * rows, 4, true};
        const int st = check_bufs(b, k);
        if (st != MXQ_OK)
            return st;
        return launched(mxq::launch_nvfp4_qdq(x, rows, cols, codes, scales, token_scales, out,
                                              (hipStream_t)stream));
    }
    if (cols > MAX_MXFP8_COLS || !mxfp8_grid_ok((rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0)
        return MXQ_ERR_SHAPE;
    if (codes) {
        b[k++] = {codes, n, 16, true};
        b[k++] = {scales, n / 32, 1, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_row_qdq(x, rows, cols, codes, scales, out,
                                              (hipStream_t)stream));
}

int mxq_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                   const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                   void *c, void *stream)
{
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_ARG;
    if (!a || !a_scales || !b || !b_scales || !c)
        return MXQ_ERR_NULL;
    if (!size_ok(M, K) || !size_ok(N, K) || !size_ok(M, 4 * N))   // C up to 4 bytes
        return MXQ_ERR_SIZE;
    if (K % 128 != 0)
        return MXQ_ERR_SHAPE;
    if (K > MAX_GEMM_K || ((M + 255) / 256) * ((N + 255) / 256) > mxq::MAX_GEMM_TILES)
        return MXQ_ERR_SIZE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    const Buf bb[5] = {{a, M * K, 16, false},
                       {a_scales, M * (K / 32), 4, false},
                       {b, N * K, 16, false},
                       {b_scales, N * (K / 32), 4, false},
                       {c, esz * M * N, esz, true}};
    const int st = check_bufs(bb, 5);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_gemm(a, a_scales, b, b_scales, M, N, K,
                                           out_dtype == MXQ_OUT_BF16, c, (hipStream_t)stream));
}

int mxq_mxfp8_grouped_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                           const uint8_t *b_scales, const int64_t *seg_offsets, int64_t n_groups,
                           int64_t total_rows, int64_t N, int64_t K, int out_dtype, void *c,
                           void *stream)
{
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_ARG;
    if (!a || !a_scales || !b || !b_scales || !seg_offsets || !c)
        return MXQ_ERR_NULL;
    if (!size_ok(total_rows, K) || !size_ok(N, K) || !size_ok(total_rows, 4 * N) || n_groups < 1 ||
        !size_ok(n_groups, N * K) || n_groups > MAX_ELEMS / 8 - 1)
        return MXQ_ERR_SIZE;
    if (K % 128 != 0)
        return MXQ_ERR_SHAPE;
    if (K > MAX_GEMM_K || total_rows > MAX_ELEMS / 4 - 255 ||
        mxq::grouped_gemm_mtiles(total_rows, n_groups) > mxq::MAX_GEMM_TILES ||
        mxq::grouped_gemm_mtiles(total_rows, n_groups) * ((N + 255) / 256) > mxq::MAX_GEMM_TILES)
        return MXQ_ERR_SIZE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    const Buf bb[6] = {{a, total_rows * K, 16, false},
                       {a_scales, total_rows * (K / 32), 4, false},
                       {b, n_groups * N * K, 16, false},
                       {b_scales, n_groups * N * (K / 32), 4, false},
                       {seg_offsets, 8 * (n_groups + 1), 8, false},
                       {c, esz * total_rows * N, esz, true}};
    const int st = check_bufs(bb, 6);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_grouped_gemm(a, a_scales, b, b_scales, seg_offsets,
                                                   n_groups, total_rows, N, K,
                                                   out_dtype == MXQ_OUT_BF16, c,
                                                   (hipStream_t)stream));
}

// Shared by the two grouped transposed entry points; rc == nullptr: the
// columnwise copy alone.
static int grouped_colt(const uint16_t *x, int64_t total_rows, int64_t cols,
                        const int64_t *seg_offsets, int64_t n_groups, uint8_t *rc, uint8_t *rs,
                        uint8_t *codes_t, uint8_t *scales_t, int64_t *block_offsets,
                        void *stream)
{
    if (!size_ok(total_rows, cols) || cols > MAX_MXFP8_COLS || n_groups < 1 ||
        n_groups > ((int64_t)1 << 40) || total_rows > MAX_ELEMS / 4)
        return MXQ_ERR_SIZE;
    const int64_t pitch = mxq::grouped_colt_pitch(total_rows, n_groups);
    if (!size_ok(pitch, cols) || !mxfp8_grid_ok(pitch / 32, cols))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0)
        return MXQ_ERR_SHAPE;
    const int64_t n = total_rows * cols;
    Buf b[7] = {{x, 2 * n, 16, false},
                {seg_offsets, 8 * (n_groups + 1), 8, false},
                {codes_t, pitch * cols, 16, true},
                {scales_t, pitch / 32 * cols, 4, true},
                {block_offsets, 8 * (n_groups + 1), 8, true},
                {rc, n, 16, true},
                {rs, n / 32, 1, true}};
    const int st = check_bufs(b, rc ? 7 : 5);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_grouped_colt(x, total_rows, cols, seg_offsets, n_groups,
                                                   rc, rs, codes_t, scales_t, block_offsets,
                                                   (hipStream_t)stream));
}

int mxq_mxfp8_grouped_colwise_t(const uint16_t *x, int64_t total_rows, int64_t cols,
                                const int64_t *seg_offsets, int64_t n_groups, uint8_t *codes_t,
                                uint8_t *scales_t, int64_t *block_offsets, void *stream)
{
    if (!x || !seg_offsets || !codes_t || !scales_t || !block_offsets)
        return MXQ_ERR_NULL;
    return grouped_colt(x, total_rows, cols, seg_offsets, n_groups, nullptr, nullptr, codes_t,
                        scales_t, block_offsets, stream);
}

int mxq_mxfp8_grouped_quantize_rowcol_t(const uint16_t *x, int64_t total_rows, int64_t cols,
                                        const int64_t *seg_offsets, int64_t n_groups,
                                        uint8_t *row_codes, uint8_t *row_scales,
                                        uint8_t *codes_t, uint8_t *scales_t,
                                        int64_t *block_offsets, void *stream)
{
    if (!x || !seg_offsets || !row_codes || !row_scales || !codes_t || !scales_t ||
        !block_offsets)
        return MXQ_ERR_NULL;
    return grouped_colt(x, total_rows, cols, seg_offsets, n_groups, row_codes, row_scales,
                        codes_t, scales_t, block_offsets, stream);
}

int mxq_mxfp8_grouped_wgrad(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                            const uint8_t *b_scales, const int64_t *block_offsets,
                            int64_t n_groups, int64_t M, int64_t N, int64_t pitch, int out_dtype,
                            void *c, void *stream)
{
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_ARG;
    if (!a || !a_scales || !b || !b_scales || !block_offsets || !c)
        return MXQ_ERR_NULL;
    if (!size_ok(M, pitch) || !size_ok(N, pitch) || !size_ok(M, 4 * N) || n_groups < 1 ||
        !size_ok(n_groups, 4 * M * N) || n_groups > MAX_ELEMS / 8 - 1)
        return MXQ_ERR_SIZE;
    if (pitch % 128 != 0)
        return MXQ_ERR_SHAPE;
    if (pitch > MAX_GEMM_K ||
        n_groups * ((M + 255) / 256) * ((N + 255) / 256) > mxq::MAX_GEMM_TILES)
        return MXQ_ERR_SIZE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    const Buf bb[6] = {{a, M * pitch, 16, false},
                       {a_scales, M * (pitch / 32), 4, false},
                       {b, N * pitch, 16, false},
                       {b_scales, N * (pitch / 32), 4, false},
                       {block_offsets, 8 * (n_groups + 1), 8, false},
                       {c, esz * n_groups * M * N, esz, true}};
    const int st = check_bufs(bb, 6);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_mxfp8_grouped_wgrad(a, a_scales, b, b_scales, block_offsets,
                                                    n_groups, M, N, pitch,
                                                    out_dtype == MXQ_OUT_BF16, c,
                                                    (hipStream_t)stream));
}

int mxq_nvfp4_grouped_gemm(const uint8_t *a, const uint8_t *a_block_scales, const float *a_scales,
                           const uint8_t *b, const uint8_t *b_block_scales, const float *b_scales,
                           const int64_t *seg_offsets, int64_t n_groups, int64_t total_rows,
                           int64_t N, int64_t K, int out_dtype, void *c, void *stream)
{
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_ARG;
    if (!a || !a_block_scales || !a_scales || !b || !b_block_scales || !b_scales ||
        !seg_offsets || !c)
        return MXQ_ERR_NULL;
    if (!size_ok(total_rows, K) || !size_ok(N, K) || !size_ok(total_rows, 4 * N) ||
        n_groups < 1 || !size_ok(n_groups, N * K) || n_groups > MAX_ELEMS / 8 - 1)
        return MXQ_ERR_SIZE;
    if (K % 64 != 0)
        return MXQ_ERR_SHAPE;
    if (K > MAX_GEMM_K || total_rows > MAX_ELEMS / 4 - 255 ||
        mxq::grouped_gemm_mtiles(total_rows, n_groups) > mxq::MAX_GEMM_TILES ||
        mxq::grouped_gemm_mtiles(total_rows, n_groups) * ((N + 255) / 256) > mxq::MAX_GEMM_TILES)
        return MXQ_ERR_SIZE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    const Buf bb[8] = {{a, total_rows * (K / 2), 16, false},
                       {a_block_scales, total_rows * (K / 16), 4, false},
                       {a_scales, 4 * total_rows, 4, false},
                       {b, n_groups * N * (K / 2), 16, false},
                       {b_block_scales, n_groups * N * (K / 16), 4, false},
                       {b_scales, 4 * n_groups, 4, false},
                       {seg_offsets, 8 * (n_groups + 1), 8, false},
                       {c, esz * total_rows * N, esz, true}};
    const int st = check_bufs(bb, 8);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_grouped_gemm(a, a_block_scales, a_scales, b,
                                                   b_block_scales, b_scales, seg_offsets,
                                                   n_groups, total_rows, N, K,
                                                   out_dtype == MXQ_OUT_BF16, c,
                                                   (hipStream_t)stream));
}

int mxq_nvfp4_gemm(const uint8_t *a, const uint8_t *a_block_scales, const float *a_scales,
                   int64_t rows_per_a_scale, const uint8_t *b, const uint8_t *b_block_scales,
                   const float *b_scales, int64_t rows_per_b_scale, int64_t M, int64_t N,
                   int64_t K, int out_dtype, void *c, void *stream)
{
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_ARG;
    if (!a || !a_block_scales || !a_scales || !b || !b_block_scales || !b_scales || !c)
        return MXQ_ERR_NULL;
    if (!size_ok(M, K) || !size_ok(N, K) || !size_ok(M, 4 * N) || rows_per_a_scale < 1 ||
        rows_per_b_scale < 1)
        return MXQ_ERR_SIZE;
    if (K % 64 != 0)
        return MXQ_ERR_SHAPE;
    if (K > MAX_GEMM_K || ((M + 255) / 256) * ((N + 255) / 256) > mxq::MAX_GEMM_TILES)
        return MXQ_ERR_SIZE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    const Buf bb[7] = {{a, M * K / 2, 16, false},
                       {a_block_scales, M * (K / 16), 4, false},
                       {a_scales, 4 * ((M + rows_per_a_scale - 1) / rows_per_a_scale), 4, false},
                       {b, N * K / 2, 16, false},
                       {b_block_scales, N * (K / 16), 4, false},
                       {b_scales, 4 * ((N + rows_per_b_scale - 1) / rows_per_b_scale), 4, false},
                       {c, esz * M * N, esz, true}};
    const int st = check_bufs(bb, 7);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_nvfp4_gemm(a, a_block_scales, a_scales, rows_per_a_scale, b,
                                           b_block_scales, b_scales, rows_per_b_scale, M, N, K,
                                           out_dtype == MXQ_OUT_BF16, c, (hipStream_t)stream));
}

int mxq_grouped_quantize(int fmt, const uint16_t *x, int64_t total_rows, int64_t cols,
                         const int64_t *seg_offsets, int64_t n_groups, const mxq_grouped_out *out,
                         void *stream)
{
    if (fmt != MXQ_FMT_MXFP8_ROWCOL && fmt != MXQ_FMT_NVFP4)
        return MXQ_ERR_ARG;
    if (!x || !seg_offsets || !out)
        return MXQ_ERR_NULL;
    if (!size_ok(total_rows, cols) || n_groups < 1 || n_groups > MAX_ELEMS / 8)
        return MXQ_ERR_SIZE;
    const int64_t n = total_rows * cols;
    if (fmt == MXQ_FMT_NVFP4) {
        if (!out->codes || !out->block_scales || !out->token_scales)
            return MXQ_ERR_NULL;
        if (total_rows > MAX_GRID_ROWS)
            return MXQ_ERR_SIZE;
        if (cols % 16 != 0)
            return MXQ_ERR_SHAPE;
        const Buf b[5] = {{x, 2 * n, 16, false},
                          {seg_offsets, 8 * (n_groups + 1), 8, false},
                          {out->codes, n / 2, 16, true},
                          {out->block_scales, n / 16, 1, true},
                          {out->token_scales, 4 * total_rows, 4, true}};
        const int st = check_bufs(b, 5);
        if (st != MXQ_OK)
            return st;
        // Per-token outputs do not depend on the segments.
        return launched(mxq::launch_nvfp4_per_token(x, total_rows, cols, out->codes,
                                                    out->block_scales, out->token_scales,
                                                    (hipStream_t)stream));
    }
    uint8_t *rc = out->row_codes, *rs = out->row_scales, *cc = out->col_codes,
            *cs = out->col_scales;
    int64_t *P = out->col_scale_offsets;
    if ((rc == nullptr) != (rs == nullptr) || (cc == nullptr) != (cs == nullptr) ||
        (cc != nullptr) != (P != nullptr) || (!rc && !cc))
        return MXQ_ERR_OFFSETS;
    if (cols % 32 != 0)
        return MXQ_ERR_SHAPE;
    if (cols > MAX_MXFP8_COLS)
        return MXQ_ERR_SIZE;
    const int64_t scale_rows = total_rows / 32 + n_groups;
    if (scale_rows > MAX_ELEMS / cols ||
        !mxfp8_grid_ok(cc ? scale_rows : (total_rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    Buf b[7];
    int k = 0;
    b[k++] = {x, 2 * n, 16, false};
    b[k++] = {seg_offsets, 8 * (n_groups + 1), 8, false};
    if (rc) {
        b[k++] = {rc, n, 16, true};
        b[k++] = {rs, n / 32, 1, true};
    }
    if (cc) {
        b[k++] = {cc, n, 16, true};
        b[k++] = {cs, scale_rows * cols, 8, true};
        b[k++] = {P, 8 * (n_groups + 1), 8, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    if (!cc) {
        // Rowwise only: identical to the dense call over all rows.
        return launched(mxq::launch_mxfp8_dense(x, total_rows, cols, rc, rs, nullptr, nullptr,
                                                nullptr, 0, (hipStream_t)stream));
    }
    return launched(mxq::launch_mxfp8_grouped(x, total_rows, cols, seg_offsets, n_groups, rc, rs,
                                              cc, cs, P, nullptr, 0, (hipStream_t)stream));
}

int mxq_grouped_quantize_dispatch(int fmt, const uint16_t *x, int64_t n_tokens, int64_t cols,
                                  int64_t top_k, const int64_t *token_rows,
                                  const int64_t *row_tokens, int64_t total_rows,
                                  const int64_t *seg_offsets, int64_t n_groups,
                                  const mxq_grouped_out *out, void *stream)
{
    if (fmt != MXQ_FMT_MXFP8_ROWCOL && fmt != MXQ_FMT_NVFP4)
        return MXQ_ERR_ARG;
    if (!x || !out)
        return MXQ_ERR_NULL;
    if (!size_ok(n_tokens, cols) || !size_ok(total_rows, cols))
        return MXQ_ERR_SIZE;
    const int64_t nx = n_tokens * cols, n = total_rows * cols;
    if (fmt == MXQ_FMT_NVFP4) {
        if (!token_rows || !out->codes || !out->block_scales || !out->token_scales)
            return MXQ_ERR_NULL;
        if (top_k < 1 || !size_ok(n_tokens, top_k) || n_tokens > MAX_GRID_ROWS)
            return MXQ_ERR_SIZE;
        if (cols % 16 != 0)
            return MXQ_ERR_SHAPE;
        const Buf b[5] = {{x, 2 * nx, 16, false},
                          {token_rows, 8 * n_tokens * top_k, 8, false},
                          {out->codes, n / 2, 16, true},
                          {out->block_scales, n / 16, 1, true},
                          {out->token_scales, 4 * total_rows, 4, true}};
        const int st = check_bufs(b, 5);
        if (st != MXQ_OK)
            return st;
        return launched(mxq::launch_nvfp4_dispatch(x, n_tokens, cols, token_rows, top_k,
                                                   total_rows, out->codes, out->block_scales,
                                                   out->token_scales, (hipStream_t)stream));
    }
    if (!row_tokens)
        return MXQ_ERR_NULL;
    uint8_t *rc = out->row_codes, *rs = out->row_scales, *cc = out->col_codes,
            *cs = out->col_scales;
    int64_t *P = out->col_scale_offsets;
    if ((rc == nullptr) != (rs == nullptr) || (cc == nullptr) != (cs == nullptr) ||
        (cc != nullptr) != (P != nullptr) || (!rc && !cc))
        return MXQ_ERR_OFFSETS;
    if (cc && !seg_offsets)
        return MXQ_ERR_NULL;
    if (cc && (n_groups < 1 || n_groups > MAX_ELEMS / 8))
        return MXQ_ERR_SIZE;
    if (cols % 32 != 0)
        return MXQ_ERR_SHAPE;
    if (cols > MAX_MXFP8_COLS)
        return MXQ_ERR_SIZE;
    const int64_t scale_rows = total_rows / 32 + (cc ? n_groups : 0);
    if (scale_rows > MAX_ELEMS / cols ||
        !mxfp8_grid_ok(cc ? scale_rows : (total_rows + 31) / 32, cols))
        return MXQ_ERR_SIZE;
    Buf b[8];
    int k = 0;
    b[k++] = {x, 2 * nx, 16, false};
    b[k++] = {row_tokens, 8 * total_rows, 8, false};
    if (rc) {
        b[k++] = {rc, n, 16, true};
        b[k++] = {rs, n / 32, 1, true};
    }
    if (cc) {
        b[k++] = {seg_offsets, 8 * (n_groups + 1), 8, false};
        b[k++] = {cc, n, 16, true};
        b[k++] = {cs, scale_rows * cols, 8, true};
        b[k++] = {P, 8 * (n_groups + 1), 8, true};
    }
    const int st = check_bufs(b, k);
    if (st != MXQ_OK)
        return st;
    if (!cc)
        return launched(mxq::launch_mxfp8_dense(x, total_rows, cols, rc, rs, nullptr, nullptr,
                                                row_tokens, n_tokens, (hipStream_t)stream));
    return launched(mxq::launch_mxfp8_grouped(x, total_rows, cols, seg_offsets, n_groups, rc, rs,
                                              cc, cs, P, row_tokens, n_tokens,
                                              (hipStream_t)stream));
}

int mxq_copy_floor(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                   void *stream)
{
    if (!src || !dst)
        return MXQ_ERR_NULL;
    if (src_bytes <= 0 || dst_bytes <= 0 || src_bytes > MAX_COPY_FLOOR_BYTES ||
        dst_bytes > MAX_COPY_FLOOR_BYTES)
        return MXQ_ERR_SIZE;
    if (src_bytes % 16 != 0 || dst_bytes % 16 != 0)
        return MXQ_ERR_SHAPE;
    const Buf b[2] = {{src, src_bytes, 16, false}, {dst, dst_bytes, 16, true}};
    const int st = check_bufs(b, 2);
    if (st != MXQ_OK)
        return st;
    return launched(mxq::launch_copy_floor(src, src_bytes, dst, dst_bytes, (hipStream_t)stream));
}

}  // extern "C"
