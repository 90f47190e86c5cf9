// mxq_mxfp8.hip -- MXFP8 rowwise 1x32 and columnwise 32x1 copies from one
// read of X (the MXFP8 format and MXFP8 recipe paragraphs of the page
// "Miles: end-to-end MXFP8 and per-token NVFP4 RL on Blackwell").
//
// Tiling.  A wavefront owns a tile of 32 rows x 64 columns (4 KB of BF16).
// Lane l holds column group g = l & 7 (8 consecutive columns, one 16-byte
// load per row) of rows 4 * (l >> 3) .. +3, so every load instruction reads
// eight 128-byte row segments.  Both reductions stay inside the wavefront:
//   rowwise 1x32 block = 4 lanes (g & 3): in-lane max over 8 values, then two
//     DPP exchanges (lane ^ 1, lane ^ 2);
//   columnwise 32x1 block = 8 lanes (l >> 3): in-lane max over 4 rows (packed
//     16-bit max), then lane ^ 8 (DPP row_ror:8), ^ 16 and ^ 32 (gfx950
//     permlane swaps).
// No LDS and no barrier.  Magnitudes are compared as integers (|x| =
// bits & 0x7FFF orders like the value).  Rowwise codes come from one
// v_cvt_scalef32_pk_fp8_bf16 per pair of elements; columnwise codes pair
// rows r and r+1 of one column (which share a scale), convert, and are
// regrouped into row order with byte permutes.
//
// Grouped variant: tiles are 32-row blocks of ragged segments; a segment's
// last tile may be short (missing rows read as 0, are not written), which
// gives the amax over existing rows.  The tile -> (segment, block) map is a
// binary search in the prefix array P that a one-workgroup kernel writes
// first.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int TILE_ROWS = 32;
constexpr int WAVE_COLS = 64;
constexpr int WAVES_PER_WG = 4;
constexpr int WG_COLS = WAVE_COLS * WAVES_PER_WG;   // 256 columns per workgroup

// Byte permute: result byte i = selected byte of {hi:lo}, selector byte i in
// 0..7 (0-3 from lo, 4-7 from hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

struct TileRows {
    int64_t row0;        // first row of the tile
    int nrows;           // rows present (1..32)
    int64_t scale_row;   // row of col_scales for this tile
};

template <bool ROW, bool COL>
__device__ __forceinline__ void mxfp8_tile(const uint16_t *__restrict__ x, int64_t cols,
                                           TileRows t, int64_t col_base,
                                           uint8_t *__restrict__ row_codes,
                                           uint8_t *__restrict__ row_scales,
                                           uint8_t *__restrict__ col_codes,
                                           uint8_t *__restrict__ col_scales)
{
    const int lane = __lane_id();
    const int g = lane & 7;
    const int rg = lane >> 3;
    const int64_t col0 = col_base + 8 * g;
    const bool col_ok = col0 < cols;     // cols % 32 == 0: a 32-column block is all in or all out
    // Element offset of this lane's first row; row i adds i * cols.
    const int64_t base = (t.row0 + 4 * rg) * cols + col0;
    const int nr = t.nrows - 4 * rg;     // rows of this lane present: r < nr

    uint32_t v[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (col_ok && i < nr) {
            uint4 q = ld_nt16(x + base + i * cols);
            v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
        } else {
            v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0u;
        }
    }

    if constexpr (ROW) {
        const int64_t nb = cols >> 5;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t m = pk_max_u16(pk_max_u16(v[i][0] & 0x7FFF7FFFu, v[i][1] & 0x7FFF7FFFu),
                                    pk_max_u16(v[i][2] & 0x7FFF7FFFu, v[i][3] & 0x7FFF7FFFu));
            uint32_t a = hmax_u16(m);
            a = max(a, dpp<DPP_XOR1>(a));
            a = max(a, dpp<DPP_XOR2>(a));
            const uint32_t b = e8m0_byte(a);
            const uint32_t c01 = mx_e4m3_pair(v[i][0], b) | (mx_e4m3_pair(v[i][1], b) << 16);
            const uint32_t c23 = mx_e4m3_pair(v[i][2], b) | (mx_e4m3_pair(v[i][3], b) << 16);
            if (col_ok && i < nr) {
                st_nt8(row_codes + base + i * cols, c01, c23);
                if ((g & 3) == 0)
                    row_scales[(base >> 5) + i * nb] = (uint8_t)b;
            }
        }
    }

    if constexpr (COL) {
        // Column amax over the 32 rows, two columns per dword.
        uint32_t m[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            m[j] = pk_max_u16(pk_max_u16(v[0][j] & 0x7FFF7FFFu, v[1][j] & 0x7FFF7FFFu),
                              pk_max_u16(v[2][j] & 0x7FFF7FFFu, v[3][j] & 0x7FFF7FFFu));
            m[j] = pk_max_u16(m[j], dpp<DPP_ROR8>(m[j]));
            m[j] = max16_pk_u16(m[j]);
            m[j] = max32_pk_u16(m[j]);
        }
        // Scale bytes: column 2j in the low half, 2j+1 in the high half.
        uint32_t sb[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            sb[j] = e8m0_byte2(m[j]);

        // Codes: pair rows (0,1) and (2,3) of each column, convert with the
        // column's scale, then regroup bytes into row order.
        // P[p][j]: bytes {col 2j: row 2p, row 2p+1 | col 2j+1: row 2p, row 2p+1}.
        uint32_t P[2][4];
#pragma unroll
        for (int p = 0; p < 2; p++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t ra = v[2 * p][j], rb = v[2 * p + 1][j];
                const uint32_t lo_pair = perm(rb, ra, 0x05040100u);   // {ra.lo, rb.lo}: column 2j
                const uint32_t hi_pair = perm(rb, ra, 0x07060302u);   // {ra.hi, rb.hi}: column 2j+1
                P[p][j] = mx_e4m3_pair(lo_pair, sb[j] & 0xFFu) |
                          (mx_e4m3_pair(hi_pair, sb[j] >> 16) << 16);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int p = i >> 1, k = i & 1;       // row 2p + k
            // Row codes for columns 0..3 (from P[p][0], P[p][1]) and 4..7.
            const uint32_t sel = k ? 0x07050301u : 0x06040200u;
            const uint32_t w0 = perm(P[p][1], P[p][0], sel);
            const uint32_t w1 = perm(P[p][3], P[p][2], sel);
            if (col_ok && i < nr)
                st_nt8(col_codes + base + i * cols, w0, w1);
        }
        if (col_ok && rg == 0) {
            const uint32_t s0 = (sb[0] & 0xFFu) | ((sb[0] >> 8) & 0xFF00u) |
                                ((sb[1] & 0xFFu) << 16) | ((sb[1] & 0xFF0000u) << 8);
            const uint32_t s1 = (sb[2] & 0xFFu) | ((sb[2] >> 8) & 0xFF00u) |
                                ((sb[3] & 0xFFu) << 16) | ((sb[3] & 0xFF0000u) << 8);
            *reinterpret_cast<uint2 *>(col_scales + t.scale_row * cols + col0) = make_uint2(s0, s1);
        }
    }
}

// Workgroup w covers column block w % ncb (256 columns) of 32-row tile
// w / ncb, so consecutive workgroups sweep one tile's rows left to right.
// Dense tensor.
template <bool ROW, bool COL>
__global__ void __launch_bounds__(256) mxfp8_dense_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ncb,
    uint8_t *__restrict__ row_codes, uint8_t *__restrict__ row_scales,
    uint8_t *__restrict__ col_codes, uint8_t *__restrict__ col_scales)
{
    const int64_t tile = (int64_t)blockIdx.x / ncb;
    const int64_t cb = (int64_t)blockIdx.x - tile * ncb;
    TileRows t;
    t.row0 = tile * TILE_ROWS;
    const int64_t left = rows - t.row0;
    t.nrows = left < TILE_ROWS ? (int)left : TILE_ROWS;
    t.scale_row = tile;
    const int64_t col_base = cb * WG_COLS + (threadIdx.x >> 6) * WAVE_COLS;
    mxfp8_tile<ROW, COL>(x, cols, t, col_base, row_codes, row_scales, col_codes, col_scales);
}

// Segment e's rows, clamped into [0, total_rows): the offsets are device data
// the host cannot check, so malformed offsets must never move an access out
// of bounds (they give meaningless bytes instead).
__device__ __forceinline__ void segment_rows(const int64_t *__restrict__ off, int64_t e,
                                             int64_t total_rows, int64_t *lo, int64_t *hi)
{
    int64_t a = off[e], b = off[e + 1];
    a = a < 0 ? 0 : (a > total_rows ? total_rows : a);
    b = b < a ? a : (b > total_rows ? total_rows : b);
    *lo = a;
    *hi = b;
}

// P[e] = sum_{f<e} ceil(n_f / 32), written to P[0..G].  One workgroup;
// sequential over chunks of 256 segments with a block scan.
__global__ void __launch_bounds__(256) grouped_prefix_kernel(const int64_t *__restrict__ off,
                                                              int64_t n_groups, int64_t total_rows,
                                                              int64_t *__restrict__ P)
{
    __shared__ int64_t part[256];
    int64_t carry = 0;
    for (int64_t base = 0; base < n_groups; base += 256) {
        const int64_t e = base + threadIdx.x;
        int64_t n = 0;
        if (e < n_groups) {
            int64_t lo, hi;
            segment_rows(off, e, total_rows, &lo, &hi);
            n = (hi - lo + 31) >> 5;
        }
        part[threadIdx.x] = n;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int64_t add = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
            __syncthreads();
            part[threadIdx.x] += add;
            __syncthreads();
        }
        if (e < n_groups)
            P[e] = carry + part[threadIdx.x] - n;   // exclusive
        const int64_t total = part[255];
        __syncthreads();
        carry += total;
    }
    if (threadIdx.x == 0)
        P[n_groups] = carry;
}

// Grouped: the grid enumerates max_tiles = total_rows/32 + n_groups tiles
// (the capacity of col_scales); tiles at or beyond P[G] exit.
template <bool ROW, bool COL>
__global__ void __launch_bounds__(256) mxfp8_grouped_kernel(
    const uint16_t *__restrict__ x, int64_t total_rows, int64_t cols, int64_t ncb,
    const int64_t *__restrict__ off, int64_t n_groups, const int64_t *__restrict__ P,
    uint8_t *__restrict__ row_codes, uint8_t *__restrict__ row_scales,
    uint8_t *__restrict__ col_codes, uint8_t *__restrict__ col_scales)
{
    const int64_t tile = (int64_t)blockIdx.x / ncb;
    const int64_t cb = (int64_t)blockIdx.x - tile * ncb;
    if (tile >= P[n_groups])
        return;
    // The last e with P[e] <= tile; then P[e] <= tile < P[e+1], so segment e
    // is not empty.
    int64_t lo = 0, hi = n_groups - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (P[mid] <= tile)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int64_t e = lo;
    int64_t s_lo, s_hi;
    segment_rows(off, e, total_rows, &s_lo, &s_hi);
    TileRows t;
    t.row0 = s_lo + (tile - P[e]) * TILE_ROWS;
    const int64_t left = s_hi - t.row0;
    t.nrows = left <= 0 ? 0 : (left < TILE_ROWS ? (int)left : TILE_ROWS);
    t.scale_row = tile;
    const int64_t col_base = cb * WG_COLS + (threadIdx.x >> 6) * WAVE_COLS;
    mxfp8_tile<ROW, COL>(x, cols, t, col_base, row_codes, row_scales, col_codes, col_scales);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_mxfp8_dense(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *rc,
                              uint8_t *rs, uint8_t *cc, uint8_t *cs, hipStream_t stream)
{
    const int64_t ncb = (cols + WG_COLS - 1) / WG_COLS;
    const int64_t tiles = (rows + TILE_ROWS - 1) / TILE_ROWS;
    const dim3 grid((unsigned)(ncb * tiles));
    const dim3 block(256);
    if (rc && cc)
        hipLaunchKernelGGL((mxfp8_dense_kernel<true, true>), grid, block, 0, stream, x, rows, cols,
                           ncb, rc, rs, cc, cs);
    else if (rc)
        hipLaunchKernelGGL((mxfp8_dense_kernel<true, false>), grid, block, 0, stream, x, rows, cols,
                           ncb, rc, rs, cc, cs);
    else
        hipLaunchKernelGGL((mxfp8_dense_kernel<false, true>), grid, block, 0, stream, x, rows, cols,
                           ncb, rc, rs, cc, cs);
    return hipGetLastError();
}

hipError_t launch_mxfp8_grouped(const uint16_t *x, int64_t total_rows, int64_t cols,
                                const int64_t *off, int64_t n_groups, uint8_t *rc, uint8_t *rs,
                                uint8_t *cc, uint8_t *cs, int64_t *P, hipStream_t stream)
{
    hipLaunchKernelGGL(grouped_prefix_kernel, dim3(1), dim3(256), 0, stream, off, n_groups,
                       total_rows, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t max_tiles = total_rows / TILE_ROWS + n_groups;
    const int64_t ncb = (cols + WG_COLS - 1) / WG_COLS;
    const dim3 grid((unsigned)(ncb * max_tiles));
    if (rc && cc)
        hipLaunchKernelGGL((mxfp8_grouped_kernel<true, true>), grid, dim3(256), 0, stream, x,
                           total_rows, cols, ncb, off, n_groups, P, rc, rs, cc, cs);
    else if (cc)
        hipLaunchKernelGGL((mxfp8_grouped_kernel<false, true>), grid, dim3(256), 0, stream, x,
                           total_rows, cols, ncb, off, n_groups, P, rc, rs, cc, cs);
    else
        hipLaunchKernelGGL((mxfp8_grouped_kernel<true, false>), grid, dim3(256), 0, stream, x,
                           total_rows, cols, ncb, off, n_groups, P, rc, rs, cc, cs);
    return hipGetLastError();
}

}  // namespace mxq
