// mxq_mxfp8.hip -- MXFP8 rowwise 1x32 and columnwise 32x1 copies from one
// read of X (the MXFP8 format and MXFP8 recipe paragraphs of the page
// "Miles: end-to-end MXFP8 and per-token NVFP4 RL on Blackwell").
//
// Tiling.  A wavefront tile is 32 rows x 128 columns (8 KB of BF16).  Lane l
// holds column group g = l & 15 (8 consecutive columns, one 16-byte load per
// row) of the 8 rows 8 * (l >> 4) .. +7, so each load or code store
// instruction covers four 256-byte (or 128-byte) row segments.  Both
// reductions stay inside the wavefront:
//   rowwise 1x32 block = the 4 lanes of a quad: in-lane max over 8 values,
//     then DPP exchanges with lane ^ 1 and lane ^ 2;
//   columnwise 32x1 block = the 4 lanes l, l^16, l^32, l^48: packed 16-bit
//     max over the lane's 8 rows, then the gfx950 permlane16/permlane32 swaps.
// No LDS, no barrier.  Magnitudes are compared as integers (|x| = bits &
// 0x7FFF orders like the value).
//
// Scale.  For a block amax a (15-bit magnitude bits = 128 E + m), the
// smallest unclipped exponent byte is max(0, E - 8 + [m > 96]) =
// max(0, a - 993) >> 7 (993 = 8 * 128 - 31); shifted left by 16 instead it is
// the byte in an f32 exponent field, which is the scale operand of the
// conversions (they use only the exponent field).
//
// Codes.  Rowwise: one v_cvt_scalef32_pk_fp8_bf16 per element pair.
// Columnwise: rows 2p and 2p+1 of one column share a scale, so they are
// paired with a byte permute, converted, and regrouped into row order.
//
// Schedule.  One tile per wavefront, every tile in one launch: wavefront w
// converts 128-column strip w % nct of tile w / nct, so the four wavefronts
// of a workgroup cover 512 consecutive columns of one 32-row band (small
// dense launches first permute workgroups so that a band's workgroups share
// an XCD: band_order).  Each
// tile's base addresses are wave-uniform (scalar registers) and lanes add
// 32-bit offsets (cols < 2^27).  For ragged segments (grouped call) tile T
// lies in the segment e with P[e] <= T < P[e+1] (binary search).
#include "mxq_dequant.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int TILE_ROWS = 32;
constexpr int TILE_COLS = 128;                  // per wavefront
static_assert(TILE_ROWS == 32 && TILE_COLS == 128, "mxfp8_tiles counts 32 x 128 tiles");

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Saturating subtraction (v_sub_u32 / v_pk_sub_u16 with clamp).
__device__ __forceinline__ uint32_t subsat(uint32_t a, uint32_t b)
{
    return __builtin_elementwise_sub_sat(a, b);
}
__device__ __forceinline__ uint32_t pk_subsat(uint32_t a, uint32_t b)
{
    ushort2_t r = __builtin_elementwise_sub_sat(__builtin_bit_cast(ushort2_t, a),
                                                __builtin_bit_cast(ushort2_t, b));
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_shr7(uint32_t a)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(ushort2_t, a) >> (unsigned short)7);
}

// Two BF16 (packed) over 2^(b-127) -> two E4M3 codes written into the low
// (HI = false) or high (HI = true) 16 bits of `old`.  `scale` carries b in
// its exponent field.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t old, uint32_t bf16pair, uint32_t scale)
{
    short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
        __builtin_bit_cast(short2_t, old), __builtin_bit_cast(bf16x2_t, bf16pair), u2f(scale), HI);
    return __builtin_bit_cast(uint32_t, r);
}

struct Tile {
    int64_t row0;      // first row
    int nrows;         // rows present, 0..32
    int64_t srow;      // row of col_scales
};

// Partial tiles (rows past the segment end, columns past cols) load from a
// clamped address and select zero: no divergent loads, which would make the
// compiler shuffle the whole tile between registers.  xt: the tile's first
// element (row0, strip column 0); lane offsets are 32-bit.
template <bool FULL>
__device__ __forceinline__ void load_tile(uint32_t (&v)[8][4], const uint16_t *__restrict__ xt,
                                          uint32_t cols, uint32_t c8, int nrows, int rg,
                                          bool col_ok)
{
    if constexpr (FULL) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint4 q = ld_nt16(xt + ((uint32_t)(8 * rg + i) * cols + c8));
            v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
        }
    } else {
        // A tile with no rows (nrows 0) reads its first row, which lies in
        // the tensor, and keeps nothing.
        const uint32_t last = nrows > 0 ? (uint32_t)(nrows - 1) : 0u;
        const uint32_t c = col_ok ? c8 : 0u;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int r = 8 * rg + i;
            const bool keep = col_ok && r < nrows;
            const uint4 q = ld_nt16(xt + ((keep ? (uint32_t)r : last) * cols + c));
            v[i][0] = keep ? q.x : 0u; v[i][1] = keep ? q.y : 0u;
            v[i][2] = keep ? q.z : 0u; v[i][3] = keep ? q.w : 0u;
        }
    }
}

// Dispatch: row r of the tile is token row_tokens[row0 + r] of x, clamped
// into [0, n_tokens) (the map is device data the host cannot check: a bad
// entry gives meaningless bytes, never an out-of-bounds read).  Rows past
// nrows read the tile's last row and select zero, as in load_tile.  Each
// token is read once per expert it is routed to, so these loads keep the
// default cache policy (measured 392 -> 320 us on 32768 tokens routed top-8
// into 262144 x 2048, against streaming loads).
template <bool FULL>
__device__ __forceinline__ void load_tile_gather(uint32_t (&v)[8][4],
                                                 const uint16_t *__restrict__ x,
                                                 const int64_t *__restrict__ row_tokens,
                                                 int64_t n_tokens, int64_t cols, int64_t row0,
                                                 int64_t col, int nrows, int rg, bool col_ok)
{
    const int last = nrows > 0 ? nrows - 1 : 0;
    const int64_t c = FULL || col_ok ? col : 0;
    int64_t tok[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = 8 * rg + i;
        const bool keep = FULL || (col_ok && r < nrows);
        int64_t t = row_tokens[row0 + (keep ? r : last)];
        tok[i] = t < 0 ? 0 : (t >= n_tokens ? n_tokens - 1 : t);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = 8 * rg + i;
        const bool keep = FULL || (col_ok && r < nrows);
        const uint4 q = ld16(x + tok[i] * cols + c);
        v[i][0] = keep ? q.x : 0u; v[i][1] = keep ? q.y : 0u;
        v[i][2] = keep ? q.z : 0u; v[i][3] = keep ? q.w : 0u;
    }
}

// Tile outputs: wave-uniform bases at (row0, strip column 0).
struct TileOut {
    uint8_t *rc, *rs, *cc, *cs;     // row codes, row scales, col codes, col scales
    uint16_t *dq;                   // dequantized rowwise copy (BF16), DQ kernels
    uint32_t ld_t, lds_t;           // transposed columnwise copy: row pitch of codes, scales
};

// Eight BF16 of one row's 8 rowwise codes (w0: columns 0..3, w1: 4..7) under
// the block's scale (byte << 23), exact (mxq_dequant.h).
__device__ __forceinline__ u32x4_t row_dq(uint32_t w0, uint32_t w1, uint32_t scale)
{
    u32x4_t o;
    const uint32_t byte = scale >> 23;
    if (byte < 247) {
        o[0] = mx_pair<false>(w0, scale);
        o[1] = mx_pair<true>(w0, scale);
        o[2] = mx_pair<false>(w1, scale);
        o[3] = mx_pair<true>(w1, scale);
    } else {
        o[0] = pack2(mx_deq1_exact(w0 & 0xFF, byte), mx_deq1_exact((w0 >> 8) & 0xFF, byte));
        o[1] = pack2(mx_deq1_exact((w0 >> 16) & 0xFF, byte), mx_deq1_exact(w0 >> 24, byte));
        o[2] = pack2(mx_deq1_exact(w1 & 0xFF, byte), mx_deq1_exact((w1 >> 8) & 0xFF, byte));
        o[3] = pack2(mx_deq1_exact((w1 >> 16) & 0xFF, byte), mx_deq1_exact(w1 >> 24, byte));
    }
    return o;
}

// DQ: also write the BF16 dequantization of the rowwise codes (o.dq); ROW
// may then be false (codes and scales computed but not stored).
// OCP: the OCP MX scale rule instead (a comparison variant): byte =
// max(0, E - 8) = max(0, a - 1024) >> 7, i.e. floor(log2 amax) - 8, under
// which x / 2^e can exceed 448.  The conversion instruction does not
// saturate (it gives NaN from 464 up), so magnitudes are first clamped to
// 448 * 2^e, whose BF16 bits are ((byte + 8) << 7) | 0x60; the nearest E4M3
// of anything at or above that is 448.
// COLT: the columnwise copy transposed, staged in LDS (the transposed
// layouts): o.cc / o.cs point at the wavefront's first row in LDS arrays of
// [column][rows] codes and [column][blocks] scale bytes with column pitches
// ld_t and lds_t; each lane writes, per column, its 8 rows as two 4-byte
// words (ld_t is a multiple of 4).
template <bool ROW, bool COL, bool FULL, bool DQ = false, bool OCP = false, bool COLT = false,
          bool LATE = false>
__device__ __forceinline__ void convert_tile(const uint32_t (&v)[8][4], uint32_t cols,
                                             uint32_t c8, int nrows, int g, int rg, bool col_ok,
                                             const TileOut &o)
{
    const int nr = nrows - 8 * rg;
    uint32_t a[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            a[i][j] = v[i][j] & 0x7FFF7FFFu;

    uint32_t rw0[8], rw1[8], rsb[8];        // LATE: rowwise codes and scale bytes, stored last
    if constexpr (ROW || DQ) {
        const uint32_t nb = cols >> 5;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t m = pk_max_u16(pk_max_u16(a[i][0], a[i][1]), pk_max_u16(a[i][2], a[i][3]));
            uint32_t am = hmax_u16(m);
            am = max(am, dpp<DPP_XOR1>(am));
            am = max(am, dpp<DPP_XOR2>(am));
            const uint32_t sc = subsat(am, OCP ? 1024u : 993u) & 0xFF80u;   // byte << 7
            const uint32_t scale = sc << 16;                     // byte << 23
            uint32_t x0 = v[i][0], x1 = v[i][1], x2 = v[i][2], x3 = v[i][3];
            if constexpr (OCP) {
                const uint32_t lim = ((sc + 0x400u) | 0x60u) * 0x10001u;
                x0 = (x0 & 0x80008000u) | pk_min_u16(a[i][0], lim);
                x1 = (x1 & 0x80008000u) | pk_min_u16(a[i][1], lim);
                x2 = (x2 & 0x80008000u) | pk_min_u16(a[i][2], lim);
                x3 = (x3 & 0x80008000u) | pk_min_u16(a[i][3], lim);
            }
            const uint32_t w0 = cvt2<true>(cvt2<false>(0u, x0, scale), x1, scale);
            const uint32_t w1 = cvt2<true>(cvt2<false>(0u, x2, scale), x3, scale);
            rw0[i] = w0;
            rw1[i] = w1;
            rsb[i] = sc >> 7;
            if (FULL || (col_ok && i < nr)) {
                const uint32_t r = (uint32_t)(8 * rg + i);
                if constexpr (ROW && !LATE) {
                    st_nt8(o.rc + (r * cols + c8), w0, w1);
                    if ((g & 3) == 0)
                        o.rs[r * nb + (c8 >> 5)] = (uint8_t)(sc >> 7);
                }
                if constexpr (DQ)
                    __builtin_nontemporal_store(row_dq(w0, w1, scale),
                                                reinterpret_cast<u32x4_t *>(o.dq + (r * cols + c8)));
            }
        }
    }

    if constexpr (COL) {
        uint32_t slo[4], shi[4], sb[4], lim[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t m = pk_max_u16(pk_max_u16(pk_max_u16(a[0][j], a[1][j]), pk_max_u16(a[2][j], a[3][j])),
                                    pk_max_u16(pk_max_u16(a[4][j], a[5][j]), pk_max_u16(a[6][j], a[7][j])));
            m = max16_pk_u16(m);
            m = max32_pk_u16(m);
            const uint32_t sc = pk_subsat(m, OCP ? 0x04000400u : 0x03E103E1u) & 0xFF80FF80u;
            slo[j] = sc << 16;                                          // column 2j
            shi[j] = sc & 0xFFFF0000u;                                  // column 2j+1
            sb[j] = pk_shr7(sc);                                        // the two bytes
            if constexpr (OCP)
                lim[j] = (sc + 0x04000400u) | 0x00600060u;              // 448 * 2^e per column
        }
        uint32_t vc[8][4];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                vc[i][j] = OCP ? (v[i][j] & 0x80008000u) | pk_min_u16(a[i][j], lim[j]) : v[i][j];
        // P[p][j] bytes: {col 2j: row 2p, 2p+1 | col 2j+1: row 2p, 2p+1}.
        uint32_t P[4][4];
#pragma unroll
        for (int p = 0; p < 4; p++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t ra = vc[2 * p][j], rb = vc[2 * p + 1][j];
                P[p][j] = cvt2<true>(cvt2<false>(0u, perm(rb, ra, 0x05040100u), slo[j]),
                                     perm(rb, ra, 0x07060302u), shi[j]);
            }
        if constexpr (!COLT) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int p = i >> 1;
                const uint32_t sel = (i & 1) ? 0x07050301u : 0x06040200u;
                const uint32_t w0 = perm(P[p][1], P[p][0], sel);
                const uint32_t w1 = perm(P[p][3], P[p][2], sel);
                if (FULL || (col_ok && i < nr))
                    st_nt8(o.cc + ((uint32_t)(8 * rg + i) * cols + c8), w0, w1);
            }
            if ((FULL || col_ok) && rg == 0) {
                const uint32_t s0 = perm(sb[1], sb[0], 0x06040200u);     // columns 0..3
                const uint32_t s1 = perm(sb[3], sb[2], 0x06040200u);     // columns 4..7
                st_nt8(o.cs + c8, s0, s1);
            }
        } else if (FULL || col_ok) {
            // Column 2j: rows 0..3 are bytes 0, 1 of P[0][j], P[1][j]; rows
            // 4..7 those of P[2][j], P[3][j].  Column 2j+1: bytes 2, 3.
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const uint32_t sel = e ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = perm(P[1][j], P[0][j], sel);
                    const uint32_t hi = perm(P[3][j], P[2][j], sel);
                    const uint32_t c = c8 + 2 * j + e;
                    uint32_t *d = reinterpret_cast<uint32_t *>(o.cc + c * o.ld_t + 8 * rg);
                    d[0] = lo;
                    d[1] = hi;
                    if (rg == 0)
                        o.cs[(size_t)c * o.lds_t] = (uint8_t)(sb[j] >> (16 * e));
                }
            }
        }
    }
    // LATE: stores count in the same counter as loads on this architecture,
    // so rowwise stores issued between the per-row waits make each later
    // wait cover more loads than the row needs; storing the rowwise copy
    // after the last load is consumed lets row i's arithmetic start as soon
    // as load i lands.  Pays where a SIMD holds few wavefronts (small grids:
    // 8192 x 2048 15.0 -> 14.5 us), not on large grids (262144 x 2048
    // grouped: 370 -> 375 us).
    if constexpr (ROW && LATE) {
        const uint32_t nb = cols >> 5;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (FULL || (col_ok && i < nr)) {
                const uint32_t r = (uint32_t)(8 * rg + i);
                st_nt8(o.rc + (r * cols + c8), rw0[i], rw1[i]);
                if ((g & 3) == 0)
                    o.rs[r * nb + (c8 >> 5)] = (uint8_t)rsb[i];
            }
        }
    }
}

struct Geometry {
    const uint16_t *x;
    int64_t rows;          // dense: rows; grouped: total rows
    int64_t cols;
    int64_t nct;           // 128-column strips
    int64_t max_tiles;     // grouped: capacity of col_scales in rows; dense transposed: rows / 32
    const int64_t *off;    // grouped: segment offsets
    const int64_t *P;      // grouped: prefix of ceil(n_e / 32)
    int64_t n_groups;
    const int64_t *row_tokens;  // dispatch: token of each (expert-sorted) row, else nullptr
    int64_t n_tokens;           // dispatch: rows of x
    // Dense launches: band order (band_order), set by the launcher.
    uint32_t bo_k;              // workgroups per 32-row band; 0: launch order
    uint32_t bo_full;           // workgroups in whole groups of 8 bo_k
    Div bo_grp;                 // division by 8 bo_k
};

// Segment e's rows clamped into [0, total_rows): offsets are device data the
// host cannot check, so malformed offsets must never move an access out of
// bounds (they give meaningless bytes instead).
__device__ __forceinline__ void segment_rows(const int64_t *__restrict__ off, int64_t e,
                                             int64_t total_rows, int64_t *lo, int64_t *hi)
{
    int64_t a = off[e], b = off[e + 1];
    a = a < 0 ? 0 : (a > total_rows ? total_rows : a);
    b = b < a ? a : (b > total_rows ? total_rows : b);
    *lo = a;
    *hi = b;
}

// Segment of tile T (grouped): the e with P[e] <= T < P[e + 1], by binary
// search (T is wave-uniform, so the loads are scalar).
__device__ __forceinline__ int64_t tile_segment(const int64_t *__restrict__ P, int64_t n_groups,
                                                int64_t T)
{
    int64_t lo = 0, hi = n_groups - 1;          // P[lo] <= T always (P[0] = 0)
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (P[mid] <= T)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Up to SCAN_MAX_GROUPS segments, a grouped kernel forms the block prefix
// P[0..G] itself instead of a separate one-workgroup launch before it (4.4 us
// plus the launch gap for 128 segments): wavefront 0 of every workgroup
// scans the offsets, 64 segments at a time, into LDS, and workgroup 0 also
// stores P for the caller.  P[e] = sum over f < e of ceil(n_f / 32) rounded
// up to a multiple of pad, each segment clamped as in segment_rows: the same
// values the prefix kernel writes.
constexpr int64_t SCAN_MAX_GROUPS = 256;
__device__ __forceinline__ void wave_block_prefix(const int64_t *__restrict__ off, int64_t G,
                                                  int64_t total_rows, int64_t pad,
                                                  int64_t *__restrict__ Ps,
                                                  int64_t *__restrict__ P_out)
{
    const int lane = (int)lane_id();
    int64_t before = 0;
    for (int64_t base = 0; base < G; base += 64) {
        const int64_t e = base + lane;
        int64_t n = 0;
        if (e < G) {
            int64_t lo, hi;
            segment_rows(off, e, total_rows, &lo, &hi);
            n = (hi - lo + 31) >> 5;
            n = (n + pad - 1) / pad * pad;
        }
        int64_t inc = n;                                // inclusive prefix over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t v = __shfl_up(inc, d);
            if (lane >= d)
                inc += v;
        }
        if (e < G) {
            Ps[e] = before + inc - n;
            if (P_out)
                P_out[e] = before + inc - n;
        }
        before += __shfl(inc, 63);
    }
    if (lane == 0) {
        Ps[G] = before;
        if (P_out)
            P_out[G] = before;
    }
}

// One tile per wavefront: wave w converts strip w % nct of tile w / nct, so
// the four wavefronts of a workgroup cover 512 consecutive columns of one
// 32-row band.  Launched over all tiles at once.
template <bool ROW, bool COL, bool GROUPED, int WPW, bool GATHER, bool DQ, bool OCP = false>
__device__ __forceinline__ void tile_body(const Geometry &G, uint8_t *__restrict__ rc,
                                          uint8_t *__restrict__ rs, uint8_t *__restrict__ cc,
                                          uint8_t *__restrict__ cs, uint16_t *__restrict__ dq,
                                          int64_t wg = -1)
{
    constexpr bool LATE = ROW && COL && !DQ && !OCP && WPW == 4;
    const int lane = (int)lane_id();
    const int g = lane & 15, rg = lane >> 4;
    const int64_t wave = (wg < 0 ? (int64_t)wg_id() : wg) * WPW + wave_in_group();
    const int64_t strip = wave % G.nct, T = wave / G.nct;
    Tile t;
    t.srow = T;
    if constexpr (!GROUPED) {
        if (T * TILE_ROWS >= G.rows)
            return;
        t.row0 = T * TILE_ROWS;
        const int64_t left = G.rows - t.row0;
        t.nrows = left < TILE_ROWS ? (int)left : TILE_ROWS;
    } else {
        int64_t ntiles = G.P[G.n_groups];
        if (ntiles > G.max_tiles)
            ntiles = G.max_tiles;
        if (T >= ntiles)
            return;
        // Dispatch: launch order T visits the tiles transposed, as a
        // G x (ntiles / G) matrix (a bijection on [0, G (ntiles / G))), so
        // tiles at about the same position of every segment run together.
        // Each segment lists its tokens in ascending order, so those tiles
        // read one narrow window of tokens, and a token's copies in several
        // segments are read close together in time: 32768 tokens routed
        // top-8 into 262144 x 2048, 320.8 -> 314.0 us.
        int64_t Tp = T;
        if constexpr (GATHER) {
            const int64_t per = ntiles / G.n_groups;
            if (T < per * G.n_groups)
                Tp = (T % G.n_groups) * per + T / G.n_groups;
        }
        t.srow = Tp;
        const int64_t e = tile_segment(G.P, G.n_groups, Tp);
        int64_t lo, hi;
        segment_rows(G.off, e, G.rows, &lo, &hi);
        t.row0 = lo + (Tp - G.P[e]) * TILE_ROWS;
        const int64_t left = hi - t.row0;
        t.nrows = left <= 0 ? 0 : (left < TILE_ROWS ? (int)left : TILE_ROWS);
    }
    const int64_t tcol = strip * TILE_COLS;              // wave-uniform
    const uint32_t cols = (uint32_t)G.cols, c8 = 8u * (uint32_t)g;
    const bool col_ok = tcol + c8 < G.cols;             // cols % 32 == 0: whole 32-column blocks
    const bool full = tcol + TILE_COLS <= G.cols && t.nrows == TILE_ROWS;
    const int64_t base = t.row0 * G.cols + tcol;
    const uint16_t *xt = G.x + base;
    TileOut o{rc + base, rs + (base >> 5), cc + base, cs + t.srow * G.cols + tcol,
              DQ ? dq + base : nullptr, 0, 0};
    uint32_t v[8][4];
    if (full) {
        if constexpr (GATHER)
            load_tile_gather<true>(v, G.x, G.row_tokens, G.n_tokens, G.cols, t.row0, tcol + c8,
                                   t.nrows, rg, col_ok);
        else
            load_tile<true>(v, xt, cols, c8, t.nrows, rg, col_ok);
        convert_tile<ROW, COL, true, DQ, OCP, false, LATE>(v, cols, c8, t.nrows, g, rg, col_ok, o);
    } else {
        if constexpr (GATHER)
            load_tile_gather<false>(v, G.x, G.row_tokens, G.n_tokens, G.cols, t.row0, tcol + c8,
                                    t.nrows, rg, col_ok);
        else
            load_tile<false>(v, xt, cols, c8, t.nrows, rg, col_ok);
        convert_tile<ROW, COL, false, DQ, OCP, false, LATE>(v, cols, c8, t.nrows, g, rg, col_ok, o);
    }
}

// Band order of dense launches.  Workgroups are dealt round-robin to the 8
// XCDs (workgroup h runs on XCD h % 8), and the k = nct / WPW workgroups of a
// 32-row band, in launch order, would land on k different XCDs.  Workgroup
// h instead takes position L (below), so that each band's k workgroups run on
// one XCD and consecutive bands on consecutive XCDs.  The rowwise scale bytes
// of a row (4 per 128-column strip) and its code segments then meet in one
// L2 and leave it as whole lines, instead of as pieces that each cost HBM a
// separate partial write.  Byte-identical; row+col 8192 x 2048 14.5 -> 14.0
// us, rowwise + BF16 copy 16.4 -> 15.9 us.  Small launches only (below
// LARGE_LAUNCH_WAVES): on large ones the effect followed where the buffers
// lay -- one-pass rowwise + dequant at 262144 x 2048 went 460 -> 440 us in
// one process and 490 -> 510 us in another -- and grouped launches showed no
// change (358-361 us either way).  The dispatch gather keeps its own order.
// L permutes each group of 8 k
// consecutive workgroups among themselves: position j of group q goes to
// 8 k q + k (j % 8) + j / 8.  A last, partial group and bands that straddle
// workgroups (nct % WPW != 0) keep launch order.  The group index is a
// multiply-high by a constant formed on the host: a division per wavefront
// delayed the loads of the small one-step launches.
__device__ __forceinline__ int64_t band_order(int64_t hw, const Geometry &G)
{
    const uint32_t h = (uint32_t)hw, k = G.bo_k;
    if (k == 0 || h >= G.bo_full)
        return hw;
    const uint32_t q0 = udiv(h, G.bo_grp) * 8 * k;   // first workgroup of h's group
    const uint32_t j = h - q0;                       // 0 .. 8 k - 1
    return (int64_t)(q0 + (j & 7) * k + (j >> 3));
}

// SCAN (grouped, G <= SCAN_MAX_GROUPS): the block prefix formed in LDS
// (wave_block_prefix; workgroup 0 stores it to P_out).
template <bool ROW, bool COL, bool GROUPED, int WPW, bool GATHER, bool SCAN = false>
__global__ void __launch_bounds__(64 * WPW) mxfp8_tile_kernel(Geometry G, uint8_t *__restrict__ rc,
                                                         uint8_t *__restrict__ rs,
                                                         uint8_t *__restrict__ cc,
                                                         uint8_t *__restrict__ cs,
                                                         int64_t *__restrict__ P_out)
{
    if constexpr (SCAN) {
        __shared__ int64_t Ps[SCAN_MAX_GROUPS + 1];
        if (wave_in_group() == 0)
            wave_block_prefix(G.off, G.n_groups, G.rows, 1, Ps, wg_id() == 0 ? P_out : nullptr);
        __syncthreads();
        G.P = Ps;
    }
    if constexpr (GATHER) {
        // Dispatch: workgroups are dealt round-robin to the 8 XCDs; position
        // L runs on the XCD that owns the L-range it falls in, so one XCD
        // visits a contiguous window of tile positions and a token's copies
        // in several segments are read by one XCD (311 -> 306.5 us on 32768
        // tokens routed top-8 into 262144 x 2048; the window is larger than
        // one L2, so most repeats still come from the memory-side cache).
        const int64_t total = (int64_t)__builtin_amdgcn_readfirstlane(
            (int)(gridDim.x)), per_xcd = total / 8;           // grid is a multiple of 8
        const int64_t hw = wg_id();
        tile_body<ROW, COL, GROUPED, WPW, GATHER, false>(G, rc, rs, cc, cs, nullptr,
                                                         (hw & 7) * per_xcd + (hw >> 3));
    } else if constexpr (!GROUPED) {
        tile_body<ROW, COL, GROUPED, WPW, GATHER, false>(G, rc, rs, cc, cs, nullptr,
                                                         band_order(wg_id(), G));
    } else {
        tile_body<ROW, COL, GROUPED, WPW, GATHER, false>(G, rc, rs, cc, cs, nullptr);
    }
}

// Rowwise quantize + BF16 dequant of the rowwise copy in one pass; ROW =
// false stores only the dequantized copy.
template <bool ROW, int WPW>
__global__ void __launch_bounds__(64 * WPW) mxfp8_row_qdq_kernel(Geometry G,
                                                            uint8_t *__restrict__ rc,
                                                            uint8_t *__restrict__ rs,
                                                            uint16_t *__restrict__ dq)
{
    tile_body<ROW, false, false, WPW, false, true>(G, rc, rs, nullptr, nullptr, dq,
                                                   band_order(wg_id(), G));
}

// Both copies under the OCP MX scale rule (comparison variant).
template <bool ROW, bool COL, int WPW>
__global__ void __launch_bounds__(64 * WPW) mxfp8_ocp_kernel(Geometry G, uint8_t *__restrict__ rc,
                                                        uint8_t *__restrict__ rs,
                                                        uint8_t *__restrict__ cc,
                                                        uint8_t *__restrict__ cs)
{
    tile_body<ROW, COL, false, WPW, false, false, true>(G, rc, rs, cc, cs, nullptr,
                                                        band_order(wg_id(), G));
}

// Grouped columnwise copy, transposed and padded (the weight-gradient
// operand layout): codes [cols][pitch], scales [cols][pitch / 32]; segment
// e's 32-row blocks, rounded up to a multiple of 4 (128 rows) with zero
// blocks, start at block P[e].  Workgroup (strip, q) converts blocks
// WPW q .. WPW q + WPW - 1 of a 128-column strip, one per wavefront (each
// finds its own segment), stages the codes in LDS as [column][32 WPW rows]
// and writes each column's 32 WPW bytes as whole lines of codes_t.  Written
// straight from the lanes, each column's bytes were 32-byte pieces of four
// lines (1.52 ms on 262144 x 2048, 17 % of the copy floor; staged, 4 waves:
// 330 us, 8 waves: 324 us, 16 waves: 325 us).  The workgroup order (below)
// keeps each XCD on a contiguous range of (q, strip), strips fastest: 302 us.
// Most of what remains over the copy floor (255 us) is the scatter itself:
// the same kernel writing each workgroup's 16 KB to one contiguous block
// took 288 us, while padding the pitch against channel aliasing changed
// nothing.  Padding blocks (no rows) load from row 0, which
// lies in the tensor, and keep nothing: zero codes and scale bytes.
// ROW: the rowwise copy [rows][cols] from the same read (the grouped
// rowwise layout, stored straight from the lanes as the tile kernel does).
// SCAN: the block prefix formed in LDS, as in mxfp8_tile_kernel.
// DENSE: the same staging for one dense tensor (the transposed layout of
// mxq_mxfp8_quantize_rowcol_t): block T is rows 32 T .. 32 T + 31, the codes'
// row pitch is rows and the scales' rows / 32, which need not be a multiple
// of 4, so scale bytes go out as dwords only where aligned and whole.
// Against each lane writing its 8 rows of a column straight to HBM (8-byte
// pieces of lines): 8192 x 2048 29.7 -> 18.0 us, 262144 x 2048 1670 -> 432
// us, byte-identical.
template <int WPW, bool ROW, bool DENSE>
__device__ __forceinline__ void colt_staged_body(const Geometry &G, uint8_t *__restrict__ rc,
                                                 uint8_t *__restrict__ rs,
                                                 uint8_t *__restrict__ cct,
                                                 uint8_t *__restrict__ cst)
{
    constexpr int LP = TILE_ROWS * WPW + 4;          // bytes per staged column (bank spread)
    constexpr int PIECES = 2 * WPW;                   // 16-byte pieces per staged column
    __shared__ __attribute__((aligned(16))) uint8_t sc[TILE_COLS * LP];
    __shared__ __attribute__((aligned(16))) uint8_t ss[TILE_COLS * WPW];
    const int lane = (int)lane_id(), w = (int)wave_in_group();
    const int g = lane & 15, rg = lane >> 4;
    const int64_t ngroups = (G.max_tiles + WPW - 1) / WPW;
    const int64_t total = ngroups * G.nct, per_xcd = (total + 7) / 8;
    // Workgroups are dealt round-robin to the 8 XCDs; position L runs on the
    // XCD that owns the L-range it falls in, strips fastest inside it.  So
    // the small pieces of one line -- a row's scale bytes (4 bytes per
    // strip) and a column's transposed scale bytes (8 bytes per workgroup)
    // -- come from neighbouring workgroups on one XCD and meet in its L2;
    // spread over XCDs, each piece reached HBM as a separate 32-byte write.
    // 262144 x 2048: 465 -> 415 us with the rowwise copy, 320 -> 302 us
    // without, byte-identical.
    const int64_t hw = wg_id();
    const int64_t wg = (hw & 7) * per_xcd + (hw >> 3);
    if (wg >= total)
        return;
    const int64_t strip = wg % G.nct, T0 = WPW * (wg / G.nct);
    int64_t ntiles = DENSE ? G.max_tiles : G.P[G.n_groups];
    if (ntiles > G.max_tiles)
        ntiles = G.max_tiles;
    if (T0 >= ntiles)                      // uniform
        return;
    const int nv = (int)min((int64_t)WPW, ntiles - T0);   // blocks of this group to write
    const int64_t tcol = strip * TILE_COLS;
    const uint32_t cols = (uint32_t)G.cols, c8 = 8u * (uint32_t)g;
    const bool col_ok = tcol + c8 < G.cols;
    if (w < nv) {                          // wave-uniform
        const int64_t T = T0 + w;
        int64_t row0;
        int nrows;
        if constexpr (DENSE) {
            row0 = T * TILE_ROWS;          // rows % 32 == 0: every block is whole
            nrows = TILE_ROWS;
        } else {
            const int64_t e = tile_segment(G.P, G.n_groups, T);
            int64_t lo, hi;
            segment_rows(G.off, e, G.rows, &lo, &hi);
            row0 = lo + (T - G.P[e]) * TILE_ROWS;
            const int64_t left = hi - row0;
            nrows = left <= 0 ? 0 : (left < TILE_ROWS ? (int)left : TILE_ROWS);
        }
        uint32_t v[8][4];
        load_tile<false>(v, G.x + (nrows > 0 ? row0 : 0) * G.cols + tcol, cols, c8, nrows, rg,
                         col_ok);
        const int64_t r0 = nrows > 0 ? row0 : 0;     // no rowwise store when nrows is 0
        const TileOut o{ROW ? rc + r0 * G.cols + tcol : nullptr,
                        ROW ? rs + r0 * (G.cols / 32) + tcol / 32 : nullptr,
                        sc + TILE_ROWS * w, ss + w, nullptr, LP, WPW};
        convert_tile<ROW, true, false, false, false, true, false>(v, cols, c8, nrows, g, rg,
                                                                  col_ok, o);
    }
    __syncthreads();
    const int t = (int)tid();
    const int64_t pitch = G.max_tiles * TILE_ROWS;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int q = t + 64 * WPW * i, c = q / PIECES, piece = q % PIECES;
        if (tcol + c < G.cols && piece < 2 * nv) {
            const uint32_t *s4 = reinterpret_cast<const uint32_t *>(sc + c * LP + 16 * piece);
            const u32x4_t val = {s4[0], s4[1], s4[2], s4[3]};
            __builtin_nontemporal_store(
                val, reinterpret_cast<u32x4_t *>(cct + (tcol + c) * pitch + TILE_ROWS * T0 +
                                                 16 * piece));
        }
    }
    // Scale bytes: WPW per column, one dword per thread.
    const bool dw = !DENSE || ((G.max_tiles & 3) == 0 && ((uintptr_t)cst & 3) == 0);
    for (int q = t; q < TILE_COLS * WPW / 4; q += 64 * WPW) {
        const int c = q / (WPW / 4), k = q % (WPW / 4);
        if (tcol + c >= G.cols || 4 * k >= nv)
            continue;
        uint8_t *d = cst + (tcol + c) * G.max_tiles + T0 + 4 * k;
        const uint8_t *src = ss + WPW * c + 4 * k;
        if (dw && 4 * k + 4 <= nv) {
            *reinterpret_cast<uint32_t *>(d) = *reinterpret_cast<const uint32_t *>(src);
        } else {
            for (int b = 0; b < 4 && 4 * k + b < nv; b++)
                d[b] = src[b];
        }
    }
}

template <int WPW, bool ROW, bool SCAN>
__global__ void __launch_bounds__(64 * WPW) mxfp8_grouped_colt_kernel(Geometry G,
                                                                      uint8_t *__restrict__ rc,
                                                                      uint8_t *__restrict__ rs,
                                                                      uint8_t *__restrict__ cct,
                                                                      uint8_t *__restrict__ cst,
                                                                      int64_t *__restrict__ P_out)
{
    if constexpr (SCAN) {
        __shared__ int64_t Ps[SCAN_MAX_GROUPS + 1];
        if (wave_in_group() == 0)
            wave_block_prefix(G.off, G.n_groups, G.rows, 4, Ps, wg_id() == 0 ? P_out : nullptr);
        __syncthreads();
        G.P = Ps;
    }
    colt_staged_body<WPW, ROW, false>(G, rc, rs, cct, cst);
}

// The transposed layout of one dense tensor through the same staging.
template <int WPW, bool ROW>
__global__ void __launch_bounds__(64 * WPW) mxfp8_colt_staged_kernel(Geometry G,
                                                                     uint8_t *__restrict__ rc,
                                                                     uint8_t *__restrict__ rs,
                                                                     uint8_t *__restrict__ cct,
                                                                     uint8_t *__restrict__ cst)
{
    colt_staged_body<WPW, ROW, true>(G, rc, rs, cct, cst);
}

// P[e] = sum_{f<e} ceil(n_f / 32) (each rounded up to a multiple of
// `pad` 32-row blocks), written to P[0..G].  One workgroup; sequential over
// chunks of 256 segments with a block scan.
__global__ void __launch_bounds__(256) grouped_prefix_kernel(const int64_t *__restrict__ off,
                                                              int64_t n_groups, int64_t total_rows,
                                                              int64_t pad,
                                                              int64_t *__restrict__ P)
{
    __shared__ int64_t part[256];
    int64_t carry = 0;
    for (int64_t base = 0; base < n_groups; base += 256) {
        const int64_t e = base + tid();
        int64_t n = 0;
        if (e < n_groups) {
            int64_t lo, hi;
            segment_rows(off, e, total_rows, &lo, &hi);
            n = (hi - lo + 31) >> 5;
            n = (n + pad - 1) / pad * pad;
        }
        part[tid()] = n;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int64_t add = tid() >= (unsigned)d ? part[tid() - d] : 0;
            __syncthreads();
            part[tid()] += add;
            __syncthreads();
        }
        if (e < n_groups)
            P[e] = carry + part[tid()] - n;   // exclusive
        const int64_t total = part[255];
        __syncthreads();
        carry += total;
    }
    if (tid() == 0)
        P[n_groups] = carry;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// Wavefronts per workgroup: 8 for large launches (measured 3% faster on the
// 262144 x 2048 grouped shape), 4 below about 8 per SIMD, where fewer, larger
// workgroups leave CUs idle (8192 x 2048: 20.5 us with 8, 17.3 us with 4).
constexpr int64_t LARGE_LAUNCH_WAVES = 32768;

// Band order (band_order) for a dense launch of `wgs` workgroups of `wpw`
// wavefronts covering `waves` tiles; launch order on large launches.
static void set_band_order(Geometry &G, int64_t waves, int64_t wgs, int wpw)
{
    G.bo_k = 0;
    G.bo_full = 0;
    G.bo_grp = Div{0, 0};
    if (waves >= LARGE_LAUNCH_WAVES || G.nct % wpw != 0 || G.nct / wpw < 2)
        return;
    const int64_t k = G.nct / wpw;          // cols <= 2^26: 8 k <= 2^20
    G.bo_k = (uint32_t)k;
    G.bo_full = (uint32_t)(wgs / (8 * k) * (8 * k));
    G.bo_grp = make_div((uint32_t)(8 * k));
}

template <bool ROW, bool COL, bool GROUPED, int WPW, bool GATHER, bool SCAN>
static hipError_t launch_wpw(const Geometry &G, int64_t waves, uint8_t *rc, uint8_t *rs,
                             uint8_t *cc, uint8_t *cs, int64_t *P_out, hipStream_t stream)
{
    const int64_t wgs = GATHER ? ((waves + WPW - 1) / WPW + 7) / 8 * 8 : (waves + WPW - 1) / WPW;
    if (wgs * 64 * WPW > MAX_GRID_ITEMS)     // checked by the caller
        return hipErrorInvalidValue;
    Geometry Gl = G;
    if (!GROUPED && !GATHER)
        set_band_order(Gl, waves, wgs, WPW);
    hipLaunchKernelGGL((mxfp8_tile_kernel<ROW, COL, GROUPED, WPW, GATHER, SCAN>),
                       dim3((unsigned)wgs), dim3(64 * WPW), 0, stream, Gl, rc, rs, cc, cs, P_out);
    return hipGetLastError();
}

template <bool ROW, bool COL, bool GROUPED, bool GATHER, bool SCAN>
static hipError_t launch_one(const Geometry &G, int64_t tiles_per_strip, uint8_t *rc,
                             uint8_t *rs, uint8_t *cc, uint8_t *cs, int64_t *P_out,
                             hipStream_t stream)
{
    const int64_t waves = tiles_per_strip * G.nct;
    if (waves >= LARGE_LAUNCH_WAVES)
        return launch_wpw<ROW, COL, GROUPED, 8, GATHER, SCAN>(G, waves, rc, rs, cc, cs, P_out,
                                                              stream);
    return launch_wpw<ROW, COL, GROUPED, 4, GATHER, SCAN>(G, waves, rc, rs, cc, cs, P_out,
                                                          stream);
}

template <bool GROUPED, bool GATHER, bool SCAN = false>
static hipError_t launch(const Geometry &G, int64_t tiles_per_strip, uint8_t *rc, uint8_t *rs,
                         uint8_t *cc, uint8_t *cs, int64_t *P_out, hipStream_t stream)
{
    if (rc && cc)
        return launch_one<true, true, GROUPED, GATHER, SCAN>(G, tiles_per_strip, rc, rs, cc, cs,
                                                             P_out, stream);
    if (rc)
        return launch_one<true, false, GROUPED, GATHER, SCAN>(G, tiles_per_strip, rc, rs, cc, cs,
                                                              P_out, stream);
    return launch_one<false, true, GROUPED, GATHER, SCAN>(G, tiles_per_strip, rc, rs, cc, cs,
                                                          P_out, stream);
}

hipError_t launch_mxfp8_dense(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *rc,
                              uint8_t *rs, uint8_t *cc, uint8_t *cs, const int64_t *row_tokens,
                              int64_t n_tokens, hipStream_t stream)
{
    Geometry G{x, rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, 0, nullptr, nullptr, 0,
               row_tokens, n_tokens};
    const int64_t tiles = (rows + TILE_ROWS - 1) / TILE_ROWS;
    if (row_tokens)
        return launch<false, true>(G, tiles, rc, rs, cc, cs, nullptr, stream);
    return launch<false, false>(G, tiles, rc, rs, cc, cs, nullptr, stream);
}

template <bool ROW, int WPW>
static hipError_t launch_qdq_wpw(const Geometry &G, int64_t waves, uint8_t *rc, uint8_t *rs,
                                 uint16_t *dq, hipStream_t stream)
{
    const int64_t wgs = (waves + WPW - 1) / WPW;
    if (wgs * 64 * WPW > MAX_GRID_ITEMS)     // checked by the caller
        return hipErrorInvalidValue;
    Geometry Gl = G;
    set_band_order(Gl, waves, wgs, WPW);
    hipLaunchKernelGGL((mxfp8_row_qdq_kernel<ROW, WPW>), dim3((unsigned)wgs), dim3(64 * WPW), 0,
                       stream, Gl, rc, rs, dq);
    return hipGetLastError();
}

hipError_t launch_mxfp8_row_qdq(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *rc,
                                uint8_t *rs, uint16_t *dq, hipStream_t stream)
{
    Geometry G{x, rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, 0, nullptr, nullptr, 0,
               nullptr, 0};
    const int64_t waves = (rows + TILE_ROWS - 1) / TILE_ROWS * G.nct;
    if (rc) {
        if (waves >= LARGE_LAUNCH_WAVES)
            return launch_qdq_wpw<true, 8>(G, waves, rc, rs, dq, stream);
        return launch_qdq_wpw<true, 4>(G, waves, rc, rs, dq, stream);
    }
    if (waves >= LARGE_LAUNCH_WAVES)
        return launch_qdq_wpw<false, 8>(G, waves, rc, rs, dq, stream);
    return launch_qdq_wpw<false, 4>(G, waves, rc, rs, dq, stream);
}

template <bool ROW, bool COL>
static hipError_t launch_ocp(const Geometry &G, int64_t waves, uint8_t *rc, uint8_t *rs,
                             uint8_t *cc, uint8_t *cs, hipStream_t stream)
{
    const int64_t wgs = (waves + 3) / 4;
    if (wgs * 256 > MAX_GRID_ITEMS)          // checked by the caller
        return hipErrorInvalidValue;
    Geometry Gl = G;
    set_band_order(Gl, waves, wgs, 4);
    hipLaunchKernelGGL((mxfp8_ocp_kernel<ROW, COL, 4>), dim3((unsigned)wgs), dim3(256), 0, stream,
                       Gl, rc, rs, cc, cs);
    return hipGetLastError();
}

hipError_t launch_mxfp8_ocp_floor(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *rc,
                                  uint8_t *rs, uint8_t *cc, uint8_t *cs, hipStream_t stream)
{
    Geometry G{x, rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, 0, nullptr, nullptr, 0,
               nullptr, 0};
    const int64_t waves = (rows + TILE_ROWS - 1) / TILE_ROWS * G.nct;
    if (rc && cc)
        return launch_ocp<true, true>(G, waves, rc, rs, cc, cs, stream);
    if (rc)
        return launch_ocp<true, false>(G, waves, rc, rs, cc, cs, stream);
    return launch_ocp<false, true>(G, waves, rc, rs, cc, cs, stream);
}

hipError_t launch_mxfp8_colt(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *rc,
                             uint8_t *rs, uint8_t *cct, uint8_t *cst, hipStream_t stream)
{
    // rows % 32 == 0: checked by the caller.
    Geometry G{x, rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, rows / TILE_ROWS, nullptr,
               nullptr, 0, nullptr, 0};
    // Four-wavefront groups below LARGE_LAUNCH_WAVES blocks x strips, as for
    // the tile kernel (8192 x 2048: 18.2 -> 17.0 us), eight above.
    if (G.max_tiles * G.nct < LARGE_LAUNCH_WAVES) {
        constexpr int WPW = 4;
        const int64_t wgs = ((G.max_tiles + WPW - 1) / WPW * G.nct + 7) / 8 * 8;
        if (rc)
            hipLaunchKernelGGL((mxfp8_colt_staged_kernel<WPW, true>), dim3((unsigned)wgs),
                               dim3(64 * WPW), 0, stream, G, rc, rs, cct, cst);
        else
            hipLaunchKernelGGL((mxfp8_colt_staged_kernel<WPW, false>), dim3((unsigned)wgs),
                               dim3(64 * WPW), 0, stream, G, rc, rs, cct, cst);
        return hipGetLastError();
    }
    constexpr int WPW = 8;
    const int64_t wgs = ((G.max_tiles + WPW - 1) / WPW * G.nct + 7) / 8 * 8;
    if (wgs * 64 * WPW > MAX_GRID_ITEMS)     // checked by the caller
        return hipErrorInvalidValue;
    if (rc)
        hipLaunchKernelGGL((mxfp8_colt_staged_kernel<WPW, true>), dim3((unsigned)wgs),
                           dim3(64 * WPW), 0, stream, G, rc, rs, cct, cst);
    else
        hipLaunchKernelGGL((mxfp8_colt_staged_kernel<WPW, false>), dim3((unsigned)wgs),
                           dim3(64 * WPW), 0, stream, G, rc, rs, cct, cst);
    return hipGetLastError();
}

hipError_t launch_mxfp8_grouped_colt(const uint16_t *x, int64_t total_rows, int64_t cols,
                                     const int64_t *off, int64_t n_groups, uint8_t *rc,
                                     uint8_t *rs, uint8_t *cct, uint8_t *cst, int64_t *P,
                                     hipStream_t stream)
{
    const int64_t max_tiles = grouped_colt_pitch(total_rows, n_groups) / TILE_ROWS;
    if (mxfp8_tiles(max_tiles, cols) > MAX_MXFP8_TILES)     // checked by the caller
        return hipErrorInvalidValue;
    const bool scan = n_groups <= SCAN_MAX_GROUPS;
    if (!scan) {
        hipLaunchKernelGGL(grouped_prefix_kernel, dim3(1), dim3(256), 0, stream, off, n_groups,
                           total_rows, (int64_t)4, P);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    Geometry G{x, total_rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, max_tiles, off, P,
               n_groups, nullptr, 0};
    constexpr int WPW = 8;
    const dim3 grid((unsigned)(((max_tiles + WPW - 1) / WPW * G.nct + 7) / 8 * 8)), block(64 * WPW);
    if (scan && rc)
        hipLaunchKernelGGL((mxfp8_grouped_colt_kernel<WPW, true, true>), grid, block, 0, stream,
                           G, rc, rs, cct, cst, P);
    else if (scan)
        hipLaunchKernelGGL((mxfp8_grouped_colt_kernel<WPW, false, true>), grid, block, 0, stream,
                           G, rc, rs, cct, cst, P);
    else if (rc)
        hipLaunchKernelGGL((mxfp8_grouped_colt_kernel<WPW, true, false>), grid, block, 0, stream,
                           G, rc, rs, cct, cst, nullptr);
    else
        hipLaunchKernelGGL((mxfp8_grouped_colt_kernel<WPW, false, false>), grid, block, 0,
                           stream, G, rc, rs, cct, cst, nullptr);
    return hipGetLastError();
}

hipError_t launch_mxfp8_grouped(const uint16_t *x, int64_t total_rows, int64_t cols,
                                const int64_t *off, int64_t n_groups, uint8_t *rc, uint8_t *rs,
                                uint8_t *cc, uint8_t *cs, int64_t *P,
                                const int64_t *row_tokens, int64_t n_tokens, hipStream_t stream)
{
    const int64_t max_tiles = total_rows / TILE_ROWS + n_groups;
    if (mxfp8_tiles(max_tiles, cols) > MAX_MXFP8_TILES)     // checked by the caller
        return hipErrorInvalidValue;
    Geometry G{x, total_rows, cols, (cols + TILE_COLS - 1) / TILE_COLS, max_tiles, off, P,
               n_groups, row_tokens, n_tokens};
    // The dispatch gather keeps the prefix launch: its tiles' loads already
    // wait on the row map, and the in-kernel prefix measured 312 -> 315 us
    // on 32768 tokens routed top-8 into 262144 x 2048.
    if (n_groups <= SCAN_MAX_GROUPS && !row_tokens)
        return launch<true, false, true>(G, max_tiles, rc, rs, cc, cs, P, stream);
    hipLaunchKernelGGL(grouped_prefix_kernel, dim3(1), dim3(256), 0, stream, off, n_groups,
                       total_rows, (int64_t)1, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (row_tokens)
        return launch<true, true>(G, max_tiles, rc, rs, cc, cs, nullptr, stream);
    return launch<true, false>(G, max_tiles, rc, rs, cc, cs, nullptr, stream);
}

}  // namespace mxq
