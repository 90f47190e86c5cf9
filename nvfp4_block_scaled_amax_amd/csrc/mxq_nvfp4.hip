// mxq_nvfp4.hip -- NVFP4 quantizers: per-token FP32 scale (the per-token
// activation paragraphs of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell") and weight export with one FP32 scale per gate/up
// pair or per tensor (its gate/up pairing paragraph).  The arithmetic is the
// page's NVFP4 format paragraph under the readings stated in mxq.h:
//   s = fp32(A_scope / 2688), b = E4M3(A_block / (6 s)), c = E2M1(x / (dec(b) s)).
//
// Layout.  A thread owns one 8-element chunk (one 16-byte load) per slot, so
// a block is a pair of adjacent lanes and every load and store instruction of
// a wavefront covers one contiguous span: the measured fastest way to stream
// HBM on this part is many small workgroups, one 16-byte access per thread,
// launched in one grid.  A block's amax is the max of the pair (one DPP
// exchange); both lanes derive the same block scale and each converts its
// own 8 elements.
// Per-token: one wavefront per row (rows of up to 4096 elements are held in
// registers; longer rows are read twice), the token amax a wavefront
// reduction.  Export: a flat array of chunks under the scope's
// FP32 scale, computed beforehand by an amax pass.
//
// Exact decisions without division.  Dividing per element is too slow and
// multiplying by a rounded reciprocal is not exact.  Every decision is
// bracketed instead: with r ~ 1/D (D = 6s for block scales, dec(b) s for codes)
// built from v_rcp_f32 (under 1 ulp) and rounded products, relative error
// below 2^-21, the kernel forms q_lo = x * r (1 - 2^-19) and
// q_hi = x * r (1 + 2^-19), so |q_lo| < |x / D| < |q_hi| with all operands
// normal.  Conversion is monotone, so when the hardware's exact nearest-even
// conversions of q_lo and q_hi agree, that code is the exactly rounded code of
// x / D.  When they differ (x / D within ~2^-18 of a rounding midpoint, a few
// per million random elements), the lane decides exactly in binary64: |x|
// against midpoint * D, a product of at most 31 significant bits, hence exact.
// Scales below 2^-101 would take the reciprocals out of the normal range; such
// scopes use a binary64 path that divides once per element.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr float S_FAST_MIN = 0x1p-101f;
constexpr float BRACKET_LO = 1.0f - 0x1p-19f;
constexpr float BRACKET_HI = 1.0f + 0x1p-19f;
constexpr float ONE_SIXTH = 1.0f / 6.0f;

// ---------------------------------------------------------------------------
// One 8-element chunk (half a block)
// ---------------------------------------------------------------------------
constexpr uint32_t MAG2 = 0x7FFF7FFFu;      // clears the sign of two BF16

// Largest |x| of the chunk as f32 bits: with the sign cleared, BF16 magnitudes
// order as unsigned integers, two per packed 16-bit max.
__device__ __forceinline__ uint32_t chunk_amax_bits(uint4 v)
{
    const uint32_t m = pk_max_u16(pk_max_u16(v.x & MAG2, v.y & MAG2),
                                  pk_max_u16(v.z & MAG2, v.w & MAG2));
    return hmax_u16(m) << 16;
}

// Block amax: the max over the lane pair (2m, 2m + 1).  Every lane of the
// wavefront must execute it.
__device__ __forceinline__ uint32_t block_amax_bits(uint32_t chunk_amax)
{
    return max(chunk_amax, dpp<DPP_XOR1>(chunk_amax));
}

// Exact block scale when the bracket straddles a midpoint: blo and blo + 1 are
// the candidates; compare A with their midpoint times 6 s exactly.
__device__ __attribute__((noinline)) uint32_t block_scale_exact(float A, float s, uint32_t blo)
{
    const double mid2 = (double)e4m3_value(blo) + (double)e4m3_value(blo + 1);  // 2 * midpoint
    const double t = mid2 * 3.0 * (double)s;                                    // midpoint * 6 s
    const double a = (double)A;
    if (a > t)
        return blo + 1;
    if (a < t)
        return blo;
    return (blo & 1u) ? blo + 1 : blo;
}

// Nibble i of the bracket results lo/hi differ: decide it exactly.  x: the
// element (BF16 bits), Dd = dec(b) s in binary64 (exact).
__device__ __forceinline__ uint32_t fix_nibble(uint32_t lo, uint32_t hi, int i, uint32_t xbits,
                                               double Dd)
{
    const uint32_t a = (lo >> (4 * i)) & 0xFu, b = (hi >> (4 * i)) & 0xFu;
    if (a == b)
        return lo;
    const uint32_t klo = a & 7u, khi = b & 7u;     // khi == klo + 1
    const double t = (e2m1_value_f64(klo) + e2m1_value_f64(khi)) * Dd;   // 2 * mid * D
    const double ax = 2.0 * fabs((double)u2f(xbits << 16));
    uint32_t k;
    if (ax > t)
        k = khi;
    else if (ax < t)
        k = klo;
    else
        k = (klo & 1u) ? khi : klo;
    return (lo & ~(0xFu << (4 * i))) | ((k | (a & 8u)) << (4 * i));
}

// Fix the nibbles of one 8-code word.  w0..w3: the 8 inputs (BF16 pairs).
__device__ __attribute__((noinline)) uint32_t codes_exact(uint32_t lo, uint32_t hi, uint32_t w0,
                                                          uint32_t w1, uint32_t w2, uint32_t w3,
                                                          float d, float s)
{
    const double D = (double)d * (double)s;
    const uint32_t w[4] = {w0, w1, w2, w3};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        lo = fix_nibble(lo, hi, i, bits, D);
    }
    return lo;
}

// The 8 codes of the chunk's values times r, with the hardware conversion.
// The four conversions overwrite all four bytes, so the first one's "old"
// operand can be any value; the first product is used.
__device__ __forceinline__ uint32_t codes8(uint4 v, float r)
{
    const float p0 = bf16_lo(v.x) * r;
    uint32_t c = e2m1_pair<0>(f2u(p0), p0, bf16_hi(v.x) * r);
    c = e2m1_pair<1>(c, bf16_lo(v.y) * r, bf16_hi(v.y) * r);
    c = e2m1_pair<2>(c, bf16_lo(v.z) * r, bf16_hi(v.z) * r);
    c = e2m1_pair<3>(c, bf16_lo(v.w) * r, bf16_hi(v.w) * r);
    return c;
}

// Per-scale constants of the fast path.
struct ScaleK {
    float s, inv_s, r6_lo, r6_hi;
};

__device__ __forceinline__ ScaleK scale_k(float s)
{
    ScaleK k;
    k.s = s;
    k.inv_s = __builtin_amdgcn_rcpf(s);
    const float r6 = k.inv_s * ONE_SIXTH;
    k.r6_lo = r6 * BRACKET_LO;
    k.r6_hi = r6 * BRACKET_HI;
    return k;
}

// Block scale byte and the chunk's 4 code bytes.
struct ChunkOut {
    uint32_t b, c;
};

// binary64 path (0 < s < 2^-101): one division per element.
__device__ __attribute__((noinline)) ChunkOut quant_chunk_f64(uint32_t w0, uint32_t w1,
                                                              uint32_t w2, uint32_t w3,
                                                              uint32_t amax_bits, float s)
{
    const uint32_t w[4] = {w0, w1, w2, w3};
    ChunkOut o;
    o.b = e4m3_code_f64((double)u2f(amax_bits) / (6.0 * (double)s));
    o.c = 0u;
    if (o.b != 0) {
        const double D = (double)e4m3_value(o.b) * (double)s;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const double xv = (double)u2f(bits << 16);
            o.c |= (e2m1_code_f64(fabs(xv) / D) | ((bits >> 12) & 8u)) << (4 * i);
        }
    }
    return o;
}

// Quantize one chunk whose block has amax bits blk_amax, under scale k.
__device__ __forceinline__ ChunkOut quant_chunk(uint4 v, uint32_t blk_amax, const ScaleK &k)
{
    ChunkOut o;
    if (k.s >= S_FAST_MIN) {
        const float A = u2f(blk_amax);
        const uint32_t bb = e4m3_pair_rne(fminf(A * k.r6_lo, 448.0f), fminf(A * k.r6_hi, 448.0f));
        o.b = bb & 0xFFu;
        if (o.b != (bb >> 8))
            o.b = block_scale_exact(A, k.s, o.b);
        o.c = 0u;
        if (o.b != 0) {
            const float d = e4m3_value(o.b);
            const float r = __builtin_amdgcn_rcpf(d) * k.inv_s;
            const uint32_t lo = codes8(v, r * BRACKET_LO), hi = codes8(v, r * BRACKET_HI);
            o.c = (lo == hi) ? lo : codes_exact(lo, hi, v.x, v.y, v.z, v.w, d, k.s);
        }
    } else if (k.s == 0.0f) {
        o.b = 0u;
        o.c = 0u;
    } else {
        o = quant_chunk_f64(v.x, v.y, v.z, v.w, blk_amax, k.s);
    }
    return o;
}

// Store the chunk's codes (4 bytes at chunk index c of a code array whose
// element 0 is chunk 0) and, from the even lane of the pair, the scale byte.
__device__ __forceinline__ void emit_chunk(ChunkOut o, int64_t c, uint8_t *__restrict__ codes,
                                           uint8_t *__restrict__ bs)
{
    st_nt4(codes + 4 * c, o.c);
    if (!(c & 1))
        bs[c >> 1] = (uint8_t)o.b;
}

__device__ __forceinline__ uint4 ld_chunk(const uint16_t *p) { return ld_nt16(p); }

// ---------------------------------------------------------------------------
// Per-token kernels: one wavefront per row; lane l holds chunks l + 64 j, so
// each 16-byte load instruction of the wavefront covers 1 KiB of the row.
// Four rows per workgroup, one launch over all rows.
// ---------------------------------------------------------------------------
constexpr int WG_THREADS = 256;
constexpr int ROWS_PER_WG = WG_THREADS / 64;

__device__ __forceinline__ float token_scale(uint32_t amax_bits, int64_t row,
                                             float *__restrict__ ts)
{
    const float s = u2f(amax_bits) / 2688.0f;
    if (lane_id() == 0)
        ts[row] = s;
    return s;
}

// Rows of up to 64 NS chunks (512 NS elements), held in registers.
template <int NS>
__global__ void __launch_bounds__(WG_THREADS) nvfp4_token_kernel(const uint16_t *__restrict__ x,
                                                                 int64_t rows, int64_t cols,
                                                                 uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ bs,
                                                                 float *__restrict__ ts)
{
    const int64_t row = (int64_t)wg_id() * ROWS_PER_WG + wave_in_group();
    if (row >= rows)
        return;
    const int lane = lane_id();
    const int64_t nchunk = cols >> 3;       // even: a pair never straddles the end
    const uint16_t *xr = x + row * cols;
    uint4 v[NS];
    uint32_t ca[NS];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int64_t c = lane + 64 * j;
        v[j] = c < nchunk ? ld_chunk(xr + 8 * c) : make_uint4(0, 0, 0, 0);
        ca[j] = chunk_amax_bits(v[j]);
        m = max(m, ca[j]);
    }
    const ScaleK k = scale_k(token_scale(__builtin_amdgcn_readfirstlane(wave_max_u32(m)), row, ts));
    uint8_t *crow = codes + row * (cols >> 1);
    uint8_t *brow = bs + row * (cols >> 4);
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int64_t c = lane + 64 * j;
        const uint32_t ba = block_amax_bits(ca[j]);
        if (c < nchunk)
            emit_chunk(quant_chunk(v[j], ba, k), c, crow, brow);
    }
}

// Longer rows: read twice (amax, then codes).
__global__ void __launch_bounds__(WG_THREADS) nvfp4_token_long_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ bs, float *__restrict__ ts)
{
    const int64_t row = (int64_t)wg_id() * ROWS_PER_WG + wave_in_group();
    if (row >= rows)
        return;
    const int lane = lane_id();
    const int64_t nchunk = cols >> 3;
    const uint16_t *xr = x + row * cols;
    uint32_t m = 0;
    for (int64_t c = lane; c < nchunk; c += 64)
        m = max(m, chunk_amax_bits(ld_chunk(xr + 8 * c)));
    const ScaleK k = scale_k(token_scale(__builtin_amdgcn_readfirstlane(wave_max_u32(m)), row, ts));
    uint8_t *crow = codes + row * (cols >> 1);
    uint8_t *brow = bs + row * (cols >> 4);
    const int64_t steps = (nchunk + 63) / 64;    // uniform trip count
    for (int64_t j = 0; j < steps; j++) {
        const int64_t c = lane + 64 * j;
        const uint4 v = c < nchunk ? ld_chunk(xr + 8 * c) : make_uint4(0, 0, 0, 0);
        const uint32_t ba = block_amax_bits(chunk_amax_bits(v));
        if (c < nchunk)
            emit_chunk(quant_chunk(v, ba, k), c, crow, brow);
    }
}

// ---------------------------------------------------------------------------
// Export: scope amax, FP32 scales, then a flat pass over the blocks.
// ---------------------------------------------------------------------------
__global__ void zero_u32_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)wg_id() * 256 + tid();
    if (i < n)
        p[i] = 0u;
}

constexpr int AMAX_LOADS = 8;                               // 16-byte loads per thread
constexpr int64_t AMAX_CHUNK = 256 * 8 * AMAX_LOADS;        // elements per workgroup

// Workgroup w reduces chunk w % chunks of scope w / chunks.  A scope is
// tensor a's slice [e * n_per, (e+1) * n_per) followed by tensor b's (if any).
// The result is the amax's BF16 magnitude bits (as u32) in amax[e].
__global__ void __launch_bounds__(256) scope_amax_kernel(const uint16_t *__restrict__ a,
                                                         const uint16_t *__restrict__ b,
                                                         int64_t n_per, int64_t chunks,
                                                         uint32_t *__restrict__ amax)
{
    __shared__ uint32_t part[4];
    const int64_t e = (int64_t)wg_id() / chunks;
    const int64_t ch = (int64_t)wg_id() - e * chunks;
    const int64_t n_scope = b ? 2 * n_per : n_per;
    uint32_t m = 0;
#pragma unroll
    for (int it = 0; it < AMAX_LOADS; it++) {
        const int64_t i = ch * AMAX_CHUNK + (int64_t)it * 2048 + 8 * tid();
        if (i < n_scope) {
            const uint16_t *p = (i < n_per) ? a + e * n_per + i : b + e * n_per + (i - n_per);
            const uint4 q = ld_nt16(p);
            m = pk_max_u16(m, pk_max_u16(pk_max_u16(q.x & 0x7FFF7FFFu, q.y & 0x7FFF7FFFu),
                                         pk_max_u16(q.z & 0x7FFF7FFFu, q.w & 0x7FFF7FFFu)));
        }
    }
    uint32_t h = wave_max_u32(hmax_u16(m));
    if (lane_id() == 0)
        part[tid() >> 6] = h;
    __syncthreads();
    if (tid() == 0) {
        h = max(max(part[0], part[1]), max(part[2], part[3]));
        atomicMax(amax + e, h);
    }
}

// amax bits -> s = fp32(amax / 2688), in place.
__global__ void scope_finalize_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)wg_id() * 256 + tid();
    if (i < n) {
        const float s = u2f(p[i] << 16) / 2688.0f;
        p[i] = f2u(s);
    }
}

// Flat export pass over one tensor of nchunk chunks (two per block); block j
// belongs to scope j / bps.  Each wavefront takes 64 SCOPED_NS consecutive
// chunks, lane l the chunks l + 64 i, like a per-token row.
constexpr int SCOPED_NS = 4;

__global__ void __launch_bounds__(WG_THREADS) nvfp4_scoped_kernel(const uint16_t *__restrict__ x,
                                                                  int64_t nchunk, Div bps,
                                                                  const float *__restrict__ scope_s,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ bs)
{
    const int64_t base = ((int64_t)wg_id() * ROWS_PER_WG + wave_in_group()) * (64 * SCOPED_NS);
    if (base >= nchunk)
        return;
    const int lane = lane_id();
    uint4 v[SCOPED_NS];
#pragma unroll
    for (int i = 0; i < SCOPED_NS; i++) {
        const int64_t c = base + lane + 64 * i;
        v[i] = c < nchunk ? ld_chunk(x + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SCOPED_NS; i++) {
        const int64_t c = base + lane + 64 * i;
        const uint32_t ba = block_amax_bits(chunk_amax_bits(v[i]));
        if (c < nchunk) {
            const uint32_t e = udiv((uint32_t)(c >> 1), bps);
            emit_chunk(quant_chunk(v[i], ba, scale_k(scope_s[e])), c, codes, bs);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <int NS>
static void launch_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                         uint8_t *bs, float *ts, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WG_THREADS);
    hipLaunchKernelGGL(nvfp4_token_kernel<NS>, grid, block, 0, stream, x, rows, cols, codes, bs,
                       ts);
}

hipError_t launch_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                  uint8_t *bs, float *ts, hipStream_t stream)
{
    // rows < 2^31: checked by the caller.
    switch ((cols / 8 + 63) / 64) {
    case 1: launch_token<1>(x, rows, cols, codes, bs, ts, stream); break;
    case 2: launch_token<2>(x, rows, cols, codes, bs, ts, stream); break;
    case 3: launch_token<3>(x, rows, cols, codes, bs, ts, stream); break;
    case 4: launch_token<4>(x, rows, cols, codes, bs, ts, stream); break;
    case 5: launch_token<5>(x, rows, cols, codes, bs, ts, stream); break;
    case 6: launch_token<6>(x, rows, cols, codes, bs, ts, stream); break;
    case 7: launch_token<7>(x, rows, cols, codes, bs, ts, stream); break;
    case 8: launch_token<8>(x, rows, cols, codes, bs, ts, stream); break;
    default: {
        const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WG_THREADS);
        hipLaunchKernelGGL(nvfp4_token_long_kernel, grid, block, 0, stream, x, rows, cols, codes,
                           bs, ts);
    }
    }
    return hipGetLastError();
}

hipError_t launch_nvfp4_scoped(const uint16_t *gate, const uint16_t *up, int64_t n_experts,
                               int64_t rows, int64_t cols, uint8_t *gc, uint8_t *gbs,
                               uint8_t *uc, uint8_t *ubs, float *scope_scales,
                               hipStream_t stream)
{
    uint32_t *amax = reinterpret_cast<uint32_t *>(scope_scales);
    const unsigned small_grid = (unsigned)((n_experts + 255) / 256);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(small_grid), dim3(256), 0, stream, amax, n_experts);
    const int64_t n_per = rows * cols;
    const int64_t n_scope = up ? 2 * n_per : n_per;
    const int64_t chunks = (n_scope + AMAX_CHUNK - 1) / AMAX_CHUNK;
    hipLaunchKernelGGL(scope_amax_kernel, dim3((unsigned)(chunks * n_experts)), dim3(256), 0,
                       stream, gate, up, n_per, chunks, amax);
    hipLaunchKernelGGL(scope_finalize_kernel, dim3(small_grid), dim3(256), 0, stream, amax,
                       n_experts);
    // Blocks in all (< 2^32) and chunks per launch: checked by the caller.
    const int64_t nchunk = n_experts * n_per / 8;
    const Div bps = make_div((uint32_t)(n_per / 16));
    const int64_t per_wg = 64 * SCOPED_NS * ROWS_PER_WG;
    const dim3 grid((unsigned)((nchunk + per_wg - 1) / per_wg)), block(WG_THREADS);
    hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, gate, nchunk, bps,
                       (const float *)scope_scales, gc, gbs);
    if (up)
        hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, up, nchunk, bps,
                           (const float *)scope_scales, uc, ubs);
    return hipGetLastError();
}

}  // namespace mxq
