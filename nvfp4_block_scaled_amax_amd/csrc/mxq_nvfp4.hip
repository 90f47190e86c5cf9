// mxq_nvfp4.hip -- NVFP4 quantizers: per-token FP32 scale (the per-token
// activation paragraphs of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell") and weight export with one FP32 scale per gate/up
// pair or per tensor (its gate/up pairing paragraph).  The arithmetic is the
// page's NVFP4 format paragraph under the readings stated in mxq.h:
//   s = fp32(A_scope / 2688), b = E4M3(A_block / (6 s)), c = E2M1(x / (dec(b) s)).
//
// Layout.  A lane owns whole 16-element blocks (two 16-byte loads each) and
// holds them as f32, so a block's amax is an in-lane max (|x| comes free as a
// source modifier: the library is built with IEEE mode off, which only
// changes how min/max treat NaN, and NaN inputs are outside the contract) and
// its scale work is done once.  Per-token: one wavefront per row, grid-stride
// over rows with many wavefronts per SIMD (measured faster than prefetching
// the next row inside a wavefront); the token amax is a wavefront reduction.
// Export:
// the tensor is a flat array of blocks (each lies in one scope), 64 blocks per
// wavefront step, with the scope's FP32 scale computed beforehand.
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

constexpr int WAVES_PER_WG = 4;
constexpr float S_FAST_MIN = 0x1p-101f;
constexpr float BRACKET_LO = 1.0f - 0x1p-19f;
constexpr float BRACKET_HI = 1.0f + 0x1p-19f;
constexpr float ONE_SIXTH = 1.0f / 6.0f;

// ---------------------------------------------------------------------------
// One 16-element block
// ---------------------------------------------------------------------------
struct Blk {
    uint32_t w[8];     // 16 BF16, packed in pairs
};

__device__ __forceinline__ void load_blk(Blk &b, const uint16_t *p)
{
    const uint4 q0 = ld_nt16(p), q1 = ld_nt16(p + 8);
    b.w[0] = q0.x; b.w[1] = q0.y; b.w[2] = q0.z; b.w[3] = q0.w;
    b.w[4] = q1.x; b.w[5] = q1.y; b.w[6] = q1.z; b.w[7] = q1.w;
}

__device__ __forceinline__ void zero_blk(Blk &b)
{
#pragma unroll
    for (int i = 0; i < 8; i++)
        b.w[i] = 0u;
}

// The block's 16 values as f32 (exact) and its largest |x| as non-negative
// f32 bits.  With IEEE mode off the max takes |x| as a source modifier.
struct BlkF {
    float x[16];
    uint32_t amax;
};

__device__ __forceinline__ BlkF unpack_blk(const Blk &b)
{
    BlkF f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        f.x[2 * i] = bf16_lo(b.w[i]);
        f.x[2 * i + 1] = bf16_hi(b.w[i]);
    }
    float m = fmaxf(fabsf(f.x[0]), fabsf(f.x[1]));
#pragma unroll
    for (int i = 2; i < 16; i += 2)
        m = fmaxf(m, fmaxf(fabsf(f.x[i]), fabsf(f.x[i + 1])));
    f.amax = f2u(m);
    return f;
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
// element (BF16 bits), D2 = 2 d s in binary64 (exact).
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

// The 8 codes of 8 values times r, written with the hardware conversion.  The
// four conversions overwrite all four bytes, so the first one's "old" operand
// can be any value; the first product is used.
__device__ __forceinline__ uint32_t codes8(const float *x, float r)
{
    const float p0 = x[0] * r;
    uint32_t c = e2m1_pair<0>(f2u(p0), p0, x[1] * r);
    c = e2m1_pair<1>(c, x[2] * r, x[3] * r);
    c = e2m1_pair<2>(c, x[4] * r, x[5] * r);
    c = e2m1_pair<3>(c, x[6] * r, x[7] * r);
    return c;
}

// Fast path for one block: codes (two words) and the block scale byte.
__device__ __forceinline__ void quant_blk_fast(const Blk &blk, const BlkF &f, float s,
                                               float inv_s, float r6_lo, float r6_hi,
                                               uint32_t *b_out, uint32_t *c0, uint32_t *c1)
{
    const float A = u2f(f.amax);
    const float plo = fminf(A * r6_lo, 448.0f);
    const float phi = fminf(A * r6_hi, 448.0f);
    const uint32_t bb = e4m3_pair_rne(plo, phi);
    uint32_t b = bb & 0xFFu;
    if (b != (bb >> 8))
        b = block_scale_exact(A, s, b);
    *b_out = b;
    if (b == 0) {
        *c0 = 0u;
        *c1 = 0u;
        return;
    }
    const float d = e4m3_value(b);
    const float r = __builtin_amdgcn_rcpf(d) * inv_s;
    const float rlo = r * BRACKET_LO, rhi = r * BRACKET_HI;
    uint32_t lo0 = codes8(f.x, rlo), hi0 = codes8(f.x, rhi);
    uint32_t lo1 = codes8(f.x + 8, rlo), hi1 = codes8(f.x + 8, rhi);
    if (lo0 != hi0)
        lo0 = codes_exact(lo0, hi0, blk.w[0], blk.w[1], blk.w[2], blk.w[3], d, s);
    if (lo1 != hi1)
        lo1 = codes_exact(lo1, hi1, blk.w[4], blk.w[5], blk.w[6], blk.w[7], d, s);
    *c0 = lo0;
    *c1 = lo1;
}

// binary64 path (0 < s < 2^-101): one division per element.  Returns the
// scale byte and the two code words (by value, so nothing goes to scratch).
struct BlkOut {
    uint32_t b, c0, c1;
};

__device__ __attribute__((noinline)) BlkOut quant_blk_f64(uint32_t w0, uint32_t w1, uint32_t w2,
                                                          uint32_t w3, uint32_t w4, uint32_t w5,
                                                          uint32_t w6, uint32_t w7,
                                                          uint32_t amax_bits, float s)
{
    const uint32_t w[8] = {w0, w1, w2, w3, w4, w5, w6, w7};
    const double A = (double)u2f(amax_bits);
    BlkOut o;
    o.b = e4m3_code_f64(A / (6.0 * (double)s));
    o.c0 = o.c1 = 0u;
    if (o.b != 0) {
        const double D = (double)e4m3_value(o.b) * (double)s;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const double xv = (double)u2f(bits << 16);
            const uint32_t k = e2m1_code_f64(fabs(xv) / D) | ((bits >> 12) & 8u);
            if (i < 8)
                o.c0 |= k << (4 * i);
            else
                o.c1 |= k << (4 * (i - 8));
        }
    }
    return o;
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

// Quantize one block under scale k (any path) and store 8 code bytes and the
// scale byte.
__device__ __forceinline__ void emit_blk(const Blk &blk, const BlkF &f, const ScaleK &k,
                                         uint8_t *__restrict__ codes8p, uint8_t *__restrict__ bsp)
{
    uint32_t b, c0, c1;
    if (k.s >= S_FAST_MIN) {
        quant_blk_fast(blk, f, k.s, k.inv_s, k.r6_lo, k.r6_hi, &b, &c0, &c1);
    } else if (k.s == 0.0f) {
        b = 0u;
        c0 = c1 = 0u;
    } else {
        const BlkOut o = quant_blk_f64(blk.w[0], blk.w[1], blk.w[2], blk.w[3], blk.w[4], blk.w[5],
                                       blk.w[6], blk.w[7], f.amax, k.s);
        b = o.b;
        c0 = o.c0;
        c1 = o.c1;
    }
    st_nt8(codes8p, c0, c1);
    *bsp = (uint8_t)b;
}

// ---------------------------------------------------------------------------
// Per-token kernel: a wavefront per row; block j of the row is held by lane
// j % 64 in slot j / 64.  NB slots cover rows of up to 1024 * NB elements.
// ---------------------------------------------------------------------------
// FULL: the row has exactly 64 NB blocks, so no lane is masked.
template <int NB, bool FULL>
__device__ __forceinline__ void load_row(Blk (&r)[NB], const uint16_t *__restrict__ xr,
                                         int64_t nblk, int lane)
{
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int64_t blk = 64 * j + lane;
        if (FULL || blk < nblk)
            load_blk(r[j], xr + 16 * blk);
        else
            zero_blk(r[j]);
    }
}

template <int NB, bool FULL>
__device__ __forceinline__ void token_row(const Blk (&r)[NB], int64_t row, int64_t cols,
                                          int64_t nblk, int lane, uint8_t *__restrict__ codes,
                                          uint8_t *__restrict__ bs, float *__restrict__ ts)
{
    BlkF f[NB];
    uint32_t A = 0;
#pragma unroll
    for (int j = 0; j < NB; j++) {
        f[j] = unpack_blk(r[j]);
        A = max(A, f[j].amax);
    }
    A = __builtin_amdgcn_readfirstlane(wave_max_u32(A));
    const float s = u2f(A) / 2688.0f;
    if (lane == 0)
        ts[row] = s;
    const ScaleK k = scale_k(s);
    uint8_t *crow = codes + row * (cols >> 1);
    uint8_t *brow = bs + row * (cols >> 4);
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int blk = 64 * j + lane;
        if (FULL || blk < nblk)
            emit_blk(r[j], f[j], k, crow + 8 * blk, brow + blk);
    }
}

template <int NB, bool FULL>
__global__ void __launch_bounds__(256) nvfp4_token_kernel(const uint16_t *__restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ bs,
                                                          float *__restrict__ ts)
{
    const int lane = __lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t nblk = cols >> 4;
    for (int64_t row = (int64_t)blockIdx.x * WAVES_PER_WG + wave_in_group(); row < rows;
         row += nwaves) {
        Blk r[NB];
        load_row<NB, FULL>(r, x + row * cols, nblk, lane);
        token_row<NB, FULL>(r, row, cols, nblk, lane, codes, bs, ts);
    }
}

// Rows longer than 4096 elements: the row is read twice (amax, then codes).
__global__ void __launch_bounds__(256) nvfp4_token_long_kernel(const uint16_t *__restrict__ x,
                                                               int64_t rows, int64_t cols,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ bs,
                                                               float *__restrict__ ts)
{
    const int lane = __lane_id();
    const int64_t row = (int64_t)blockIdx.x * WAVES_PER_WG + wave_in_group();
    if (row >= rows)
        return;
    const int64_t nblk = cols >> 4;
    const uint16_t *xr = x + row * cols;
    uint32_t A = 0;
    for (int64_t blk = lane; blk < nblk; blk += 64) {
        Blk b;
        load_blk(b, xr + 16 * blk);
        A = max(A, unpack_blk(b).amax);
    }
    A = wave_max_u32(A);
    const float s = u2f(A) / 2688.0f;
    if (lane == 0)
        ts[row] = s;
    const ScaleK k = scale_k(s);
    for (int64_t blk = lane; blk < nblk; blk += 64) {
        Blk b;
        load_blk(b, xr + 16 * blk);
        emit_blk(b, unpack_blk(b), k, codes + row * (cols >> 1) + 8 * blk,
                 bs + row * (cols >> 4) + blk);
    }
}

// ---------------------------------------------------------------------------
// Export: scope amax, FP32 scales, then a flat pass over the blocks.
// ---------------------------------------------------------------------------
__global__ void zero_u32_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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
    const int64_t e = (int64_t)blockIdx.x / chunks;
    const int64_t ch = (int64_t)blockIdx.x - e * chunks;
    const int64_t n_scope = b ? 2 * n_per : n_per;
    uint32_t m = 0;
#pragma unroll
    for (int it = 0; it < AMAX_LOADS; it++) {
        const int64_t i = ch * AMAX_CHUNK + (int64_t)it * 2048 + 8 * threadIdx.x;
        if (i < n_scope) {
            const uint16_t *p = (i < n_per) ? a + e * n_per + i : b + e * n_per + (i - n_per);
            const uint4 q = ld_nt16(p);
            m = pk_max_u16(m, pk_max_u16(pk_max_u16(q.x & 0x7FFF7FFFu, q.y & 0x7FFF7FFFu),
                                         pk_max_u16(q.z & 0x7FFF7FFFu, q.w & 0x7FFF7FFFu)));
        }
    }
    uint32_t h = wave_max_u32(hmax_u16(m));
    if (__lane_id() == 0)
        part[threadIdx.x >> 6] = h;
    __syncthreads();
    if (threadIdx.x == 0) {
        h = max(max(part[0], part[1]), max(part[2], part[3]));
        atomicMax(amax + e, h);
    }
}

// amax bits -> s = fp32(amax / 2688), in place.
__global__ void scope_finalize_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float s = u2f(p[i] << 16) / 2688.0f;
        p[i] = f2u(s);
    }
}

// Flat export pass over one tensor of nblk blocks; block j belongs to scope
// j / bps (bps = blocks per scope).  Step t covers blocks 64 t .. 64 t + 63;
// when bps >= 64 a step spans at most two scopes, so the scope comes from one
// wave-uniform division and a compare.
__device__ __forceinline__ void scoped_step(const Blk &blk, int64_t t, int lane, int64_t nblk,
                                            int64_t bps, const float *__restrict__ scope_s,
                                            uint8_t *__restrict__ codes, uint8_t *__restrict__ bs)
{
    const int64_t j = 64 * t + lane;
    int64_t e;
    if (bps >= 64) {
        const int64_t e0 = (64 * t) / bps;                 // wave-uniform
        e = e0 + (j >= (e0 + 1) * bps ? 1 : 0);
    } else {
        e = j / bps;
    }
    if (j >= nblk)
        return;
    const ScaleK k = scale_k(scope_s[e]);
    emit_blk(blk, unpack_blk(blk), k, codes + 8 * j, bs + j);
}

__global__ void __launch_bounds__(256) nvfp4_scoped_kernel(const uint16_t *__restrict__ x,
                                                           int64_t nblk, int64_t bps,
                                                           const float *__restrict__ scope_s,
                                                           uint8_t *__restrict__ codes,
                                                           uint8_t *__restrict__ bs)
{
    const int lane = __lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t nsteps = (nblk + 63) >> 6;
    for (int64_t t = (int64_t)blockIdx.x * WAVES_PER_WG + wave_in_group(); t < nsteps;
         t += nwaves) {
        const int64_t j = 64 * t + lane;
        Blk b;
        if (j < nblk)
            load_blk(b, x + 16 * j);
        else
            zero_blk(b);
        scoped_step(b, t, lane, nblk, bps, scope_s, codes, bs);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// Workgroups for a grid-stride kernel: OVERSUBSCRIBE times what the device
// holds at once (measured: more wavefronts in flight keep more loads
// outstanding than in-wave prefetching), at most one wavefront per unit of
// work.
constexpr int OVERSUBSCRIBE = 8;

static unsigned grid_for(const void *kernel, int64_t work_waves)
{
    int64_t w = resident_workgroups(kernel, 64 * WAVES_PER_WG) * WAVES_PER_WG * OVERSUBSCRIBE;
    if (w > work_waves)
        w = work_waves;
    return (unsigned)((w + WAVES_PER_WG - 1) / WAVES_PER_WG);
}

template <int NB, bool FULL>
static void launch_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                         uint8_t *bs, float *ts, hipStream_t stream)
{
    const dim3 grid(grid_for((const void *)nvfp4_token_kernel<NB, FULL>, rows));
    hipLaunchKernelGGL((nvfp4_token_kernel<NB, FULL>), grid, dim3(64 * WAVES_PER_WG), 0, stream,
                       x, rows, cols, codes, bs, ts);
}

hipError_t launch_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                  uint8_t *bs, float *ts, hipStream_t stream)
{
    const int64_t nblk = cols >> 4;
    const int64_t nb = (nblk + 63) / 64;
    const bool full = nblk == 64 * nb;
    switch (nb) {
    case 1: full ? launch_token<1, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_token<1, false>(x, rows, cols, codes, bs, ts, stream); break;
    case 2: full ? launch_token<2, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_token<2, false>(x, rows, cols, codes, bs, ts, stream); break;
    case 3: full ? launch_token<3, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_token<3, false>(x, rows, cols, codes, bs, ts, stream); break;
    case 4: full ? launch_token<4, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_token<4, false>(x, rows, cols, codes, bs, ts, stream); break;
    default: {
        const dim3 g2((unsigned)((rows + WAVES_PER_WG - 1) / WAVES_PER_WG));
        hipLaunchKernelGGL(nvfp4_token_long_kernel, g2, dim3(64 * WAVES_PER_WG), 0, stream, x,
                           rows, cols, codes, bs, ts);
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
    const int64_t nblk = n_experts * n_per / 16;
    const int64_t bps = n_per / 16;
    const dim3 grid(grid_for((const void *)nvfp4_scoped_kernel, (nblk + 63) / 64));
    const dim3 block(64 * WAVES_PER_WG);
    hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, gate, nblk, bps,
                       (const float *)scope_scales, gc, gbs);
    if (up)
        hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, up, nblk, bps,
                           (const float *)scope_scales, uc, ubs);
    return hipGetLastError();
}

}  // namespace mxq
