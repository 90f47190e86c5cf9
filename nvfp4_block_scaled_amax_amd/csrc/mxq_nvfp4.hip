// mxq_nvfp4.hip -- NVFP4 quantizers: per-token FP32 scale (the per-token
// activation paragraphs of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell") and scoped weight export with one FP32 scale per
// gate/up pair or per tensor (its gate/up pairing paragraph).  The arithmetic
// is the page's NVFP4 format paragraph under the readings stated in mxq.h:
//   s = fp32(A_scope / 2688), b = E4M3(A_block / (6 s)), c = E2M1(x / (dec(b) s)).
//
// Layout.  One wavefront owns one row.  The row is read in chunks of 512
// elements; in chunk c lane l holds elements 512c + 8l .. +7 (one 16-byte
// load), so a 16-element block is the lane pair (2m, 2m+1): the block amax is
// an in-lane max and one DPP exchange, the token amax a wavefront reduction.
// For rows up to 4096 elements the whole row stays in registers (one HBM
// read); longer rows are read twice.
//
// Exact decisions without division.  Dividing per element is too slow and
// multiplying by a rounded reciprocal is not exact.  Instead every decision is
// bracketed: with r ~ 1/D (D = 6s for block scales, dec(b) s for codes) built
// from v_rcp_f32 and rounded products, relative error below 2^-21, the kernel
// forms q_lo = x * r(1 - 2^-19) and q_hi = x * r(1 + 2^-19), which satisfy
// |q_lo| < |x / D| < |q_hi| (strictly; all operands normal on this path).
// Rounding is monotone, so when the hardware's exact nearest-even conversions
// of q_lo and q_hi agree, that code is the exactly rounded code of x / D.
// When they differ (x / D within 2^-18 of a rounding midpoint, which random
// data hits a few times per million elements), the lane decides exactly in
// binary64: |x| against midpoint * D, a product with at most 31 significant
// bits, hence exact.  Rows whose scope amax is below 2^-90 (an FP32 scale
// below 2^-101) would take the reciprocals out of the normal range; they go to
// a binary64 path that divides once per element.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int ROWS_PER_WG = 4;               // one row per wavefront
constexpr uint32_t FAST_MIN_AMAX = 0x1280u;  // BF16 bits of 2^-90
constexpr float BRACKET_LO = 1.0f - 0x1p-19f;
constexpr float BRACKET_HI = 1.0f + 0x1p-19f;
constexpr float ONE_SIXTH = 1.0f / 6.0f;

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

// Fix the nibbles where the bracket codes differ.  lo/hi: 8 codes each; xs:
// the 8 inputs as f32; D = d s exactly as (d, s).
__device__ __attribute__((noinline)) uint32_t codes_exact(uint32_t lo, uint32_t hi,
                                                          const float *xs, float d, float s)
{
    const double D = (double)d * (double)s;
    uint32_t out = lo;
#pragma unroll 1
    for (int i = 0; i < 8; i++) {
        const uint32_t a = (lo >> (4 * i)) & 0xFu, b = (hi >> (4 * i)) & 0xFu;
        if (a == b)
            continue;
        const uint32_t klo = a & 7u, khi = b & 7u;     // khi == klo + 1
        const double t = (e2m1_value_f64(klo) + e2m1_value_f64(khi)) * D;  // 2 * mid * D
        const double ax = 2.0 * fabs((double)xs[i]);
        uint32_t k;
        if (ax > t)
            k = khi;
        else if (ax < t)
            k = klo;
        else
            k = (klo & 1u) ? khi : klo;
        out = (out & ~(0xFu << (4 * i))) | ((k | (a & 8u)) << (4 * i));
    }
    return out;
}

// One 8-element slice (a lane's half of a 16-block) on the fast path.
// Returns 8 packed codes; *b_out gets the block scale byte.
__device__ __forceinline__ uint32_t quant8_fast(const uint32_t (&v)[4], uint32_t bamax, float s,
                                                float inv_s, float r6_lo, float r6_hi,
                                                uint32_t *b_out)
{
    const float A = u2f(bamax << 16);
    const float plo = fminf(A * r6_lo, 448.0f);
    const float phi = fminf(A * r6_hi, 448.0f);
    const uint32_t bb = e4m3_pair_rne(plo, phi);
    uint32_t b = bb & 0xFFu;
    if (b != (bb >> 8))
        b = block_scale_exact(A, s, b);
    *b_out = b;
    if (b == 0)
        return 0u;
    const float d = e4m3_value(b);
    const float r = __builtin_amdgcn_rcpf(d) * inv_s;
    const float rlo = r * BRACKET_LO, rhi = r * BRACKET_HI;
    float xs[8];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        xs[2 * j] = bf16_lo(v[j]);
        xs[2 * j + 1] = bf16_hi(v[j]);
    }
    uint32_t lo = 0, hi = 0;
    lo = e2m1_pair<0>(lo, xs[0] * rlo, xs[1] * rlo);
    hi = e2m1_pair<0>(hi, xs[0] * rhi, xs[1] * rhi);
    lo = e2m1_pair<1>(lo, xs[2] * rlo, xs[3] * rlo);
    hi = e2m1_pair<1>(hi, xs[2] * rhi, xs[3] * rhi);
    lo = e2m1_pair<2>(lo, xs[4] * rlo, xs[5] * rlo);
    hi = e2m1_pair<2>(hi, xs[4] * rhi, xs[5] * rhi);
    lo = e2m1_pair<3>(lo, xs[6] * rlo, xs[7] * rlo);
    hi = e2m1_pair<3>(hi, xs[6] * rhi, xs[7] * rhi);
    if (lo != hi)
        lo = codes_exact(lo, hi, xs, d, s);
    return lo;
}

// One 8-element slice on the binary64 path (tiny scopes).
__device__ __attribute__((noinline)) uint32_t quant8_f64(const uint32_t *v, uint32_t bamax,
                                                         float s, uint32_t *b_out)
{
    const double A = (double)u2f(bamax << 16);
    const uint32_t b = e4m3_code_f64(A / (6.0 * (double)s));
    *b_out = b;
    if (b == 0)
        return 0u;
    const double D = (double)e4m3_value(b) * (double)s;
    uint32_t out = 0;
    for (int i = 0; i < 8; i++) {
        const uint32_t bits = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
        const double xv = (double)u2f(bits << 16);
        const uint32_t k = e2m1_code_f64(fabs(xv) / D) | ((bits >> 12) & 8u);
        out |= k << (4 * i);
    }
    return out;
}

// Block amax of this lane's 8 values, exchanged with the partner lane.
__device__ __forceinline__ uint32_t slice_amax(const uint32_t (&v)[4])
{
    const uint32_t m = pk_max_u16(pk_max_u16(v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu),
                                  pk_max_u16(v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu));
    const uint32_t h = hmax_u16(m);
    return max(h, dpp<DPP_XOR1>(h));
}

// Quantize one slice and store its codes (and, from even lanes, the block
// scale).  k0 = index of the slice's first element in the row.
__device__ __forceinline__ void emit_slice(const uint32_t (&v)[4], uint32_t bamax, uint32_t A,
                                           float s, float inv_s, float r6_lo, float r6_hi,
                                           int64_t k0, uint8_t *__restrict__ codes_row,
                                           uint8_t *__restrict__ bs_row, int lane)
{
    uint32_t b, c;
    if (A >= FAST_MIN_AMAX) {
        c = quant8_fast(v, bamax, s, inv_s, r6_lo, r6_hi, &b);
    } else if (A == 0) {
        b = 0;
        c = 0;
    } else {
        c = quant8_f64(v, bamax, s, &b);
    }
    st_nt4(codes_row + (k0 >> 1), c);
    if ((lane & 1) == 0)
        bs_row[k0 >> 4] = (uint8_t)b;
}

// SCOPED == false: the scope is the row itself (per-token scale, written to
// token_scales).  SCOPED == true: the scope amax (BF16 bits as u32) is
// scope_amax[row / rows_per_scope]; rows at or beyond `rows_a` come from the
// second tensor (x_b, codes_b, bs_b) -- the up half of a gate/up pair.
// NC > 0: the row (<= 512 * NC elements) is kept in registers; NC == 0:
// generic length, read twice.
template <int NC, bool SCOPED>
__global__ void __launch_bounds__(256) nvfp4_kernel(
    const uint16_t *__restrict__ x_a, const uint16_t *__restrict__ x_b, int64_t rows_a,
    int64_t rows, int64_t cols, uint8_t *__restrict__ codes_a, uint8_t *__restrict__ codes_b,
    uint8_t *__restrict__ bs_a, uint8_t *__restrict__ bs_b, float *__restrict__ token_scales,
    const uint32_t *__restrict__ scope_amax, int64_t rows_per_scope)
{
    const int64_t row_all = (int64_t)blockIdx.x * ROWS_PER_WG + (threadIdx.x >> 6);
    if (row_all >= rows)
        return;
    const int lane = __lane_id();
    const bool second = SCOPED && row_all >= rows_a;
    const int64_t row = second ? row_all - rows_a : row_all;
    const uint16_t *xr = (second ? x_b : x_a) + row * cols;
    uint8_t *codes_row = (second ? codes_b : codes_a) + row * (cols >> 1);
    uint8_t *bs_row = (second ? bs_b : bs_a) + row * (cols >> 4);

    if constexpr (NC > 0) {
        uint32_t v[NC][4];
        uint32_t bam[NC];
        uint32_t rmax = 0;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int64_t k0 = 512 * c + 8 * lane;
            if (k0 < cols) {
                const uint4 q = ld_nt16(xr + k0);
                v[c][0] = q.x; v[c][1] = q.y; v[c][2] = q.z; v[c][3] = q.w;
            } else {
                v[c][0] = v[c][1] = v[c][2] = v[c][3] = 0u;
            }
        }
#pragma unroll
        for (int c = 0; c < NC; c++) {
            bam[c] = slice_amax(v[c]);
            rmax = max(rmax, bam[c]);
        }
        uint32_t A;
        if constexpr (SCOPED) {
            A = scope_amax[row / rows_per_scope];
        } else {
            A = wave_max_u32(rmax);
        }
        const float s = u2f(A << 16) / 2688.0f;
        if (!SCOPED && lane == 0)
            token_scales[row] = s;
        const float inv_s = __builtin_amdgcn_rcpf(s);
        const float r6 = inv_s * ONE_SIXTH;
        const float r6_lo = r6 * BRACKET_LO, r6_hi = r6 * BRACKET_HI;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int64_t k0 = 512 * c + 8 * lane;
            if (k0 < cols)
                emit_slice(v[c], bam[c], A, s, inv_s, r6_lo, r6_hi, k0, codes_row, bs_row, lane);
        }
    } else {
        uint32_t A;
        if constexpr (SCOPED) {
            A = scope_amax[row / rows_per_scope];
        } else {
            uint32_t rmax = 0;
            for (int64_t k0 = 8 * lane; k0 < cols; k0 += 512) {
                const uint4 q = ld16(xr + k0);
                const uint32_t v[4] = {q.x, q.y, q.z, q.w};
                const uint32_t m = pk_max_u16(pk_max_u16(v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu),
                                              pk_max_u16(v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu));
                rmax = max(rmax, hmax_u16(m));
            }
            A = wave_max_u32(rmax);
        }
        const float s = u2f(A << 16) / 2688.0f;
        if (!SCOPED && lane == 0)
            token_scales[row] = s;
        const float inv_s = __builtin_amdgcn_rcpf(s);
        const float r6 = inv_s * ONE_SIXTH;
        const float r6_lo = r6 * BRACKET_LO, r6_hi = r6 * BRACKET_HI;
        // Uniform trip count so the DPP exchange sees every lane active.
        for (int64_t base = 0; base < cols; base += 512) {
            const int64_t k0 = base + 8 * lane;
            uint32_t v[4] = {0u, 0u, 0u, 0u};
            if (k0 < cols) {
                const uint4 q = ld16(xr + k0);
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            }
            const uint32_t bam = slice_amax(v);
            if (k0 < cols)
                emit_slice(v, bam, A, s, inv_s, r6_lo, r6_hi, k0, codes_row, bs_row, lane);
        }
    }
}

// ---------------------------------------------------------------------------
// Scope amax for the weight export: zero, reduce (atomic max per workgroup),
// and the final conversion of the amax bits to the FP32 scale.
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
            const uint4 q = ld16(p);
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

__global__ void scope_finalize_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float s = u2f(p[i] << 16) / 2688.0f;
        p[i] = f2u(s);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <bool SCOPED>
static hipError_t launch_nvfp4(const uint16_t *xa, const uint16_t *xb, int64_t rows_a,
                               int64_t rows, int64_t cols, uint8_t *ca, uint8_t *cb, uint8_t *ba,
                               uint8_t *bb, float *ts, const uint32_t *scope_amax,
                               int64_t rows_per_scope, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG));
    const dim3 block(64 * ROWS_PER_WG);
    const int64_t nc = (cols + 511) / 512;
#define MXQ_NVFP4_CASE(N)                                                                     \
    hipLaunchKernelGGL((nvfp4_kernel<N, SCOPED>), grid, block, 0, stream, xa, xb, rows_a, rows, \
                       cols, ca, cb, ba, bb, ts, scope_amax, rows_per_scope)
    switch (nc) {
    case 1: MXQ_NVFP4_CASE(1); break;
    case 2: MXQ_NVFP4_CASE(2); break;
    case 3: MXQ_NVFP4_CASE(3); break;
    case 4: MXQ_NVFP4_CASE(4); break;
    case 5:
    case 6: MXQ_NVFP4_CASE(6); break;
    case 7:
    case 8: MXQ_NVFP4_CASE(8); break;
    default: MXQ_NVFP4_CASE(0); break;
    }
#undef MXQ_NVFP4_CASE
    return hipGetLastError();
}

hipError_t launch_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                  uint8_t *bs, float *ts, hipStream_t stream)
{
    return launch_nvfp4<false>(x, nullptr, rows, rows, cols, codes, nullptr, bs, nullptr, ts,
                               nullptr, 1, stream);
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
    const int64_t rows_a = n_experts * rows;
    const int64_t rows_all = up ? 2 * rows_a : rows_a;
    hipError_t err = launch_nvfp4<true>(gate, up, rows_a, rows_all, cols, gc, uc, gbs, ubs,
                                        nullptr, amax, rows, stream);
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(scope_finalize_kernel, dim3(small_grid), dim3(256), 0, stream, amax,
                       n_experts);
    return hipGetLastError();
}

}  // namespace mxq
