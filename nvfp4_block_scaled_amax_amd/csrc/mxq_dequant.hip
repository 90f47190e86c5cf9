// mxq_dequant.hip -- BF16 dequantization of the exact forward operands (the
// dequantized-backward paragraph of the page "Miles: end-to-end MXFP8 and
// per-token NVFP4 RL on Blackwell").  y = BF16(dec(code) * dec(scale) [* s]),
// rounded once from the exact product, ties to even, saturating at 0x7F7F.
//
// Work unit: 16 consecutive elements of the flattened [rows][cols] array
// (cols is a multiple of 16, so the 16 share a row, and for NVFP4 a block):
// one 16-byte (MXFP8) or 8-byte (NVFP4) code load, 32 bytes of BF16 out.
// Grid-stride over units with many wavefronts per SIMD.
//
// MXFP8.  dec(c) 2^e has at most 4 significant bits, so it is a BF16 value
// unless it lies below the BF16 normal range or overflows.  One
// v_cvt_scalef32_pk_bf16_fp8 per element pair computes it (the E8M0 byte sits
// in the exponent field of the scale operand); measured exact for every code
// and every scale byte, BF16 subnormals included, except that it returns Inf
// instead of saturating, which only happens for scale bytes >= 247 -- those
// units take an exact path.  Rowwise: one scale per unit (index f / 32).
// Columnwise: one scale per element, so each pair is converted twice and the
// halves merged.
//
// NVFP4.  dec(c) dec(b) is exact (at most 6 bits) and p = fp32(dec(c) dec(b) s)
// is its one f32 rounding.  The f32 -> BF16 conversion (nearest-even) is the
// second; the two can differ from one rounding of the exact product only when
// p lands exactly on a BF16 midpoint without being exact.  Within a block,
// dec(c) dec(b) s = 2^j d s or 2^j 3 d s, so p is 2^j fp32(d s) or
// 2^j fp32(3 d s): checking those two products once per block settles every
// element.  Blocks where that check fires, whose values could overflow BF16,
// or whose FP32 scale is below 2^-100 take an exact binary64 path.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int WAVES_PER_WG = 4;
constexpr int OVERSUBSCRIBE = 8;
constexpr float NV_FAST_MIN_S = 0x1p-100f;
constexpr float BF16_MAX = 0x1.FEp127f;

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// f32 -> BF16 bits, nearest-even, saturating (for finite inputs, or Inf from
// an f32 overflow).
__device__ __forceinline__ uint32_t bf16_rne_sat(uint32_t u)
{
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((r & 0x7F80u) == 0x7F80u) ? ((r & 0x8000u) | 0x7F7Fu) : r;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Exact BF16 of dec(c) * 2^(b - 127): the product is exact in f32 (possibly
// subnormal, at least 2^-136) or overflows to Inf, which saturates.
__device__ __forceinline__ uint32_t mx_deq1_exact(uint32_t c, uint32_t b)
{
    const float y = ldexpf(e4m3_value(c), (int)b - 127);
    return bf16_rne_sat(f2u(y));
}

// Two codes (bytes of the low or high half of `w`) under one scale byte.
template <bool HI>
__device__ __forceinline__ uint32_t mx_pair(uint32_t w, uint32_t scale_bits)
{
    const bf16x2v_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, u2f(scale_bits), HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 1 iff some byte of w is >= 247.
__device__ __forceinline__ uint32_t any_byte_ge247(uint32_t w)
{
    return (((w & 0x7F7F7F7Fu) + 0x09090909u) & w & 0x80808080u) != 0u;
}

// Unsigned division of n < 2^32 by a fixed d via a multiply and a shift
// (round-up method: m = floor(2^32 (2^l - d) / d) + 1, l = ceil(log2 d)).
struct Div {
    uint32_t m, l;
};
__device__ __forceinline__ uint32_t udiv(uint32_t n, Div d)
{
    return (uint32_t)(((uint64_t)__umulhi(n, d.m) + n) >> d.l);
}

template <bool COL>
__global__ void __launch_bounds__(256) dequant_mxfp8_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t units, int64_t cols,
                                                            Div per_row, uint16_t *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
        const int64_t f = u * 16;
        const uint4 cq = ld_nt16(codes + f);
        const uint32_t cw[4] = {cq.x, cq.y, cq.z, cq.w};
        uint32_t o[8];
        if constexpr (!COL) {
            const uint32_t b = scales[f >> 5];
            const uint32_t sbits = b << 23;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                o[2 * j] = mx_pair<false>(cw[j], sbits);
                o[2 * j + 1] = mx_pair<true>(cw[j], sbits);
            }
            if (b >= 247u) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    o[2 * j] = pack2(mx_deq1_exact(cw[j] & 0xFF, b),
                                     mx_deq1_exact((cw[j] >> 8) & 0xFF, b));
                    o[2 * j + 1] = pack2(mx_deq1_exact((cw[j] >> 16) & 0xFF, b),
                                         mx_deq1_exact(cw[j] >> 24, b));
                }
            }
        } else {
            const uint32_t row = udiv((uint32_t)u, per_row);
            const int64_t k = f - (int64_t)row * cols;
            const uint4 sq = ld16(scales + (int64_t)(row >> 5) * cols + k);
            const uint32_t sw[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t s = sw[j];
                const uint32_t lo_a = mx_pair<false>(cw[j], (s & 0xFFu) << 23);
                const uint32_t lo_b = mx_pair<false>(cw[j], ((s >> 8) & 0xFFu) << 23);
                const uint32_t hi_a = mx_pair<true>(cw[j], ((s >> 16) & 0xFFu) << 23);
                const uint32_t hi_b = mx_pair<true>(cw[j], (s >> 24) << 23);
                o[2 * j] = __builtin_amdgcn_perm(lo_b, lo_a, 0x07060100u);
                o[2 * j + 1] = __builtin_amdgcn_perm(hi_b, hi_a, 0x07060100u);
            }
            if (any_byte_ge247(sw[0]) | any_byte_ge247(sw[1]) | any_byte_ge247(sw[2]) |
                any_byte_ge247(sw[3])) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t c = cw[j], s = sw[j];
                    o[2 * j] = pack2(mx_deq1_exact(c & 0xFF, s & 0xFF),
                                     mx_deq1_exact((c >> 8) & 0xFF, (s >> 8) & 0xFF));
                    o[2 * j + 1] = pack2(mx_deq1_exact((c >> 16) & 0xFF, (s >> 16) & 0xFF),
                                         mx_deq1_exact(c >> 24, s >> 24));
                }
            }
        }
        st_nt16(out + f, o[0], o[1], o[2], o[3]);
        st_nt16(out + f + 8, o[4], o[5], o[6], o[7]);
    }
}

// BF16 of the exact product y (binary64, exact), nearest-even, saturating.
__device__ __forceinline__ uint32_t bf16_from_f64(double y)
{
    const uint32_t sign = signbit(y) ? 0x8000u : 0u;
    const double a = fabs(y);
    if (a >= (double)BF16_MAX)
        return sign | 0x7F7Fu;
    if (a == 0.0)
        return sign;
    int e = 0;
    (void)frexp(a, &e);
    int E = e - 1;
    if (E < -126)
        E = -126;
    const double n = rint(ldexp(a, 7 - E));        // exact scaling, nearest-even
    const float r = (float)ldexp(n, E - 7);         // a BF16 value: exact in f32
    return sign | (f2u(r) >> 16);
}

// 1 iff fp32(a * s) is a BF16 midpoint that is not the exact product.
__device__ __forceinline__ bool bf16_tie_hazard(float a, float s)
{
    const float p = a * s;
    return (f2u(p) & 0xFFFFu) == 0x8000u && __builtin_fmaf(a, s, -p) != 0.0f;
}

// Exact BF16 pair for one code byte (two E2M1 codes) under (d, s).
__device__ __attribute__((noinline)) uint32_t nv_pair_exact(uint32_t byte, float d, float s)
{
    const float2_t v = e2m1_values(byte);
    return pack2(bf16_from_f64((double)v[0] * (double)d * (double)s),
                 bf16_from_f64((double)v[1] * (double)d * (double)s));
}

__global__ void __launch_bounds__(256) dequant_nvfp4_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ bscales,
                                                            const float *__restrict__ fp32_scales,
                                                            int64_t units, Div per_scale,
                                                            uint16_t *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
        const uint2 cq = *reinterpret_cast<const uint2 *>(codes + u * 8);
        const float d = e4m3_value(bscales[u]);
        const float s = fp32_scales[udiv((uint32_t)u, per_scale)];
        uint32_t o[8];
        const bool fast = s >= NV_FAST_MIN_S && fabsf((6.0f * d) * s) <= BF16_MAX &&
                          !bf16_tie_hazard(d, s) && !bf16_tie_hazard(3.0f * d, s);
        if (fast) {
            const uint32_t cw[2] = {cq.x, cq.y};
#pragma unroll
            for (int w = 0; w < 2; w++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float2_t v = e2m1_values((cw[w] >> (8 * j)) & 0xFFu);
                    const bf16x2v_t r = {(__bf16)((v[0] * d) * s), (__bf16)((v[1] * d) * s)};
                    o[4 * w + j] = __builtin_bit_cast(uint32_t, r);
                }
        } else {
            const uint32_t cw[2] = {cq.x, cq.y};
            for (int i = 0; i < 8; i++)
                o[i] = nv_pair_exact((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu, d, s);
        }
        st_nt16(out + u * 16, o[0], o[1], o[2], o[3]);
        st_nt16(out + u * 16 + 8, o[4], o[5], o[6], o[7]);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static Div make_div(uint32_t d)
{
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d)
        l++;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return Div{(uint32_t)m, l};
}

template <class K>
static unsigned grid_for(K kernel, int64_t units)
{
    int64_t wgs = resident_workgroups((const void *)kernel, 256) * OVERSUBSCRIBE;
    const int64_t need = (units + 255) / 256;
    if (wgs > need)
        wgs = need;
    return (unsigned)(wgs < 1 ? 1 : wgs);
}

hipError_t launch_dequant_mxfp8(bool col, const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream)
{
    const int64_t units = rows * cols / 16;     // < 2^32: checked by the caller
    const Div per_row = make_div((uint32_t)(cols / 16));
    if (col)
        hipLaunchKernelGGL((dequant_mxfp8_kernel<true>), dim3(grid_for(dequant_mxfp8_kernel<true>, units)),
                           dim3(256), 0, stream, codes, scales, units, cols, per_row, out);
    else
        hipLaunchKernelGGL((dequant_mxfp8_kernel<false>), dim3(grid_for(dequant_mxfp8_kernel<false>, units)),
                           dim3(256), 0, stream, codes, scales, units, cols, per_row, out);
    return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t *codes, const uint8_t *bscales, const float *fs,
                                int64_t rows_per_scale, int64_t rows, int64_t cols, uint16_t *out,
                                hipStream_t stream)
{
    const int64_t units = rows * cols / 16;     // < 2^32: checked by the caller
    const int64_t per = (cols / 16) * rows_per_scale;   // units per FP32 scale
    const Div per_scale = make_div((uint32_t)(per < units ? per : units));
    hipLaunchKernelGGL(dequant_nvfp4_kernel, dim3(grid_for(dequant_nvfp4_kernel, units)), dim3(256),
                       0, stream, codes, bscales, fs, units, per_scale, out);
    return hipGetLastError();
}

}  // namespace mxq
