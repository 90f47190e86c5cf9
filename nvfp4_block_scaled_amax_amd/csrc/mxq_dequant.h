// mxq_dequant.h -- exact BF16 dequantization of MXFP8 and NVFP4 codes, shared
// by the dequant kernels and the kernels that emit the dequantized operand
// next to the codes (the dequantized-backward paragraph of the page "Miles:
// end-to-end MXFP8 and per-token NVFP4 RL on Blackwell").  y = BF16(dec(code)
// * dec(scale) [* s]), rounded once from the exact product, ties to even,
// saturating at 0x7F7F.
//
// MXFP8.  dec(c) 2^e has at most 4 significant bits, so it is a BF16 value
// unless it lies below the BF16 normal range or overflows.  One
// v_cvt_scalef32_pk_bf16_fp8 per element pair computes it (the E8M0 byte sits
// in the exponent field of the scale operand); measured exact for every code
// and every scale byte, BF16 subnormals included, except that it returns Inf
// instead of saturating, which only happens for scale bytes >= 247 -- those
// take an exact path.
//
// NVFP4.  dec(c) dec(b) is exact (at most 6 bits) and p = fp32(dec(c) dec(b) s)
// is its one f32 rounding.  The f32 -> BF16 conversion (nearest-even) is the
// second; the two can differ from one rounding of the exact product only when
// p lands exactly on a BF16 midpoint without being exact.  Within a block,
// dec(c) dec(b) s = 2^j d s or 2^j 3 d s, so p is 2^j fp32(d s) or
// 2^j fp32(3 d s): checking those two products once per block settles every
// element.  Blocks where that check fires, whose values could overflow BF16,
// or whose FP32 scale is below 2^-100 take an exact binary64 path.
#pragma once
#include "mxq_device.h"

namespace mxq {

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

// Eight BF16 (16 bytes) of one MXFP8 chunk: codes cw (8 bytes), scales sw
// (one byte per element for the columnwise layout, else the chunk's one
// scale byte in every byte).
template <bool COL>
__device__ __forceinline__ u32x4_t mx_chunk(uint2 cq, uint2 sq)
{
    const uint32_t cw[2] = {cq.x, cq.y}, sw[2] = {sq.x, sq.y};
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const uint32_t c = cw[j], s = sw[j];
        if constexpr (!COL) {
            o[2 * j] = mx_pair<false>(c, (s & 0xFFu) << 23);
            o[2 * j + 1] = mx_pair<true>(c, (s & 0xFFu) << 23);
        } else {
            // Each conversion applies one scale to both codes of a pair:
            // convert under each element's scale and keep its half.
            const uint32_t lo_a = mx_pair<false>(c, (s & 0xFFu) << 23);
            const uint32_t lo_b = mx_pair<false>(c, ((s >> 8) & 0xFFu) << 23);
            const uint32_t hi_a = mx_pair<true>(c, ((s >> 16) & 0xFFu) << 23);
            const uint32_t hi_b = mx_pair<true>(c, (s >> 24) << 23);
            o[2 * j] = __builtin_amdgcn_perm(lo_b, lo_a, 0x07060100u);
            o[2 * j + 1] = __builtin_amdgcn_perm(hi_b, hi_a, 0x07060100u);
        }
    }
    if (any_byte_ge247(sw[0]) | any_byte_ge247(sw[1])) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const uint32_t c = cw[j], s = sw[j];
            o[2 * j] = pack2(mx_deq1_exact(c & 0xFF, s & 0xFF),
                             mx_deq1_exact((c >> 8) & 0xFF, (s >> 8) & 0xFF));
            o[2 * j + 1] = pack2(mx_deq1_exact((c >> 16) & 0xFF, (s >> 16) & 0xFF),
                                 mx_deq1_exact(c >> 24, s >> 24));
        }
    }
    return o;
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
    return ((int)((f2u(p) & 0xFFFFu) == 0x8000u) & (int)(__builtin_fmaf(a, s, -p) != 0.0f)) != 0;
}

// Exact BF16 pair for one code byte (two E2M1 codes) under (d, s).  Inlined
// into the dequant kernel (an out-of-line call there cost 8192 x 2048
// 9.8 -> 10.8 us); the one-pass quantize + dequant kernels call it out of
// line, since inlined it would add to their register pressure (the
// quantizers spilled when their own binary64 path was inlined).
__device__ __forceinline__ uint32_t nv_pair_exact_inl(uint32_t byte, float d, float s)
{
    const float2_t v = e2m1_values(byte);
    return pack2(bf16_from_f64((double)v[0] * (double)d * (double)s),
                 bf16_from_f64((double)v[1] * (double)d * (double)s));
}
static __device__ __attribute__((noinline)) uint32_t nv_pair_exact(uint32_t byte, float d, float s)
{
    return nv_pair_exact_inl(byte, d, s);
}

// Whether a block with decoded block scale d under FP32 scale s takes the
// fast path: every element's f32 product rounds to the same BF16 as the
// exact product (no tie hazard, no overflow, s not tiny).
__device__ __forceinline__ bool nv_fast(float d, float s)
{
    // Bitwise, not short-circuit: all four tests are cheap, and evaluating
    // them all keeps the check free of branches.
    return ((int)(s >= NV_FAST_MIN_S) & (int)(fabsf((6.0f * d) * s) <= BF16_MAX) &
            (int)!bf16_tie_hazard(d, s) & (int)!bf16_tie_hazard(3.0f * d, s)) != 0;
}

// Fast-path BF16 pair of the two E2M1 codes in byte J of w (the conversion
// reads the byte itself, so no shift is spent on it): dec(c) d is exact in
// f32, and the product with s is rounded to f32 and then to BF16.
template <int J>
__device__ __forceinline__ uint32_t nv_pair_fast(uint32_t w, float d, float s)
{
    const float2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J);
    const bf16x2v_t r = {(__bf16)((v[0] * d) * s), (__bf16)((v[1] * d) * s)};
    return __builtin_bit_cast(uint32_t, r);
}

// Eight BF16 (16 bytes) of one NVFP4 chunk: 8 codes (4 bytes) of a block
// with decoded block scale d under FP32 scale s, on the fast path.
__device__ __forceinline__ u32x4_t nv_chunk_fast(uint32_t cw, float d, float s)
{
    return u32x4_t{nv_pair_fast<0>(cw, d, s), nv_pair_fast<1>(cw, d, s),
                   nv_pair_fast<2>(cw, d, s), nv_pair_fast<3>(cw, d, s)};
}

// The same eight BF16 on the exact binary64 path.
__device__ __forceinline__ u32x4_t nv_chunk_exact(uint32_t cw, float d, float s)
{
    u32x4_t o;
    for (int j = 0; j < 4; j++)
        o[j] = nv_pair_exact_inl((cw >> (8 * j)) & 0xFFu, d, s);
    return o;
}

// Sixteen BF16 of one NVFP4 block (codes c0: elements 0..7, c1: 8..15), the
// fast-path check made once for the block.
__device__ __forceinline__ void nv_block16(uint32_t c0, uint32_t c1, float d, float s,
                                           u32x4_t &lo, u32x4_t &hi)
{
    if (nv_fast(d, s)) {
        lo = nv_chunk_fast(c0, d, s);
        hi = nv_chunk_fast(c1, d, s);
    } else {
        for (int j = 0; j < 4; j++) {
            lo[j] = nv_pair_exact((c0 >> (8 * j)) & 0xFFu, d, s);
            hi[j] = nv_pair_exact((c1 >> (8 * j)) & 0xFFu, d, s);
        }
    }
}

}  // namespace mxq
