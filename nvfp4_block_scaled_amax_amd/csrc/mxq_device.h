// mxq_device.h -- device-side helpers shared by the libmxq kernels (gfx950).
//
// Format facts used here (the pages name the formats; layouts are the
// textbook ones): BF16 = 1-8-7, E4M3 = 1-4-3 without infinities (max 448),
// E8M0 = 2^(b-127), E2M1 = 1-2-1 (max 6).
//
// Hardware conversions relied upon, each verified bit-exactly by the GPU
// tests against the CPU oracle on every input class the kernels feed them:
//   v_cvt_scalef32_pk_fp8_bf16: x / 2^E(scale) rounded to E4M3,
//       nearest-even, sign kept, exact for |x / 2^E| <= 448 (MXFP8 never
//       exceeds that: the scale is chosen so the block maximum fits).
//       Only the scale's exponent field E is used, so an E8M0 byte b placed
//       in the exponent field (b << 23) is the scale operand.
//   v_cvt_pk_fp8_f32: f32 -> E4M3 nearest-even; values >= 480 give NaN, so
//       callers clamp to 448 first.
//   v_cvt_scalef32_pk_fp4_f32 (scale 1.0): f32 -> E2M1 nearest-even on the
//       full f32 value, saturating at +-6, sign kept.
//   v_cvt_f32_fp8 / v_cvt_scalef32_pk_f32_fp4: exact decoders.
//   v_cvt_scalef32_pk_bf16_fp8: E4M3 x 2^E(scale) to BF16, exact except that
//       it overflows to Inf (instead of saturating) for scale bytes >= 247.
//   v_rcp_f32: reciprocal within 1 ulp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef unsigned uint2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// BF16 halves of a packed dword as f32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return u2f(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return u2f(v & 0xFFFF0000u); }

// Element-wise max of the two unsigned 16-bit halves (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    ushort2_t r = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                            __builtin_bit_cast(ushort2_t, b));
    return __builtin_bit_cast(uint32_t, r);
}

// Element-wise min of the two unsigned 16-bit halves (v_pk_min_u16).
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    ushort2_t r = __builtin_elementwise_min(__builtin_bit_cast(ushort2_t, a),
                                            __builtin_bit_cast(ushort2_t, b));
    return __builtin_bit_cast(uint32_t, r);
}

// Max of the two halves of a dword, as a u32 in [0, 0xFFFF].
__device__ __forceinline__ uint32_t hmax_u16(uint32_t a)
{
    uint32_t lo = a & 0xFFFFu, hi = a >> 16;
    return lo > hi ? lo : hi;
}

// Work-item, workgroup and lane indices straight from the hardware (the HIP
// blockIdx / threadIdx / gridDim accessors and __umulhi are device-library
// functions built with IEEE mode on, which the compiler will not inline into
// this library's IEEE-off kernels: each use would be a call).  Grid-stride
// kernels take their grid size as an argument.
__device__ __forceinline__ uint32_t tid() { return __builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ uint32_t wg_id() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ uint32_t lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
__device__ __forceinline__ uint32_t mulhi(uint32_t a, uint32_t b)
{
    return (uint32_t)(((uint64_t)a * b) >> 32);
}

// Index of this wavefront within its workgroup, as a wave-uniform value (so
// that everything derived from it lives in scalar registers).
__device__ __forceinline__ int wave_in_group()
{
    return __builtin_amdgcn_readfirstlane((int)(tid() >> 6));
}

// ---------------------------------------------------------------------------
// Cross-lane exchanges.  DPP patterns act within rows of 16 lanes; the
// gfx950 permlane swaps exchange rows (16-lane) and halves (32-lane).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// Reductions across lane ^ 16 and lane ^ 32 with the gfx950 permlane swaps.
// Called with both operands equal to v, a swap leaves one register holding
// the even 16-lane rows (or the low 32-lane half) in both slots of each pair
// and the other register the odd rows (or the high half); combining the two
// registers gives every lane the combination over its pair, whichever
// register holds which.
__device__ __forceinline__ uint32_t max16_u32(uint32_t v)
{
    uint2_t r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t max32_u32(uint32_t v)
{
    uint2_t r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t max16_pk_u16(uint32_t v)
{
    uint2_t r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return pk_max_u16(r[0], r[1]);
}
__device__ __forceinline__ uint32_t max32_pk_u16(uint32_t v)
{
    uint2_t r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return pk_max_u16(r[0], r[1]);
}

// Max over all 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp<DPP_XOR1>(v));
    v = max(v, dpp<DPP_XOR2>(v));
    v = max(v, dpp<DPP_HALF_MIRROR>(v));
    v = max(v, dpp<DPP_MIRROR>(v));
    v = max16_u32(v);
    v = max32_u32(v);
    return v;
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------

// f32 -> E4M3 nearest-even for 0 <= a, b <= 448 (codes in bits 0-7, 8-15).
__device__ __forceinline__ uint32_t e4m3_pair_rne(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float e4m3_value(uint32_t code)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// Two f32 -> two E2M1 codes (nearest-even, saturating, sign kept) placed in
// byte `SEL` of `old` (first value in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

__device__ __forceinline__ float2_t e2m1_values(uint32_t byte)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
}

// ---------------------------------------------------------------------------
// Exact decisions in binary64 (rare paths).  For q >= 0 given as an exact
// quotient rounded once to binary64: the exact quotients these kernels form
// are either on a rounding midpoint or at least ~2^-32 away from one in
// relative terms, far above binary64's 2^-53, so rounding the binary64
// quotient to the nearest format value gives the exactly rounded result.
// ---------------------------------------------------------------------------

// Nearest E4M3 magnitude code (0..0x7E) to q >= 0, ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_code_f64(double q)
{
    if (!(q < 448.0))
        return 0x7E;
    int e = 0;
    (void)frexp(q, &e);                 // q = f * 2^e, f in [.5, 1)
    int E = e - 1;                      // floor(log2 q)
    if (E < -6)
        E = -6;                         // subnormal grid 2^-9
    double n = rint(ldexp(q, 3 - E));   // q / 2^(E-3): exact scaling, RNE
    // n in [0, 16]; n == 16 moves to the next binade.
    int ni = (int)n;
    if (q < 0x1p-6) {                   // subnormal region: code = n (n may be 8 -> 0x08 = 2^-6)
        return (uint32_t)ni;
    }
    if (ni == 16) {
        E += 1;
        ni = 8;
    }
    return (uint32_t)(((E + 7) << 3) | (ni - 8));
}

// Nearest E2M1 magnitude code (0..7) to q >= 0, ties to even, saturating.
__device__ __forceinline__ uint32_t e2m1_code_f64(double q)
{
    // Midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 between codes k and k+1; at a
    // tie the even code wins.
    uint32_t k = 0;
    k += (q > 0.25);
    k += (q >= 0.75);
    k += (q > 1.25);
    k += (q >= 1.75);
    k += (q > 2.5);
    k += (q >= 3.5);
    k += (q > 5.0);
    return k;
}

// ---------------------------------------------------------------------------
// Global memory access (native vector types, so the nontemporal builtins
// apply: streaming data is touched once).
// ---------------------------------------------------------------------------
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_nt16(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
// Unsigned division of n < 2^32 by a fixed d via a multiply and a shift
// (round-up method: m = floor(2^32 (2^l - d) / d) + 1, l = ceil(log2 d)),
// exact for every n < 2^32 and 1 <= d < 2^32.
struct Div {
    uint32_t m, l;
};
__device__ __forceinline__ uint32_t udiv(uint32_t n, Div d)
{
    return (uint32_t)(((uint64_t)mulhi(n, d.m) + n) >> d.l);
}
static inline Div make_div(uint32_t d)
{
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d)
        l++;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return Div{(uint32_t)m, l};
}

// Gathered rows are re-read (a token by each expert it is routed to), so
// they are loaded with the default cache policy.
__device__ __forceinline__ uint4 ld16(const void *p)
{
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_nt8(const void *p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint2 ld8(const void *p)
{
    const u32x2_t v = *reinterpret_cast<const u32x2_t *>(p);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld_nt4(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ void st_nt8(void *p, uint32_t a, uint32_t b)
{
    const u32x2_t v = {a, b};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(p));
}
__device__ __forceinline__ void st8(void *p, uint32_t a, uint32_t b)
{
    const u32x2_t v = {a, b};
    *reinterpret_cast<u32x2_t *>(p) = v;
}

}  // namespace mxq
