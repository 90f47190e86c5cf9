// mxq_dequant.hip -- BF16 dequantization of the exact forward operands (the
// dequantized-backward paragraph of the page "Miles: end-to-end MXFP8 and
// per-token NVFP4 RL on Blackwell").  y = BF16(dec(code) * dec(scale) [* s]),
// rounded once from the exact product, ties to even, saturating at 0x7F7F.
//
// Each thread handles 16 consecutive elements of the flattened [rows][cols]
// array (cols is a multiple of 16, so the 16 share a row and, for NVFP4, a
// block): one 16-byte (MXFP8) or 8-byte (NVFP4) code load, 32 bytes of BF16
// out.
//
// Exactness.  MXFP8: dec(c) * 2^e has at most 4 significant bits and is at
// least 2^-136, so it is exact in f32 (subnormal f32 included) unless it
// overflows; the f32 -> BF16 step is then the only rounding.  NVFP4:
// dec(c) dec(b) is exact (at most 6 bits); p = fp32(dec(c) dec(b) s) rounds
// once more, which can only matter when p lands exactly on a BF16 midpoint;
// then the exact error e = fma(cd, s, -p) (exact while s >= 2^-100) says
// which way the true product lies.  Scales below 2^-100 use binary64.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

// f32 -> BF16 bits, nearest-even, saturating at the largest finite BF16.
// `adj`: when the f32 value sits exactly on a BF16 midpoint, +1 rounds the
// magnitude up, -1 down, 0 keeps nearest-even.
__device__ __forceinline__ uint32_t bf16_rne_sat(uint32_t u, int adj)
{
    const uint32_t lsb = (u >> 16) & 1u;
    uint32_t add = 0x7FFFu + lsb;
    if (adj != 0 && (u & 0xFFFFu) == 0x8000u)
        add = adj > 0 ? 0x8000u : 0x7FFFu;
    uint32_t r = (u + add) >> 16;          // may carry into the exponent (correct)
    if ((r & 0x7F80u) == 0x7F80u)          // overflowed to Inf (inputs are finite)
        r = (r & 0x8000u) | 0x7F7Fu;
    return r;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// BF16 bits of dec(c) * 2^(b - 127) for an E4M3 code c and an E8M0 byte b.
__device__ __forceinline__ uint32_t mx_deq1(uint32_t c, uint32_t b)
{
    const float y = ldexpf(e4m3_value(c), (int)b - 127);
    return bf16_rne_sat(f2u(y), 0);
}

// COL == false: scales[row][cols/32]; COL == true: scales[row/32][cols].
template <bool COL>
__global__ void __launch_bounds__(256) dequant_mxfp8_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t rows, int64_t cols,
                                                            uint16_t *__restrict__ out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t f = t * 16;
    if (f >= rows * cols)
        return;
    const int64_t row = f / cols, k = f - row * cols;
    const uint4 cq = ld_nt16(codes + f);
    const uint32_t cw[4] = {cq.x, cq.y, cq.z, cq.w};
    uint32_t sw[4];
    if (COL) {
        const uint4 sq = ld16(scales + (row >> 5) * cols + k);
        sw[0] = sq.x; sw[1] = sq.y; sw[2] = sq.z; sw[3] = sq.w;
    } else {
        const uint32_t b = scales[row * (cols >> 5) + (k >> 5)];
        sw[0] = sw[1] = sw[2] = sw[3] = b * 0x01010101u;
    }
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t c = cw[j], s = sw[j];
        o[2 * j] = pack2(mx_deq1(c & 0xFF, s & 0xFF), mx_deq1((c >> 8) & 0xFF, (s >> 8) & 0xFF));
        o[2 * j + 1] = pack2(mx_deq1((c >> 16) & 0xFF, (s >> 16) & 0xFF),
                             mx_deq1(c >> 24, s >> 24));
    }
    st_nt16(out + f, o[0], o[1], o[2], o[3]);
    st_nt16(out + f + 8, o[4], o[5], o[6], o[7]);
}

// BF16 of the exact product y (binary64, exact), nearest-even, saturating.
__device__ __attribute__((noinline)) uint32_t bf16_from_f64(double y)
{
    const uint32_t sign = signbit(y) ? 0x8000u : 0u;
    const double a = fabs(y);
    const double BF16_MAX = 0x1.FEp127;
    if (a >= BF16_MAX)
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

constexpr float NV_DEQ_FAST_MIN_S = 0x1p-100f;

__global__ void __launch_bounds__(256) dequant_nvfp4_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ bscales,
                                                            const float *__restrict__ fp32_scales,
                                                            int64_t rows_per_scale, int64_t rows,
                                                            int64_t cols, uint16_t *__restrict__ out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t f = t * 16;
    if (f >= rows * cols)
        return;
    const int64_t row = f / cols, k = f - row * cols;
    const uint2 cq = *reinterpret_cast<const uint2 *>(codes + (f >> 1));
    const uint32_t b = bscales[row * (cols >> 4) + (k >> 4)];
    const float s = fp32_scales[row / rows_per_scale];
    const float d = e4m3_value(b);
    uint32_t o[8];
    const uint32_t cw[2] = {cq.x, cq.y};
    if (s >= NV_DEQ_FAST_MIN_S) {
#pragma unroll
        for (int w = 0; w < 2; w++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float2_t v = e2m1_values((cw[w] >> (8 * j)) & 0xFFu);
                uint32_t h[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const float cd = v[i] * d;                 // exact
                    const float p = cd * s;
                    const uint32_t u = f2u(p);
                    int adj = 0;
                    if ((u & 0xFFFFu) == 0x8000u) {
                        const float e = __builtin_fmaf(cd, s, -p);   // exact error
                        adj = (e == 0.0f) ? 0 : (((e > 0.0f) == (p > 0.0f)) ? 1 : -1);
                    }
                    h[i] = bf16_rne_sat(u, adj);
                }
                o[4 * w + j] = pack2(h[0], h[1]);
            }
        }
    } else {
        for (int w = 0; w < 2; w++) {
            for (int j = 0; j < 4; j++) {
                const float2_t v = e2m1_values((cw[w] >> (8 * j)) & 0xFFu);
                const uint32_t lo = bf16_from_f64((double)v[0] * (double)d * (double)s);
                const uint32_t hi = bf16_from_f64((double)v[1] * (double)d * (double)s);
                o[4 * w + j] = pack2(lo, hi);
            }
        }
    }
    st_nt16(out + f, o[0], o[1], o[2], o[3]);
    st_nt16(out + f + 8, o[4], o[5], o[6], o[7]);
}

hipError_t launch_dequant_mxfp8(bool col, const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream)
{
    const int64_t threads = rows * cols / 16;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (col)
        hipLaunchKernelGGL((dequant_mxfp8_kernel<true>), grid, dim3(256), 0, stream, codes, scales,
                           rows, cols, out);
    else
        hipLaunchKernelGGL((dequant_mxfp8_kernel<false>), grid, dim3(256), 0, stream, codes,
                           scales, rows, cols, out);
    return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t *codes, const uint8_t *bscales, const float *fs,
                                int64_t rows_per_scale, int64_t rows, int64_t cols, uint16_t *out,
                                hipStream_t stream)
{
    const int64_t threads = rows * cols / 16;
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL(dequant_nvfp4_kernel, grid, dim3(256), 0, stream, codes, bscales, fs,
                       rows_per_scale, rows, cols, out);
    return hipGetLastError();
}

}  // namespace mxq
