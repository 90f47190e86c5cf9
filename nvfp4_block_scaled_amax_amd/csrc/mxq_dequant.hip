// mxq_dequant.hip -- BF16 dequantization of the exact forward operands (the
// dequantized-backward paragraph of the page "Miles: end-to-end MXFP8 and
// per-token NVFP4 RL on Blackwell").  y = BF16(dec(code) * dec(scale) [* s]),
// rounded once from the exact product, ties to even, saturating at 0x7F7F.
//
// Work layout: each wavefront takes 1024 (MXFP8) or 2048 (NVFP4) consecutive
// elements of the flattened [rows][cols] array per step; lane l converts the
// 8-element chunks starting at 8l + 512h (h = 0, 1, or 0..3; cols is a
// multiple of 16, so a chunk never straddles a row or an NVFP4 block).  Every
// 16-byte store instruction of the wave then covers 1 KiB of contiguous
// output, whole cache lines: 32 contiguous bytes per lane would leave each
// store instruction writing half lines, which the streaming stores turn into
// extra HBM write traffic.  Grid-stride over wave steps.
//
// NVFP4 issues every load of a step before using any of them (chunks past
// the end load from element 0 and are not stored), and reads the FP32 scale
// with one scalar load when the step lies within one scale's rows.  Measured
// against two chunks per lane with the loads in bounds branches (which made
// the first chunk's loads land before the second's were issued): 8192 x 2048
// 11.9 -> 10.7 us, 262144 x 2048 254 -> 232 us; eight chunks per lane were
// slower (12.3 and 236 us), and so was decoding the codes through a byte-
// permute table of the block's eight BF16 products instead of converting
// them (11.2 and 242 us).  The MXFP8 kernels keep two chunks per lane: four
// were no faster at 8192 x 2048 and slower at 262144 x 2048 (254 -> 264 us).
//
// NVFP4 takes the fast/exact choice once per chunk for the whole wave (one
// uniform branch; the check itself is branch-free) and stores each chunk as
// soon as it is converted.  Against a per-lane branch per chunk, which left
// a wait for the previous store before each store: 262144 x 2048 234 -> 227
// us, 8192 x 2048 unchanged (10.0-10.4 us).  Converting all four chunks
// before the first store was slower at 8192 x 2048 (11.7 us): with one step
// per wavefront the writes then start late.
//
// The arithmetic (exact conversion instructions, and the exact fallbacks)
// is in mxq_dequant.h.  MXFP8 rowwise: one scale per unit (index f / 32);
// columnwise: one scale per element, so each pair is converted twice and the
// halves merged.
#include "mxq_dequant.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int WAVES_PER_WG = 4;
// Grid size in multiples of the resident workgroups (0: one wave step per
// wavefront, the whole array in one launch wave).  Measured on the 262144 x
// 2048 grouped shape.
constexpr int MXFP8_OVERSUBSCRIBE = 0;
constexpr int NVFP4_OVERSUBSCRIBE = 16;
constexpr int64_t WAVE_SPAN = 1024;     // MXFP8: elements per wavefront step
constexpr int64_t HALF_SPAN = 512;
constexpr int NV_CHUNKS = 4;            // NVFP4: chunks per lane per step
constexpr int64_t NV_SPAN = HALF_SPAN * NV_CHUNKS;

// COL == false: scales[row][cols/32]; COL == true: scales[row/32][cols].
// n = rows * cols elements; per_row16 divides by cols / 16.
template <bool COL>
__global__ void __launch_bounds__(256) dequant_mxfp8_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t n, int64_t cols,
                                                            Div per_row16, uint32_t nwg,
                                                            uint16_t *__restrict__ out)
{
    const int64_t lane8 = (tid() & 63) * 8;
    const int64_t waves = (int64_t)nwg * WAVES_PER_WG;
    for (int64_t w = (int64_t)wg_id() * WAVES_PER_WG + wave_in_group(); w * WAVE_SPAN < n;
         w += waves) {
        int64_t f[2];
        uint2 cq[2], sq[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            f[h] = w * WAVE_SPAN + h * HALF_SPAN + lane8;
            cq[h] = make_uint2(0, 0);
            sq[h] = make_uint2(0, 0);
            if (f[h] < n) {
                cq[h] = ld_nt8(codes + f[h]);
                if constexpr (COL) {
                    const uint32_t row = udiv((uint32_t)(f[h] >> 4), per_row16);
                    const int64_t k = f[h] - (int64_t)row * cols;
                    sq[h] = ld8(scales + (int64_t)(row >> 5) * cols + k);
                } else {
                    const uint32_t b = scales[f[h] >> 5] * 0x01010101u;
                    sq[h] = make_uint2(b, b);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const u32x4_t o = mx_chunk<COL>(cq[h], sq[h]);
            if (f[h] < n)
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t *>(out + f[h]));
        }
    }
}

// n = rows * cols elements; per_scale divides a block index by the blocks
// per FP32 scale.
__global__ void __launch_bounds__(256) dequant_nvfp4_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ bscales,
                                                            const float *__restrict__ fp32_scales,
                                                            int64_t n, Div per_scale,
                                                            uint32_t nwg,
                                                            uint16_t *__restrict__ out)
{
    const int64_t lane8 = (tid() & 63) * 8;
    const int64_t waves = (int64_t)nwg * WAVES_PER_WG;
    for (int64_t w = (int64_t)wg_id() * WAVES_PER_WG + wave_in_group(); w * NV_SPAN < n;
         w += waves) {
        int64_t f[NV_CHUNKS];
        bool ok[NV_CHUNKS];
        uint32_t cw[NV_CHUNKS], bb[NV_CHUNKS];
        float s[NV_CHUNKS];
        // One FP32 scale for the whole step?  (Wave-uniform.)
        const int64_t f0 = w * NV_SPAN;
        const int64_t f1 = (f0 + NV_SPAN <= n ? f0 + NV_SPAN : n) - 1;
        const uint32_t s0 = udiv((uint32_t)(f0 >> 4), per_scale);
        const bool one = s0 == udiv((uint32_t)(f1 >> 4), per_scale);
#pragma unroll
        for (int h = 0; h < NV_CHUNKS; h++) {
            f[h] = f0 + h * HALF_SPAN + lane8;
            ok[h] = f[h] < n;
            const int64_t blk = ok[h] ? f[h] >> 4 : 0;
            cw[h] = ld_nt4(codes + 8 * blk + ((f[h] >> 1) & 4));
            bb[h] = bscales[blk];
            s[h] = one ? 0.0f : fp32_scales[udiv((uint32_t)blk, per_scale)];
        }
        __builtin_amdgcn_sched_barrier(0);      // keep the vector loads ahead of their uses
        if (one) {
            const float su = fp32_scales[s0];
#pragma unroll
            for (int h = 0; h < NV_CHUNKS; h++)
                s[h] = su;
        }
        // Chunk by chunk: the fast/exact choice is made for the whole wave
        // (one branch, no divergence) and each chunk is stored as soon as it
        // is converted, so the wave's first store leaves early.
#pragma unroll
        for (int h = 0; h < NV_CHUNKS; h++) {
            const float dh = e4m3_value(ok[h] ? bb[h] : 0u);     // code 0 decodes to 0
            const uint32_t ch = ok[h] ? cw[h] : 0u;
            const bool fast = nv_fast(dh, s[h]);
            const u32x4_t o = __builtin_amdgcn_ballot_w64(!fast) == 0
                                  ? nv_chunk_fast(ch, dh, s[h])
                                  : (fast ? nv_chunk_fast(ch, dh, s[h])
                                          : nv_chunk_exact(ch, dh, s[h]));
            if (ok[h])
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t *>(out + f[h]));
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <class K>
static unsigned grid_for(K kernel, int64_t n, int64_t span, int oversubscribe)
{
    const int64_t need = (n + span * WAVES_PER_WG - 1) / (span * WAVES_PER_WG);
    int64_t wgs = need;
    if (oversubscribe > 0) {
        const int64_t cap = resident_workgroups((const void *)kernel, 64 * WAVES_PER_WG) *
                            oversubscribe;
        if (wgs > cap)
            wgs = cap;
    }
    if (wgs > MAX_GRID_ITEMS / (64 * WAVES_PER_WG))     // grid-stride covers the rest
        wgs = MAX_GRID_ITEMS / (64 * WAVES_PER_WG);
    return (unsigned)(wgs < 1 ? 1 : wgs);
}

hipError_t launch_dequant_mxfp8(bool col, const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream)
{
    const int64_t n = rows * cols;              // n / 16 < 2^32: checked by the caller
    const Div per_row16 = make_div((uint32_t)(cols / 16));
    const dim3 block(64 * WAVES_PER_WG);
    if (col) {
        const unsigned g =
            grid_for(dequant_mxfp8_kernel<true>, n, WAVE_SPAN, MXFP8_OVERSUBSCRIBE);
        hipLaunchKernelGGL((dequant_mxfp8_kernel<true>), dim3(g), block, 0, stream, codes, scales,
                           n, cols, per_row16, g, out);
    } else {
        const unsigned g =
            grid_for(dequant_mxfp8_kernel<false>, n, WAVE_SPAN, MXFP8_OVERSUBSCRIBE);
        hipLaunchKernelGGL((dequant_mxfp8_kernel<false>), dim3(g), block, 0, stream, codes,
                           scales, n, cols, per_row16, g, out);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t *codes, const uint8_t *bscales, const float *fs,
                                int64_t rows_per_scale, int64_t rows, int64_t cols, uint16_t *out,
                                hipStream_t stream)
{
    const int64_t n = rows * cols;              // n / 16 < 2^32: checked by the caller
    const int64_t blocks = n / 16;
    const int64_t per = (cols / 16) * rows_per_scale;   // blocks per FP32 scale
    const Div per_scale = make_div((uint32_t)(per < blocks ? per : blocks));
    const unsigned g = grid_for(dequant_nvfp4_kernel, n, NV_SPAN, NVFP4_OVERSUBSCRIBE);
    hipLaunchKernelGGL(dequant_nvfp4_kernel, dim3(g), dim3(64 * WAVES_PER_WG), 0, stream, codes,
                       bscales, fs, n, per_scale, g, out);
    return hipGetLastError();
}

}  // namespace mxq
