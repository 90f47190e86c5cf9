// mxq_gemm.hip -- block-scaled GEMM consuming the MXFP8 operands the
// quantizers produce: C[m][n] = sum_k dec(a[m][k]) 2^(ea[m][k/32]) *
// dec(b[n][k]) 2^(eb[n][k/32]), with both operands K-contiguous (the rowwise
// 1x32 copies: activations [M][K] and weights [N][K]), fp32 accumulation and
// an fp32 or BF16 (nearest-even) result.  This is the forward GEMM that the
// MXFP8 recipe paragraph of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell" feeds; the E8M0 scale per 32 elements along K is
// the block format of gfx950's scaled matrix instructions.
//
// Matrix instruction.  v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32x64
// A block by a 64x32 B block.  Measured lane layout (a probe on MI355X):
// lane l serves row (or column) l % 32; of the 64 K values, the two 32-wide
// scale blocks are split across the lane halves h = l / 32: bytes 0..15 of
// lane (r, h) are k = 16h .. 16h+15 of block 0 and bytes 16..31 are k = 32 +
// 16h .. of block 1; block 0 takes lane r's scale byte, block 1 lane r+32's.
// The accumulator (16 floats per lane) holds column l % 32, rows 8(i/4) +
// 4h + i%4.
//
// Tiling.  A workgroup of four wavefronts computes a 256x256 tile of C in K
// steps of 128; wavefront (wm, wn) owns a 128x128 quarter: 4x4 instruction
// tiles, 256 fp32 accumulators per lane.  Each K step, the workgroup copies
// the 256x128-byte A and B slices (and their 4 scale bytes per row) from
// global memory to LDS; 16-byte chunks of each 128-byte LDS row are XOR-
// swizzled by the row index, so the 32 rows one fragment read touches fall
// in distinct banks.  Two LDS buffers: the next step's global loads are in
// flight while the current step computes, then land in the other buffer.
// Rows past M or N read the last valid row and are not stored.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GEMM_BM = 256, GEMM_BN = 256, GEMM_BK = 128;
constexpr int GEMM_THREADS = 256;
constexpr int GEMM_TILE_BYTES = GEMM_BM * GEMM_BK;              // 32 KiB per operand

struct GemmSmem {
    u32x4_t a[2][GEMM_BM * GEMM_BK / 16];
    u32x4_t b[2][GEMM_BN * GEMM_BK / 16];
    uint32_t as[2][GEMM_BM];          // 4 scale bytes (the K step's 4 blocks) per row
    uint32_t bs[2][GEMM_BN];
};

// 16-byte chunk c of LDS row r (8 chunks per 128-byte row), swizzled.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Thread t's share of one K step: rows t/8 + 32 i (i < 8) at chunk t % 8 of
// each operand, and one scale word per operand (row t).  The row offsets are
// 32-bit and fixed for the whole K loop (rows past M or N clamped to the
// last row); the K step only moves the wave-uniform base pointers.
struct GemmStage {
    u32x4_t a[8], b[8];
    uint32_t as, bs;
};
struct GemmOffsets {
    uint32_t a[8], b[8];    // (row - tile row 0) * K + 16 (t % 8)
    uint32_t as, bs;        // (row - tile row 0) * K / 32
};

__device__ __forceinline__ GemmOffsets gemm_offsets(int64_t m0, int64_t n0, int64_t M, int64_t N,
                                                    int64_t K, int t)
{
    GemmOffsets o;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = (t >> 3) + 32 * i;
        const int64_t ra = m0 + r < M ? r : M - 1 - m0;
        const int64_t rb = n0 + r < N ? r : N - 1 - n0;
        o.a[i] = (uint32_t)(ra * K + 16 * c);
        o.b[i] = (uint32_t)(rb * K + 16 * c);
    }
    const int64_t ra = m0 + t < M ? t : M - 1 - m0;
    const int64_t rb = n0 + t < N ? t : N - 1 - n0;
    o.as = (uint32_t)(ra * (K >> 5));
    o.bs = (uint32_t)(rb * (K >> 5));
    return o;
}

// a, b: the tile's first row at column k0; as_, bs_: its scale row at block k0/32.
__device__ __forceinline__ void gemm_load(GemmStage &st, const GemmOffsets &o,
                                          const uint8_t *__restrict__ a,
                                          const uint8_t *__restrict__ as_,
                                          const uint8_t *__restrict__ b,
                                          const uint8_t *__restrict__ bs_)
{
#pragma unroll
    for (int i = 0; i < 8; i++) {
        st.a[i] = *reinterpret_cast<const u32x4_t *>(a + o.a[i]);
        st.b[i] = *reinterpret_cast<const u32x4_t *>(b + o.b[i]);
    }
    st.as = *reinterpret_cast<const uint32_t *>(as_ + o.as);
    st.bs = *reinterpret_cast<const uint32_t *>(bs_ + o.bs);
}

__device__ __forceinline__ void gemm_store_lds(GemmSmem &sm, int buf, const GemmStage &st, int t)
{
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = (t >> 3) + 32 * i;
        sm.a[buf][swz(r, c)] = st.a[i];
        sm.b[buf][swz(r, c)] = st.b[i];
    }
    sm.as[buf][t] = st.as;
    sm.bs[buf][t] = st.bs;
}

// One 32x64 fragment (A rows or B columns r0 .. r0+31) of K sub-step s for
// this lane, and its scale word shifted so that byte 2s holds the lane's
// block scale.
__device__ __forceinline__ i32x8_t gemm_frag(const u32x4_t *__restrict__ tile, int r, int h, int s)
{
    const u32x4_t lo = tile[swz(r, 4 * s + h)];
    const u32x4_t hi = tile[swz(r, 4 * s + 2 + h)];
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) mxfp8_gemm_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, int64_t M, int64_t N, int64_t K, uint32_t tiles_n,
    void *__restrict__ C)
{
    __shared__ GemmSmem sm;
    const int t = (int)tid();
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t tile = wg_id();
    const int64_t m0 = (int64_t)(tile / tiles_n) * GEMM_BM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * GEMM_BN;
    const int64_t ksteps = K / GEMM_BK;

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = f32x16_t{};

    const GemmOffsets off = gemm_offsets(m0, n0, M, N, K, t);
    const uint8_t *a = A + m0 * K, *b = B + n0 * K;
    const uint8_t *as_ = As + m0 * (K >> 5), *bs_ = Bs + n0 * (K >> 5);
    GemmStage st;
    gemm_load(st, off, a, as_, b, bs_);
    gemm_store_lds(sm, 0, st, t);
    __syncthreads();

    for (int64_t ks = 0; ks < ksteps; ks++) {
        const int buf = (int)(ks & 1);
        const bool more = ks + 1 < ksteps;
        if (more) {
            const int64_t k1 = (ks + 1) * GEMM_BK;
            gemm_load(st, off, a + k1, as_ + (k1 >> 5), b + k1, bs_ + (k1 >> 5));
        }
        uint32_t sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            sa[i] = sm.as[buf][128 * wm + 32 * i + r32] >> (8 * h);
            sb[i] = sm.bs[buf][128 * wn + 32 * i + r32] >> (8 * h);
        }
#pragma unroll
        for (int s = 0; s < 2; s++) {
            i32x8_t fb[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                fb[j] = gemm_frag(sm.b[buf], 128 * wn + 32 * j + r32, h, s);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const i32x8_t fa = gemm_frag(sm.a[buf], 128 * wm + 32 * i + r32, h, s);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if (s == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa, fb[j], acc[i][j], 0, 0, 0, (int)sa[i], 0, (int)sb[j]);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa, fb[j], acc[i][j], 0, 0, 2, (int)sa[i], 2, (int)sb[j]);
                }
            }
        }
        if (more)
            gemm_store_lds(sm, buf ^ 1, st, t);
        __syncthreads();
    }

    // Epilogue: lane holds column n of each instruction tile, rows 8(e/4) +
    // 4h + e%4.
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t n = n0 + 128 * wn + 32 * j + r32;
        if (n >= N)
            continue;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t m = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) {
                    if constexpr (BF16_OUT) {
                        const uint32_t u = f2u(acc[i][j][e]);
                        reinterpret_cast<uint16_t *>(C)[m * N + n] =
                            (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                    } else {
                        reinterpret_cast<float *>(C)[m * N + n] = acc[i][j][e];
                    }
                }
            }
    }
}

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                             const uint8_t *b_scales, int64_t M, int64_t N, int64_t K,
                             bool bf16_out, void *c, hipStream_t stream)
{
    const int64_t tm = (M + GEMM_BM - 1) / GEMM_BM, tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (tm * tn > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(tm * tn)), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(mxfp8_gemm_kernel<true>, grid, block, 0, stream, a, a_scales, b,
                           b_scales, M, N, K, (uint32_t)tn, c);
    else
        hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, grid, block, 0, stream, a, a_scales, b,
                           b_scales, M, N, K, (uint32_t)tn, c);
    return hipGetLastError();
}

}  // namespace mxq
