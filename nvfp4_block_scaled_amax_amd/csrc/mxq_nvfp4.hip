// mxq_nvfp4.hip -- NVFP4 quantizers: per-token FP32 scale (the per-token
// activation paragraphs of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell") and weight export with one FP32 scale per gate/up
// pair or per tensor (its gate/up pairing paragraph).  The arithmetic is the
// page's NVFP4 format paragraph under the readings stated in mxq.h:
//   s = fp32(A_scope / 2688), b = E4M3(A_block / (6 s)), c = E2M1(x / (dec(b) s)).
//
// Layout.  A lane owns whole 16-element blocks (two 16-byte loads each), so a
// block's amax, scale and reciprocal are computed once, in one lane.  The
// element conversions (about 10 cycles per instruction on this part, against
// 2-4 for a multiply or an integer op) dominate the arithmetic, so everything
// else is kept per block or per row.  Per-token: one wavefront per row (rows
// of up to 4096 elements are held in registers; longer rows are read twice),
// every row in one launch; the token amax is a wavefront reduction.  Export:
// the same over the flat block array, under the scope's FP32 scale, computed
// beforehand by an amax pass.
//
// Token scale.  s = fp32(A / 2688) for a BF16 magnitude A is q0 = A * R
// (R = fp32(1 / 2688)), then one FMA correction: fma(fma(-q0, 2688, A), R, q0).
// This equals the correctly rounded quotient for every finite BF16 A,
// subnormal results included (checked exhaustively against exact rational
// arithmetic), at three instructions instead of a full division.
//
// Exact decisions without division.  Dividing per element is too slow and
// multiplying by a rounded reciprocal is not exact.  Every decision is
// bracketed instead: with r ~ 1/D (D = 6s for block scales, dec(b) s for codes)
// built from v_rcp_f32 (under 1 ulp) and rounded products, relative error
// below 2^-21, the kernel forms q_lo = x * r (1 - 2^-19) and
// q_hi = x * r (1 + 2^-19), so |q_lo| < |x / D| < |q_hi| with all operands
// normal.  Conversion is monotone, so when the hardware's exact nearest-even
// conversions of q_lo and q_hi agree, that code is the exactly rounded code of
// x / D.  When they differ (x / D within ~2^-18 of a rounding midpoint), the
// lane decides exactly with one FMA: the sign of midpoint * c * s - |x|, which
// FP32 gets right (see block_scale_fix).  Scales below 2^-101 would take the
// reciprocals out of the normal range; such scopes use a binary64 path that
// divides once per element.
#include "mxq_dequant.h"
#include "mxq_launch.h"

namespace mxq {

constexpr float S_FAST_MIN = 0x1p-101f;
constexpr float BRACKET_LO = 1.0f - 0x1p-19f;
constexpr float BRACKET_HI = 1.0f + 0x1p-19f;
constexpr float ONE_SIXTH = 1.0f / 6.0f;
constexpr float RCP_2688 = 0x1.861862p-12f;     // fp32(1 / 2688)

// fp32(A / 2688), correctly rounded, for a non-negative BF16 value A.
__device__ __forceinline__ float div2688(float A)
{
    const float q0 = A * RCP_2688;
    return __builtin_fmaf(__builtin_fmaf(-q0, 2688.0f, A), RCP_2688, q0);
}

// ---------------------------------------------------------------------------
// One 16-element block
// ---------------------------------------------------------------------------
struct Blk {
    uint32_t w[8];     // 16 BF16, packed in pairs
};

// A lane reads its block as two 16-byte halves in two instructions, each
// covering half of every line it touches.  Default-policy loads keep the
// lines for the second instruction: per token 262144 x 2048 241 -> 224 us,
// export gate/up pair 312 -> 296 us.  NT: streaming loads, which measured
// better where the kernel also writes more than it reads (one-pass quantize
// + dequant on large grids: 439 against 467 us) or scatters its outputs
// (dispatch: 76 against 81 us).
template <bool NT = false>
__device__ __forceinline__ void load_blk(Blk &b, const uint16_t *p)
{
    const uint4 q0 = NT ? ld_nt16(p) : ld16(p), q1 = NT ? ld_nt16(p + 8) : ld16(p + 8);
    b.w[0] = q0.x; b.w[1] = q0.y; b.w[2] = q0.z; b.w[3] = q0.w;
    b.w[4] = q1.x; b.w[5] = q1.y; b.w[6] = q1.z; b.w[7] = q1.w;
}

// The block's 16 values as f32 (exact) and its largest |x| (f32 bits).  With
// IEEE mode off the max takes |x| as a source modifier (three operands per
// instruction); NaN inputs are outside the contract.
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

// Exact decisions where the bracket straddles a midpoint (fast path only,
// s >= 2^-101).  For a midpoint m of the target format and a divisor
// D = c s (c = 6 for block scales, c = dec(b) for codes), m c has at most 7
// significant bits, so it is exact in FP32, and fma(m c, s, -a) rounds the
// exact m c s - a once.  Rounding keeps the sign, and the exact difference is
// 0 or a nonzero multiple of 2^-135 (m c is a multiple of 2^-11, s one of
// 2^-124, a BF16 value one of 2^-133), which FP32 (denormals kept) represents,
// so the FMA's sign is the sign of m c s - a and a tie is exactly t == 0.
// These cases are far more common than random quotients would suggest: with
// BF16 inputs of 8 significant bits and 2688 = 2^7 * 21, quotients such as
// x 2688 / (dec(b) A) often equal a midpoint before the inexact s moves them
// by a relative 2^-24, so the decision stays inline (an out-of-line binary64
// fix-up measured 12.7 us against 10.0 us without it on 8192 x 2048).

// Block scale: the candidates are blo and blo + 1; 6 * midpoint =
// 3 (dec(blo) + dec(blo + 1)).
__device__ __forceinline__ uint32_t block_scale_fix(float A, float s, uint32_t blo)
{
    const float m6 = 3.0f * (e4m3_value(blo) + e4m3_value(blo + 1u));
    const float t = __builtin_fmaf(m6, s, -A);
    return t < 0.0f ? blo + 1u : (t > 0.0f ? blo : ((blo & 1u) ? blo + 1u : blo));
}

// The nibbles of one 8-code word where the bracket words lo and hi differ
// (there the magnitudes are klo and klo + 1): decided against the midpoint.
// x: the word's 8 elements as f32.
__device__ __forceinline__ uint32_t codes_fix(uint32_t lo, uint32_t hi, const float *x, float d,
                                              float s)
{
    const uint32_t diff = lo ^ hi;
    uint32_t out = lo;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        if ((diff >> (4 * i)) & 0xFu) {
            const uint32_t a = (lo >> (4 * i)) & 0xFu, klo = a & 7u;
            const float2_t v = e2m1_values(klo | ((klo + 1u) << 4));
            const float md = (0.5f * (v[0] + v[1])) * d;
            const float t = __builtin_fmaf(md, s, -fabsf(x[i]));
            const uint32_t k = t < 0.0f ? klo + 1u : (t > 0.0f ? klo : ((klo & 1u) ? klo + 1u : klo));
            out = (out & ~(0xFu << (4 * i))) | ((k | (a & 8u)) << (4 * i));
        }
    }
    return out;
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

// Block scale byte and the two code words.
struct BlkOut {
    uint32_t b, c0, c1;
};

// binary64 path (0 < s < 2^-101): one division per element.
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

// Quantize one block under scale k (any path).  APPROX (an opt-in variant,
// not the contract): the block scale and the codes each from one conversion
// of a reciprocal-multiply (v_rcp_f32, about 1 ulp) with no exactness
// fix-up, so a quotient within about 2^-21 of a rounding midpoint may take
// the other neighbour; the FP32 scale and the tiny-scale binary64 path are
// unchanged.
template <bool APPROX = false>
__device__ __forceinline__ BlkOut quant_blk(const Blk &blk, const BlkF &f, const ScaleK &k)
{
    BlkOut o;
    if (APPROX && k.s >= S_FAST_MIN) {
        const float A = u2f(f.amax);
        const float r6 = k.inv_s * ONE_SIXTH;
        o.b = e4m3_pair_rne(fminf(A * r6, 448.0f), 0.0f) & 0xFFu;
        o.c0 = o.c1 = 0u;
        if (o.b != 0) {
            const float r = __builtin_amdgcn_rcpf(e4m3_value(o.b)) * k.inv_s;
            o.c0 = codes8(f.x, r);
            o.c1 = codes8(f.x + 8, r);
        }
    } else if (k.s >= S_FAST_MIN) {
        const float A = u2f(f.amax);
        const uint32_t bb = e4m3_pair_rne(fminf(A * k.r6_lo, 448.0f), fminf(A * k.r6_hi, 448.0f));
        o.b = bb & 0xFFu;
        if (o.b != (bb >> 8))
            o.b = block_scale_fix(A, k.s, o.b);
        o.c0 = o.c1 = 0u;
        if (o.b != 0) {
            const float d = e4m3_value(o.b);
            const float r = __builtin_amdgcn_rcpf(d) * k.inv_s;
            const float rlo = r * BRACKET_LO, rhi = r * BRACKET_HI;
            const uint32_t lo0 = codes8(f.x, rlo), hi0 = codes8(f.x, rhi);
            const uint32_t lo1 = codes8(f.x + 8, rlo), hi1 = codes8(f.x + 8, rhi);
            o.c0 = lo0 == hi0 ? lo0 : codes_fix(lo0, hi0, f.x, d, k.s);
            o.c1 = lo1 == hi1 ? lo1 : codes_fix(lo1, hi1, f.x + 8, d, k.s);
        }
    } else if (k.s == 0.0f) {
        o.b = 0u;
        o.c0 = o.c1 = 0u;
    } else {
        o = quant_blk_f64(blk.w[0], blk.w[1], blk.w[2], blk.w[3], blk.w[4], blk.w[5], blk.w[6],
                          blk.w[7], f.amax, k.s);
    }
    return o;
}

// Store block j's 8 code bytes and its scale byte.  NT: streaming code
// stores.  A dispatched token's codes go to several scattered rows; those
// are stored with the default policy (measured 91 -> 86 us on 32768 tokens
// routed top-8, against streaming stores).
template <bool NT = true>
__device__ __forceinline__ void emit_blk(const BlkOut &o, int64_t j, uint8_t *__restrict__ codes,
                                         uint8_t *__restrict__ bs)
{
    if constexpr (NT) {
        // Keeps the store where it is: with one block per lane, the
        // optimizer otherwise merges the stores that follow the arithmetic
        // paths of quant_blk and drops their non-temporal mark.
        asm volatile("" ::: "memory");
        st_nt8(codes + 8 * j, o.c0, o.c1);
    } else
        st8(codes + 8 * j, o.c0, o.c1);
    bs[j] = (uint8_t)o.b;
}

// ---------------------------------------------------------------------------
// Per-token kernels: one wavefront per row; lane l owns blocks l + 64 k.
// One launch over all rows.
// ---------------------------------------------------------------------------
// One wavefront per workgroup: a finished wavefront's slot is released at
// once instead of when the slowest of its group ends (measured 9% faster on
// the 262144 x 2048 shape than four wavefronts per group).
constexpr int WG_THREADS = 64;
constexpr int ROWS_PER_WG = WG_THREADS / 64;

// Row order of the split kernel: workgroup h takes row L(h), so that 32
// consecutive rows -- one 128-byte line of FP32 token scales -- run on one
// XCD (workgroups are dealt round-robin to the 8 XCDs) and consecutive 32-row
// runs on consecutive XCDs; a last, partial group of 256 keeps launch order.
// Each XCD's L2 then holds whole lines of token scales instead of 4-byte
// pieces that each cost HBM a partial write.  Byte-identical; 8192 x 2048
// per token 10.9 -> 10.5 us, 2048 x 2048 5.5 -> 5.0 us.  The one-wavefront
// rows of large grids keep launch order: there it was no faster per token
// (262144 x 2048, 233 us either way) and slower with the BF16 copy (one-pass
// quantize + dequant 420 -> 435 us).
__device__ __forceinline__ int64_t row_order(int64_t h, int64_t rows)
{
    if (h >= (rows >> 8) << 8)
        return h;
    return (h & ~(int64_t)255) | ((h & 7) << 5) | ((h >> 3) & 31);
}

// Where a row's outputs go.  Per-token call: row i of the input is row i of
// the outputs.  Dispatch call: the input rows are tokens, and token t's
// outputs are written to each valid row dest[t * copies + c] of the outputs
// (the expert-sorted rows holding that token); a row index outside
// [0, out_rows) is skipped, so a malformed map cannot move a write out of
// bounds.
struct Dest {
    const int64_t *dest;    // nullptr: identity
    int64_t copies;
    int64_t out_rows;
    uint16_t *dq;           // quantize-dequant kernels: BF16 [rows][cols]
};

// Block j's 16 dequantized BF16 values (32 bytes at out + 16 j): the exact
// product of the codes, the block scale and s, rounded once (mxq_dequant.h).
// Default-policy stores: each store instruction covers half of the lines it
// touches, and the other half follows at once from the same wavefront.
__device__ __forceinline__ void emit_dq(const BlkOut &o, int64_t j, float s,
                                        uint16_t *__restrict__ out)
{
    const float d = e4m3_value(o.b);
    u32x4_t lo, hi;
    nv_block16(o.c0, o.c1, d, s, lo, hi);
    *reinterpret_cast<u32x4_t *>(out + 16 * j) = lo;
    *reinterpret_cast<u32x4_t *>(out + 16 * j + 8) = hi;
}

// Destination rows c0 .. c0+63 of dispatched row `row`, one per lane (-1 past
// the last copy): one vector load, issued before the quantize so that its
// latency is hidden, instead of a dependent scalar load per copy.
__device__ __forceinline__ int64_t dest_chunk(const Dest &d, int64_t row, int64_t c0, int lane)
{
    const int64_t c = c0 + lane;
    return c < d.copies ? d.dest[row * d.copies + c] : -1;
}
__device__ __forceinline__ bool dest_ok(const Dest &d, int64_t r)
{
    return r >= 0 && r < d.out_rows;
}
// Lane c's 64-bit value, wave-uniform.
__device__ __forceinline__ int64_t lane_i64(int64_t v, int c)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, c);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), c);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Rows of up to 64 NB blocks (1024 NB elements), held in registers.  FULL:
// exactly 64 NB blocks (no lane idle); otherwise missing blocks load a valid
// address and are zeroed (no divergent loads) and are not stored.
// Full rows of up to 2048 elements fit 64 VGPRs (8 wavefronts per SIMD)
// without spilling; partial or longer rows are left to the compiler's
// occupancy choice (a partial row of 65..127 blocks spilled at 64).
// DQ: also the dequantized row (dst.dq); codes/bs and ts may then be null
// (not stored).
template <int NB, bool FULL, bool SCATTER, bool DQ, bool APPROX = false>
__device__ __forceinline__ void token_body(const uint16_t *__restrict__ x, int64_t rows,
                                           int64_t cols, uint8_t *__restrict__ codes,
                                           uint8_t *__restrict__ bs, float *__restrict__ ts,
                                           const Dest &dst)
{
    const int64_t row = (int64_t)wg_id() * ROWS_PER_WG + wave_in_group();
    if (row >= rows)
        return;
    const int lane = lane_id();
    const int nblk = (int)(cols >> 4);                  // cols <= 4096 here
    const uint16_t *xr = x + row * cols;
    const int64_t dmine = SCATTER ? dest_chunk(dst, row, 0, lane) : 0;
    Blk r[NB];
#pragma unroll
    for (int k = 0; k < NB; k++) {
        const int j = lane + 64 * k;
        if (FULL) {
            load_blk<SCATTER || DQ>(r[k], xr + 16 * j);
        } else {
            const bool ok = j < nblk;
            load_blk<SCATTER || DQ>(r[k], xr + 16 * (ok ? j : 0));
#pragma unroll
            for (int i = 0; i < 8; i++)
                r[k].w[i] = ok ? r[k].w[i] : 0u;
        }
    }
    BlkF f[NB];
    uint32_t A = 0;
#pragma unroll
    for (int k = 0; k < NB; k++) {
        f[k] = unpack_blk(r[k]);
        A = max(A, f[k].amax);
    }
    const float s = div2688(u2f(__builtin_amdgcn_readfirstlane(wave_max_u32(A))));
    const ScaleK sk = scale_k(s);
    if constexpr (!SCATTER) {
        if (lane == 0 && (!DQ || ts))
            ts[row] = s;
        uint8_t *crow = codes + row * (cols >> 1);
        uint8_t *brow = bs + row * (cols >> 4);
        // DQ: the row's BF16 goes through LDS (32 bytes per block at block
        // j), so that every global store instruction writes 1 KiB of whole
        // lines; lane-owned 32-byte pieces would leave each instruction
        // writing half lines.  One wavefront per workgroup, so the buffer is
        // the wavefront's own.
        static_assert(ROWS_PER_WG == 1, "LDS staging assumes one row per workgroup");
        __shared__ u32x4_t stage[DQ ? 128 * NB : 1];
#pragma unroll
        for (int k = 0; k < NB; k++) {
            const int j = lane + 64 * k;
            if (FULL || j < nblk) {
                const BlkOut o = quant_blk<APPROX>(r[k], f[k], sk);
                if (!DQ || codes)
                    emit_blk(o, j, crow, brow);
                if constexpr (DQ)
                    nv_block16(o.c0, o.c1, e4m3_value(o.b), s, stage[2 * j], stage[2 * j + 1]);
            }
        }
        if constexpr (DQ) {
            __syncthreads();
            uint16_t *out = dst.dq + row * cols;
#pragma unroll
            for (int q = 0; q < 2 * NB; q++) {
                const int u = 64 * q + lane;            // 16-byte unit of the row
                if (FULL || u < 2 * nblk)
                    __builtin_nontemporal_store(stage[u], reinterpret_cast<u32x4_t *>(out + 8 * u));
            }
        }
    } else {
        BlkOut o[NB];
#pragma unroll
        for (int k = 0; k < NB; k++)
            o[k] = quant_blk(r[k], f[k], sk);
        for (int64_t c0 = 0; c0 < dst.copies; c0 += 64) {
            const int64_t mine = c0 == 0 ? dmine : dest_chunk(dst, row, c0, lane);
            if (dest_ok(dst, mine))
                ts[mine] = s;
            const int n = dst.copies - c0 < 64 ? (int)(dst.copies - c0) : 64;
            for (int c = 0; c < n; c++) {
                const int64_t orow = lane_i64(mine, c);
                if (!dest_ok(dst, orow))
                    continue;
                uint8_t *crow = codes + orow * (cols >> 1);
                uint8_t *brow = bs + orow * (cols >> 4);
#pragma unroll
                for (int k = 0; k < NB; k++) {
                    const int j = lane + 64 * k;
                    if (FULL || j < nblk)
                        emit_blk<false>(o[k], j, crow, brow);
                }
            }
        }
    }
}

template <int NB, bool FULL, bool SCATTER>
__global__ void __launch_bounds__(WG_THREADS)
__attribute__((amdgpu_waves_per_eu(NB == 1 || (NB == 2 && FULL) ? 8 : 1, 8)))
nvfp4_token_kernel(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                   uint8_t *__restrict__ codes, uint8_t *__restrict__ bs,
                   float *__restrict__ ts, Dest dst)
{
    token_body<NB, FULL, SCATTER, false>(x, rows, cols, codes, bs, ts, dst);
}

template <int NB, bool FULL>
__global__ void __launch_bounds__(WG_THREADS)
__attribute__((amdgpu_waves_per_eu(NB == 1 || (NB == 2 && FULL) ? 8 : 1, 8)))
nvfp4_token_approx_kernel(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                          uint8_t *__restrict__ codes, uint8_t *__restrict__ bs,
                          float *__restrict__ ts, Dest dst)
{
    token_body<NB, FULL, false, false, true>(x, rows, cols, codes, bs, ts, dst);
}

template <int NB, bool FULL>
__global__ void __launch_bounds__(WG_THREADS)
__attribute__((amdgpu_waves_per_eu(NB == 1 || (NB == 2 && FULL) ? 8 : 1, 8)))
nvfp4_token_qdq_kernel(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                       uint8_t *__restrict__ codes, uint8_t *__restrict__ bs,
                       float *__restrict__ ts, Dest dst)
{
    token_body<NB, FULL, false, true>(x, rows, cols, codes, bs, ts, dst);
}

// Small launches: each row split over the two wavefronts of a workgroup,
// wavefront w taking blocks [64 NB w, 64 NB (w + 1)) (lane l the blocks
// 64 NB w + l + 64 k); the token amax is combined through LDS.  Twice the
// wavefronts, each with half the arithmetic: when the grid is about one
// round of resident wavefronts, the arithmetic that follows the last loads
// is halved (2048 x 2048: 8.1 -> 6.4 us, 8192 x 2048: 13.6 -> 13.2 us); on
// large grids the one-wavefront rows are faster (262144 x 2048: 248 against
// 274 us).
template <int NB, bool FULL, bool DQ>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(8, 8)))
nvfp4_token_split_kernel(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                         uint8_t *__restrict__ codes, uint8_t *__restrict__ bs,
                         float *__restrict__ ts, uint16_t *__restrict__ dq)
{
    const int64_t row = row_order(wg_id(), rows);
    if (row >= rows)                    // uniform over the workgroup
        return;
    const int w = wave_in_group();
    const int lane = lane_id();
    const int nblk = (int)(cols >> 4);
    const uint16_t *xr = x + row * cols;
    Blk r[NB];
    BlkF f[NB];
    uint32_t A = 0;
#pragma unroll
    for (int k = 0; k < NB; k++) {
        const int j = 64 * NB * w + lane + 64 * k;
        if (FULL) {
            load_blk(r[k], xr + 16 * j);
        } else {
            const bool ok = j < nblk;
            load_blk(r[k], xr + 16 * (ok ? j : 0));
#pragma unroll
            for (int i = 0; i < 8; i++)
                r[k].w[i] = ok ? r[k].w[i] : 0u;
        }
    }
#pragma unroll
    for (int k = 0; k < NB; k++) {
        f[k] = unpack_blk(r[k]);
        A = max(A, f[k].amax);
    }
    __shared__ uint32_t part[2];
    const uint32_t Aw = __builtin_amdgcn_readfirstlane(wave_max_u32(A));
    if (lane == 0)
        part[w] = Aw;
    __syncthreads();
    const float s = div2688(u2f(max(part[0], part[1])));
    const ScaleK sk = scale_k(s);
    if (w == 0 && lane == 0 && (!DQ || ts))
        ts[row] = s;
    uint8_t *crow = codes + row * (cols >> 1);
    uint8_t *brow = bs + row * (cols >> 4);
    // DQ: each wavefront stages its half of the BF16 row in LDS (32 bytes
    // per block), so that every global store instruction writes 1 KiB of
    // whole lines.
    __shared__ u32x4_t stage[DQ ? 2 * 128 * NB : 1];
#pragma unroll
    for (int k = 0; k < NB; k++) {
        const int j = 64 * NB * w + lane + 64 * k;
        if (FULL || j < nblk) {
            const BlkOut o = quant_blk(r[k], f[k], sk);
            if (!DQ || codes)
                emit_blk(o, j, crow, brow);
            if constexpr (DQ) {
                const int jl = lane + 64 * k;           // block within the wavefront's half
                nv_block16(o.c0, o.c1, e4m3_value(o.b), s, stage[128 * NB * w + 2 * jl],
                           stage[128 * NB * w + 2 * jl + 1]);
            }
        }
    }
    if constexpr (DQ) {
        __syncthreads();
        uint16_t *out = dq + row * cols + 16 * (64 * NB * w);
        const int units = 2 * (nblk - 64 * NB * w);     // 16-byte units in this half
#pragma unroll
        for (int q = 0; q < 2 * NB; q++) {
            const int u = 64 * q + lane;
            if (FULL || u < units)
                __builtin_nontemporal_store(stage[128 * NB * w + u],
                                            reinterpret_cast<u32x4_t *>(out + 8 * u));
        }
    }
}

// Longer rows: read twice (amax, then codes).  Dispatch: each block is
// written to every destination row as it is produced.
template <bool SCATTER, bool DQ>
__global__ void __launch_bounds__(WG_THREADS) nvfp4_token_long_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ bs, float *__restrict__ ts, Dest dst)
{
    const int64_t row = (int64_t)wg_id() * ROWS_PER_WG + wave_in_group();
    if (row >= rows)
        return;
    const int lane = lane_id();
    const int64_t nblk = cols >> 4;
    const uint16_t *xr = x + row * cols;
    uint32_t A = 0;
    for (int64_t j = lane; j < nblk; j += 64) {
        Blk b;
        load_blk<SCATTER>(b, xr + 16 * j);
        A = max(A, unpack_blk(b).amax);
    }
    const float s = div2688(u2f(__builtin_amdgcn_readfirstlane(wave_max_u32(A))));
    const ScaleK sk = scale_k(s);
    if constexpr (!SCATTER) {
        if (lane == 0 && (!DQ || ts))
            ts[row] = s;
        for (int64_t j = lane; j < nblk; j += 64) {
            Blk b;
            load_blk<SCATTER>(b, xr + 16 * j);
            const BlkOut o = quant_blk(b, unpack_blk(b), sk);
            if (!DQ || codes)
                emit_blk(o, j, codes + row * (cols >> 1), bs + row * (cols >> 4));
            if constexpr (DQ)
                emit_dq(o, j, s, dst.dq + row * cols);
        }
    } else {
        // Copies in chunks of 64 (the row is re-read per chunk; top-k is
        // normally far below 64).
        for (int64_t c0 = 0; c0 < dst.copies; c0 += 64) {
            const int64_t mine = dest_chunk(dst, row, c0, lane);
            if (dest_ok(dst, mine))
                ts[mine] = s;
            const int n = dst.copies - c0 < 64 ? (int)(dst.copies - c0) : 64;
            for (int64_t j = lane; j < nblk; j += 64) {
                Blk b;
                load_blk<SCATTER>(b, xr + 16 * j);
                const BlkOut o = quant_blk(b, unpack_blk(b), sk);
                for (int c = 0; c < n; c++) {
                    const int64_t orow = lane_i64(mine, c);
                    if (dest_ok(dst, orow))
                        emit_blk<false>(o, j, codes + orow * (cols >> 1),
                                        bs + orow * (cols >> 4));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Export: scope amax (per-chunk partial maxima, then one wavefront per scope),
// FP32 scales, then a flat pass over the blocks.  Atomics on one word per
// scope serialize (hundreds of workgroups per scope), so the partials are
// written to distinct words: the start of the gate code array, which the
// code pass overwrites afterwards (stream order; the code array is always
// large enough, see launch_nvfp4_scoped).
// ---------------------------------------------------------------------------
constexpr int AMAX_THREADS = 64;                            // one wavefront per workgroup
constexpr int AMAX_LOADS = 8;                               // 16-byte loads per thread
constexpr int64_t AMAX_CHUNK = AMAX_THREADS * 8 * AMAX_LOADS;   // elements per workgroup
static_assert(AMAX_THREADS == 64, "scoped_amax_workgroups counts 64-lane workgroups");

int64_t scoped_amax_workgroups(int64_t n_experts, int64_t n_per, bool pair)
{
    const int64_t n_scope = pair ? 2 * n_per : n_per;
    return (n_scope + AMAX_CHUNK - 1) / AMAX_CHUNK * n_experts;
}

// Workgroup w reduces chunk w % chunks of scope w / chunks into partial[w]
// (BF16 magnitude bits as u32).  A scope is tensor a's slice
// [e * n_per, (e+1) * n_per) followed by tensor b's (if any).
__global__ void __launch_bounds__(AMAX_THREADS) scope_amax_kernel(const uint16_t *__restrict__ a,
                                                                  const uint16_t *__restrict__ b,
                                                                  int64_t n_per, int64_t chunks,
                                                                  uint32_t *__restrict__ partial)
{
    const int64_t e = (int64_t)wg_id() / chunks;
    const int64_t ch = (int64_t)wg_id() - e * chunks;
    const int64_t n_scope = b ? 2 * n_per : n_per;
    uint32_t m = 0;
#pragma unroll
    for (int it = 0; it < AMAX_LOADS; it++) {
        const int64_t i = ch * AMAX_CHUNK + (int64_t)it * (8 * AMAX_THREADS) + 8 * tid();
        if (i < n_scope) {
            const uint16_t *p = (i < n_per) ? a + e * n_per + i : b + e * n_per + (i - n_per);
            const uint4 q = ld_nt16(p);
            m = pk_max_u16(m, pk_max_u16(pk_max_u16(q.x & 0x7FFF7FFFu, q.y & 0x7FFF7FFFu),
                                         pk_max_u16(q.z & 0x7FFF7FFFu, q.w & 0x7FFF7FFFu)));
        }
    }
    const uint32_t h = wave_max_u32(hmax_u16(m));
    if (lane_id() == 0)
        partial[wg_id()] = h;
}

// One wavefront per scope: the max of its partials -> s = fp32(amax / 2688).
__global__ void __launch_bounds__(64) scope_finalize_kernel(const uint32_t *__restrict__ partial,
                                                            int64_t chunks,
                                                            float *__restrict__ scope_s)
{
    const int64_t e = wg_id();
    uint32_t m = 0;
    for (int64_t c = lane_id(); c < chunks; c += 64)
        m = max(m, partial[e * chunks + c]);
    m = wave_max_u32(m);
    if (lane_id() == 0)
        scope_s[e] = div2688(u2f(m << 16));
}

// Scope scales from amaxes the caller supplies (BF16 magnitudes, the sign bit
// ignored): one lane per scope.
__global__ void __launch_bounds__(64) scope_scale_from_amax_kernel(
    const uint16_t *__restrict__ amax, int64_t n_experts, float *__restrict__ scope_s)
{
    const int64_t e = (int64_t)wg_id() * 64 + lane_id();
    if (e < n_experts)
        scope_s[e] = div2688(u2f((uint32_t)(amax[e] & 0x7FFFu) << 16));
}

// Flat export pass over one tensor of nblk blocks; block j belongs to scope
// j / bps.  Each wavefront takes 64 SCOPED_NB consecutive blocks, lane l the
// blocks base + l + 64 k.  When the wavefront's span lies in one scope (the
// usual case) the scale constants are computed once.
constexpr int SCOPED_NB = 2;

__global__ void __launch_bounds__(WG_THREADS) nvfp4_scoped_kernel(const uint16_t *__restrict__ x,
                                                                  int64_t nblk, Div bps,
                                                                  const float *__restrict__ scope_s,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ bs)
{
    const int64_t base = ((int64_t)wg_id() * ROWS_PER_WG + wave_in_group()) * (64 * SCOPED_NB);
    if (base >= nblk)
        return;
    const int lane = lane_id();
    const int64_t last = (base + 64 * SCOPED_NB <= nblk ? base + 64 * SCOPED_NB : nblk) - 1;
    Blk r[SCOPED_NB];
#pragma unroll
    for (int k = 0; k < SCOPED_NB; k++) {
        const int64_t j = base + lane + 64 * k;
        const bool ok = j <= last;
        load_blk(r[k], x + 16 * (ok ? j : last));
    }
    const uint32_t e0 = udiv((uint32_t)base, bps), e1 = udiv((uint32_t)last, bps);
    if (e0 == e1) {
        const ScaleK sk = scale_k(scope_s[e0]);
#pragma unroll
        for (int k = 0; k < SCOPED_NB; k++) {
            const int64_t j = base + lane + 64 * k;
            if (j <= last)
                emit_blk(quant_blk(r[k], unpack_blk(r[k]), sk), j, codes, bs);
        }
    } else {
#pragma unroll
        for (int k = 0; k < SCOPED_NB; k++) {
            const int64_t j = base + lane + 64 * k;
            if (j <= last) {
                const ScaleK sk = scale_k(scope_s[udiv((uint32_t)j, bps)]);
                emit_blk(quant_blk(r[k], unpack_blk(r[k]), sk), j, codes, bs);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <int NB, bool FULL, bool SCATTER, bool DQ>
static void launch_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                         uint8_t *bs, float *ts, Dest dst, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WG_THREADS);
    if constexpr (DQ)
        hipLaunchKernelGGL((nvfp4_token_qdq_kernel<NB, FULL>), grid, block, 0, stream, x, rows,
                           cols, codes, bs, ts, dst);
    else
        hipLaunchKernelGGL((nvfp4_token_kernel<NB, FULL, SCATTER>), grid, block, 0, stream, x,
                           rows, cols, codes, bs, ts, dst);
}

template <bool SCATTER, bool DQ = false>
static hipError_t launch_rows(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                              uint8_t *bs, float *ts, Dest dst, hipStream_t stream)
{
    if (rows > MAX_TOKEN_ROWS)          // checked by the caller
        return hipErrorInvalidValue;
    const int64_t nblk = cols >> 4;
    const int64_t nb = (nblk + 63) / 64;
    const bool full = nblk == 64 * nb;
    switch (nb) {
    case 1: full ? launch_token<1, true, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream)
                 : launch_token<1, false, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream); break;
    case 2: full ? launch_token<2, true, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream)
                 : launch_token<2, false, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream); break;
    case 3: full ? launch_token<3, true, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream)
                 : launch_token<3, false, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream); break;
    case 4: full ? launch_token<4, true, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream)
                 : launch_token<4, false, SCATTER, DQ>(x, rows, cols, codes, bs, ts, dst, stream); break;
    default: {
        const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WG_THREADS);
        hipLaunchKernelGGL((nvfp4_token_long_kernel<SCATTER, DQ>), grid, block, 0, stream, x,
                           rows, cols, codes, bs, ts, dst);
    }
    }
    return hipGetLastError();
}

// Rows of 65..256 blocks use the split kernel on grids of up to one round of
// resident one-wavefront rows (up to 128 blocks) or two (129..256 blocks):
// 8192 and 16384 rows on 256 CUs, the measured crossovers (2048 x 2048:
// 8.0 -> 6.4 us, 8192 x 4096: 26.8 -> 21.5 us; 16384 x 2048: 20.8 against
// 21.6 us split).  The round scales with the device's CU count.
static bool use_split(int64_t rows, int64_t nblk)
{
    if (nblk <= 64 || nblk > 256)
        return false;
    const int64_t round =
        resident_workgroups((const void *)nvfp4_token_kernel<2, true, false>, WG_THREADS);
    return rows <= (nblk <= 128 ? round : 2 * round);
}

template <int NB, bool FULL, bool DQ>
static void launch_split(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                         uint8_t *bs, float *ts, uint16_t *dq, hipStream_t stream)
{
    hipLaunchKernelGGL((nvfp4_token_split_kernel<NB, FULL, DQ>), dim3((unsigned)rows), dim3(128),
                       0, stream, x, rows, cols, codes, bs, ts, dq);
}

// Two wavefronts of NB blocks per lane: 64 NB < nblk <= 128 NB.
template <bool DQ>
static hipError_t launch_split_rows(const uint16_t *x, int64_t rows, int64_t cols,
                                    uint8_t *codes, uint8_t *bs, float *ts, uint16_t *dq,
                                    hipStream_t stream)
{
    const int64_t nblk = cols >> 4;
    if (nblk <= 128)
        nblk == 128 ? launch_split<1, true, DQ>(x, rows, cols, codes, bs, ts, dq, stream)
                    : launch_split<1, false, DQ>(x, rows, cols, codes, bs, ts, dq, stream);
    else
        nblk == 256 ? launch_split<2, true, DQ>(x, rows, cols, codes, bs, ts, dq, stream)
                    : launch_split<2, false, DQ>(x, rows, cols, codes, bs, ts, dq, stream);
    return hipGetLastError();
}

hipError_t launch_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                                  uint8_t *bs, float *ts, hipStream_t stream)
{
    if (use_split(rows, cols >> 4))
        return launch_split_rows<false>(x, rows, cols, codes, bs, ts, nullptr, stream);
    return launch_rows<false>(x, rows, cols, codes, bs, ts, Dest{nullptr, 1, rows, nullptr},
                              stream);
}

template <int NB, bool FULL>
static void launch_approx(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                          uint8_t *bs, float *ts, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WG_THREADS);
    hipLaunchKernelGGL((nvfp4_token_approx_kernel<NB, FULL>), grid, block, 0, stream, x, rows,
                       cols, codes, bs, ts, Dest{nullptr, 1, rows, nullptr});
}

hipError_t launch_nvfp4_approx(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                               uint8_t *bs, float *ts, hipStream_t stream)
{
    // cols <= 4096 (checked by the caller): rows held in registers.
    const int64_t nblk = cols >> 4;
    const int64_t nb = (nblk + 63) / 64;
    const bool full = nblk == 64 * nb;
    switch (nb) {
    case 1: full ? launch_approx<1, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_approx<1, false>(x, rows, cols, codes, bs, ts, stream); break;
    case 2: full ? launch_approx<2, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_approx<2, false>(x, rows, cols, codes, bs, ts, stream); break;
    case 3: full ? launch_approx<3, true>(x, rows, cols, codes, bs, ts, stream)
                 : launch_approx<3, false>(x, rows, cols, codes, bs, ts, stream); break;
    default: full ? launch_approx<4, true>(x, rows, cols, codes, bs, ts, stream)
                  : launch_approx<4, false>(x, rows, cols, codes, bs, ts, stream);
    }
    return hipGetLastError();
}

hipError_t launch_nvfp4_qdq(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                            uint8_t *bs, float *ts, uint16_t *dq, hipStream_t stream)
{
    if (use_split(rows, cols >> 4))
        return launch_split_rows<true>(x, rows, cols, codes, bs, ts, dq, stream);
    return launch_rows<false, true>(x, rows, cols, codes, bs, ts, Dest{nullptr, 1, rows, dq},
                                    stream);
}

hipError_t launch_nvfp4_dispatch(const uint16_t *x, int64_t n_tokens, int64_t cols,
                                 const int64_t *token_rows, int64_t top_k, int64_t out_rows,
                                 uint8_t *codes, uint8_t *bs, float *ts, hipStream_t stream)
{
    return launch_rows<true>(x, n_tokens, cols, codes, bs, ts,
                             Dest{token_rows, top_k, out_rows, nullptr}, stream);
}

// The code pass of the export over both tensors under scope_scales.
static void launch_scoped_codes(const uint16_t *gate, const uint16_t *up, int64_t n_experts,
                                int64_t n_per, uint8_t *gc, uint8_t *gbs, uint8_t *uc,
                                uint8_t *ubs, const float *scope_scales, hipStream_t stream)
{
    // Blocks in all below 2^32: checked by the caller.
    const int64_t nblk = n_experts * n_per / 16;
    const Div bps = make_div((uint32_t)(n_per / 16));
    const int64_t per_wg = 64 * SCOPED_NB * ROWS_PER_WG;
    const dim3 grid((unsigned)((nblk + per_wg - 1) / per_wg)), block(WG_THREADS);
    hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, gate, nblk, bps,
                       scope_scales, gc, gbs);
    if (up)
        hipLaunchKernelGGL(nvfp4_scoped_kernel, grid, block, 0, stream, up, nblk, bps,
                           scope_scales, uc, ubs);
}

hipError_t launch_nvfp4_scoped_amax(const uint16_t *gate, const uint16_t *up,
                                    const uint16_t *scope_amax, int64_t n_experts, int64_t rows,
                                    int64_t cols, uint8_t *gc, uint8_t *gbs, uint8_t *uc,
                                    uint8_t *ubs, float *scope_scales, hipStream_t stream)
{
    if (n_experts > MAX_GRID_ITEMS / 64)    // checked by the caller
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(scope_scale_from_amax_kernel, dim3((unsigned)((n_experts + 63) / 64)),
                       dim3(64), 0, stream, scope_amax, n_experts, scope_scales);
    launch_scoped_codes(gate, up, n_experts, rows * cols, gc, gbs, uc, ubs, scope_scales, stream);
    return hipGetLastError();
}

hipError_t launch_nvfp4_scoped(const uint16_t *gate, const uint16_t *up, int64_t n_experts,
                               int64_t rows, int64_t cols, uint8_t *gc, uint8_t *gbs,
                               uint8_t *uc, uint8_t *ubs, float *scope_scales,
                               hipStream_t stream)
{
    // Partials: chunks * n_experts words at the start of gate_codes, whose
    // n_experts * n_per / 2 bytes always suffice: chunks <= 2 n_per / 4096 + 1
    // and n_per >= 16, so 4 * chunks <= n_per / 512 + 4 <= n_per / 2.
    const int64_t n_per = rows * cols;
    const int64_t n_scope = up ? 2 * n_per : n_per;
    const int64_t chunks = (n_scope + AMAX_CHUNK - 1) / AMAX_CHUNK;
    // Grid limits (checked by the caller): chunks * n_experts and n_experts
    // workgroups of 64 lanes.
    if (chunks * n_experts > MAX_SCOPED_AMAX_WORKGROUPS || n_experts > MAX_GRID_ITEMS / 64)
        return hipErrorInvalidValue;
    uint32_t *partial = reinterpret_cast<uint32_t *>(gc);
    hipLaunchKernelGGL(scope_amax_kernel, dim3((unsigned)(chunks * n_experts)), dim3(AMAX_THREADS),
                       0, stream, gate, up, n_per, chunks, partial);
    hipLaunchKernelGGL(scope_finalize_kernel, dim3((unsigned)n_experts), dim3(64), 0, stream,
                       (const uint32_t *)partial, chunks, scope_scales);
    launch_scoped_codes(gate, up, n_experts, n_per, gc, gbs, uc, ubs, scope_scales, stream);
    return hipGetLastError();
}

}  // namespace mxq
