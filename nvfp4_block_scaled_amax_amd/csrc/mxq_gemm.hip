// mxq_gemm.hip -- block-scaled GEMMs consuming the operands the quantizers
// produce.  MXFP8: C[m][n] = sum_k dec(a[m][k]) 2^(ea[m][k/32]) *
// dec(b[n][k]) 2^(eb[n][k/32]), with both operands K-contiguous (the rowwise
// 1x32 copies: activations [M][K] and weights [N][K]), fp32 accumulation and
// an fp32 or BF16 (nearest-even) result.  This is the forward GEMM that the
// MXFP8 recipe paragraph of the page "Miles: end-to-end MXFP8 and per-token
// NVFP4 RL on Blackwell" feeds; the E8M0 scale per 32 elements along K is
// the block format of gfx950's scaled matrix instructions.  NVFP4 (further
// down): the same tile with the E4M3 block scales applied while
// dequantizing to FP16.  Each has a dense kernel and a grouped one (the MoE
// expert layer: expert-sorted rows times each expert's weight).
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
// Tiling.  A workgroup of four wavefronts computes a 256x256 tile of C;
// wavefront (wm, wn) owns a 128x128 quarter: 4x4 instruction tiles, 256
// fp32 accumulators per lane.  A and B go from global memory straight into
// LDS (global_load_lds: lane l of a wavefront writes the 16 bytes at LDS
// base + 16 l) through a ring of K steps, and 16-byte chunks of each LDS
// row are XOR-swizzled by the row index (each lane fetches the global chunk
// that belongs in its slot), so the rows one fragment read touches fall in
// distinct banks.  Rows past M or N read the last valid row and are not
// stored.  The MXFP8 kernel's pipeline is described at the kernel.
//
// BF16 result: the accumulators go through LDS (rows padded to 272 bytes, so
// the row groups a store instruction writes miss each other's banks) and
// leave as 16-byte stores that cover 256 contiguous bytes of a row.
//
// Measured (2048x8192x2048, BF16 result, one workgroup's clock counters):
// the earlier form of the MXFP8 kernel (K steps of 128, two LDS stages, the
// next step's copies waited for at the end of the current one, BF16 values
// written to LDS one at a time) spent 65k cycles in its K loop, 48k of them
// with its global copies switched off, and 14.5k in the epilogue; the
// pipelined form spends 58k (49k without copies) and 10.4k, and takes
// 43.9 us against 46.5 us per call (8192x8192x2048: 163 us against 170 us).
// Without copies the loop issues a matrix instruction every ~95 cycles
// against its 64-cycle occupancy; the clock under this load is 1.6-2.0 GHz.
// Issuing a step's eight copies one after each of its later matrix
// instructions (rather than all after the barrier, where the matrix unit
// waited for them) took 2048x8192x2048 from 40.3 to 37.1 us (counters
// before: LDS busy 14 % of the time, bank conflicts 13 % of that, so the
// copies' issue, not LDS bandwidth, was the cost); issuing them a step
// earlier as well (four steps ahead) measured the same.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t *lds_ptr_t;

constexpr int GEMM_BM = 256, GEMM_BN = 256;
constexpr int GEMM_THREADS = 256;
static_assert(GEMM_BM == 256 && GEMM_BN == 256 && GEMM_THREADS == 256,
              "MAX_GEMM_TILES counts 256 x 256 tiles of 256 threads");
constexpr int GEMM_EPI_ROW = 128 * 2 + 16;                      // padded BF16 row of a quarter
constexpr int GEMM_EPI_BYTES = 4 * 128 * GEMM_EPI_ROW;
constexpr int GEMM_SCALE_BYTES = 2 * GEMM_BM * 4;                // epilogue row and column scales
constexpr int GEMM_LDS_BYTES = GEMM_EPI_BYTES + GEMM_SCALE_BYTES;  // 138 KiB

// MXFP8 ring: four 64-deep K steps of A and B codes (16 KiB each) and three
// buffers of scale words (one 4-block word per row of A and of B).
constexpr int MXG_BK = 64;
constexpr int MXG_STAGES = 4, MXG_SCALE_BUFS = 3;
constexpr int MXG_OP_BYTES = GEMM_BM * MXG_BK;
constexpr int MXG_STAGE_BYTES = 2 * MXG_OP_BYTES;
constexpr int MXG_SCALE_BYTES = 2 * GEMM_BM * 4;
constexpr int MXG_SCALE_BASE = MXG_STAGES * MXG_STAGE_BYTES;
static_assert(MXG_SCALE_BASE + MXG_SCALE_BUFS * MXG_SCALE_BYTES <= GEMM_LDS_BYTES,
              "the ring fits in the epilogue's LDS");
// Loads one wavefront issues per step: four 16-byte copies each of A and B,
// and on even steps one scale word each of A and B.
constexpr int MXG_LOADS_ODD = 8, MXG_LOADS_EVEN = 10;
// Rows per block of the grouped transposed columnwise copy (its offsets
// count 32-row blocks).
constexpr int64_t TILE_K_BLOCK = 32;

// 16-byte chunk c of LDS row r (8 chunks per 128-byte row), swizzled by
// (r / 2) % 8.  A 16-byte read serves 16 lanes per cycle (64 banks: 16
// slots of 16 bytes); a fragment read's 16 lanes are 16 consecutive rows at
// one logical chunk, and 8 (r % 2) + (c ^ (r / 2) % 8) is distinct over any
// 16 consecutive rows.  (Swizzling by r % 8 left rows r and r + 8 in one
// slot: half of all LDS cycles were bank conflicts.)
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// The same for 64-byte rows (4 chunks): slot 4 (r % 4) + (c ^ (r / 4) % 4)
// is distinct over any 16 consecutive rows.
__device__ __forceinline__ int swz64(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Per-lane global offsets of one MXFP8 step, fixed over the K loop (the
// step only moves the wave-uniform base pointers).  Copy i of wavefront w
// fills LDS chunks 64 (4i + w) .. +63: lane l lands in row r = 64i + 16w +
// l/4, physical chunk l%4, which holds logical chunk (l%4) ^ ((r/4) % 4) =
// (l%4) ^ ((l/16) % 4) (the same for every i).  Scale words: row 64w + l.
// Rows past M or N are clamped to the last row.
struct MxgOffsets {
    uint32_t r0, c16;           // first row of copy 0 (16w + l/4), 16 * logical chunk
    uint32_t ra_max, rb_max;    // last valid row of the A and B tiles
    uint32_t K;                 // row pitch of A and B (bytes)
    uint32_t as, bs;            // scale-row offsets (clamped row * pitch / 32)
    __device__ __forceinline__ uint32_t a(int i) const
    {
        const uint32_t r = r0 + 64 * i;
        return (r < ra_max ? r : ra_max) * K + c16;
    }
    __device__ __forceinline__ uint32_t b(int i) const
    {
        const uint32_t r = r0 + 64 * i;
        return (r < rb_max ? r : rb_max) * K + c16;
    }
};
__device__ __forceinline__ MxgOffsets mxg_offsets(int64_t m0, int64_t n0, int64_t M, int64_t N,
                                                  int64_t ld, int w, int lane)
{
    MxgOffsets o;
    o.r0 = (uint32_t)(16 * w + (lane >> 2));
    o.c16 = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    o.ra_max = (uint32_t)(M - 1 - m0 < GEMM_BM ? M - 1 - m0 : GEMM_BM - 1);
    o.rb_max = (uint32_t)(N - 1 - n0 < GEMM_BN ? N - 1 - n0 : GEMM_BN - 1);
    o.K = (uint32_t)ld;
    const uint32_t r = (uint32_t)(64 * w + lane);
    o.as = (r < o.ra_max ? r : o.ra_max) * (uint32_t)(ld >> 5);
    o.bs = (r < o.rb_max ? r : o.rb_max) * (uint32_t)(ld >> 5);
    return o;
}

// Global -> LDS copies of one wavefront: lane l's bytes land at LDS byte
// address lds + size * l.  Issued as instructions the compiler does not
// track, so that it does not make the current step's LDS reads wait for
// later steps' copies (it cannot tell the buffers apart and would wait for
// all of them); the kernel orders them itself: every wavefront waits for
// its own copies of a step (a vmcnt that leaves only the later steps'
// copies outstanding) before the barrier that publishes it.
__device__ __forceinline__ void lds_copy16(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

// Codes of step s (K columns 64s .. 64s+63 of the tile's A and B rows) into
// ring stage s % 4 at LDS byte address ring: the wavefront's eight copies,
// copy c moving 64 rows of A (c even) or B (c odd).
__device__ __forceinline__ void mxg_copy(uint32_t ring, uint32_t s, int c, const MxgOffsets &o,
                                         const uint8_t *a, const uint8_t *b, int w)
{
    const uint32_t st = ring + (s & 3u) * MXG_STAGE_BYTES;
    const uint32_t q = (uint32_t)(4 * (c >> 1) + w) * 1024u;
    if ((c & 1) == 0)
        lds_copy16(a + (size_t)s * MXG_BK, o.a(c >> 1), st + q);
    else
        lds_copy16(b + (size_t)s * MXG_BK, o.b(c >> 1), st + MXG_OP_BYTES + q);
}
__device__ __forceinline__ void mxg_issue_codes(uint32_t ring, uint32_t s, const MxgOffsets &o,
                                                const uint8_t *a, const uint8_t *b, int w)
{
#pragma unroll
    for (int c = 0; c < 8; c++)
        mxg_copy(ring, s, c, o, a, b, w);
}
// Scale group g (blocks 4g .. 4g+3 of every row: steps 2g and 2g + 1) into
// scale buffer g % 3.
__device__ __forceinline__ void mxg_issue_scales(uint32_t ring, uint32_t g, const MxgOffsets &o,
                                                 const uint8_t *as_, const uint8_t *bs_, int w)
{
    const uint32_t sb = ring + MXG_SCALE_BASE + (g % 3u) * MXG_SCALE_BYTES;
    lds_copy4(as_ + 4 * (size_t)g, o.as, sb + 256 * w);
    lds_copy4(bs_ + 4 * (size_t)g, o.bs, sb + GEMM_BM * 4 + 256 * w);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt not waited), then a workgroup
// barrier.  The empty asm statements keep the compiler from moving LDS
// accesses across the barrier.
template <int N>
__device__ __forceinline__ void mxg_sync()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One lane's operands of step t: for each of its 4 row blocks of A and of
// B, 32 bytes of codes (bytes 0..15: k = 16h .. 16h+15, chunk h; bytes
// 16..31: k = 32 + 16h .., chunk 2 + h) and the row's scale byte for the
// lane's block of the step (block 2 (t % 2) + h of the scale word), read
// alone so that it arrives in byte 0 of the register: the matrix
// instruction takes block 0's scale from lanes h = 0 and block 1's from
// lanes h = 1, both at byte 0 (no VALU shift before the instructions; with
// shifts, the instructions ran ~13 cycles apart more).
struct MxgFrags {
    i32x8_t a[4], b[4];
    uint32_t sa[4], sb[4];
};
__device__ __forceinline__ i32x8_t mxg_frag(const u32x4_t *tile, int r, int h)
{
    const u32x4_t lo = tile[swz64(r, h)];
    const u32x4_t hi = tile[swz64(r, 2 + h)];
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <int PAR>       // t % 2
__device__ __forceinline__ void mxg_read(MxgFrags &f, const uint8_t *lds, uint32_t t, int wm,
                                         int wn, int r32, int h)
{
    const uint8_t *st = lds + (t & 3u) * MXG_STAGE_BYTES;
    const u32x4_t *ta = reinterpret_cast<const u32x4_t *>(st);
    const u32x4_t *tb = reinterpret_cast<const u32x4_t *>(st + MXG_OP_BYTES);
    const uint8_t *sb = lds + MXG_SCALE_BASE + ((t >> 1) % 3u) * MXG_SCALE_BYTES + 2 * PAR + h;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int ra = 128 * wm + 32 * i + r32, rb = 128 * wn + 32 * i + r32;
        f.a[i] = mxg_frag(ta, ra, h);
        f.b[i] = mxg_frag(tb, rb, h);
        f.sa[i] = sb[4 * ra];
        f.sb[i] = sb[4 * (GEMM_BM + rb)];
    }
}
// The step's 16 matrix instructions.  B is the instruction's first operand,
// so the accumulator of block (i, j) holds C transposed: lane (r, h) holds
// C[32i + r][32j + 8g + 4h + e] in element 4g + e, four consecutive columns.
__device__ __forceinline__ void mxg_mfma(f32x16_t (&acc)[4][4], const MxgFrags &f)
{
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f.b[j], f.a[i], acc[i][j], 0, 0, 0, (int)f.sb[j], 0, (int)f.sa[i]);
}

// Tile order.  Workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2, so workgroup w runs on XCD w % 8.  Workgroup w takes position
// L = (w % 8) * per_xcd + w / 8 of a grouped order (GM tile rows at a time,
// column-major inside a group), so each XCD's L2 serves one compact block
// of the tile grid and fetches only that block's A rows and B columns
// (2048 x 8192 x 2048: 48 MiB from memory instead of 160 MiB).
struct GemmGrid {
    uint32_t tiles_m, tiles_n, per_xcd, group_m;
};
__device__ __forceinline__ bool gemm_tile(const GemmGrid &g, uint32_t w, uint32_t *mt,
                                          uint32_t *nt)
{
    const uint32_t L = (w & 7) * g.per_xcd + (w >> 3);
    if (L >= g.tiles_m * g.tiles_n)
        return false;
    const uint32_t span = g.group_m * g.tiles_n;
    const uint32_t grp = L / span, r = L % span;
    const uint32_t rows = g.tiles_m - grp * g.group_m < g.group_m ? g.tiles_m - grp * g.group_m
                                                                  : g.group_m;
    *mt = grp * g.group_m + r % rows;
    *nt = r / rows;
    return true;
}

// Order of a step's instructions for the scheduler: the next step's 24 LDS
// reads (16 fragment halves, 8 scale bytes) go out among the first matrix
// instructions, four after each of the first six, so that they return under
// the step's matrix work instead of delaying its final wait.
__device__ __forceinline__ void mxg_interleave()
{
#pragma unroll
    for (int k = 0; k < 6; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // matrix
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// One step's 16 matrix instructions with the next step's LDS reads among
// the first six (as mxg_interleave) and the copies of step sc (and scale
// group g when SCALES) one after each of the later ones, so that their issue
// overlaps the matrix unit's work instead of following the barrier.
template <bool SCALES>
__device__ __forceinline__ void mxg_step(f32x16_t (&acc)[4][4], const MxgFrags &f, uint32_t ring,
                                         uint32_t sc, uint32_t g, const MxgOffsets &o,
                                         const uint8_t *a, const uint8_t *b,
                                         const uint8_t *as_, const uint8_t *bs_, int w)
{
#pragma unroll
    for (int q = 0; q < 7; q++)
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[q & 3], f.a[q >> 2], acc[q >> 2][q & 3], 0, 0, 0, (int)f.sb[q & 3], 0,
            (int)f.sa[q >> 2]);
#pragma unroll
    for (int k = 0; k < 6; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // matrix
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 7; q < 16; q++) {
        if (q < 15)
            mxg_copy(ring, sc, q - 7, o, a, b, w);
        else if (SCALES)
            mxg_issue_scales(ring, g, o, as_, bs_, w);
        __builtin_amdgcn_sched_barrier(0);
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[q & 3], f.a[q >> 2], acc[q >> 2][q & 3], 0, 0, 0, (int)f.sb[q & 3], 0,
            (int)f.sa[q >> 2]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Write the wavefront's 128x128 quarter of the C tile from transposed
// accumulators (B was the matrix instructions' first operand): lane (r, h)
// holds, for each block (i, j) and g = 0..3, C[32i + r][32j + 8g + 4h .. +3]
// in elements 4g .. 4g+3.  SCALED: multiply by the FP32 scales of the row
// (sa[m / rows_per_a]) and of the column (sb[n / rows_per_b]), as
// fp32(fp32(acc * sa) * sb).  BF16: through LDS (rows padded to 272 bytes;
// one 8-byte write per four values) and out as 16-byte stores covering 256
// contiguous bytes of a row; the caller has synchronised the workgroup, so
// LDS is free.  FP32: one 16-byte store per four values.
template <bool BF16_OUT, bool SCALED>
__device__ __forceinline__ void gemm_epilogue(const f32x16_t (&acc)[4][4], uint8_t *lds, int wave,
                                              int lane, int64_t m0, int64_t n0, int64_t M,
                                              int64_t N, void *__restrict__ C,
                                              const float *__restrict__ sa, int64_t rows_per_a,
                                              const float *__restrict__ sb, int64_t rows_per_b)
{
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    // SCALED: the tile's 256 row and 256 column scales go to LDS past the
    // staging area (one of each per thread), so that a lane's 64 columns
    // take 16 reads of four consecutive scales and no division each.
    float rs[4] = {1.0f, 1.0f, 1.0f, 1.0f};     // row scales of the lane's 4 rows
    const float *csc = nullptr;                 // the tile's column scales in LDS
    if constexpr (SCALED) {
        float *sc = reinterpret_cast<float *>(lds + GEMM_EPI_BYTES);
        const int t = 64 * wave + lane;
        const int64_t m = m0 + t < M ? m0 + t : M - 1;
        const int64_t n = n0 + t < N ? n0 + t : N - 1;
        sc[t] = sa[m / rows_per_a];
        sc[GEMM_BM + t] = sb[n / rows_per_b];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; i++)
            rs[i] = sc[128 * wm + 32 * i + r32];
        csc = sc + GEMM_BM + 128 * wn;
    }
    // The four values of block (i, j), group g, scaled.
    auto quad = [&](int i, int j, int g) {
        f32x4_t v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
        if constexpr (SCALED) {
            const f32x4_t cs = *reinterpret_cast<const f32x4_t *>(csc + 32 * j + 8 * g + 4 * h);
            v = (v * rs[i]) * cs;
        }
        return v;
    };
    if constexpr (BF16_OUT) {
        uint8_t *q = lds + wave * (128 * GEMM_EPI_ROW);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const f32x4_t v = quad(i, j, g);
                    const bf16x2_t lo = {(__bf16)v[0], (__bf16)v[1]};
                    const bf16x2_t hi = {(__bf16)v[2], (__bf16)v[3]};
                    const int r = 32 * i + r32, c = 32 * j + 8 * g + 4 * h;
                    *reinterpret_cast<uint2_t *>(q + r * GEMM_EPI_ROW + 2 * c) =
                        uint2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                }
        __syncthreads();
        const int64_t col = n0 + 128 * wn + 8 * (lane & 15);
        uint16_t *c = reinterpret_cast<uint16_t *>(C);
        // 16-byte stores need every row start 16-byte aligned.
        const bool vec = (N & 7) == 0 && ((uintptr_t)C & 15) == 0;
        for (int rr = 0; rr < 128; rr += 4) {
            const int r = rr + (lane >> 4);
            const int64_t m = m0 + 128 * wm + r;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(q + r * GEMM_EPI_ROW +
                                                                  16 * (lane & 15));
            if (m < M) {
                if (vec && col + 8 <= N) {
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(c + m * N + col));
                } else {
                    const uint16_t *p = reinterpret_cast<const uint16_t *>(&v);
                    for (int e = 0; e < 8 && col + e < N; e++)
                        c[m * N + col + e] = p[e];
                }
            }
        }
    } else {
        float *c = reinterpret_cast<float *>(C);
        const bool vec = (N & 3) == 0 && ((uintptr_t)C & 15) == 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t m = m0 + 128 * wm + 32 * i + r32;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int64_t n = n0 + 128 * wn + 32 * j + 8 * g + 4 * h;
                    const f32x4_t v = quad(i, j, g);
                    if (vec && n + 4 <= N) {
                        const u32x4_t u = {f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])};
                        __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t *>(c + m * N + n));
                    } else {
                        for (int e = 0; e < 4 && n + e < N; e++)
                            c[m * N + n + e] = v[e];
                    }
                }
        }
    }
}

// MXFP8 GEMM.  A workgroup of four wavefronts computes a 256x256 tile of C
// in K steps of 64 (one matrix instruction deep); wavefront (wm, wn) owns a
// 128x128 quarter: 4x4 instruction tiles, 256 fp32 accumulators per lane.
// Pipeline, per step s: issue the global -> LDS copies of step s + 3 into
// ring stage (s + 3) % 4 (the stage step s - 1 used, read by everyone
// before the previous barrier); read step s + 1's fragments and scale words
// into registers; run step s's 16 matrix instructions on the registers read
// during step s - 1; wait for this wavefront's copies of step s + 2 and for
// its LDS reads; barrier.  So a copy has three steps to land, and LDS reads
// run under the matrix instructions.  Scale groups (4 blocks, two steps)
// travel with the even steps into a ring of three buffers.  The loop is
// unrolled by two so that the registers of alternate steps and the scale
// byte selectors are static.
// One 256x256 tile of C = A B^T at (m0, n0), C row-major [M][N].
template <bool BF16_OUT>
// A and B rows have pitch ld bytes (scale rows ld / 32); the product runs
// over K <= ld columns (K % 128 == 0; K == 0 gives a zero tile).
__device__ __forceinline__ void mxg_tile(uint8_t *lds, const uint8_t *__restrict__ A,
                                         const uint8_t *__restrict__ As,
                                         const uint8_t *__restrict__ B,
                                         const uint8_t *__restrict__ Bs, int64_t M, int64_t N,
                                         int64_t K, int64_t ld, int64_t m0, int64_t n0,
                                         void *__restrict__ C)
{
    const int t = (int)tid();
    const int lane = t & 63, wave = (int)wave_in_group();    // wave index: uniform
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t nsteps = (uint32_t)(K / MXG_BK);          // even: K % 128 == 0

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = f32x16_t{};
    if (nsteps == 0) {
        gemm_epilogue<BF16_OUT, false>(acc, lds, wave, lane, m0, n0, M, N, C, nullptr, 1,
                                       nullptr, 1);
        return;
    }

    const MxgOffsets off = mxg_offsets(m0, n0, M, N, ld, wave, lane);
    const uint8_t *a = A + m0 * ld, *b = B + n0 * ld;
    const uint8_t *as_ = As + m0 * (ld >> 5), *bs_ = Bs + n0 * (ld >> 5);
    const uint32_t ring = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

    // Prologue: steps 0, 1 and 2 in flight; wait for steps 0 and 1.
    mxg_issue_codes(ring, 0, off, a, b, wave);
    mxg_issue_scales(ring, 0, off, as_, bs_, wave);
    mxg_issue_codes(ring, 1, off, a, b, wave);
    if (nsteps > 2) {
        mxg_issue_codes(ring, 2, off, a, b, wave);
        mxg_issue_scales(ring, 1, off, as_, bs_, wave);
        mxg_sync<MXG_LOADS_EVEN>();
    } else {
        mxg_sync<0>();
    }
    MxgFrags f0, f1;
    mxg_read<0>(f0, lds, 0, wm, wn, r32, h);

    // Steady state: both steps issue copies.
    uint32_t s = 0;
    for (; s + 4 < nsteps; s += 2) {
        // Step s (even): matrix work on f0; read step s + 1 into f1.
        mxg_read<1>(f1, lds, s + 1, wm, wn, r32, h);
        mxg_step<false>(acc, f0, ring, s + 3, 0, off, a, b, as_, bs_, wave);
        mxg_sync<MXG_LOADS_ODD>();
        // Step s + 1 (odd): matrix work on f1; read step s + 2 into f0.
        mxg_read<0>(f0, lds, s + 2, wm, wn, r32, h);
        mxg_step<true>(acc, f1, ring, s + 4, (s + 4) >> 1, off, a, b, as_, bs_, wave);
        mxg_sync<MXG_LOADS_EVEN>();
    }
    // The last two or four steps (s = nsteps - 4 or nsteps - 2).
    if (s + 4 == nsteps) {
        mxg_read<1>(f1, lds, s + 1, wm, wn, r32, h);
        mxg_step<false>(acc, f0, ring, s + 3, 0, off, a, b, as_, bs_, wave);
        mxg_sync<MXG_LOADS_ODD>();
        mxg_read<0>(f0, lds, s + 2, wm, wn, r32, h);
        mxg_mfma(acc, f1);
        mxg_interleave();
        mxg_sync<0>();
    }
    mxg_read<1>(f1, lds, nsteps - 1, wm, wn, r32, h);
    mxg_mfma(acc, f0);
    mxg_interleave();
    mxg_sync<0>();
    mxg_mfma(acc, f1);

    // Every copy has landed and every LDS read returned (the last syncs wait
    // for all); after this barrier no wavefront reads the ring.
    __syncthreads();
    gemm_epilogue<BF16_OUT, false>(acc, lds, wave, lane, m0, n0, M, N, C, nullptr, 1, nullptr, 1);
}

template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) mxfp8_gemm_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, int64_t M, int64_t N, int64_t K, GemmGrid grid,
    void *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GEMM_LDS_BYTES];
    uint32_t mt, nt;
    if (!gemm_tile(grid, wg_id(), &mt, &nt))
        return;
    mxg_tile<BF16_OUT>(lds, A, As, B, Bs, M, N, K, K, (int64_t)mt * GEMM_BM,
                       (int64_t)nt * GEMM_BN, C);
}

// ---------------------------------------------------------------------------
// Grouped MXFP8 GEMM (the MoE expert layer): rows seg_offsets[e] ..
// seg_offsets[e+1] of A (the expert-sorted rowwise copy that the grouped
// quantizer writes) times expert e's weight B_e [N][K]:
// C[r][n] = sum_k dec(a[r][k]) 2^(sa[r][k/32]) dec(b_e[n][k]) 2^(sb_e[n][k/32]).
// Each segment is cut into 256-row tiles; global m-tile mg (the segments'
// tiles concatenated) and n-tile nt come from the workgroup index, dealt to
// the XCDs in contiguous runs so each XCD works on few experts.
// ---------------------------------------------------------------------------
struct GroupedGemmGrid {
    uint32_t tiles_n, per_xcd, max_mtiles;
};

// The segment that global m-tile mg falls in, by a wavefront prefix sum of
// the segments' tile counts, 64 segments at a time (offsets are device data
// the host cannot check: each segment is clamped into [0, rows), so
// malformed offsets give meaningless rows, never an access out of bounds).
// Every output is wave-uniform.  False if mg lies past the last tile.
__device__ __forceinline__ bool grouped_mtile(const int64_t *__restrict__ off, int64_t G,
                                              int64_t rows, int64_t mg, int64_t *e_out,
                                              int64_t *lo_out, int64_t *n_out, int64_t *mt_out)
{
    const int lane = (int)lane_id();
    int64_t before = 0;
    for (int64_t base = 0; base < G; base += 64) {
        const int64_t e = base + lane;
        int64_t lo = 0, hi = 0;
        if (e < G) {
            lo = off[e];
            hi = off[e + 1];
            lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
            hi = hi < lo ? lo : (hi > rows ? rows : hi);
        }
        const int64_t n = (hi - lo + GEMM_BM - 1) / GEMM_BM;
        int64_t inc = n;                                      // inclusive prefix over lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t v = __shfl_up(inc, d);
            if (lane >= d)
                inc += v;
        }
        const int64_t total = __shfl(inc, 63);
        if (mg < before + total) {
            const unsigned long long hit = __ballot(before + inc > mg);
            const int l = (int)__builtin_amdgcn_readfirstlane((uint32_t)(__ffsll((long long)hit) - 1));
            *e_out = base + l;
            *lo_out = __shfl(lo, l);
            *n_out = __shfl(hi - lo, l);
            *mt_out = mg - before - (__shfl(inc, l) - __shfl(n, l));
            return true;
        }
        before += total;
    }
    return false;
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) mxfp8_grouped_gemm_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const int64_t *__restrict__ off, int64_t G, int64_t rows,
    int64_t N, int64_t K, GroupedGemmGrid grid, void *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GEMM_LDS_BYTES];
    const uint32_t w = wg_id();
    const uint32_t L = (w & 7) * grid.per_xcd + (w >> 3);
    const uint32_t mg = L / grid.tiles_n, nt = L % grid.tiles_n;
    if (mg >= grid.max_mtiles)
        return;
    int64_t e, lo, n, mt;
    if (!grouped_mtile(off, G, rows, mg, &e, &lo, &n, &mt))
        return;
    e = uniform_i64(e);
    lo = uniform_i64(lo);
    n = uniform_i64(n);
    mt = uniform_i64(mt);
    const int64_t esz = BF16_OUT ? 2 : 4;
    mxg_tile<BF16_OUT>(lds, A + lo * K, As + lo * (K >> 5), B + e * N * K, Bs + e * N * (K >> 5),
                       n, N, K, K, mt * GEMM_BM, (int64_t)nt * GEMM_BN,
                       reinterpret_cast<uint8_t *>(C) + lo * N * esz);
}

// ---------------------------------------------------------------------------
// NVFP4 GEMM: C[m][n] = sa[m / rows_per_a] sb[n / rows_per_b] sum_k
// dec(ca[m][k]) dec(ba[m][k/16]) dec(cb[n][k]) dec(bb[n][k/16]).  The
// per-16 E4M3 block scales are not an E8M0 power of two, so the fp4 matrix
// instructions cannot apply them; but dec(code) dec(block scale) has at most
// 6 significant bits and lies in [2^-10, 2688], so it is exactly an FP16
// value (and a BF16 one).  The kernel dequantizes each K step to FP16 on its
// way into LDS (register-staged: the next step's codes and scales are loaded
// while the current step's FP16 matrix instructions run) and applies the
// FP32 scales in the epilogue.  FP16 rather than BF16 because gfx950 has a
// packed FP16 multiply and an fp4 -> FP16 pair conversion selecting its
// code byte: one conversion and one packed multiply per code pair, against
// an fp4 -> f32 conversion, two multiplies and a byte permute for BF16
// (byte-identical results, 2048x8192x2048 80 -> 77 us, 8192x8192x2048
// 276 -> 265 us).
//
// FP16 instruction: v_mfma_f32_32x32x16_f16, lane (r, h) holds 8
// consecutive K values: chunk 2s + h (16 bytes) of the 64-element step for
// slice s.  LDS rows are 64 FP16 = 128 bytes, swizzled as above.
//
// Measured (2048x8192x2048, BF16 result): the earlier form, which ran the
// step's 64 matrix instructions and then the next step's dequantization,
// took 104 us; interleaving the dequantization with the matrix instructions
// (and the transposed epilogue) 80 us (8192x8192x2048: 372 -> 287 us),
// byte-identical.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
constexpr int NVG_BK = 64;                                       // K elements per step
constexpr int NVG_STAGE_BYTES = 2 * GEMM_BM * NVG_BK * 2;       // A and B FP16 slices

// Thread t's share of one step: row t of A and of B (clamped), 64 codes
// (32 bytes) and 4 block-scale bytes each.
struct NvStage {
    u32x4_t ca[2], cb[2];
    uint32_t sa, sb;
};

__device__ __forceinline__ void nv_load(NvStage &st, const uint8_t *a, const uint8_t *ab,
                                        const uint8_t *b, const uint8_t *bb, uint32_t ra,
                                        uint32_t rb, uint32_t half_k, uint32_t blk_k)
{
    st.ca[0] = *reinterpret_cast<const u32x4_t *>(a + ra * half_k);
    st.ca[1] = *reinterpret_cast<const u32x4_t *>(a + ra * half_k + 16);
    st.cb[0] = *reinterpret_cast<const u32x4_t *>(b + rb * half_k);
    st.cb[1] = *reinterpret_cast<const u32x4_t *>(b + rb * half_k + 16);
    st.sa = *reinterpret_cast<const uint32_t *>(ab + ra * blk_k);
    st.sb = *reinterpret_cast<const uint32_t *>(bb + rb * blk_k);
}

// Code pair (byte J of codes) times d2 = {d, d}: the conversion is exact
// (E2M1 values are FP16 values) and so is the product (at most 6
// significant bits, within FP16's normal range).  Low half: the low nibble.
template <int J>
__device__ __forceinline__ uint32_t nv_pair_f16(uint32_t codes, half2_t d2)
{
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, J) * d2);
}
// 8 FP16 (one 16-byte chunk) from 4 code bytes under block scale d.
__device__ __forceinline__ u32x4_t nv_chunk_f16(uint32_t codes, half2_t d2)
{
    return u32x4_t{nv_pair_f16<0>(codes, d2), nv_pair_f16<1>(codes, d2),
                   nv_pair_f16<2>(codes, d2), nv_pair_f16<3>(codes, d2)};
}
__device__ __forceinline__ half2_t nv_scale_f16(uint32_t byte)
{
    const _Float16 d = (_Float16)e4m3_value(byte);      // exact: E4M3 values are FP16 values
    return half2_t{d, d};
}

__device__ __forceinline__ void nv_store_row(u32x4_t *tile, int r, const u32x4_t (&c)[2],
                                             uint32_t scales)
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        tile[swz(r, j)] = nv_chunk_f16(c[j >> 2][j & 3],
                                       nv_scale_f16((scales >> (8 * (j >> 1))) & 0xFFu));
    }
}

__device__ __forceinline__ u32x4_t *nvg_tile_a(uint8_t *lds, int buf)
{
    return reinterpret_cast<u32x4_t *>(lds + buf * NVG_STAGE_BYTES);
}
__device__ __forceinline__ u32x4_t *nvg_tile_b(uint8_t *lds, int buf)
{
    return reinterpret_cast<u32x4_t *>(lds + buf * NVG_STAGE_BYTES + GEMM_BM * NVG_BK * 2);
}

// Fragments of slice sl (16 K values) for the wavefront's 4 row blocks of A
// and of B.
__device__ __forceinline__ void nvg_frags(f16x8_t (&fa)[4], f16x8_t (&fb)[4],
                                          const u32x4_t *ta, const u32x4_t *tb, int sl, int wm,
                                          int wn, int r32, int h)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        fa[i] = __builtin_bit_cast(f16x8_t, ta[swz(128 * wm + 32 * i + r32, 2 * sl + h)]);
        fb[i] = __builtin_bit_cast(f16x8_t, tb[swz(128 * wn + 32 * i + r32, 2 * sl + h)]);
    }
}
// One K step: the 64 matrix instructions on LDS stage buf (B is their
// first operand, so the accumulators hold C transposed, the layout
// gemm_epilogue takes) and, if CONVERT, the dequantization of the next step
// (registers nx: row t of A and of B) into the other stage.  The order is
// fixed by scheduling fences: per slice, the next slice's fragments are read
// first; then per row block i, each of its 4 independent instructions is
// followed by one code pair of conversion chunk 4 sl + i (A's 8 chunks, then
// B's), and the chunk's LDS write ends the group.  So the VALU work issues
// while the matrix unit is busy, and no two instructions on one accumulator
// are adjacent.
template <bool CONVERT>
__device__ __forceinline__ void nvg_step(f32x16_t (&acc)[4][4], uint8_t *lds, int buf,
                                         const NvStage &nx, int t, int wm, int wn, int r32, int h)
{
    const u32x4_t *ta = nvg_tile_a(lds, buf), *tb = nvg_tile_b(lds, buf);
    f16x8_t fa[2][4], fb[2][4];
    nvg_frags(fa[0], fb[0], ta, tb, 0, wm, wn, r32, h);
#pragma unroll
    for (int sl = 0; sl < 4; sl++) {
        if (sl < 3)
            nvg_frags(fa[(sl + 1) & 1], fb[(sl + 1) & 1], ta, tb, sl + 1, wm, wn, r32, h);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = 4 * sl + i, j8 = u & 7;
            const bool isb = u >= 8;
            const uint32_t codes = (isb ? nx.cb : nx.ca)[j8 >> 2][j8 & 3];
            const half2_t d2 = nv_scale_f16(((isb ? nx.sb : nx.sa) >> (8 * (j8 >> 1))) & 0xFFu);
            u32x4_t o;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[sl & 1][j], fa[sl & 1][i],
                                                                   acc[i][j], 0, 0, 0);
                if constexpr (CONVERT) {
                    o[j] = j == 0 ? nv_pair_f16<0>(codes, d2)
                         : j == 1 ? nv_pair_f16<1>(codes, d2)
                         : j == 2 ? nv_pair_f16<2>(codes, d2)
                                  : nv_pair_f16<3>(codes, d2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (CONVERT)
                (isb ? nvg_tile_b(lds, buf ^ 1) : nvg_tile_a(lds, buf ^ 1))[swz(t, j8)] = o;
        }
    }
}

// lgkmcnt(0) (this wavefront's LDS writes and reads done) and a workgroup
// barrier, leaving global loads in flight (the compiler waits for those
// where their registers are used).
__device__ __forceinline__ void nvg_sync()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Pipeline: step ks computes from LDS stage ks % 2 while the registers of
// step ks + 1 (loaded one step earlier) are dequantized into the other
// stage and step ks + 2 is loaded into the registers step ks used.  The
// loop is unrolled by two so that the two register sets keep their roles.
// One 256x256 tile of the NVFP4 GEMM at (m0, n0), C row-major [M][N].
template <bool BF16_OUT>
__device__ __forceinline__ void nvg_tile(uint8_t *lds, const uint8_t *__restrict__ A,
                                         const uint8_t *__restrict__ Ab,
                                         const float *__restrict__ As, int64_t rows_per_a,
                                         const uint8_t *__restrict__ B,
                                         const uint8_t *__restrict__ Bb,
                                         const float *__restrict__ Bs, int64_t rows_per_b,
                                         int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                         void *__restrict__ C)
{
    const int t = (int)tid();
    const int lane = t & 63, wave = (int)wave_in_group();
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t ksteps = K / NVG_BK;
    const uint32_t half_k = (uint32_t)(K >> 1), blk_k = (uint32_t)(K >> 4);
    const uint32_t ra = (uint32_t)(m0 + t < M ? t : M - 1 - m0);
    const uint32_t rb = (uint32_t)(n0 + t < N ? t : N - 1 - n0);
    const uint8_t *a = A + m0 * (K >> 1), *b = B + n0 * (K >> 1);
    const uint8_t *ab = Ab + m0 * (K >> 4), *bb = Bb + n0 * (K >> 4);
    auto load = [&](NvStage &st, int64_t step) {
        const int64_t k = step * NVG_BK;
        nv_load(st, a + (k >> 1), ab + (k >> 4), b + (k >> 1), bb + (k >> 4), ra, rb, half_k,
                blk_k);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = f32x16_t{};

    // Loads past the last step re-read the last step (valid memory); their
    // conversions land in a stage no later step reads.  So the loop body has
    // no branch and the register sets of alternate steps stay static.
    const int64_t last = ksteps - 1;
    NvStage s0, s1;
    load(s0, 0);
    load(s1, last < 1 ? last : 1);
    nv_store_row(nvg_tile_a(lds, 0), t, s0.ca, s0.sa);
    nv_store_row(nvg_tile_b(lds, 0), t, s0.cb, s0.sb);
    nvg_sync();

    int64_t ks = 0;
    for (; ks + 1 < ksteps; ks += 2) {
        load(s0, ks + 2 < last ? ks + 2 : last);
        nvg_step<true>(acc, lds, 0, s1, t, wm, wn, r32, h);
        nvg_sync();
        load(s1, ks + 3 < last ? ks + 3 : last);
        nvg_step<true>(acc, lds, 1, s0, t, wm, wn, r32, h);
        nvg_sync();
    }
    if (ks < ksteps)                        // odd step count: the last step
        nvg_step<false>(acc, lds, 0, s0, t, wm, wn, r32, h);
    // No wavefront reads the stages after this barrier.
    __syncthreads();
    gemm_epilogue<BF16_OUT, true>(acc, lds, wave, lane, m0, n0, M, N, C, As, rows_per_a, Bs,
                                  rows_per_b);
}

template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) nvfp4_gemm_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ Ab, const float *__restrict__ As,
    int64_t rows_per_a, const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bb,
    const float *__restrict__ Bs, int64_t rows_per_b, int64_t M, int64_t N, int64_t K,
    GemmGrid grid, void *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GEMM_LDS_BYTES];
    uint32_t mt, nt;
    if (!gemm_tile(grid, wg_id(), &mt, &nt))
        return;
    nvg_tile<BF16_OUT>(lds, A, Ab, As, rows_per_a, B, Bb, Bs, rows_per_b, M, N, K,
                       (int64_t)mt * GEMM_BM, (int64_t)nt * GEMM_BN, C);
}

// Grouped NVFP4 GEMM (the MoE expert layer on per-token NVFP4 rows): rows of
// segment e (codes, block scales and one FP32 scale per row, as the grouped
// quantizer writes them) times expert e's NVFP4 weight [N][K/2] with its one
// FP32 scope scale Bs[e]; tiles found as in the grouped MXFP8 kernel.
template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) nvfp4_grouped_gemm_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ Ab, const float *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bb, const float *__restrict__ Bs,
    const int64_t *__restrict__ off, int64_t G, int64_t rows, int64_t N, int64_t K,
    GroupedGemmGrid grid, void *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GEMM_LDS_BYTES];
    const uint32_t w = wg_id();
    const uint32_t L = (w & 7) * grid.per_xcd + (w >> 3);
    const uint32_t mg = L / grid.tiles_n, nt = L % grid.tiles_n;
    if (mg >= grid.max_mtiles)
        return;
    int64_t e, lo, n, mt;
    if (!grouped_mtile(off, G, rows, mg, &e, &lo, &n, &mt))
        return;
    e = uniform_i64(e);
    lo = uniform_i64(lo);
    n = uniform_i64(n);
    mt = uniform_i64(mt);
    const int64_t esz = BF16_OUT ? 2 : 4;
    nvg_tile<BF16_OUT>(lds, A + lo * (K >> 1), Ab + lo * (K >> 4), As + lo, 1,
                       B + e * N * (K >> 1), Bb + e * N * (K >> 4), Bs + e, N, n, N, K,
                       mt * GEMM_BM, (int64_t)nt * GEMM_BN,
                       reinterpret_cast<uint8_t *>(C) + lo * N * esz);
}

hipError_t launch_nvfp4_grouped_gemm(const uint8_t *a, const uint8_t *a_block_scales,
                                     const float *a_scales, const uint8_t *b,
                                     const uint8_t *b_block_scales, const float *b_scales,
                                     const int64_t *seg_offsets, int64_t n_groups, int64_t rows,
                                     int64_t N, int64_t K, bool bf16_out, void *c,
                                     hipStream_t stream)
{
    const int64_t tm = grouped_gemm_mtiles(rows, n_groups), tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (tm * tn > MAX_GEMM_TILES)            // checked by the caller
        return hipErrorInvalidValue;
    GroupedGemmGrid g;
    g.tiles_n = (uint32_t)tn;
    g.max_mtiles = (uint32_t)tm;
    g.per_xcd = (uint32_t)((tm * tn + 7) / 8);
    const dim3 grid(8 * g.per_xcd), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(nvfp4_grouped_gemm_kernel<true>, grid, block, 0, stream, a,
                           a_block_scales, a_scales, b, b_block_scales, b_scales, seg_offsets,
                           n_groups, rows, N, K, g, c);
    else
        hipLaunchKernelGGL(nvfp4_grouped_gemm_kernel<false>, grid, block, 0, stream, a,
                           a_block_scales, a_scales, b, b_block_scales, b_scales, seg_offsets,
                           n_groups, rows, N, K, g, c);
    return hipGetLastError();
}

hipError_t launch_nvfp4_gemm(const uint8_t *a, const uint8_t *a_block_scales,
                             const float *a_scales, int64_t rows_per_a, const uint8_t *b,
                             const uint8_t *b_block_scales, const float *b_scales,
                             int64_t rows_per_b, int64_t M, int64_t N, int64_t K, bool bf16_out,
                             void *c, hipStream_t stream)
{
    const int64_t tm = (M + GEMM_BM - 1) / GEMM_BM, tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (tm * tn > MAX_GEMM_TILES)            // checked by the caller
        return hipErrorInvalidValue;
    GemmGrid g;
    g.tiles_m = (uint32_t)tm;
    g.tiles_n = (uint32_t)tn;
    g.per_xcd = (uint32_t)((tm * tn + 7) / 8);
    g.group_m = (uint32_t)(tm < 8 ? tm : 8);
    const dim3 grid(8 * g.per_xcd), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(nvfp4_gemm_kernel<true>, grid, block, 0, stream, a, a_block_scales,
                           a_scales, rows_per_a, b, b_block_scales, b_scales, rows_per_b, M, N, K,
                           g, c);
    else
        hipLaunchKernelGGL(nvfp4_gemm_kernel<false>, grid, block, 0, stream, a, a_block_scales,
                           a_scales, rows_per_a, b, b_block_scales, b_scales, rows_per_b, M, N, K,
                           g, c);
    return hipGetLastError();
}

// Grouped product over each segment's rows (the expert layer's weight
// gradient): for expert e, C_e[m][n] = sum over k in [32 P[e], 32 P[e+1])
// of A[m][k] B[n][k], where A [M][ld] and B [N][ld] are grouped transposed
// padded columnwise copies (scales [.][ld / 32]) whose segment e occupies
// columns 32 P[e] .. 32 P[e+1] (a multiple of 128 wide); C [G][M][N].
// P is device data: each range is clamped into [0, ld) and cut to whole
// 128-column steps, so malformed offsets give meaningless tiles, never an
// access out of bounds.
template <bool BF16_OUT>
__global__ void __launch_bounds__(GEMM_THREADS) mxfp8_grouped_wgrad_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const int64_t *__restrict__ P, int64_t G, int64_t M,
    int64_t N, int64_t ld, GroupedGemmGrid grid, void *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GEMM_LDS_BYTES];
    const uint32_t w = wg_id();
    const uint32_t L = (w & 7) * grid.per_xcd + (w >> 3);
    const uint32_t per_e = grid.max_mtiles * grid.tiles_n;
    const int64_t e = L / per_e;
    if (e >= G)
        return;
    const uint32_t r = L % per_e, mt = r / grid.tiles_n, nt = r % grid.tiles_n;
    int64_t k0 = P[e] * TILE_K_BLOCK, k1 = P[e + 1] * TILE_K_BLOCK;
    k0 = k0 < 0 ? 0 : (k0 > ld ? ld : k0) & ~(int64_t)127;
    k1 = k1 < k0 ? k0 : (k1 > ld ? ld : k1);
    const int64_t K = (k1 - k0) & ~(int64_t)127;
    const int64_t esz = BF16_OUT ? 2 : 4;
    mxg_tile<BF16_OUT>(lds, A + k0, As + (k0 >> 5), B + k0, Bs + (k0 >> 5), M, N, K, ld,
                       (int64_t)mt * GEMM_BM, (int64_t)nt * GEMM_BN,
                       reinterpret_cast<uint8_t *>(C) + e * M * N * esz);
}

hipError_t launch_mxfp8_grouped_wgrad(const uint8_t *a, const uint8_t *a_scales,
                                      const uint8_t *b, const uint8_t *b_scales,
                                      const int64_t *block_offsets, int64_t n_groups, int64_t M,
                                      int64_t N, int64_t ld, bool bf16_out, void *c,
                                      hipStream_t stream)
{
    const int64_t tm = (M + GEMM_BM - 1) / GEMM_BM, tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (n_groups * tm * tn > MAX_GEMM_TILES)  // checked by the caller
        return hipErrorInvalidValue;
    GroupedGemmGrid g;
    g.tiles_n = (uint32_t)tn;
    g.max_mtiles = (uint32_t)tm;
    g.per_xcd = (uint32_t)((n_groups * tm * tn + 7) / 8);
    const dim3 grid(8 * g.per_xcd), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(mxfp8_grouped_wgrad_kernel<true>, grid, block, 0, stream, a, a_scales,
                           b, b_scales, block_offsets, n_groups, M, N, ld, g, c);
    else
        hipLaunchKernelGGL(mxfp8_grouped_wgrad_kernel<false>, grid, block, 0, stream, a,
                           a_scales, b, b_scales, block_offsets, n_groups, M, N, ld, g, c);
    return hipGetLastError();
}

hipError_t launch_mxfp8_grouped_gemm(const uint8_t *a, const uint8_t *a_scales,
                                     const uint8_t *b, const uint8_t *b_scales,
                                     const int64_t *seg_offsets, int64_t n_groups, int64_t rows,
                                     int64_t N, int64_t K, bool bf16_out, void *c,
                                     hipStream_t stream)
{
    const int64_t tm = grouped_gemm_mtiles(rows, n_groups), tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (tm * tn > MAX_GEMM_TILES)            // checked by the caller
        return hipErrorInvalidValue;
    GroupedGemmGrid g;
    g.tiles_n = (uint32_t)tn;
    g.max_mtiles = (uint32_t)tm;
    g.per_xcd = (uint32_t)((tm * tn + 7) / 8);
    const dim3 grid(8 * g.per_xcd), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(mxfp8_grouped_gemm_kernel<true>, grid, block, 0, stream, a, a_scales,
                           b, b_scales, seg_offsets, n_groups, rows, N, K, g, c);
    else
        hipLaunchKernelGGL(mxfp8_grouped_gemm_kernel<false>, grid, block, 0, stream, a, a_scales,
                           b, b_scales, seg_offsets, n_groups, rows, N, K, g, c);
    return hipGetLastError();
}

hipError_t launch_mxfp8_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b,
                             const uint8_t *b_scales, int64_t M, int64_t N, int64_t K,
                             bool bf16_out, void *c, hipStream_t stream)
{
    const int64_t tm = (M + GEMM_BM - 1) / GEMM_BM, tn = (N + GEMM_BN - 1) / GEMM_BN;
    if (tm * tn > MAX_GEMM_TILES)            // checked by the caller
        return hipErrorInvalidValue;
    GemmGrid g;
    g.tiles_m = (uint32_t)tm;
    g.tiles_n = (uint32_t)tn;
    g.per_xcd = (uint32_t)((tm * tn + 7) / 8);
    g.group_m = (uint32_t)(tm < 8 ? tm : 8);
    const dim3 grid(8 * g.per_xcd), block(GEMM_THREADS);
    if (bf16_out)
        hipLaunchKernelGGL(mxfp8_gemm_kernel<true>, grid, block, 0, stream, a, a_scales, b,
                           b_scales, M, N, K, g, c);
    else
        hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, grid, block, 0, stream, a, a_scales, b,
                           b_scales, M, N, K, g, c);
    return hipGetLastError();
}

}  // namespace mxq
