// mxq_floor.hip -- the measurement reference beside the quantizers: a kernel
// that reads a given number of bytes and writes a given number of bytes with
// no arithmetic beyond an XOR fold, in the quantizers' launch style (a
// one-shot grid, every thread moving 16-byte chunks, every load and store
// instruction coalesced across its wavefront).  Its time for a workload's read
// and write bytes is the floor that any kernel moving exactly those bytes
// meets on the device, so a quantizer's time can be stated against it as well
// as against the HBM peak.
//
//   reads >= writes (fold):   out chunk j = XOR of in chunks j + i n_w, over
//                             every i with j + i n_w < n_r.
//   reads <  writes (spread): out chunk j = in chunk floor(j m / 2^32), with
//                             m = floor(n_r 2^32 / n_w) (a multiply, not a
//                             division, per thread); the threads of a
//                             wavefront read adjacent chunks, so each input
//                             line is fetched once.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int FLOOR_THREADS = 256;
constexpr int FLOOR_BATCH = 8;

template <bool FOLD>
__global__ void __launch_bounds__(FLOOR_THREADS)
    copy_floor_kernel(const u32x4_t *__restrict__ src, int64_t n_r, u32x4_t *__restrict__ dst,
                      int64_t n_w, uint64_t k)
{
    const int64_t j = (int64_t)wg_id() * FLOOR_THREADS + tid();
    if (j >= n_w)
        return;
    u32x4_t v;
    if constexpr (FOLD) {
        // Eight loads in flight per thread before any is consumed (a plain
        // loop waits for each load before issuing the next, which makes a
        // read-heavy floor latency-bound: 4 reads per write took 9.5 us on
        // 33.5 MB in + 9.5 MB out).
        v = __builtin_nontemporal_load(src + j);
        for (int64_t i0 = 1; i0 < (int64_t)k; i0 += FLOOR_BATCH) {
            u32x4_t t[FLOOR_BATCH];
#pragma unroll
            for (int u = 0; u < FLOOR_BATCH; u++) {
                const int64_t c = j + (i0 + u) * n_w;
                t[u] = u32x4_t{0u, 0u, 0u, 0u};
                if (i0 + u < (int64_t)k && c < n_r)
                    t[u] = __builtin_nontemporal_load(src + c);
            }
#pragma unroll
            for (int u = 0; u < FLOOR_BATCH; u++)
                v ^= t[u];
        }
    } else {
        v = src[((uint64_t)j * k) >> 32];      // k = m: n_w <= 2^31, so j m < 2^63
    }
    __builtin_nontemporal_store(v, dst + j);
}

hipError_t launch_copy_floor(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                             hipStream_t stream)
{
    const int64_t n_r = src_bytes / 16, n_w = dst_bytes / 16;
    if (n_w > MAX_GRID_ITEMS)           // checked by the caller
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n_w + FLOOR_THREADS - 1) / FLOOR_THREADS)), block(FLOOR_THREADS);
    const u32x4_t *s = reinterpret_cast<const u32x4_t *>(src);
    u32x4_t *d = reinterpret_cast<u32x4_t *>(dst);
    if (n_r >= n_w)
        hipLaunchKernelGGL(copy_floor_kernel<true>, grid, block, 0, stream, s, n_r, d, n_w,
                           (uint64_t)((n_r + n_w - 1) / n_w));
    else    // n_r < n_w <= 2^31: m < 2^32
        hipLaunchKernelGGL(copy_floor_kernel<false>, grid, block, 0, stream, s, n_r, d, n_w,
                           (uint64_t)(((unsigned __int128)n_r << 32) / (uint64_t)n_w));
    return hipGetLastError();
}

}  // namespace mxq
