// mxq_runtime.cpp -- launch geometry for the grid-stride kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxq_launch.h"

namespace mxq {

namespace {

struct Entry {
    const void *kernel;
    int device;
    int block;
    int64_t wgs;
};

constexpr int CACHE = 64;
Entry cache[CACHE];
int cache_n = 0;
std::mutex cache_mu;

}  // namespace

int64_t resident_workgroups(const void *kernel, int block_threads)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1024;
    }
    {
        std::lock_guard<std::mutex> lock(cache_mu);
        for (int i = 0; i < cache_n; i++)
            if (cache[i].kernel == kernel && cache[i].device == dev &&
                cache[i].block == block_threads)
                return cache[i].wgs;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) !=
            hipSuccess) {
        (void)hipGetLastError();
        return 1024;
    }
    if (per_cu < 1)
        per_cu = 1;
    const int64_t wgs = (int64_t)cus * per_cu;
    std::lock_guard<std::mutex> lock(cache_mu);
    if (cache_n < CACHE)
        cache[cache_n++] = Entry{kernel, dev, block_threads, wgs};
    return wgs;
}

}  // namespace mxq
