// Launch geometry helpers: compute-unit count and resident blocks per kernel.
#include <mutex>
#include <unordered_map>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Blocks of kern (launched with `threads` threads each) that are resident on
// the current device at once (occupancy per compute unit times compute units),
// cached per (kernel, device): each kernel is launched with one block size.
int resident_blocks(const void* kern, int threads)
{
    static std::mutex mu;
    static std::unordered_map<const void*, int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache[dev].find(kern);
    if (it != cache[dev].end()) return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, 0) != hipSuccess || nb < 1) nb = 1;
    const int blocks = nb * device_cus();
    cache[dev][kern] = blocks;
    return blocks;
}

}  // namespace tq
