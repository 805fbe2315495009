// Resident-workgroup counts for the launchers that size their grids to what
// the GPU holds at once.  Queried once per (device, kernel, shape) and cached.
#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

struct OccEntry {
    int dev;
    const void *fn;
    int threads;
    size_t lds;
    int blocks;
};

std::mutex g_mu;
OccEntry g_cache[128];
int g_used = 0;

}  // namespace

int resident_blocks(const void *fn, int threads, size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();  // clear it: the launch reports its own
        return 0;
    }
    {
        std::lock_guard<std::mutex> lock(g_mu);
        for (int i = 0; i < g_used; i++) {
            const OccEntry &c = g_cache[i];
            if (c.dev == dev && c.fn == fn && c.threads == threads && c.lds == lds) return c.blocks;
        }
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_used < 128) g_cache[g_used++] = OccEntry{dev, fn, threads, lds, cus * per_cu};
    return cus * per_cu;
}

}  // namespace ep
