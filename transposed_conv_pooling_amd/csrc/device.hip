// device.hip - per-device facts the launchers size their grids with, queried
// once and cached: the compute-unit count of each device, the occupancy of
// each (kernel, block size, dynamic LDS) on each device, and the largest
// dynamic-LDS size already granted to a kernel on each device.  Every lookup
// after the first is a read under a mutex (no HIP call besides the
// thread-local hipGetDevice).
#include <mutex>
#include <vector>

#include "ct_internal.h"

namespace ct {
namespace {

struct OccKey {
    int dev;
    const void *fn;
    int threads;
    size_t lds;
    int value;
};

struct LdsKey {
    int dev;
    const void *fn;
    int granted;
};

std::mutex g_mu;
std::vector<int> g_cus;           // by device ordinal; 0 = not yet queried
std::vector<OccKey> g_occ;
std::vector<LdsKey> g_lds;

}  // namespace

int current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

int device_cus()
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_cus.size() <= dev) g_cus.resize(dev + 1, 0);
    if (g_cus[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;                    // MI355X
        g_cus[dev] = cus;
    }
    return g_cus[dev];
}

int occupancy(const void *fn, int threads, size_t lds)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    for (const OccKey &k : g_occ)
        if (k.dev == dev && k.fn == fn && k.threads == threads && k.lds == lds) return k.value;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    g_occ.push_back({dev, fn, threads, lds, per_cu});
    return per_cu;
}

hipError_t allow_dynamic_lds(const void *fn, size_t lds)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    for (LdsKey &k : g_lds)
        if (k.dev == dev && k.fn == fn) {
            if ((size_t)k.granted >= lds) return hipSuccess;
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e == hipSuccess) k.granted = (int)lds;
            return e;
        }
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess) g_lds.push_back({dev, fn, (int)lds});
    return e;
}

}  // namespace ct
