// Device workspace for launches that need scratch memory (the split-K
// partial products).  Allocation is stream-ordered from a memory pool owned
// by this library, one per device: a block freed on a stream is reused by
// the next allocation on any stream once the free is ordered before it, and
// up to kKeep bytes stay reserved between calls, so steady-state calls do not
// go to the driver or synchronize.
#include <mutex>

#include "kernels.h"

namespace sgemm {

namespace {
constexpr int kMaxDevices = 64;
constexpr uint64_t kKeep = uint64_t(256) << 20;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t pool_for(hipStream_t s, hipMemPool_t* out) {
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (!g_pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if ((e = hipMemPoolCreate(&p, &props)) != hipSuccess) return e;
        uint64_t keep = kKeep;
        if ((e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return e;
        }
        g_pools[dev] = p;
    }
    *out = g_pools[dev];
    return hipSuccess;
}
}  // namespace

hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t s) {
    hipMemPool_t pool;
    const hipError_t e = pool_for(s, &pool);
    if (e != hipSuccess) return e;
    return hipMallocFromPoolAsync(p, bytes, pool, s);
}

hipError_t workspace_free(void* p, hipStream_t s) { return hipFreeAsync(p, s); }

}  // namespace sgemm
