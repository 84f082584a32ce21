// The library's static device scratch: the scratch memory of the entry point
// that allocates nothing (sgemm_f32_ex_split_noalloc), for callers that may
// not allocate device memory.
//
// The array below is part of the library's code object, so every device the
// library runs on holds one copy of it, at that device's own address, from
// the code object's load until the process ends.  In host code its name is
// only a host-side handle: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and kernels take that address as an argument.  Every call on a device
// shares the device's copy, which keeps the last call's contents; nothing in
// it needs to start at zero (packed copies and partial products are written
// in full before they are read).  Calls that overlap in time on one device,
// from different streams or threads, race on it.
#include <mutex>

#include "kernels.h"

namespace sgemm {

static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];  // device address per device, once looked up
}  // namespace

hipError_t static_scratch(hipStream_t s, FixedScratch* out) {
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t f = hipSetDevice(cur);
            if (e == hipSuccess) e = f;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    out->ptr = g_scratch_ptr[dev];
    out->bytes = kStaticScratchBytes;
    return hipSuccess;
}

}  // namespace sgemm
