// Device workspace for launches that need scratch memory (the split-K
// partial products).
//
// Each device keeps one cached buffer, allocated stream-ordered from a
// memory pool this library owns and grown on demand, so that a steady
// stream of calls makes no allocator call at all.  Uses on one stream are
// ordered by the stream itself, and as long as every use has been on one
// stream nothing else is done (an event per call costs about 2 us of GPU
// time between back-to-back calls).  The first use on a second stream waits
// for the whole device once (the earlier stream may no longer exist, so its
// work cannot be waited for through it); from then on every use records the
// device's event on its stream after its last launch, and a use on another
// stream first waits for that event.  A request larger than kCacheMax gets a
// buffer of its own, allocated and freed stream-ordered around that one
// call.
#include <mutex>

#include "kernels.h"

namespace sgemm {

namespace {
constexpr size_t kCacheMax = size_t(256) << 20;

struct DeviceWorkspace {
    std::mutex mu;
    hipMemPool_t pool = nullptr;
    hipEvent_t done = nullptr;     // recorded after the latest use
    hipStream_t last = nullptr;    // stream of the latest use
    bool used = false;
    bool multi = false;            // used from more than one stream: events recorded
    void* buf = nullptr;
    size_t cap = 0;
};
DeviceWorkspace g_ws[kMaxDevices];

hipError_t device_of(hipStream_t s, int* dev) {
    return s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
}

// Pool and event of a device, created on first use (caller holds the lock).
hipError_t init(DeviceWorkspace& w, int dev) {
    hipError_t e;
    if (!w.pool) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if ((e = hipMemPoolCreate(&p, &props)) != hipSuccess) return e;
        uint64_t keep = kCacheMax;
        if ((e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return e;
        }
        w.pool = p;
    }
    if (!w.done && (e = hipEventCreateWithFlags(&w.done, hipEventDisableTiming)) != hipSuccess)
        return e;
    return hipSuccess;
}
}  // namespace

hipError_t workspace_acquire(size_t bytes, hipStream_t s, Workspace* out) {
    int dev = 0;
    hipError_t e = device_of(s, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceWorkspace& w = g_ws[dev];
    std::unique_lock<std::mutex> lock(w.mu);
    if ((e = init(w, dev)) != hipSuccess) return e;
    if (bytes > kCacheMax) {
        out->own = true;
        out->dev = dev;
        return hipMallocFromPoolAsync(&out->ptr, bytes, w.pool, s);
    }
    // Order this use after the latest one when it ran on another stream.
    if (w.used && w.last != s) {
        if (!w.multi) {
            if ((e = hipDeviceSynchronize()) != hipSuccess) return e;
            w.multi = true;
        } else if ((e = hipStreamWaitEvent(s, w.done, 0)) != hipSuccess) {
            return e;
        }
    }
    if (bytes > w.cap) {
        size_t cap = w.cap ? w.cap : (size_t(4) << 20);
        while (cap < bytes) cap *= 2;
        if (cap > kCacheMax) cap = kCacheMax;
        void* p = nullptr;
        if ((e = hipMallocFromPoolAsync(&p, cap, w.pool, s)) != hipSuccess) return e;
        if (w.buf) (void)hipFreeAsync(w.buf, s);
        w.buf = p;
        w.cap = cap;
    }
    out->ptr = w.buf;
    out->own = false;
    out->dev = dev;
    out->lock = std::move(lock);
    return hipSuccess;
}

hipError_t workspace_release(Workspace* ws, hipStream_t s) {
    if (ws->own) return hipFreeAsync(ws->ptr, s);
    DeviceWorkspace& w = g_ws[ws->dev];
    const hipError_t e = w.multi ? hipEventRecord(w.done, s) : hipSuccess;
    w.last = s;
    w.used = true;
    ws->lock.unlock();
    return e;
}

}  // namespace sgemm
