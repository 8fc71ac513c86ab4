// The workspace of the allocation-free entry point (ssd_fwd_noalloc): a
// fixed array in each GPU's memory, held from the library's load until the
// process ends.  Host code never uses the array's name as an address: it asks
// HIP for the array's device address once per device, with that device
// current, and keeps it (each GPU holds its own copy at its own address).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <string>

#include "ssd.h"

namespace ssd {

static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_WORKSPACE_BYTES];

namespace {
std::mutex g_scratch_mutex;
void *g_scratch_ptr[64];
}  // namespace

// Device address of `scratch` on device `dev`; nullptr with *err set on
// failure.
void *noalloc_scratch(int dev, std::string *err) {
    char buf[256];
    if (dev < 0 || dev >= 64) {
        snprintf(buf, sizeof(buf), "device %d out of range", dev);
        *err = buf;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        *err = "hipGetDevice failed";
        return nullptr;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        snprintf(buf, sizeof(buf), "hipSetDevice(%d) failed", dev);
        *err = buf;
        return nullptr;
    }
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        snprintf(buf, sizeof(buf), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        *err = buf;
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace ssd
