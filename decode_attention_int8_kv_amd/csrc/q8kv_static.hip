// q8kv_static.hip -- q8_decode_step_static: the decode step for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It runs the kernels of q8_decode_step,
// with the partial records they need kept in `scratch`, a device array of
// this library instead of a caller workspace.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy at its own address until the process ends.  In host
// code its name is only a stand-in for that symbol, so the device address is
// looked up with hipGetSymbolAddress once per device (with that device
// current) and every launch gets the looked-up pointer.
#include <mutex>

#include "q8kv_internal.hpp"

namespace q8kv {

constexpr size_t kScratchBytes = 16u << 20;   // 16 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

// The device address of this device's `scratch` (looked up on first use).
hipError_t static_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace q8kv
