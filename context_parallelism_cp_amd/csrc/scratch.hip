// scratch.hip -- the library's own device scratch memory, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// One file-scope device array holds the per-row dvec of the backward pass
// (dout . out, Hq x rows floats) for cp_ring_bwd_noalloc.  Every GPU the
// library runs on holds its own copy, at its own address, from the time the
// code object is loaded until the process ends.  In host code the array's
// name is only a stand-in for the device symbol: its device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels.
#include "cp_kernels.h"

#include <mutex>

namespace cpattn {

namespace {

__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_floats(float **ptr)
{
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_ptr[dev] = (float *)p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace cpattn
