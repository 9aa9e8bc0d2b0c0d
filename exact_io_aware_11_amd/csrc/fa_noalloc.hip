// fa_noalloc.hip -- the static scratch buffer behind fa_decode_noalloc.
//
// fa_decode_noalloc serves callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops).  The split-KV decode needs
// scratch for its per-chunk partial results (o_s, lse_s), which fa_decode
// takes from a caller-provided workspace; here it lives in a file-scope
// device array instead.  The array is part of the library's code object, so
// each GPU the library runs on holds its own copy, at its own address, until
// the process ends.
//
// In host code the name `scratch` is only a host-side stand-in for that
// array, not a device address.  The device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and cached; the
// kernels receive that pointer as their partials buffer.
//
// Every call on one device shares that device's array and overwrites what the
// last call left there (the split kernels write every partial before the
// merge reads it, so nothing needs clearing).  Calls that overlap in time on
// one device -- on different streams, or from different host threads without
// ordering -- race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

namespace fa {

namespace {

static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // first call on this device, which is current: its own copy of
            // the array, at its own device address
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace fa
