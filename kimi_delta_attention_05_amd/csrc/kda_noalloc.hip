// Fixed device scratch for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): kda_chunk_fwd_noalloc runs the chunkwise prefill with its
// workspace in this file-scope array instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of the array (allocated when
// the code object is loaded on that device, kept until the process ends). In
// host code the array's name is only a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress and that
// address is what reaches the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "kda_internal.h"

static __device__ __align__(256) unsigned char scratch[kda::kNoAllocScratchBytes];

namespace kda {

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (a == 0) {
        // first call on this device (it is current): look up this device's copy
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        a = (uintptr_t)p;
        g_scratch_addr[dev].store(a, std::memory_order_release);
    }
    *ptr = (void *)a;
    return hipSuccess;
}

}  // namespace kda
