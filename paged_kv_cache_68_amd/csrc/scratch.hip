// Library-owned scratch memory for paged_attention_decode_noalloc: a fixed array in the
// code object's device data, one copy per GPU, so that the call allocates nothing.
//
// Host code never uses the array's name as an address (on the host it only names the
// symbol): the device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is the only pointer handed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace pkv {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace pkv
