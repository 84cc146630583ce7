// Fixed device workspace of the entry point that allocates nothing
// (mt_prefill_noalloc in include/mt.h): the prefill row workspace in a
// file-scope device array instead of memory from hipMalloc.  Each GPU the
// library runs on holds its own copy of the array until the process ends.
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address: the address of this device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current (at
// mt_create) and kept per device.  Only that pointer is ever passed to
// kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mt_internal.h"

namespace {

constexpr size_t kScratchFloats = size_t(9) << 20;  // 36 MiB
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

std::mutex g_mu;
float* g_scratch[kMaxDevices] = {};

}  // namespace

namespace mt {

size_t noalloc_scratch_floats() { return kScratchFloats; }

hipError_t noalloc_scratch_setup(int device, float** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[device] = static_cast<float*>(p);
    }
    *out = g_scratch[device];
    return hipSuccess;
}

}  // namespace mt
