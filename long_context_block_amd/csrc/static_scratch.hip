// static_scratch.hip — the library's one device-resident scratch array, for callers that cannot
// allocate (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in the code object: each device the library runs on holds its own copy from
// the first use until the process ends.  Host code never passes the array's name to a kernel
// (in host code that name is only a stand-in for the symbol); the device address of the current
// device's copy is looked up once per device with hipGetSymbolAddress and cached.

#include <mutex>

#include "bsa_internal.hpp"

namespace bsa {
namespace {

static __device__ __align__(256) unsigned char scratch[BSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace bsa
