// noalloc.hip -- the scratch memory of the entry points that allocate nothing.
//
// A file-scope device array, one copy per GPU the library runs on, held until the process
// ends.  In host code its name is only a host-side stand-in, so the device address is
// looked up once per device with hipGetSymbolAddress, with that device current, and kept;
// every launch takes that address.  Every call on a GPU shares the GPU's copy: calls that
// overlap on one GPU (on different streams, or from different threads) race.
#include <mutex>

#include "ulp_kernels.h"

namespace ulp {
namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_pointer(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ulp
