// mhc_scratch.hip -- the device memory behind mhc_pre_forward_noalloc: a file-scope device
// array of kScratchBytes that every GPU the library runs on holds from module load to the
// end of the process (zero-filled at load), used as that call's workspace.
//
// In host code the array's name is only a stand-in for the symbol, not a device address:
// its address on a device comes from hipGetSymbolAddress, called once per device with that
// device current, and only that address is ever handed to a kernel or a copy.
#include <hip/hip_runtime.h>

#include <array>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "mhc_plan.h"

namespace mhc {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
std::array<void*, kMaxDevices> g_addr{};   // per device: the array's address there, once looked up

}  // namespace

int scratch_for_current_device(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return 0;
}

}  // namespace mhc
