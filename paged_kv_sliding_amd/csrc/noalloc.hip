// noalloc.hip -- the library's fixed device scratch array, used by
// pkvs_decode_noalloc in place of caller workspaces.
//
// Every device the library runs on holds its own copy of `scratch` (the code
// object's data, loaded with the library's kernels) until the process ends.
// Host code never passes the array's name to a kernel or a copy: on the host
// that name is a stand-in, not a device address.  The device address is read
// once per device with hipGetSymbolAddress, with that device current, and
// kept; every later use goes through the kept pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkvs_internal.h"

static __device__ __align__(256) uint8_t scratch[PKVS_NOALLOC_SCRATCH_BYTES];

namespace pkvs {

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t scratch_for_device(int device, void **ptr)
{
    *ptr = nullptr;
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;  // the caller makes it current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace pkvs
