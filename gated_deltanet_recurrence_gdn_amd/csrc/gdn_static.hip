// gdn_static.hip -- the fixed device array behind gdn_forward_noalloc.
//
// gdn_forward_noalloc serves callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The scratch its kernels need lives in one file-scope device array
// of a fixed size instead of a handle's allocation.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device memory):
// the first call on a device, with that device current, resolves the array's
// device address with hipGetSymbolAddress and keeps it per device; every later
// use goes through that address.
#include "gdn_launch.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[gdn::STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES];       // resolved device address of `scratch`, per device
bool g_checked[MAX_DEVICES];    // the device was checked to be a gfx950

}  // namespace

namespace gdn {

hipError_t static_scratch(int device, void **ptr, bool *is_gfx950) {
    *ptr = nullptr;
    *is_gfx950 = false;
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_checked[device]) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, device);
        if (e != hipSuccess) return e;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return hipSuccess;  // *is_gfx950 stays false
        g_checked[device] = true;
    }
    *is_gfx950 = true;
    if (!g_ptr[device]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != device) (void)hipSetDevice(prev);
        if (e != hipSuccess) return e;
        g_ptr[device] = p;
    }
    *ptr = g_ptr[device];
    return hipSuccess;
}

}  // namespace gdn
