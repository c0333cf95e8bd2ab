// Library-owned scratch for twomamba_fwd_noalloc: the forward's workspace for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// The buffer is a file-scope device array, so the loader places one copy on
// every GPU the library's code object is loaded on, and it lives until the
// process ends.  Host code never passes the array's name to a kernel or a copy
// (on the host it names a stand-in, not device memory): the device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and kept in a table.  Every call on one GPU shares that GPU's array; calls
// that overlap on one GPU (other streams, other host threads) race on it.
#include <mutex>

#include "internal.h"

#include <hip/hip_runtime.h>

namespace {

static __device__ __align__(256) unsigned char scratch[TWOMAMBA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];   // scratch's device address per device, NULL until looked up

}  // namespace

namespace twm {

int noalloc_scratch(void* stream, void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TWOMAMBA_ERR_DEVICE;
    if (stream != nullptr) {
        // the scratch of the stream's device is used; it must be the current one, whose
        // symbol address is looked up below
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess || sdev != dev) return TWOMAMBA_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TWOMAMBA_ERR_DEVICE;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return TWOMAMBA_OK;
}

}  // namespace twm
