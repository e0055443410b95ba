// noalloc.hip -- the static workspace of wave_run_blocked_noalloc.
//
// The time-blocked leapfrog needs two more fields of the grid's shape for
// the intermediate time levels.  For callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc), those two fields live in this file-scope device array
// instead: each GPU the library runs on holds its own copy from the first
// use until the process ends.
//
// In host code the name `scratch` is only the host-side stand-in of the
// array, not a device address.  Its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and cached; kernels
// and copies are only ever given that address.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "stencil3d.h"

static __device__ __align__(256) unsigned char scratch[2 * (size_t)ST_NOALLOC_FIELD_BYTES_MAX];

namespace st {
namespace {

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not yet)
std::mutex g_scratch_mutex;

}  // namespace

int noalloc_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ST_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();  // leave no sticky error for the next call
            return ST_ERR_DEVICE;
        }
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = sizeof(scratch);
    return ST_OK;
}

}  // namespace st
