// kda_scratch.hip -- the library's one file-scope device buffer, the workspace
// of kda_chunk_fwd_noalloc (for callers that cannot allocate device memory).
//
// `scratch` is a static __device__ array: every device the library runs on
// holds its own copy, at its own address, for the life of the process.  In
// host code its name is only a host-side stand-in, so its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; every later use takes that address.
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.hpp"

namespace kda {

static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once found
}  // namespace

hipError_t noalloc_scratch(int device, void **ptr) {
    *ptr = nullptr;
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (device != current || device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace kda
