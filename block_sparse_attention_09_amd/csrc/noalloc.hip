// noalloc.hip -- the scratch memory of msa_sparse_attn_prefill_noalloc: one
// static device array per GPU, so that callers that cannot allocate (code
// under graph capture, tight serving loops) still get the prefill's remap
// workspace.
//
// The array is a module global: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Host code must not use
// the array's name as a device address (on the host it names a stand-in);
// the address on the current device comes from hipGetSymbolAddress, looked up
// once per device and kept.
#include "msa_internal.h"

#include <mutex>

namespace msa {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace msa
