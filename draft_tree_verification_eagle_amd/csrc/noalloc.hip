// Tree attention for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
// kernels as eagle_tree_attention, with the split-KV partials in a file-scope
// device array instead of a caller workspace.
//
// Each GPU that runs this entry point holds its own copy of the array until the
// process ends.  Its device address is taken once per device with
// hipGetSymbolAddress (the array's name in host code is only a host-side stand-in)
// and kept per device.  The partials need no initialisation (every slot the merge
// reads is written earlier in the same call), so nothing is cleared; calls that
// overlap on one GPU share the array and race.
#include <mutex>

#include "launchers.hpp"

namespace eagle {
namespace {

static __device__ __align__(256) unsigned char scratch[EAGLE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once taken

// The array's device address on the current device (taken on the first call there).
hipError_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_attention_noalloc(const eagle_attn_desc& d, const void* q, const void* k, const void* v,
                                    const uint64_t* mask, void* o, float* lse, hipStream_t stream) {
    void* ws = nullptr;
    hipError_t e = scratch_for_current_device(&ws);
    if (e != hipSuccess) return e;
    return launch_attention(d, q, k, v, mask, o, lse, ws, stream);
}

}  // namespace eagle
