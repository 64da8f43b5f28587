// The fused forward for callers that cannot allocate: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc. It runs
// moe_fused_fwd with the library's own device scratch array as the
// workspace instead of one the caller brings.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy, at its own address, from module load until the
// process ends. Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in, not a device address): once per device,
// with that device current, its address comes from hipGetSymbolAddress and is
// kept in a per-device table, and that pointer is what the kernels get.
//
// Every call on one GPU shares that GPU's array and leaves the last call's
// contents in it; the fused forward needs nothing in its workspace on entry
// (every segment is written before it is read), so nothing is cleared. Calls
// that overlap on one GPU (two streams, or two host threads) race on the
// array: callers order them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "moe_internal.h"
#include "moeffn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device.
int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::report_error(MOE_ERR_HIP, "hipGetDevice", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return moe::report_error(MOE_ERR_UNSUPPORTED, "device index", "beyond 64");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return moe::report_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch)", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_fused_fwd_noalloc(const moe_fused_args_t* args, moe_stream_t stream) {
    size_t need = 0;
    int rc = moe_fused_workspace_size(args, &need);
    if (rc != MOE_OK) return rc;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
        char msg[160];
        snprintf(msg, sizeof msg, "this call needs %zu bytes, the built-in scratch holds %zu", need,
                 (size_t)MOE_NOALLOC_SCRATCH_BYTES);
        return moe::report_error(MOE_ERR_WORKSPACE, "moe_fused_fwd_noalloc", msg);
    }
    void* ws = nullptr;
    if ((rc = scratch_of_current_device(&ws)) != MOE_OK) return rc;
    return moe_fused_fwd(args, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
