// conv2d_fwd_noalloc: conv2d_fwd for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). The workspace of the planned form is a file-scope device
// array of kNoAllocScratchBytes that every GPU holds from the library's load
// until the process ends; the caller still passes x, w and y.
//
// In host code the array's name is a host-side stand-in, not a device
// address, so its address on each device is taken once, with that device
// current, by hipGetSymbolAddress on the first call there, and only that
// pointer is handed to kernels. Calls on one GPU share its array: calls that
// overlap on one GPU (two streams, or threads) race on it. No kernel of the
// library relies on the workspace's earlier contents (every element read is
// written first in the same call), so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "im2win_conv2d.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) static unsigned char scratch[IM2WIN_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// the array's address on the current device, taken once per device
conv2d_status_t scratch_on_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONV2D_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CONV2D_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return CONV2D_OK;
}

}  // namespace

extern "C" conv2d_status_t conv2d_fwd_noalloc(const conv2d_desc_t *d, const void *x, const void *w,
                                               void *y, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_plan_t p;
    const conv2d_status_t st = conv2d_plan(d, &p);
    if (st != CONV2D_OK) return st;
    if (p.ws_bytes > int64_t(IM2WIN_NOALLOC_SCRATCH_BYTES)) return CONV2D_ERR_SCRATCH;
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        const conv2d_status_t s2 = scratch_on_current_device(&ws);
        if (s2 != CONV2D_OK) return s2;
    }
    return conv2d_fwd(d, x, w, y, ws, stream);
}
