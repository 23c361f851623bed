// noalloc.hip -- coli_moe_route_forward_noalloc: the one-call layer step of
// coli_moe_route_forward with its scratch in a static device array instead
// of a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates: the array is part of the library's
// code object, present on every device the library is loaded on until the
// process ends.
#include <mutex>

#include "common.h"

// The scratch of every call on one device (the workspace of
// coli_moe_route_forward).  In host code this name only identifies the
// symbol for the lookup below; it is never used as a device address.
static __device__ __align__(256) uint8_t scratch[COLI_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// Device address of the current device's copy of `scratch`: looked up once
// per device, with that device current, on its first call.
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COLI_E_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();  // clear the error the failed lookup left
            return COLI_E_DEVICE;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return COLI_OK;
}

}  // namespace

extern "C" int coli_moe_route_forward_noalloc(const coli_moe_layer *L, const float *x, int32_t T,
                                              float top_p, int32_t *topk_ids, float *topk_w,
                                              int32_t *union_ids, int32_t *offsets,
                                              int32_t *slots, int32_t *n_union, int32_t act_mode,
                                              float *y, void *hip_stream)
{
    // every host check of coli_moe_route_forward, then COLI_E_SCRATCH for a
    // shape beyond the array, then the lookup
    return coli::route_forward_scratch(L, x, T, top_p, topk_ids, topk_w, union_ids, offsets, slots,
                                       n_union, act_mode, y, hip_stream,
                                       scratch_of_current_device);
}
