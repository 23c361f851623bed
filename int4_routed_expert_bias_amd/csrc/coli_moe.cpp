// coli_moe.cpp -- host entry points of libcoli_moe.so (C ABI declared in
// include/coli_moe.h).  Every argument, shape and alignment check runs on
// the host before the first HIP call; kernels are enqueued on the caller's
// stream (the grouped GEMM of up to 1,024 tokens also on two side streams
// forked from it and joined back, created once per device); nothing is
// allocated, freed or synchronised here.
#include "../../include/coli_moe.h"

#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"

using namespace coli;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(int32_t H, int32_t I, int32_t E, int32_t k, int32_t T)
{
    if (H < 64 || H > COLI_MAX_H || H % 64) return COLI_E_SHAPE;
    if (I < 64 || I > COLI_MAX_I || I % 64) return COLI_E_SHAPE;
    if (E < 1 || E > COLI_MAX_E) return COLI_E_SHAPE;
    if (k < 1 || k > COLI_MAX_K || k > E) return COLI_E_SHAPE;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    return COLI_OK;
}

int check_layer(const coli_moe_layer *L, bool need_experts)
{
    if (!L) return COLI_E_ARG;
    if (L->n_shared != 0 && L->n_shared != 1) return COLI_E_SHAPE;
    if (int st = check_dims(L->H, L->I, L->E, L->k, 0)) return st;
    if (!L->router_w || !L->router_bias) return COLI_E_ARG;
    if (!aligned16(L->router_w) || !aligned16(L->router_bias)) return COLI_E_ALIGN;
    if (need_experts) {
        if (!L->w13 || !L->s13 || !L->w2 || !L->s2) return COLI_E_ARG;
        if (!aligned16(L->w13) || !aligned16(L->s13) || !aligned16(L->w2) || !aligned16(L->s2))
            return COLI_E_ALIGN;
        const bool any_sh = L->sh_w13 || L->sh_s13 || L->sh_w2 || L->sh_s2;
        const bool all_sh = L->sh_w13 && L->sh_s13 && L->sh_w2 && L->sh_s2;
        if (L->n_shared ? !all_sh : any_sh) return COLI_E_ARG;
        if (L->n_shared && (!aligned16(L->sh_w13) || !aligned16(L->sh_s13) ||
                            !aligned16(L->sh_w2) || !aligned16(L->sh_s2)))
            return COLI_E_ALIGN;
    }
    return COLI_OK;
}

std::atomic<int> g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

int device_check()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return COLI_E_DEVICE;
    if (dev < 0 || dev >= 64) return COLI_E_DEVICE;
    int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return COLI_E_DEVICE;
        s = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_state[dev].store(s, std::memory_order_relaxed);
    }
    return s == 1 ? COLI_OK : COLI_E_UNSUPPORTED;
}

std::atomic<int> g_dev_cus[64];  // 0 unknown, else the CU count

}  // namespace

int coli::device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = g_dev_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_dev_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

struct SideSlot {
    std::once_flag once;
    std::mutex mu;
    bool ok = false;
    SideSet set{};
};
SideSlot g_side[64];

void side_create(SideSlot &sl)
{
    SideSet &q = sl.set;
    bool ok = hipEventCreateWithFlags(&q.fork, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; i < 2 && ok; ++i)
        ok = hipStreamCreateWithFlags(&q.s[i], hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&q.join[i], hipEventDisableTiming) == hipSuccess;
    sl.ok = ok;
}

}  // namespace

SideSet *coli::side_fork(hipStream_t st, int n)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || n < 1 || n > 2) return nullptr;
    SideSlot &sl = g_side[dev];
    std::call_once(sl.once, side_create, std::ref(sl));
    if (!sl.ok) return nullptr;
    sl.mu.lock();
    SideSet *q = &sl.set;
    bool ok = hipEventRecord(q->fork, st) == hipSuccess;
    for (int i = 0; i < n && ok; ++i) ok = hipStreamWaitEvent(q->s[i], q->fork, 0) == hipSuccess;
    if (!ok) {
        sl.mu.unlock();
        return nullptr;
    }
    return q;
}

hipError_t coli::side_join(SideSet *q, hipStream_t st, int n)
{
    hipError_t err = hipSuccess;
    for (int i = 0; i < n; ++i) {
        if (err == hipSuccess) err = hipEventRecord(q->join[i], q->s[i]);
        if (err == hipSuccess) err = hipStreamWaitEvent(st, q->join[i], 0);
    }
    // the lock of the device whose set this is
    for (auto &sl : g_side)
        if (&sl.set == q) sl.mu.unlock();
    return err;
}

namespace {

LayerDev to_dev(const coli_moe_layer *L)
{
    LayerDev d;
    d.H = L->H; d.I = L->I; d.E = L->E; d.k = L->k; d.n_shared = L->n_shared;
    d.router_w = L->router_w; d.router_bias = L->router_bias;
    d.w13 = L->w13; d.s13 = L->s13; d.w2 = L->w2; d.s2 = L->s2;
    d.sh_w13 = L->sh_w13; d.sh_s13 = L->sh_s13; d.sh_w2 = L->sh_w2; d.sh_s2 = L->sh_s2;
    return d;
}

int status_of(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_E_DEVICE; }

}  // namespace

extern "C" {

int coli_moe_abi_version(void) { return COLI_MOE_ABI_VERSION; }

size_t coli_moe_workspace_bytes(int32_t H, int32_t I, int32_t E, int32_t k, int32_t T,
                                int32_t act_mode)
{
    if (check_dims(H, I, E, k, T) != COLI_OK) return 0;
    if (act_mode != COLI_ACT_F32 && act_mode != COLI_ACT_I8) return 0;
    return workspace_layout(H, I, E, k, T, act_mode, 1).total;
}

size_t coli_moe_acc_dump_bytes(int32_t H, int32_t I, int32_t k, int32_t T, int32_t n_shared)
{
    if (check_dims(H, I, k, k, T) != COLI_OK) return 0;
    if (n_shared != 0 && n_shared != 1) return 0;
    return dump_layout(H, I, k, T, n_shared).total;
}

int coli_moe_i8_workspace_offsets(int32_t H, int32_t I, int32_t E, int32_t k, int32_t T,
                                  int32_t n_shared, size_t *out)
{
    if (!out || (n_shared != 0 && n_shared != 1)) return COLI_E_ARG;
    if (check_dims(H, I, E, k, T) != COLI_OK || T <= kI8StreamTMax) return COLI_E_SHAPE;
    const Workspace w = workspace_layout(H, I, E, k, T, COLI_ACT_I8, n_shared);
    out[0] = w.o;
    out[1] = w.qh;
    out[2] = w.sh;
    return COLI_OK;
}

const char *coli_moe_strerror(int status)
{
    switch (status) {
    case COLI_OK: return "COLI_OK";
    case COLI_E_ARG: return "COLI_E_ARG: null pointer or invalid argument";
    case COLI_E_SHAPE: return "COLI_E_SHAPE: shape outside the supported limits";
    case COLI_E_ALIGN: return "COLI_E_ALIGN: tensor pointer not 16-byte aligned";
    case COLI_E_WORKSPACE: return "COLI_E_WORKSPACE: workspace too small";
    case COLI_E_DEVICE: return "COLI_E_DEVICE: HIP call or kernel launch failed";
    case COLI_E_UNSUPPORTED: return "COLI_E_UNSUPPORTED: device is not gfx950 or mode unknown";
    case COLI_E_SCRATCH:
        return "COLI_E_SCRATCH: shape needs more than the static scratch of the no-allocation "
               "entry point";
    default: return "unknown coli status";
    }
}

int coli_moe_device_check(void) { return device_check(); }

static int route_impl(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                      int32_t *topk_ids, float *topk_w, void *workspace, size_t workspace_bytes,
                      void *hip_stream)
{
    if (int st = check_layer(L, false)) return st;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    if (!(top_p > 0.0f)) return COLI_E_ARG;  // also rejects NaN
    if (T == 0) return COLI_OK;
    if (!x || !topk_ids || !topk_w || !workspace) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(workspace))
        return COLI_E_ALIGN;
    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, COLI_ACT_F32, L->n_shared);
    if (workspace_bytes < lay.route_end) return COLI_E_WORKSPACE;
    if (int st = device_check()) return st;
    RouteIO io{x, T, topk_ids, topk_w,
               reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + lay.logits), top_p};
    return status_of(launch_route(to_dev(L), io, static_cast<hipStream_t>(hip_stream)));
}

int coli_moe_route(const coli_moe_layer *L, const float *x, int32_t T, int32_t *topk_ids,
                   float *topk_w, void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return route_impl(L, x, T, 1.0f, topk_ids, topk_w, workspace, workspace_bytes, hip_stream);
}

int coli_moe_route_topp(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                        int32_t *topk_ids, float *topk_w, void *workspace, size_t workspace_bytes,
                        void *hip_stream)
{
    return route_impl(L, x, T, top_p, topk_ids, topk_w, workspace, workspace_bytes, hip_stream);
}

int coli_moe_route_union(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                         int32_t *topk_ids, float *topk_w, int32_t *union_ids, int32_t *offsets,
                         int32_t *slots, int32_t *n_union, void *workspace,
                         size_t workspace_bytes, void *hip_stream)
{
    if (int st = check_layer(L, false)) return st;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    if (!(top_p > 0.0f)) return COLI_E_ARG;  // also rejects NaN
    if (!n_union || !union_ids || !offsets) return COLI_E_ARG;
    if (!aligned16(union_ids) || !aligned16(offsets) || !aligned16(n_union)) return COLI_E_ALIGN;
    if (T == 0) {
        if (int st = device_check()) return st;
        return status_of(launch_union(nullptr, 0, L->k, L->E, union_ids, offsets, slots, n_union,
                                      static_cast<hipStream_t>(hip_stream)));
    }
    if (!x || !topk_ids || !topk_w || !slots || !workspace) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(slots) ||
        !aligned16(workspace))
        return COLI_E_ALIGN;
    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, COLI_ACT_F32, L->n_shared);
    if (workspace_bytes < lay.route_end) return COLI_E_WORKSPACE;
    if (int st = device_check()) return st;
    RouteIO io{x, T, topk_ids, topk_w,
               reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + lay.logits), top_p};
    UnionIO un{union_ids, offsets, slots, n_union};
    return status_of(launch_route(to_dev(L), io, static_cast<hipStream_t>(hip_stream), &un));
}

int coli_moe_union(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t *union_ids,
                   int32_t *offsets, int32_t *slots, int32_t *n_union, void *hip_stream)
{
    if (E < 1 || E > COLI_MAX_E) return COLI_E_SHAPE;
    if (k < 1 || k > COLI_MAX_K || k > E) return COLI_E_SHAPE;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    if (!n_union || !union_ids || !offsets) return COLI_E_ARG;
    if (T > 0 && (!topk_ids || !slots)) return COLI_E_ARG;
    if (!aligned16(union_ids) || !aligned16(offsets) || !aligned16(n_union) ||
        (T > 0 && (!aligned16(topk_ids) || !aligned16(slots))))
        return COLI_E_ALIGN;
    if (int st = device_check()) return st;
    return status_of(launch_union(topk_ids, T, k, E, union_ids, offsets, slots, n_union,
                                  static_cast<hipStream_t>(hip_stream)));
}

static int forward_impl(const coli_moe_layer *L, const float *x, int32_t T,
                        const int32_t *topk_ids, const float *topk_w, const int32_t *union_ids,
                        const int32_t *offsets, const int32_t *slots, const int32_t *n_union,
                        int32_t act_mode, float *y, void *workspace, size_t workspace_bytes,
                        int32_t *acc_dump, void *hip_stream, Marks *mk)
{
    if (int st = check_layer(L, true)) return st;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    if (act_mode != COLI_ACT_F32 && act_mode != COLI_ACT_I8) return COLI_E_UNSUPPORTED;
    if (acc_dump && act_mode != COLI_ACT_I8) return COLI_E_ARG;
    if (mk) {
        const int need = 2 * forward_kernel_count(act_mode, T);
        if (!mk->ev || mk->n < need) return COLI_E_ARG;
        for (int i = 0; i < need; ++i)
            if (!mk->ev[i]) return COLI_E_ARG;
    }
    if (T == 0) return COLI_OK;
    if (!x || !topk_ids || !topk_w || !union_ids || !offsets || !slots || !n_union || !y ||
        !workspace)
        return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(union_ids) ||
        !aligned16(offsets) || !aligned16(slots) || !aligned16(n_union) || !aligned16(y) ||
        !aligned16(workspace) || (acc_dump && !aligned16(acc_dump)))
        return COLI_E_ALIGN;
    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, act_mode, L->n_shared);
    if (workspace_bytes < lay.forward_end) return COLI_E_WORKSPACE;
    if (int st = device_check()) return st;
    ForwardIO io{};
    io.x = x; io.T = T; io.ids = topk_ids; io.w = topk_w;
    io.union_ids = union_ids; io.offsets = offsets; io.slots = slots; io.n_union = n_union;
    io.y = y; io.ws = static_cast<uint8_t *>(workspace); io.lay = lay;
    io.acc_dump = acc_dump;
    io.dump = dump_layout(L->H, L->I, L->k, T, L->n_shared);
    const LayerDev d = to_dev(L);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    return status_of(act_mode == COLI_ACT_I8 ? launch_forward_i8(d, io, st, mk)
                                             : launch_forward_f32(d, io, st, mk));
}

int coli_moe_forward(const coli_moe_layer *L, const float *x, int32_t T,
                     const int32_t *topk_ids, const float *topk_w, const int32_t *union_ids,
                     const int32_t *offsets, const int32_t *slots, const int32_t *n_union,
                     int32_t act_mode, float *y, void *workspace, size_t workspace_bytes,
                     int32_t *acc_dump, void *hip_stream)
{
    return forward_impl(L, x, T, topk_ids, topk_w, union_ids, offsets, slots, n_union, act_mode,
                        y, workspace, workspace_bytes, acc_dump, hip_stream, nullptr);
}

int coli_moe_forward_profiled(const coli_moe_layer *L, const float *x, int32_t T,
                              const int32_t *topk_ids, const float *topk_w,
                              const int32_t *union_ids, const int32_t *offsets,
                              const int32_t *slots, const int32_t *n_union, int32_t act_mode,
                              float *y, void *workspace, size_t workspace_bytes,
                              int32_t *acc_dump, void **events, int32_t n_events,
                              void *hip_stream)
{
    if (!events || n_events < 1) return COLI_E_ARG;
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    return forward_impl(L, x, T, topk_ids, topk_w, union_ids, offsets, slots, n_union, act_mode,
                        y, workspace, workspace_bytes, acc_dump, hip_stream, &mk);
}

// Kernels of the self-routing route + forward: router GEMV + the forward's.
static int route_forward_kernels(int32_t act_mode, int32_t T)
{
    return 1 + forward_kernel_count(act_mode, T);
}

// T <= 4 tokens (the int8 family: one), E <= 256: router GEMV, then the
// forward whose gate/up kernel routes the tokens itself (the top-k launch
// is saved).
static bool route_forward_fused(const coli_moe_layer *L, int32_t T, int32_t act_mode)
{
    return T >= 1 && T <= 4 && L->E <= 256 && (act_mode == COLI_ACT_F32 || T == 1);
}

// scratch (the no-allocation entry point): the workspace arguments are
// ignored; after every host check the call takes its scratch from
// scratch() (COLI_E_SCRATCH first if the shape needs more than
// COLI_NOALLOC_SCRATCH_BYTES).
static int route_forward_impl(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                              int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                              int32_t *offsets, int32_t *slots, int32_t *n_union, int32_t act_mode,
                              float *y, void *workspace, size_t workspace_bytes, void *hip_stream,
                              Marks *mk, ScratchFn scratch = nullptr)
{
    if (int st = check_layer(L, true)) return st;
    if (T < 0 || T > COLI_MAX_T) return COLI_E_SHAPE;
    if (act_mode != COLI_ACT_F32 && act_mode != COLI_ACT_I8) return COLI_E_UNSUPPORTED;
    if (!(top_p > 0.0f)) return COLI_E_ARG;  // also rejects NaN
    const bool fused = route_forward_fused(L, T, act_mode);
    if (mk) {
        if (!fused) return COLI_E_UNSUPPORTED;
        if (mk->tl) {  // timeline: the fp32 family's kernels write it
            if (act_mode != COLI_ACT_F32) return COLI_E_UNSUPPORTED;
            if (mk->tl_cap < 1 || ((uintptr_t)mk->tl & 7u)) return COLI_E_ARG;
        } else {
            const int need = 2 * route_forward_kernels(act_mode, T);
            if (!mk->ev || mk->n < need) return COLI_E_ARG;
            for (int i = 0; i < need; ++i)
                if (!mk->ev[i]) return COLI_E_ARG;
        }
    }
    if (!n_union || !union_ids || !offsets) return COLI_E_ARG;
    if (!aligned16(union_ids) || !aligned16(offsets) || !aligned16(n_union)) return COLI_E_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (T == 0) {
        if (int s = device_check()) return s;
        return status_of(launch_union(nullptr, 0, L->k, L->E, union_ids, offsets, slots, n_union, st));
    }
    if (!x || !topk_ids || !topk_w || !slots || !y || (!workspace && !scratch)) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(slots) ||
        !aligned16(y) || (!scratch && !aligned16(workspace)))
        return COLI_E_ALIGN;
    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, act_mode, L->n_shared);
    if (scratch) {
        if (coli_moe_workspace_bytes(L->H, L->I, L->E, L->k, T, act_mode) >
            COLI_NOALLOC_SCRATCH_BYTES)
            return COLI_E_SCRATCH;
    } else if (workspace_bytes < (fused ? lay.fused_end : std::max(lay.route_end, lay.forward_end))) {
        return COLI_E_WORKSPACE;
    }
    if (int s = device_check()) return s;
    if (scratch) {
        if (int s = scratch(&workspace)) return s;
        workspace_bytes = COLI_NOALLOC_SCRATCH_BYTES;
    }
    const LayerDev d = to_dev(L);
    ForwardIO io{};
    io.x = x; io.T = T; io.ids = topk_ids; io.w = topk_w;
    io.union_ids = union_ids; io.offsets = offsets; io.slots = slots; io.n_union = n_union;
    io.y = y; io.ws = static_cast<uint8_t *>(workspace); io.lay = lay;
    if (fused) return status_of(launch_route_forward_small(d, io, act_mode, top_p, st, mk));
    // (the forward buffers alias the route scratch: stream-ordered)
    RouteIO rio{x, T, topk_ids, topk_w, reinterpret_cast<float *>(io.ws + lay.logits), top_p};
    UnionIO un{union_ids, offsets, slots, n_union};
    if (int s = status_of(launch_route(d, rio, st, &un))) return s;
    io.dump = dump_layout(L->H, L->I, L->k, T, L->n_shared);
    return status_of(act_mode == COLI_ACT_I8 ? launch_forward_i8(d, io, st, nullptr)
                                             : launch_forward_f32(d, io, st, nullptr));
}

int coli_moe_route_forward(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                           int32_t *topk_ids, float *topk_w, int32_t *union_ids, int32_t *offsets,
                           int32_t *slots, int32_t *n_union, int32_t act_mode, float *y,
                           void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return route_forward_impl(L, x, T, top_p, topk_ids, topk_w, union_ids, offsets, slots,
                              n_union, act_mode, y, workspace, workspace_bytes, hip_stream,
                              nullptr);
}

}  // extern "C"

int coli::route_forward_scratch(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                                int32_t *topk_ids, float *topk_w, int32_t *union_ids,
                                int32_t *offsets, int32_t *slots, int32_t *n_union,
                                int32_t act_mode, float *y, void *hip_stream, ScratchFn scratch)
{
    return route_forward_impl(L, x, T, top_p, topk_ids, topk_w, union_ids, offsets, slots,
                              n_union, act_mode, y, nullptr, 0, hip_stream, nullptr, scratch);
}

extern "C" {

int coli_moe_route_forward_profiled(const coli_moe_layer *L, const float *x, int32_t T,
                                    float top_p, int32_t *topk_ids, float *topk_w,
                                    int32_t *union_ids, int32_t *offsets, int32_t *slots,
                                    int32_t *n_union, int32_t act_mode, float *y,
                                    void *workspace, size_t workspace_bytes, void **events,
                                    int32_t n_events, void *hip_stream)
{
    if (!events || n_events < 1) return COLI_E_ARG;
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    return route_forward_impl(L, x, T, top_p, topk_ids, topk_w, union_ids, offsets, slots,
                              n_union, act_mode, y, workspace, workspace_bytes, hip_stream, &mk);
}

int coli_moe_route_forward_timeline(const coli_moe_layer *L, const float *x, int32_t T,
                                    float top_p, int32_t *topk_ids, float *topk_w,
                                    int32_t *union_ids, int32_t *offsets, int32_t *slots,
                                    int32_t *n_union, int32_t act_mode, float *y,
                                    void *workspace, size_t workspace_bytes, uint64_t *timeline,
                                    int32_t waves_cap, void *hip_stream)
{
    if (!timeline || waves_cap < 1) return COLI_E_ARG;
    Marks mk;
    mk.tl = timeline;
    mk.tl_cap = waves_cap;
    return route_forward_impl(L, x, T, top_p, topk_ids, topk_w, union_ids, offsets, slots,
                              n_union, act_mode, y, workspace, workspace_bytes, hip_stream, &mk);
}

int coli_moe_route_forward_kernel_count(int32_t act_mode, int32_t T)
{
    if (act_mode != COLI_ACT_F32 && act_mode != COLI_ACT_I8) return 0;
    if (T < 1 || T > 4 || (act_mode == COLI_ACT_I8 && T != 1)) return 0;
    return route_forward_kernels(act_mode, T);
}

const char *coli_moe_route_forward_kernel_name(int32_t act_mode, int32_t T, int32_t i)
{
    if (i < 0 || i >= coli_moe_route_forward_kernel_count(act_mode, T)) return nullptr;
    return i == 0 ? "logits_gemv_kernel" : coli_moe_forward_kernel_name(act_mode, T, i - 1);
}

int coli_moe_forward_kernel_count(int32_t act_mode, int32_t T)
{
    return forward_kernel_count(act_mode, T);
}

const char *coli_moe_forward_kernel_name(int32_t act_mode, int32_t T, int32_t i)
{
    static const char *f32_one[] = {"gateup_t1_kernel", "down_t1c_kernel"};
    static const char *f32_few[] = {"gateup_mt_kernel", "down_mt_kernel", "combine_kernel"};
    static const char *f32[] = {"gateup_f32_kernel", "down_f32_kernel", "combine_kernel"};
    static const char *i8_few[] = {"quant_rows_kernel", "gateup_i8v_kernel", "down_i8v_kernel",
                                   "combine_kernel"};
    static const char *i8[] = {"quant_rows_kernel",           "schedule_kernel",
                               "ggemm_kernel<gateup,full>",   "ggemm_kernel<gateup,partial>",
                               "ggemm_kernel<gateup,small>",  "ggemm_kernel<down,full>",
                               "ggemm_kernel<down,partial>",  "ggemm_kernel<down,small>",
                               "combine_kernel"};
    if (i < 0 || i >= forward_kernel_count(act_mode, T)) return nullptr;
    if (act_mode == COLI_ACT_F32) return T == 1 ? f32_one[i] : T <= 4 ? f32_few[i] : f32[i];
    return T <= kI8StreamTMax ? i8_few[i] : i8[i];
}

int coli_rmsnorm(const float *x, float *xhat, int32_t T, int32_t H, float eps, void *hip_stream)
{
    if (T < 0 || T > COLI_MAX_T || H < 64 || H > COLI_MAX_H || H % 64) return COLI_E_SHAPE;
    if (!(eps >= 0.0f)) return COLI_E_ARG;
    if (T == 0) return COLI_OK;
    if (!x || !xhat) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(xhat)) return COLI_E_ALIGN;
    if (int st = device_check()) return st;
    return status_of(launch_rmsnorm(x, xhat, T, H, eps, static_cast<hipStream_t>(hip_stream)));
}

int coli_add_inplace(float *x, const float *y, int64_t n, void *hip_stream)
{
    if (n < 0) return COLI_E_ARG;
    if (n == 0) return COLI_OK;
    if (!x || !y) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(y)) return COLI_E_ALIGN;
    if (int st = device_check()) return st;
    return status_of(launch_add(x, y, n, static_cast<hipStream_t>(hip_stream)));
}

int coli_add_rmsnorm(float *x, const float *y, float *xhat, int32_t T, int32_t H, float eps,
                     void *hip_stream)
{
    if (T < 0 || T > COLI_MAX_T || H < 64 || H > COLI_MAX_H || H % 64) return COLI_E_SHAPE;
    if (!(eps >= 0.0f)) return COLI_E_ARG;
    if (T == 0) return COLI_OK;
    if (!x || !y || !xhat) return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(y) || !aligned16(xhat)) return COLI_E_ALIGN;
    if (int st = device_check()) return st;
    return status_of(launch_add_rmsnorm(x, y, xhat, T, H, eps, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
