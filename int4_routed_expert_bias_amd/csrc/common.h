// common.h -- internal helpers of libcoli_moe.so (device utilities, the
// workspace layout and the launcher interface between the host entry points
// and the kernel translation units).  Written for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/coli_moe.h"

namespace coli {

constexpr int kWave = 64;
#define COLI_MAX_K_DEV 16    // must equal COLI_MAX_K of the public header
#define COLI_MAX_E_DEV 1024  // must equal COLI_MAX_E of the public header
#define COLI_MAX_H_DEV 8192  // must equal COLI_MAX_H of the public header

// ---------------------------------------------------------------------------
// device helpers

// IEEE binary16 bit pattern -> fp32 (exact; one v_cvt_f32_f16).
__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float wave_sum(float v)
{
    // fixed butterfly over lane bits 5..0: same tree for every value
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Position of element kk (within a row) in the permuted int8 activation
// layout used by the integer kernels: inside every 8-element block the
// order is [0,2,4,6,1,3,5,7], matching how a packed int4 dword splits into
// its even-element and odd-element bytes.
__device__ __forceinline__ int perm8_pos(int kk)
{
    int b = kk & 7;
    return (kk & ~7) | ((b & 1) << 2) | (b >> 1);
}

// The int8 family's fp32 epilogue forms each group term as acc * s from the
// exact int32 group accumulator acc and the activation scale s rounded to 22
// significant bits (to nearest, ties up; a relative change of at most
// 2^-23): epi_act_scale(s).  Then kEpiM * s' is exact in fp32 (kEpiM = 3 *
// 2^22), so the grouped GEMM forms the term as one FMA on the accumulator
// offset by kEpiM inside the matrix core (as fp32, kEpiM + acc is exact for
// |acc| < 2^22): fma(kEpiM + acc, s', -kEpiM * s') = round(acc * s'), bit
// for bit float(acc) * s', which the streaming kernels compute.
constexpr float kEpiM = 12582912.0f;         // 3 * 2^22 = 1.5 * 2^23
constexpr int32_t kEpiMBits = 0x4B400000;    // its bit pattern (unit 1 in the last place)
__device__ __forceinline__ float epi_act_scale(float s)
{
    return __uint_as_float((__float_as_uint(s) + 2u) & ~3u);
}

// ---------------------------------------------------------------------------
// workspace layout (offsets in bytes, each region 256-byte aligned)

struct Workspace {
    size_t logits;   // route: [T][E] f32 sigmoid scores, or [S][T][E] f64 logit partials
    size_t route_end;
    // forward, shared by both families
    size_t o;        // [R][H] f32 expert outputs per slot / shared row
    // fp32 family
    size_t h;        // [R][I] f32 SwiGLU outputs
    // int8 family
    size_t qx, sx;   // [T][H] i8 (permuted), [T][H/64] f32
    size_t qh, sh;   // [R][I] i8 (permuted), [R][I/64] f32
    size_t tiles;    // [max_tiles] int2 (entry, first row) + [2] list sizes
    size_t forward_end;
    // route + forward in one call (one token): the scores stay readable
    // while gate/up writes h, so they sit past the forward buffers
    size_t scores;   // [E] f32
    size_t fused_end;
    size_t total;
    int64_t R;       // rows: T*k + n_shared*T
    int64_t cap;     // min(E, T*k)
    int64_t max_tiles;
};

constexpr int kTileM = 128;  // token rows per integer-GEMM tile
// Batches up to this size run the streaming kernels of the integer family
// (and, for T >= 2, of the fp32 family).
constexpr int kI8StreamTMax = 4;

// Router: batches of up to kGemvTMax tokens stream Wr once (GEMV, fp32
// logits); larger batches run an fp64 MFMA GEMM split over K whose fp64
// partial sums [S][T][E] are added in split order by the top-k kernel.
constexpr int kGemvTMax = 8;
constexpr int kLogitTile = 64;  // tokens x experts per GEMM workgroup

// K-splits of the router GEMM for T tokens: S splits of bps 16-wide
// k-blocks each (S == 0: GEMV path).  A function of the shape only (never of
// the device), so that the workspace size and the launch agree: about 512
// workgroups, at least four k-blocks per split, at most 64 MiB of partials
// unless S == 1, and every split non-empty ((S-1)*bps < H/16 <= S*bps).
struct RouteSplit {
    int S, bps;
};

inline RouteSplit route_split(int64_t T, int64_t H, int64_t E)
{
    if (T <= kGemvTMax) return {0, 0};
    const int64_t tiles = ((T + kLogitTile - 1) / kLogitTile) * ((E + kLogitTile - 1) / kLogitTile);
    const int64_t nb = H / 16;
    int64_t s = (512 + tiles - 1) / tiles;
    if (s > nb / 4) s = nb / 4;
    const int64_t cap = (int64_t(64) << 20) / (T * E * 8);
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    const int64_t bps = (nb + s - 1) / s;
    return {(int)((nb + bps - 1) / bps), (int)bps};
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline Workspace workspace_layout(int64_t H, int64_t I, int64_t E, int64_t k, int64_t T,
                                  int act_mode, int64_t n_shared)
{
    Workspace w{};
    w.R = T * k + n_shared * T;
    w.cap = (T * k < E) ? T * k : E;
    w.max_tiles = (T * k + kTileM - 1) / kTileM + w.cap + n_shared * ((T + kTileM - 1) / kTileM);
    size_t p = 0;
    const int S = route_split(T, H, E).S;
    w.logits = p; p = align256(p + (S == 0 ? (size_t)T * E * 4 : (size_t)S * T * E * 8));
    w.route_end = p;
    p = 0;  // forward buffers alias the route scratch (stream-ordered)
    w.o = p; p = align256(p + (size_t)w.R * H * 4);
    if (act_mode == 0) {
        w.h = p; p = align256(p + (size_t)w.R * I * 4);
    } else {
        w.qx = p; p = align256(p + (size_t)T * H);
        w.sx = p; p = align256(p + (size_t)T * (H / 64) * 4);
        w.qh = p; p = align256(p + (size_t)w.R * I);
        w.sh = p; p = align256(p + (size_t)w.R * (I / 64) * 4);
        w.tiles = p; p = align256(p + (size_t)(w.max_tiles + 2) * 8);
        if (T <= kI8StreamTMax) {  // the small-batch kernels pass h in fp32
            w.h = p; p = align256(p + (size_t)w.R * I * 4);
        }
    }
    w.forward_end = p;
    w.scores = p; p = align256(p + (size_t)(T <= 4 ? T : 1) * E * 4);
    w.fused_end = p;
    w.total = w.route_end > w.fused_end ? w.route_end : w.fused_end;
    if (w.total == 0) w.total = 256;
    return w;
}

// acc_dump regions (see coli_moe.h)
struct DumpLayout {
    size_t acc13, acc2, qh, sh, qx, sx, total;
};

inline DumpLayout dump_layout(int64_t H, int64_t I, int64_t k, int64_t T, int64_t n_shared)
{
    DumpLayout d{};
    int64_t R = T * k + n_shared * T;
    size_t p = 0;
    d.acc13 = p; p = align256(p + (size_t)R * 2 * I * (H / 64) * 4);
    d.acc2 = p;  p = align256(p + (size_t)R * H * (I / 64) * 4);
    d.qh = p;    p = align256(p + (size_t)R * I);
    d.sh = p;    p = align256(p + (size_t)R * (I / 64) * 4);
    d.qx = p;    p = align256(p + (size_t)T * H);
    d.sx = p;    p = align256(p + (size_t)T * (H / 64) * 4);
    d.total = p;
    return d;
}

// ---------------------------------------------------------------------------
// launcher interface (each returns hipError_t of the launch)

// Optional profiling marks: caller-created events, two per kernel of a call
// (ev[2i], ev[2i + 1]), set to the start and the end of kernel i by its own
// dispatch (hipExtLaunchKernel), i.e. the durations a kernel trace reports.
// Optional timeline (coli_moe_route_forward_timeline): per kernel of the
// call, 8 real-time-counter marks per wave (see tl_mark).
struct Marks {
    void **ev = nullptr;
    int n = 0;  // events available
    int i = 0;  // kernels launched so far
    uint64_t *tl = nullptr;
    int tl_cap = 0;  // waves recorded per kernel
    // timeline records of the kernel launched next (null: none)
    uint64_t *tl_next() const { return tl ? tl + (size_t)i * tl_cap * 8 : nullptr; }
    bool next(hipEvent_t &start, hipEvent_t &end)
    {
        const int j = 2 * i++;
        if (!ev || j + 1 >= n) return false;
        start = static_cast<hipEvent_t>(ev[j]);
        end = static_cast<hipEvent_t>(ev[j + 1]);
        return true;
    }
};

// Every kernel of a forward call is launched through this: a plain launch,
// or with marks one whose dispatch records the kernel's start and end.
template <typename F, typename... Args>
inline void launch(Marks *mk, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                   Args... args)
{
    hipEvent_t a, b;
    if (mk && mk->next(a, b)) hipExtLaunchKernelGGL(kernel, grid, block, lds, st, a, b, 0, args...);
    else hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

struct LayerDev {
    int32_t H, I, E, k, n_shared;
    const float *router_w, *router_bias;
    const uint8_t *w13; const uint16_t *s13;
    const uint8_t *w2; const uint16_t *s2;
    const uint8_t *sh_w13; const uint16_t *sh_s13;
    const uint8_t *sh_w2; const uint16_t *sh_s2;
};

struct RouteIO {
    const float *x; int32_t T;
    int32_t *ids; float *w;
    float *logits;  // workspace
    float top_p;    // >= 1: plain top-k
};

// Compute units of the current device (cached per device on first use).
int device_cu_count();

// Union outputs for launch_route (NULL: route only).
struct UnionIO {
    int32_t *union_ids, *offsets, *slots, *n_union;
};

// Route; with un, also the batch-union of the routed slots (in the top-k
// launch itself for T <= 4, else by launch_union after it).
hipError_t launch_route(const LayerDev &L, const RouteIO &io, hipStream_t st,
                        const UnionIO *un = nullptr);

// Sigmoid scores of T <= 8 tokens (the router GEMV alone) into scores [T][E].
hipError_t launch_scores(const LayerDev &L, const float *x, int32_t T, float *scores,
                         hipStream_t st, Marks *mk = nullptr);

hipError_t launch_union(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *union_ids,
                        int32_t *offsets, int32_t *slots, int32_t *n_union, hipStream_t st);

// A batch of at most 4 tokens that routes itself inside its gate/up kernel
// (see launch_route_forward_small): the tokens' sigmoid scores and the
// selection outputs the gate/up kernel's workgroup 0 writes.
struct RouteSelf {
    const float *scores, *bias;  // [T][E] sigmoid scores, [E] selection bias
    int T, E, k, cap;
    float top_p;
    int32_t *ids;                // [T][k]
    float *w;                    // [T][k]
    int32_t *union_ids, *offsets, *slots, *n_union;
};

struct ForwardIO {
    const float *x; int32_t T;
    const int32_t *ids; const float *w;
    const int32_t *union_ids, *offsets, *slots, *n_union;
    float *y;
    uint8_t *ws; Workspace lay;
    int32_t *acc_dump; DumpLayout dump;
    // false: the expert outputs stay in the workspace (o) and y is not
    // written; the placed forward combines once after its last pass
    bool combine = true;
    // set: one token whose gate/up kernel selects and unions it (the union
    // lists above are then written by that kernel)
    const RouteSelf *route = nullptr;
};

// Kernels one forward call launches (without acc_dump): fp32 family gate/up,
// down, combine; integer family quant, [schedule,] gate/up, down, combine
// (batches of at most kI8StreamTMax tokens stream without a tile schedule;
// larger ones run each grouped GEMM as two launches, full then partial
// tiles).
inline int forward_kernel_count(int act_mode, int T)
{
    if (act_mode == 0) return T == 1 ? 2 : 3;  // T == 1: down and combine in one launch
    if (act_mode == 1) return T <= kI8StreamTMax ? 4 : 9;
    return 0;
}

hipError_t launch_forward_f32(const LayerDev &L, const ForwardIO &io, hipStream_t st, Marks *mk);
// Route and forward of T <= 4 tokens (E <= 256; the int8 family T == 1):
// router GEMV (scores into io.ws + io.lay.scores), then the family's forward
// whose gate/up kernel selects and unions the tokens itself (writing io.ids
// / io.w / the union).
hipError_t launch_route_forward_small(const LayerDev &L, const ForwardIO &io, int act_mode,
                                      float top_p, hipStream_t st, Marks *mk);
hipError_t launch_forward_i8(const LayerDev &L, const ForwardIO &io, hipStream_t st, Marks *mk);
hipError_t launch_forward_i8_small(const LayerDev &L, const ForwardIO &io, const int8_t *qx,
                                   const float *sx, float *h, float *o, hipStream_t st, Marks *mk);
// The one-call layer step of coli_moe_route_forward with its scratch from
// scratch() instead of a caller workspace (coli_moe_route_forward_noalloc):
// scratch() runs after every host check and returns a COLI_* status and
// the device address of COLI_NOALLOC_SCRATCH_BYTES of scratch.
typedef int (*ScratchFn)(void **ws);
int route_forward_scratch(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                          int32_t *topk_ids, float *topk_w, int32_t *union_ids, int32_t *offsets,
                          int32_t *slots, int32_t *n_union, int32_t act_mode, float *y,
                          void *hip_stream, ScratchFn scratch);
// Side streams of one device for launches of a call that may run
// concurrently with the caller's stream (created once per device with the
// default priority, non-blocking, kept until the process ends).  Between
// side_fork and side_join the enqueueing thread holds the device's lock, so
// concurrent calls on one device cannot interleave their fork and join
// events.  side_fork makes side streams 0..n-1 wait for everything enqueued
// on st so far and returns them (null: none available -- the caller then
// enqueues on st); side_join makes st wait for everything enqueued on them
// since, and releases the lock.
struct SideSet {
    hipStream_t s[2];
    hipEvent_t fork, join[2];
};
SideSet *side_fork(hipStream_t st, int n);
hipError_t side_join(SideSet *ss, hipStream_t st, int n);
hipError_t launch_combine(const float *o, const int32_t *ids, const float *w, int32_t T, int32_t k,
                          int32_t H, int32_t n_shared, float *y, hipStream_t st,
                          Marks *mk = nullptr);
hipError_t launch_rmsnorm(const float *x, float *xhat, int32_t T, int32_t H, float eps,
                          hipStream_t st);
hipError_t launch_add(float *x, const float *y, int64_t n, hipStream_t st);
hipError_t launch_add_rmsnorm(float *x, const float *y, float *xhat, int32_t T, int32_t H,
                              float eps, hipStream_t st);

}  // namespace coli
