/*
 * coli_moe.h -- C ABI of libcoli_moe.so: one Mixture-of-Experts FFN layer
 * with int4 (group size 64) routed experts, on AMD Instinct MI355X (gfx950).
 *
 * The layer follows the per-token path the Colibri pages describe -- route,
 * union, then expert compute -- for experts resident in device memory (the
 * placement of experts from pinned host memory is in coli_place.h, the
 * compressed-KV attention in coli_mla.h):
 *   [Start]  Colibri getting-started page (cti.vibequant.cc), section
 *            "토큰당 처리 경로 (The Per-Token Path)": Route picks the experts,
 *            Union de-duplicates experts shared by tokens of a batch, Place
 *            changes only speed, never router decisions or precision.
 *   [Guide]  "Colibri 完全ガイド — 25GB のメモリで 744B パラメータの大規模モデルを
 *            動かす" (dashen-tech.com): table "コア技術のハイライト" (DeepSeek-V3
 *            sigmoid router with shared experts; int8 and packed-int4 integer
 *            dot kernels) and walk-through "詳細解説" step 3 (single-token
 *            decode in f32, batched prefill on the integer kernel).
 *   [Skill]  "Colibri" (mcpfield.com), section "コアアーキテクチャ" item 1.
 *   [Heart]  "colibri解説｜GLM-5.2（744B MoE）を25GB RAMで動かす純Cランタイムの
 *            実測速度" (ai-heartland.com), section "なぜ25GBで動くのか" (top-8
 *            experts per MoE layer, ~19 MB int4 experts).
 *   [Hysen]  "colibri: 744B MoEをストレージから推論するCエンジン"
 *            (hysenlabs.com), sections "トークンごとの5ステップパス..." and
 *            "エンドツーエンドの測定で地位を獲得する技術" (batched expert union;
 *            the default policy never silently changes precision or router
 *            semantics).
 *
 * Conventions for every entry point
 *  - Memory: every tensor pointer is DEVICE memory owned by the caller; the
 *    library never allocates or frees device memory, keeps no state between
 *    calls (coli_moe_route_forward_noalloc's static scratch array aside) and
 *    never synchronises.  Work is enqueued on `hip_stream` (a
 *    hipStream_t; NULL = the null stream) and buffers must stay valid until
 *    the caller synchronises that stream.  (The int8 grouped GEMM of 5 to
 *    1,024 tokens also runs on two side streams of the library, created once
 *    per device with the default priority; they wait for the caller's
 *    stream and the caller's stream waits for them, so ordering is that of
 *    one stream, under HIP graph capture as well.)  The layer descriptor itself is
 *    host memory and may be reused or freed when the call returns.
 *  - Layouts are row-major.  int4 codes are two's complement in [-8, 7];
 *    byte b of a packed row holds element 2b in its low nibble and element
 *    2b+1 in its high nibble.  Scales are IEEE fp16 bit patterns, one per
 *    row per 64-wide group along the reduction axis.
 *  - Alignment: every tensor pointer must be 16-byte aligned.
 *  - Errors: argument, shape and alignment checks run on the host before any
 *    HIP call and return a nonzero COLI_E_* code (nothing is enqueued then).
 *    A failed launch returns COLI_E_DEVICE.  Faults inside kernels surface
 *    at the caller's next synchronisation.  Non-finite inputs give
 *    unspecified (but memory-safe) results.  No C++ exception crosses the ABI.
 *  - Threading: calls are thread-safe; concurrent calls must use distinct
 *    output and workspace buffers.
 *  - Determinism: for a given input every result is bitwise reproducible
 *    from run to run (no floating-point atomics), and a token's results do
 *    not depend on the other tokens of the batch within one arithmetic
 *    family (act_mode).
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_MOE_ABI_VERSION 1

enum coli_status {
    COLI_OK = 0,
    COLI_E_ARG = 1,         /* NULL pointer or invalid scalar argument        */
    COLI_E_SHAPE = 2,       /* H, I, E, k, T, n_shared outside the limits     */
    COLI_E_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned        */
    COLI_E_WORKSPACE = 4,   /* workspace smaller than coli_moe_workspace_bytes */
    COLI_E_DEVICE = 5,      /* a HIP call or kernel launch failed             */
    COLI_E_UNSUPPORTED = 6, /* current device is not gfx950, or unknown mode  */
    COLI_E_SCRATCH = 7      /* shape needs more scratch than the static array
                               of coli_moe_route_forward_noalloc holds      */
};

/* Arithmetic family of the expert matmuls ([Guide] "詳細解説" step 3; the
 * pages' IDOT switch made an explicit argument, so batching never changes
 * the function silently -- [Hysen] "エンドツーエンドの測定で...").        */
enum coli_act_mode {
    COLI_ACT_F32 = 0, /* fp32 activations x dequantised int4 weights       */
    COLI_ACT_I8 = 1   /* int8 per-token gs64 activations x int4 weights,
                         exact int32 group accumulators, fp32 scaling     */
};

/* Shape limits checked by every entry point. */
#define COLI_MAX_H 8192     /* H % 64 == 0, 64 <= H <= COLI_MAX_H          */
#define COLI_MAX_I 8192     /* I % 64 == 0, 64 <= I <= COLI_MAX_I          */
#define COLI_MAX_E 1024     /* 1 <= E <= COLI_MAX_E                        */
#define COLI_MAX_K 16       /* 1 <= k <= min(E, COLI_MAX_K)                */
#define COLI_MAX_T 65536    /* 0 <= T <= COLI_MAX_T                        */

/* One MoE layer resident in device memory (descriptor in host memory). */
typedef struct coli_moe_layer {
    int32_t H;             /* hidden size                                   */
    int32_t I;             /* expert intermediate size                     */
    int32_t E;             /* routed experts                                */
    int32_t k;             /* experts selected per token                    */
    int32_t n_shared;      /* 0 or 1 shared expert of the same shape        */
    const float *router_w;     /* [E][H] fp32                               */
    const float *router_bias;  /* [E] fp32, used for selection only         */
    const uint8_t *w13;        /* [E][2I][H/2] int4; rows [0,I) gate,
                                  rows [I,2I) up                            */
    const uint16_t *s13;       /* [E][2I][H/64] fp16 scales                 */
    const uint8_t *w2;         /* [E][H][I/2] int4 down projection          */
    const uint16_t *s2;        /* [E][H][I/64] fp16 scales                  */
    const uint8_t *sh_w13;     /* shared expert [2I][H/2]; NULL iff n_shared==0 */
    const uint16_t *sh_s13;    /* [2I][H/64]                                */
    const uint8_t *sh_w2;      /* [H][I/2]                                  */
    const uint16_t *sh_s2;     /* [H][I/64]                                 */
} coli_moe_layer;

/* Bytes of device workspace needed by coli_moe_route, coli_moe_union,
 * coli_moe_forward and coli_moe_route_forward for this shape and arithmetic
 * family (one buffer of this size serves all these calls on one stream; its
 * contents are scratch).
 * Returns 0 for an invalid shape or mode. */
size_t coli_moe_workspace_bytes(int32_t H, int32_t I, int32_t E, int32_t k, int32_t T,
                                int32_t act_mode);

/* Route ([Skill] "コアアーキテクチャ" item 1, [Guide] "コア技術のハイライト":
 * a DeepSeek-V3 style sigmoid router; [Heart] "なぜ25GBで動くのか": top-8).
 * For each token t of x [T][H] fp32:
 *   l[e]  = fp32( sum_h x[t][h] * router_w[e][h] ), accumulated in fp64,
 *   s[e]  = fp32( 1 / (1 + exp(-l[e])) ) evaluated in fp64,
 *   key[e] = s[e] + router_bias[e]  (fp32),
 *   topk_ids[t][0..k) = the k largest keys, largest first, equal keys
 *                       ordered by lower expert index,
 *   topk_w[t][j] = s[topk_ids[t][j]] / sum_j' s[topk_ids[t][j']]  (fp32).
 * topk_ids [T][k] int32, topk_w [T][k] fp32 are written.  T == 0 is a no-op. */
int coli_moe_route(const coli_moe_layer *L, const float *x, int32_t T, int32_t *topk_ids,
                   float *topk_w, void *workspace, size_t workspace_bytes, void *hip_stream);

/* Route with adaptive expert top-p ([Heart] "速度を稼ぐ実用ノブ", knob
 * list: an adaptive expert top-p, `--topp 0.7`, reading 30-40% fewer expert
 * bytes; the pages give no formula, this is the library's reading).  The
 * top-k selection of coli_moe_route, then per token: with the routing
 * weights w[0..k) in selection order,
 *   c_m = w[0] + ... + w[m-1]                 (fp32, in order),
 *   k'  = the least m in [1, k] with c_m >= top_p (k if none),
 *   topk_ids[t][j] = the selection for j < k', -1 for j >= k',
 *   topk_w[t][j]   = s[id_j] / (s[id_0] + ... + s[id_{k'-1}]) for j < k',
 *                    0 for j >= k'.
 * top_p >= 1 gives exactly coli_moe_route; top_p must be > 0 (COLI_E_ARG
 * otherwise).  coli_moe_union and coli_moe_forward skip the slots marked -1,
 * so only the kept experts' weights are read. */
int coli_moe_route_topp(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                        int32_t *topk_ids, float *topk_w, void *workspace,
                        size_t workspace_bytes, void *hip_stream);

/* Union ([Start] "토큰당 처리 경로": batch-union of the experts chosen by
 * several tokens; [Hysen] "エンドツーエンドの測定で...": batched expert union).
 * From topk_ids [T][k] (each row holds distinct ids in [0, E), or -1 for
 * a slot the top-p router dropped):
 *   n_union[0]     = U, the number of distinct experts,
 *   union_ids[u]   = the distinct experts in ascending order (u < U),
 *   offsets[u]     = first position in slots of expert union_ids[u],
 *                    offsets[U] = n_kept, the number of slots with an expert
 *                    (T*k without dropped slots),
 *   slots[p]       = slot index t*k + j, grouped by expert in union order,
 *                    ascending within an expert (p < n_kept).
 * Capacities: union_ids [min(E, T*k)], offsets [min(E, T*k) + 1],
 * slots [T*k].  Entries past U are set to -1 (union_ids) and n_kept
 * (offsets); slots past n_kept are unspecified.  All results stay on the
 * device.  Other out-of-range ids are skipped like -1 (memory-safe). */
int coli_moe_union(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t *union_ids,
                   int32_t *offsets, int32_t *slots, int32_t *n_union, void *hip_stream);

/* Route and union in one call: exactly coli_moe_route_topp(L, x, T, top_p,
 * topk_ids, topk_w, ...) (coli_moe_route when top_p >= 1) followed by
 * coli_moe_union(topk_ids, T, L->k, L->E, union_ids, offsets, slots,
 * n_union) -- the same outputs, bit for bit -- with both steps in one kernel
 * launch for T <= 4 (one workgroup routes the tokens and unions their slots),
 * so a decode or verify step launches one kernel fewer.  Argument checks of
 * both calls; top_p must be > 0.  T == 0 only writes the empty union. */
int coli_moe_route_union(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                         int32_t *topk_ids, float *topk_w, int32_t *union_ids, int32_t *offsets,
                         int32_t *slots, int32_t *n_union, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* Forward: expert compute and combine for the routed batch
 * ([Guide] "詳細解説" step 3; [Start] "토큰당 처리 경로").
 * For every union expert e and each of its slots (t, j), and for the shared
 * expert with every token (weight 1, ungated):
 *   g, u = x[t] . W13_e^T    (gate rows, up rows)
 *   h    = g / (1 + exp(-g)) * u                        (SwiGLU, fp32)
 *   o    = h . W2_e^T
 *   y[t] = sum_j topk_w[t][j] * o_(t,j) + o_shared(t)   (j ascending, slots
 *          with topk_ids -1 skipped)
 * act_mode COLI_ACT_F32: dot products of fp32 x / h with the dequantised
 *   weights (code * scale), fp32 accumulation.
 * act_mode COLI_ACT_I8: x and h quantised per token per 64-group to int8
 *   (scale = amax / 127, q = clamp(rint(v / scale), -127, 127), amax == 0
 *   gives scale 0), exact int32 accumulators per 64-group, output
 *   sum_g acc * act_scale * weight_scale in fp32, the groups added in
 *   ascending order by one fp32 FMA chain per output.  Every batch size runs
 *   this same arithmetic (streaming kernels for T <= 4, the grouped GEMM
 *   above), so a token's y does not depend on its batch.
 * Inputs are the outputs of coli_moe_route and coli_moe_union for the same
 * x and T; y [T][H] fp32 is written.
 * acc_dump (COLI_ACT_I8 only; NULL in production) receives, for every row r
 * in [0, R), R = T*k + n_shared*T (r < T*k: slot r; else shared token
 * r - T*k), in this order:
 *   int32  acc13 [R][2I][H/64]   gate/up group accumulators,
 *   int32  acc2  [R][H][I/64]    down group accumulators,
 *   int8   qh    [R][I]          int8 codes of h (natural element order),
 *   fp32   sh    [R][I/64]       their scales,
 *   int8   qx    [T][H]          int8 codes of x (natural element order),
 *   fp32   sx    [T][H/64]       their scales,
 * each region starting at a 256-byte aligned offset; coli_moe_acc_dump_bytes
 * gives the total size.  Every batch size fills it from the kernels that
 * serve that batch size in production. */
int coli_moe_forward(const coli_moe_layer *L, const float *x, int32_t T,
                     const int32_t *topk_ids, const float *topk_w, const int32_t *union_ids,
                     const int32_t *offsets, const int32_t *slots, const int32_t *n_union,
                     int32_t act_mode, float *y, void *workspace, size_t workspace_bytes,
                     int32_t *acc_dump, void *hip_stream);

/* Profiling variant of coli_moe_forward: the same work, and in addition
 * events[2i] and events[2i + 1] (hipEvent_t values created by the caller,
 * with timing) receive the start and the end of the i-th kernel the call
 * launches, recorded by that kernel's own dispatch (hipExtLaunchKernel), so
 * hipEventElapsedTime(events[2i], events[2i + 1]) is the kernel's duration
 * as a kernel trace reports it.  i < n = coli_moe_forward_kernel_count(
 * act_mode, T); requires n_events >= 2n (else COLI_E_ARG, nothing enqueued).
 * For measurement only; the production path is coli_moe_forward. */
int coli_moe_forward_profiled(const coli_moe_layer *L, const float *x, int32_t T,
                              const int32_t *topk_ids, const float *topk_w,
                              const int32_t *union_ids, const int32_t *offsets,
                              const int32_t *slots, const int32_t *n_union, int32_t act_mode,
                              float *y, void *workspace, size_t workspace_bytes,
                              int32_t *acc_dump, void **events, int32_t n_events,
                              void *hip_stream);

/* One step of the layer: coli_moe_route_union(L, x, T, top_p, topk_ids,
 * topk_w, union_ids, offsets, slots, n_union, ...) followed by
 * coli_moe_forward(L, x, T, topk_ids, topk_w, union_ids, offsets, slots,
 * n_union, act_mode, y, ...) without acc_dump -- the same outputs, bit for
 * bit (topk_ids, topk_w, the union and y).  For T <= 4 tokens with E <= 256
 * (the int8 family: T == 1) the top-k launch is saved: the router GEMV
 * writes the sigmoid scores, and every workgroup of the gate/up kernel
 * selects the top k and forms the union itself before streaming its share
 * of the experts (its workgroup 0 writes them out) -- at T == 1 three
 * launches in the fp32 family (the down kernel also forms y), five in the
 * int8 family.  Otherwise it runs the two calls.
 * Argument checks of both calls (the layer's experts must be present);
 * top_p > 0; workspace_bytes >= coli_moe_workspace_bytes.  T == 0 only
 * writes the empty union. */
int coli_moe_route_forward(const coli_moe_layer *L, const float *x, int32_t T, float top_p,
                           int32_t *topk_ids, float *topk_w, int32_t *union_ids, int32_t *offsets,
                           int32_t *slots, int32_t *n_union, int32_t act_mode, float *y,
                           void *workspace, size_t workspace_bytes, void *hip_stream);

/* coli_moe_route_forward for the self-routing case only (see above; else
 * COLI_E_UNSUPPORTED, nothing enqueued), recording events[2i] /
 * events[2i + 1] at the start / end of its i-th kernel through the kernel's
 * own dispatch (n_events >= 2 * coli_moe_route_forward_kernel_count(
 * act_mode, T), hipEvent_t values created by the caller with timing);
 * coli_moe_route_forward_kernel_name(act_mode, T, i) names kernel i as a
 * profiler trace shows it (template arguments omitted; NULL out of range;
 * count 0 when the case does not route itself).  For measurement only. */
int coli_moe_route_forward_profiled(const coli_moe_layer *L, const float *x, int32_t T,
                                    float top_p, int32_t *topk_ids, float *topk_w,
                                    int32_t *union_ids, int32_t *offsets, int32_t *slots,
                                    int32_t *n_union, int32_t act_mode, float *y,
                                    void *workspace, size_t workspace_bytes, void **events,
                                    int32_t n_events, void *hip_stream);
int coli_moe_route_forward_kernel_count(int32_t act_mode, int32_t T);
const char *coli_moe_route_forward_kernel_name(int32_t act_mode, int32_t T, int32_t i);

/* coli_moe_route_forward for the self-routing fp32 family (T <= 4; else
 * COLI_E_UNSUPPORTED, nothing enqueued), where the waves of its kernels also
 * write a timeline: timeline is device memory of
 * coli_moe_route_forward_kernel_count(act_mode, T) * waves_cap * 8 uint64_t,
 * zeroed by the caller; wave w (its workgroup index times the waves per
 * workgroup plus its wave index, recorded for w < waves_cap) of kernel i
 * writes mark j to timeline[(i * waves_cap + w) * 8 + j]: the chip's
 * 100 MHz real-time counter (s_memrealtime) at the kernel's points j:
 * 0 entry, 7 exit; the self-routing gate/up kernels 1 routing done, 2
 * activations staged, 3 first reduction batch written; the fused down +
 * combine 1 first entry's rows done, 2 / 3 before / after the workgroup
 * barrier.  Marks a kernel does not reach stay 0.  waves_cap >= 1.  The
 * outputs are those of coli_moe_route_forward.  For measurement only. */
int coli_moe_route_forward_timeline(const coli_moe_layer *L, const float *x, int32_t T,
                                    float top_p, int32_t *topk_ids, float *topk_w,
                                    int32_t *union_ids, int32_t *offsets, int32_t *slots,
                                    int32_t *n_union, int32_t act_mode, float *y,
                                    void *workspace, size_t workspace_bytes, uint64_t *timeline,
                                    int32_t waves_cap, void *hip_stream);

/* coli_moe_route_forward for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same call, arguments and outputs (bit for bit) without the
 * workspace: its scratch is one static device array of
 * COLI_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held
 * from the library's load until the process ends.  The caller still owns x,
 * the routing and union outputs and y.  Nothing is allocated or freed: the
 * array's device address is looked up once per device (hipGetSymbolAddress,
 * on the first call with that device current).
 *  - Size limit: a shape whose coli_moe_workspace_bytes(H, I, E, k, T,
 *    act_mode) exceeds COLI_NOALLOC_SCRATCH_BYTES returns COLI_E_SCRATCH
 *    and enqueues nothing.  On the H 6144 / I 2048 / E 256 / top-8 layer
 *    this admits up to 113 tokens in the fp32 family and 135 in the int8
 *    family (decode, verify and small batches).
 *  - Every call on one GPU shares that GPU's array, and nothing in it must
 *    start at zero (its contents are scratch, as in coli_moe_route_forward).
 *    Calls that overlap on one GPU (concurrent streams, or threads without
 *    ordering between their streams) race on the array: the caller orders
 *    them, e.g. on one stream.
 *  - Errors as in coli_moe_route_forward; COLI_E_DEVICE if the symbol lookup
 *    fails. */
#define COLI_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int coli_moe_route_forward_noalloc(const coli_moe_layer *L, const float *x, int32_t T,
                                   float top_p, int32_t *topk_ids, float *topk_w,
                                   int32_t *union_ids, int32_t *offsets, int32_t *slots,
                                   int32_t *n_union, int32_t act_mode, float *y,
                                   void *hip_stream);

/* Number of kernels coli_moe_forward launches for act_mode and a batch of
 * T tokens without acc_dump (0 if the mode is unknown), and the name of the
 * i-th one: the HIP kernel function as it appears in a profiler trace
 * (template arguments omitted).  Both depend on T: T == 1 and 2 <= T <= 4
 * run streaming kernels in the fp32 family (at T == 1 the down projection
 * and the combine share one launch), T <= 4 streaming kernels in the int8
 * family (no tile schedule).  NULL if out of range. */
int coli_moe_forward_kernel_count(int32_t act_mode, int32_t T);
const char *coli_moe_forward_kernel_name(int32_t act_mode, int32_t T, int32_t i);

/* Size in bytes of the acc_dump buffer of coli_moe_forward (0 if invalid). */
size_t coli_moe_acc_dump_bytes(int32_t H, int32_t I, int32_t k, int32_t T, int32_t n_shared);

/* Where a coli_moe_forward call in the int8 family with T > 4 tokens (the
 * grouped GEMM) leaves its intermediate results inside the workspace, for
 * tests and diagnostics; they stay valid until the next call that uses the
 * workspace.  R = T*k + n_shared*T rows.  out[0..2] receive byte offsets:
 *   out[0]  o   fp32 [R][H]     expert outputs, row = slot t*k + j, or
 *                               T*k + t for the shared expert;
 *   out[1]  qh  int8 [R][I]     int8 codes of h, row = union position (the
 *                               slot's index in the union's slot list, or
 *                               T*k + t for the shared expert), inside
 *                               every 8-element block in the element order
 *                               [0,2,4,6,1,3,5,7];
 *   out[2]  sh  fp32 [R][I/64]  the codes' scales, rows as qh.
 * Returns COLI_OK; COLI_E_ARG (out NULL, n_shared not 0 or 1) or
 * COLI_E_SHAPE (dimensions outside the limits, or T <= 4: the streaming
 * kernels keep h in fp32 and quantise it in registers). */
int coli_moe_i8_workspace_offsets(int32_t H, int32_t I, int32_t E, int32_t k, int32_t T,
                                  int32_t n_shared, size_t *out);

/* Human-readable name of a status code (static string). */
const char *coli_moe_strerror(int status);

/* COLI_MOE_ABI_VERSION of the loaded library. */
int coli_moe_abi_version(void);

/* COLI_OK when the current HIP device is a gfx950, else COLI_E_UNSUPPORTED
 * (or COLI_E_DEVICE when no device can be queried). */
int coli_moe_device_check(void);

/* ---- Measurement ---------------------------------------------------------
 * For measurement only (not part of the layer): reads bytes (a multiple of
 * 1024, at most 1 GiB) of device memory at buf with the load pattern of the
 * streaming expert kernels -- 16-byte buffer loads per lane, 1 KB per wave
 * instruction, 8 loads in flight per wave -- on n_groups workgroups of 4
 * waves (1..65536), and writes one XOR checksum per workgroup to
 * out[n_groups] (uint32).  Timing it gives the practical HBM read rate the
 * streaming kernels' GB/s are compared against. */
int coli_stream_read(const void *buf, size_t bytes, uint32_t *out, int32_t n_groups,
                     void *hip_stream);

/* For measurement only: whether one SIMD issues int8 MFMAs and fp32 vector
 * FMAs in parallel (it sets the int8 GEMM's ceiling, whose epilogue is
 * vector work).  n_groups workgroups of 8 waves (two per SIMD; 1..65536)
 * run 2048 iterations of: mode 0, 4 independent v_mfma_i32_16x16x64_i8 per
 * wave; mode 1, 16 independent fp32 FMAs per wave; mode 2, waves 0-3 the
 * MFMAs of mode 0 and waves 4-7 the FMAs of mode 1; mode 3, every wave both,
 * interleaved; mode 4, the FMAs of mode 1 in waves 0-3 only (one wave per
 * SIMD); mode 5, 16 independent fp32 FMAs per wave whose three sources are
 * distinct VGPRs (the VOP3 form).  ticks[n_groups] (uint64) receives each workgroup's duration
 * in wall-clock (100 MHz) ticks; sink (one int32) is written only to keep
 * the work.  COLI_E_ARG for a bad mode, count or pointer, COLI_E_ALIGN for a
 * misaligned one. */
int coli_issue_probe(int32_t mode, int32_t n_groups, uint64_t *ticks, int32_t *sink,
                     void *hip_stream);

/* ---- Glue for stacking layers (outside the MoE layer itself) ------------
 * The pages do not describe the blocks around the MoE layer.  To run a
 * stack of synthetic layers without overflow, a unit-gain RMS pre-norm and
 * a residual add are provided (the reading of a GLM-style pre-norm block). */

/* xhat[t][h] = x[t][h] / sqrt(mean_h(x[t][h]^2) + eps), fp32, [T][H]. */
int coli_rmsnorm(const float *x, float *xhat, int32_t T, int32_t H, float eps,
                 void *hip_stream);

/* x[i] += y[i] for i < n (fp32). */
int coli_add_inplace(float *x, const float *y, int64_t n, void *hip_stream);

/* Both of the above in one pass, as they meet between stacked layers:
 * x[t][h] += y[t][h], then xhat = rmsnorm(x) of the updated x; x and xhat
 * are bitwise those of coli_add_inplace(x, y, T*H) followed by
 * coli_rmsnorm(x, xhat, T, H, eps).  x, y, xhat [T][H] fp32, distinct
 * buffers; same limits and errors as coli_rmsnorm. */
int coli_add_rmsnorm(float *x, const float *y, float *xhat, int32_t T, int32_t H, float eps,
                     void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_MOE_H */
