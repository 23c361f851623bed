/*
 * coli_place.h -- expert placement across pinned host memory and device
 * memory, with copy/compute overlap, for the MoE layer of coli_moe.h.
 * Part of libcoli_moe.so.
 *
 * What the pages describe:
 *   [Start]  Colibri getting-started page (cti.vibequant.cc), section
 *            "토큰당 처리 경로 (The Per-Token Path)": after Route and Union,
 *            Place decides where each expert is fetched from (VRAM before
 *            RAM before disk) and changes only speed, never the router's
 *            decisions or the weights' precision; Overlap computes with the
 *            resident experts while an I/O pool brings in the missing ones.
 *   [Hysen]  "colibri: 744B MoEをストレージから推論するCエンジン"
 *            (hysenlabs.com), section "なぜ744Bモデルが25GBのRAMで動くのか":
 *            routed experts are streamed on demand through a per-layer LRU
 *            cache.
 * Here the fast tier is a pool of expert slots in device memory and the slow
 * tier is pinned host memory that holds every expert of the layer; the
 * pages' disk tier, learned pinning and look-ahead prefetch are not part of
 * this library.
 *
 * The placer is host-side state for ONE layer: which expert occupies which
 * device slot, the LRU clock, and (created on first device use) pinned host
 * staging buffers and HIP events.  It owns no device memory: the slot pool,
 * its slot table, the host tier and the device scratch of
 * coli_moe_forward_placed belong to the caller.  Calls on one placer must
 * not overlap (one thread at a time, one compute stream); different placers
 * are independent.  The residency describes the device memory named by the
 * tiers descriptor: a call whose descriptor names other slot memory starts
 * again from empty slots.
 *
 * Residency policy (coli_moe_place_plan), per call with union U:
 *   - the clock advances by one;
 *   - a union expert already in a slot is a hit: it is computed in pass 0
 *     and its slot's last use becomes the current clock;
 *   - the misses, in union order, are split into passes 1, 2, ... of at most
 *     `chunk` experts each; each miss gets a victim slot, chosen as
 *       (a) the lowest-index empty slot, else
 *       (b) among slots no pass of this call reads, the least recently used
 *           (lowest index on ties), else
 *       (c) among slots read by an earlier pass q of this call, the one with
 *           the smallest q (lowest index on ties); its copy then waits until
 *           pass q has finished on the device;
 *     the victim's previous expert is no longer resident.
 * Hits are never evicted by the same call's policy (b); with n_slots >= U
 * rule (c) is never needed.
 */
#ifndef COLI_PLACE_H
#define COLI_PLACE_H

#include <stddef.h>
#include <stdint.h>

#include "coli_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct coli_moe_placer coli_moe_placer;

/* The two tiers of one layer's routed experts (descriptor in host memory).
 * Per-expert layouts are those of coli_moe_layer: w13 [2I][H/2],
 * s13 [2I][H/64], w2 [H][I/2], s2 [H][I/64]. */
typedef struct coli_moe_tiers {
    const uint8_t *host_w13;  /* [E][2I][H/2]  pinned host memory (hipHostMalloc) */
    const uint16_t *host_s13; /* [E][2I][H/64] pinned host memory                 */
    const uint8_t *host_w2;   /* [E][H][I/2]   pinned host memory                 */
    const uint16_t *host_s2;  /* [E][H][I/64]  pinned host memory                 */
    uint8_t *slot_w13;        /* [n_slots][2I][H/2]  device memory                */
    uint16_t *slot_s13;       /* [n_slots][2I][H/64] device memory                */
    uint8_t *slot_w2;         /* [n_slots][H][I/2]   device memory                */
    uint16_t *slot_s2;        /* [n_slots][H][I/64]  device memory                */
    int32_t *slot_table;      /* [E] device memory: the slot of each expert or -1,
                                 written only by the placer (its contents need no
                                 initialisation)                                  */
} coli_moe_tiers;

/* Per-call counts reported by coli_moe_forward_placed. */
typedef struct coli_moe_place_stats {
    int32_t n_union;   /* U of the call                                     */
    int32_t hits;      /* union experts found resident                      */
    int32_t loads;     /* experts copied from host memory (U - hits)        */
    int32_t passes;    /* compute passes (1 + ceil(loads / chunk))          */
} coli_moe_place_stats;

/* Create a placer for a layer of shape (H, I, E, k) with n_slots device
 * slots, calls of at most T_max tokens, and at most `chunk` loaded experts
 * per compute pass (1 <= chunk <= n_slots, 1 <= n_slots <= E).  All slots
 * start empty.  Host memory only (no HIP call): usable without a device.
 * Returns COLI_E_SHAPE / COLI_E_ARG on invalid arguments (*out untouched). */
int coli_moe_placer_create(int32_t H, int32_t I, int32_t E, int32_t k, int32_t n_slots,
                           int32_t T_max, int32_t chunk, coli_moe_placer **out);

/* Release the placer, its events and its pinned staging (NULL is a no-op).
 * The caller must have synchronised the streams of its last call. */
void coli_moe_placer_destroy(coli_moe_placer *P);

/* Forget every residency: all slots empty, the clock restarts. */
int coli_moe_placer_reset(coli_moe_placer *P);

/* Slot holding expert e, or -1 when e is not resident (or out of range). */
int32_t coli_moe_placer_slot_of(const coli_moe_placer *P, int32_t e);

/* The residency policy above as a pure host function, which also commits
 * the new residency to the placer (used by coli_moe_forward_placed; exposed
 * for callers that issue their own copies, and for tests).
 * union_ids [n_union] host memory, ascending distinct ids in [0, E).
 * Outputs (host arrays of n_union entries each):
 *   entry_slot[u]  slot that holds union_ids[u] when its pass runs,
 *   entry_pass[u]  0 for a hit, else the pass that computes it,
 *   load_entry[i]  union position of the i-th copy, in issue order,
 *   load_wait[i]   pass that must finish before copy i starts, or -1,
 *   counts[0..3)   hits, loads, passes.
 * On an invalid union (COLI_E_ARG) the placer is unchanged. */
int coli_moe_place_plan(coli_moe_placer *P, const int32_t *union_ids, int32_t n_union,
                        int32_t *entry_slot, int32_t *entry_pass, int32_t *load_entry,
                        int32_t *load_wait, int32_t *counts);

/* Bytes of device scratch (place_ws) coli_moe_forward_placed needs for
 * calls of at most T tokens (0 if the shape is invalid). */
size_t coli_moe_place_ws_bytes(int32_t E, int32_t k, int32_t T);

/* Place + Overlap + forward for one routed batch ([Start] "토큰당 처리
 * 경로").  Computes exactly what coli_moe_forward computes for the same
 * inputs on a layer whose routed experts are the host tier -- bitwise the
 * same y, since every expert entry runs the same kernels on the same bytes
 * -- while only n_slots experts live in device memory:
 *   1. a kernel splits the union (outputs of coli_moe_union on hip_stream)
 *      against the device slot table: the resident experts form pass 0;
 *      with a shared expert, pass 0 (hits + shared expert) and a combine are
 *      enqueued at once;
 *   2. the host waits until the union has reached it (the one blocking
 *      step; pass 0 keeps the device busy meanwhile) and assigns slots with
 *      coli_moe_place_plan; with no miss the call is complete;
 *   3. otherwise the misses are copied from the host tier into their slots
 *      on copy_stream (4 copies per expert) while pass 0 runs; pass p >= 1
 *      waits for its own copies only, so the copies of later passes overlap
 *      the compute of earlier ones;
 *   4. the combine (topk_w-weighted sum in slot order plus the shared
 *      expert) runs again after the last pass and overwrites y.
 * L supplies H, I, E, k, n_shared and the shared expert (device memory);
 * its w13/s13/w2/s2 are not read and may be NULL; the shape must match the
 * placer's.  T <= T_max.  acc_dump is not available here.  workspace as for
 * coli_moe_forward (coli_moe_workspace_bytes), place_ws of at least
 * coli_moe_place_ws_bytes(E, k, T) bytes, both device memory.  stats may be
 * NULL.  copy_stream may equal hip_stream (no overlap, same results).
 * The host tier must be pinned host memory (pageable memory makes each copy
 * synchronous).  The placer binds to the device current at its first call;
 * a later call on another device is COLI_E_ARG.  On COLI_E_DEVICE the
 * placer forgets all residency (the next call reloads every expert).
 * On COLI_E_ARG after step 1 (inputs that are not a union) y is
 * unspecified and the residency unchanged.
 * Returns when all work is enqueued (after step 2's wait). */
int coli_moe_forward_placed(const coli_moe_layer *L, const coli_moe_tiers *tiers,
                            coli_moe_placer *P, const float *x, int32_t T,
                            const int32_t *topk_ids, const float *topk_w,
                            const int32_t *union_ids, const int32_t *offsets,
                            const int32_t *slots, const int32_t *n_union, int32_t act_mode,
                            float *y, void *workspace, size_t workspace_bytes, void *place_ws,
                            size_t place_ws_bytes, coli_moe_place_stats *stats,
                            void *hip_stream, void *copy_stream);

/* Make the listed experts resident (experts [n] host memory, distinct, in
 * [0, E), n <= n_slots): one call of the residency policy with these
 * experts as the union and all misses in one pass, their copies on
 * copy_stream ordered after the work already on hip_stream, and hip_stream
 * made to wait for the copies.  Nothing is computed.  Used to warm the
 * cache before a run. */
int coli_moe_place_prefetch(coli_moe_placer *P, const coli_moe_tiers *tiers,
                            const int32_t *experts, int32_t n, void *hip_stream,
                            void *copy_stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_PLACE_H */
