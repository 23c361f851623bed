// place.hip -- expert placement over pinned host memory and a pool of
// device slots, with copy/compute overlap (C ABI in include/coli_place.h).
//
// Colibri getting-started page, section "토큰당 처리 경로 (The Per-Token
// Path)": Place picks where an expert is read from and changes only speed;
// Overlap computes with resident experts while missing ones are brought in.
// hysenlabs.com "colibri: 744B MoE...", section "なぜ744Bモデルが25GBの
// RAMで動くのか": a per-layer LRU cache in front of the slow tier.
//
// One call of coli_moe_forward_placed (with a shared expert):
//   compute stream: split the union against the device slot table (hits ->
//                   pass 0's sub-union, everything packed for the host),
//                   copy the packed union to pinned host memory, pass 0
//                   (hits + shared expert), combine
//   host:           waits for the packed union only (pass 0 keeps the device
//                   busy meanwhile), plans slots (LRU); if nothing is missing
//                   the call is complete
//   otherwise       uploads the sub-unions of passes 1.. and the new slot
//                   table; copy stream: [wait done[q]] H2D copies of pass
//                   p's experts, ready[p]; compute stream: [wait ready[p]]
//                   pass p ..., combine again (the first one saw only pass 0)
// Every pass runs the unchanged forward kernels on a sub-union whose entries
// name device slots instead of experts, and without the combine; the expert
// outputs land in the workspace by slot index, so the combine after the last
// pass sees exactly what one resident forward would have produced.
// Without a shared expert pass 0 may be empty, so the host plans first and
// launches pass 0 only if it has hits.
#include "../../include/coli_place.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "common.h"

using namespace coli;

struct coli_moe_placer {
    int32_t H, I, E, k, n_slots, T_max, chunk, cap_max;
    int64_t tick = 0;
    std::vector<int32_t> slot_of;    // [E] slot of expert, -1 if absent
    std::vector<int32_t> expert_in;  // [n_slots] expert in slot, -1 if empty
    std::vector<int64_t> last_use;   // [n_slots] clock of the last call that used it
    std::vector<int32_t> slot_pass;  // [n_slots] reader pass in the current call, -1 none
    // plan results of the current call (forward_placed)
    std::vector<int32_t> entry_slot, entry_pass, load_entry, load_wait;
    // the device memory the residency describes; a different one on a later
    // call means the slots hold nothing known
    const void *bound[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    bool table_dirty = true;  // the device slot table must be rewritten before use
    // device-side resources, created on first device use
    int device = -1;
    int32_t *stage_in = nullptr;   // pinned host: the packed union
    int32_t *stage_out = nullptr;  // pinned host: the sub-unions of passes 1..
    int32_t *stage_tab = nullptr;  // pinned host: the slot table
    size_t stage_in_ints = 0, stage_out_ints = 0;
    std::vector<hipEvent_t> ready, done;  // per pass
    // packed: the packed union reached the host; tab / sub: the last upload
    // from stage_tab / stage_out finished; order: prefetch ordering
    hipEvent_t packed = nullptr, tab = nullptr, sub = nullptr, order[2] = {nullptr, nullptr};
};

namespace {

inline size_t pad4(size_t n) { return (n + 3) & ~size_t(3); }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int32_t cap_of(int32_t E, int32_t k, int32_t T)
{
    const int64_t tk = (int64_t)T * k;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(E, tk));
}

// int32 regions of place_ws (each a multiple of 4 ints):
//   packed union for the host: n_union, n_hits, union_ids[cap], offsets[cap+1], slots[T*k]
size_t packed_ints(int32_t cap, int64_t tk) { return pad4(3 + 2 * (size_t)cap + (size_t)tk); }
//   pass 0 (built on the device): n (4), entries pad4(cap), offsets pad4(cap+1), slots pad4(T*k)
size_t sub0_ints(int32_t cap, int64_t tk)
{
    return 4 + pad4(cap) + pad4((size_t)cap + 1) + pad4(std::max<int64_t>(tk, 1));
}
//   passes 1.. (built on the host): per pass n (4) + entries pad4(n) +
//   offsets pad4(n + 1) + slots pad4(max(S, 1)) <= 2n + S + 15; at most cap
//   passes with sum n <= cap and sum S <= T*k
size_t subunion_ints(int32_t cap, int64_t tk) { return 17 * (size_t)cap + (size_t)tk + 16; }

// ---- residency policy -------------------------------------------------------

// Victim slot for a miss computed in pass p; *wait = pass to wait for or -1.
int32_t pick_victim(const coli_moe_placer &P, int32_t p, int32_t *wait)
{
    for (int32_t s = 0; s < P.n_slots; ++s)  // (a) an empty slot
        if (P.expert_in[s] < 0) {
            *wait = -1;
            return s;
        }
    int32_t best = -1;  // (b) least recently used, not read in this call
    for (int32_t s = 0; s < P.n_slots; ++s)
        if (P.slot_pass[s] < 0 && (best < 0 || P.last_use[s] < P.last_use[best])) best = s;
    if (best >= 0) {
        *wait = -1;
        return best;
    }
    for (int32_t s = 0; s < P.n_slots; ++s)  // (c) read by the earliest earlier pass
        if (P.slot_pass[s] >= 0 && P.slot_pass[s] < p &&
            (best < 0 || P.slot_pass[s] < P.slot_pass[best]))
            best = s;
    *wait = best >= 0 ? P.slot_pass[best] : -1;
    return best;
}

int plan_impl(coli_moe_placer &P, const int32_t *uid, int32_t U, int32_t chunk,
              int32_t *entry_slot, int32_t *entry_pass, int32_t *load_entry, int32_t *load_wait,
              int32_t *counts)
{
    if (U < 0 || U > P.E) return COLI_E_ARG;
    for (int32_t u = 0; u < U; ++u)
        if (uid[u] < 0 || uid[u] >= P.E || (u > 0 && uid[u] <= uid[u - 1])) return COLI_E_ARG;
    ++P.tick;
    std::fill(P.slot_pass.begin(), P.slot_pass.end(), -1);
    std::vector<char> miss(U);
    int32_t hits = 0;
    for (int32_t u = 0; u < U; ++u) {
        const int32_t s = P.slot_of[uid[u]];
        miss[u] = s < 0;
        if (s >= 0) {
            entry_slot[u] = s;
            entry_pass[u] = 0;
            P.last_use[s] = P.tick;
            P.slot_pass[s] = 0;
            ++hits;
        }
    }
    int32_t nl = 0;
    for (int32_t u = 0; u < U; ++u) {
        if (!miss[u]) continue;
        const int32_t p = 1 + nl / chunk;
        int32_t wait = -1;
        const int32_t s = pick_victim(P, p, &wait);
        // unreachable while chunk <= n_slots: at most chunk - 1 slots are
        // read by pass p itself when its next victim is chosen
        if (s < 0) return COLI_E_ARG;
        if (P.expert_in[s] >= 0) P.slot_of[P.expert_in[s]] = -1;
        P.expert_in[s] = uid[u];
        P.slot_of[uid[u]] = s;
        P.last_use[s] = P.tick;
        P.slot_pass[s] = p;
        entry_slot[u] = s;
        entry_pass[u] = p;
        load_entry[nl] = u;
        load_wait[nl] = wait;
        ++nl;
    }
    counts[0] = hits;
    counts[1] = nl;
    counts[2] = 1 + (nl + chunk - 1) / chunk;
    return COLI_OK;
}

void forget(coli_moe_placer &P)
{
    std::fill(P.slot_of.begin(), P.slot_of.end(), -1);
    std::fill(P.expert_in.begin(), P.expert_in.end(), -1);
    std::fill(P.last_use.begin(), P.last_use.end(), 0);
    std::fill(P.slot_pass.begin(), P.slot_pass.end(), -1);
    P.tick = 0;
    P.table_dirty = true;
}

// ---- device side ------------------------------------------------------------

// Splits the union against the slot table: the resident experts become pass
// 0's sub-union (device slots instead of experts, offsets and slot lists
// compacted, union order kept), and the whole union is packed for one copy
// to the host.  One workgroup of 1024 threads (U <= cap <= 1024).
// Memory-safe for any contents of the inputs (indices are clamped), exact
// for the outputs of coli_moe_union.
__global__ __launch_bounds__(1024) void place_split_kernel(
    const int32_t *__restrict__ n_union, const int32_t *__restrict__ union_ids,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ table, int E, int cap, int tk, int32_t *__restrict__ packed,
    int32_t *__restrict__ sub0)
{
    __shared__ int32_t s_off[COLI_MAX_E_DEV + 1];
    __shared__ int32_t s_pos[COLI_MAX_E_DEV];  // pass-0 entry of a hit, -1 for a miss
    __shared__ int32_t s_row[COLI_MAX_E_DEV];  // its first pass-0 row
    __shared__ int32_t s_wsum[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int U_raw = n_union[0];
    const int U = min(max(U_raw, 0), cap);
    int32_t *ent0 = sub0 + 4;
    int32_t *off0 = ent0 + ((cap + 3) & ~3);
    int32_t *sl0 = off0 + ((cap + 4) & ~3);
    int hit = 0, cnt = 0, slot = -1;
    if (tid < U) {
        const int e = union_ids[tid];
        slot = (e >= 0 && e < E) ? table[e] : -1;
        hit = slot >= 0;
        const int a = offsets[tid], b = offsets[tid + 1];
        cnt = max(b - a, 0);
        s_off[tid] = a;
        if (tid == U - 1) s_off[U] = b;
    }
    // block-wide exclusive scans of hit and hit * cnt
    const int hc = hit ? cnt : 0;
    int ih = hit, ir = hc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int a = __shfl_up(ih, d, 64), b = __shfl_up(ir, d, 64);
        if (lane >= d) {
            ih += a;
            ir += b;
        }
    }
    if (lane == 63) {
        s_wsum[0][wv] = ih;
        s_wsum[1][wv] = ir;
    }
    __syncthreads();
    int n0 = 0, before_h = 0, before_r = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wv) {
            before_h += s_wsum[0][w];
            before_r += s_wsum[1][w];
        }
        n0 += s_wsum[0][w];
    }
    const int pos = before_h + ih - hit, row = before_r + ir - hc;
    if (tid < U) {
        s_pos[tid] = hit ? pos : -1;
        s_row[tid] = row;
        if (hit) {
            ent0[pos] = slot;
            off0[pos + 1] = row + cnt;
        }
    }
    if (tid == 0) {
        sub0[0] = n0;
        sub0[1] = sub0[2] = sub0[3] = 0;
        off0[0] = 0;
    }
    __syncthreads();
    // the hits' slot lists, compacted
    const int total = U > 0 ? min(max(s_off[U], 0), tk) : 0;
    for (int r = tid; r < total; r += blockDim.x) {
        int lo = 0, hi = U - 1;  // the entry u with s_off[u] <= r < s_off[u + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        if (s_pos[lo] >= 0) {
            const int dst = s_row[lo] + (r - s_off[lo]);
            if (dst >= 0 && dst < tk) sl0[dst] = slots[r];
        }
    }
    // the union for the host: n_union, n_hits, union_ids, offsets, slots
    const int npk = 3 + 2 * cap + tk;
    for (int i = tid; i < npk; i += blockDim.x) {
        int32_t v;
        if (i == 0) v = U_raw;
        else if (i == 1) v = n0;
        else if (i < 2 + cap) v = union_ids[i - 2];
        else if (i < 3 + 2 * cap) v = offsets[i - 2 - cap];
        else v = slots[i - 3 - 2 * cap];
        packed[i] = v;
    }
}

bool make_event(hipEvent_t &e)
{
    if (e) return true;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess) return true;
    e = nullptr;
    return false;
}

bool host_alloc(int32_t *&p, size_t ints)
{
    if (p) return true;
    if (hipHostMalloc(reinterpret_cast<void **>(&p), ints * 4, hipHostMallocDefault) == hipSuccess)
        return true;
    p = nullptr;
    return false;
}

int ensure_device(coli_moe_placer &P)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return COLI_E_DEVICE;
    if (P.device >= 0) return dev == P.device ? COLI_OK : COLI_E_ARG;
    // allocate what an earlier failed attempt left missing
    const int64_t tk = (int64_t)P.T_max * P.k;
    P.stage_in_ints = packed_ints(P.cap_max, tk);
    P.stage_out_ints = subunion_ints(P.cap_max, tk);
    if (!host_alloc(P.stage_in, P.stage_in_ints) || !host_alloc(P.stage_out, P.stage_out_ints) ||
        !host_alloc(P.stage_tab, pad4(P.E)))
        return COLI_E_DEVICE;
    const size_t n_ev = (size_t)P.cap_max + 1;  // passes <= 1 + misses <= 1 + cap
    P.ready.resize(n_ev, nullptr);
    P.done.resize(n_ev, nullptr);
    for (size_t i = 0; i < n_ev; ++i)
        if (!make_event(P.ready[i]) || !make_event(P.done[i])) return COLI_E_DEVICE;
    if (!make_event(P.packed) || !make_event(P.tab) || !make_event(P.sub) ||
        !make_event(P.order[0]) || !make_event(P.order[1]))
        return COLI_E_DEVICE;
    P.device = dev;
    return COLI_OK;
}

// The residency describes the memory of `t`: a call with other memory
// starts from empty slots.
void bind(coli_moe_placer &P, const coli_moe_tiers &t)
{
    const void *now[5] = {t.slot_table, t.slot_w13, t.slot_s13, t.slot_w2, t.slot_s2};
    if (!std::equal(now, now + 5, P.bound)) {
        forget(P);
        std::copy(now, now + 5, P.bound);
    }
}

// Uploads the host slot table to the device (stream-ordered on st).
hipError_t upload_table(coli_moe_placer &P, const coli_moe_tiers &t, hipStream_t st)
{
    hipError_t err;
    if ((err = hipEventSynchronize(P.tab)) != hipSuccess) return err;  // stage_tab is free
    std::copy(P.slot_of.begin(), P.slot_of.end(), P.stage_tab);
    if ((err = hipMemcpyAsync(t.slot_table, P.stage_tab, (size_t)P.E * 4, hipMemcpyHostToDevice,
                              st)) != hipSuccess)
        return err;
    if ((err = hipEventRecord(P.tab, st)) != hipSuccess) return err;
    P.table_dirty = false;
    return hipSuccess;
}

// Bytes of one expert in each of the four arrays.
struct ExpertBytes {
    size_t w13, s13, w2, s2;
};

ExpertBytes expert_bytes(const coli_moe_placer &P)
{
    const size_t H = P.H, I = P.I;
    return {2 * I * (H / 2), 2 * I * (H / 64) * 2, H * (I / 2), H * (I / 64) * 2};
}

hipError_t copy_expert(const coli_moe_placer &P, const coli_moe_tiers &t, int32_t e, int32_t s,
                       hipStream_t cs)
{
    const ExpertBytes b = expert_bytes(P);
    const uint8_t *hw13 = t.host_w13 + (size_t)e * b.w13;
    const uint8_t *hs13 = reinterpret_cast<const uint8_t *>(t.host_s13) + (size_t)e * b.s13;
    const uint8_t *hw2 = t.host_w2 + (size_t)e * b.w2;
    const uint8_t *hs2 = reinterpret_cast<const uint8_t *>(t.host_s2) + (size_t)e * b.s2;
    uint8_t *dw13 = t.slot_w13 + (size_t)s * b.w13;
    uint8_t *ds13 = reinterpret_cast<uint8_t *>(t.slot_s13) + (size_t)s * b.s13;
    uint8_t *dw2 = t.slot_w2 + (size_t)s * b.w2;
    uint8_t *ds2 = reinterpret_cast<uint8_t *>(t.slot_s2) + (size_t)s * b.s2;
    hipError_t err;
    if ((err = hipMemcpyAsync(dw13, hw13, b.w13, hipMemcpyHostToDevice, cs)) != hipSuccess) return err;
    if ((err = hipMemcpyAsync(ds13, hs13, b.s13, hipMemcpyHostToDevice, cs)) != hipSuccess) return err;
    if ((err = hipMemcpyAsync(dw2, hw2, b.w2, hipMemcpyHostToDevice, cs)) != hipSuccess) return err;
    return hipMemcpyAsync(ds2, hs2, b.s2, hipMemcpyHostToDevice, cs);
}

int check_tiers(const coli_moe_tiers *t)
{
    if (!t) return COLI_E_ARG;
    if (!t->host_w13 || !t->host_s13 || !t->host_w2 || !t->host_s2 || !t->slot_w13 ||
        !t->slot_s13 || !t->slot_w2 || !t->slot_s2 || !t->slot_table)
        return COLI_E_ARG;
    if (!aligned16(t->host_w13) || !aligned16(t->host_s13) || !aligned16(t->host_w2) ||
        !aligned16(t->host_s2) || !aligned16(t->slot_w13) || !aligned16(t->slot_s13) ||
        !aligned16(t->slot_w2) || !aligned16(t->slot_s2) || !aligned16(t->slot_table))
        return COLI_E_ALIGN;
    return COLI_OK;
}

int placed_impl(const coli_moe_layer *L, const coli_moe_tiers &tiers, coli_moe_placer &P,
                const float *x, int32_t T, const int32_t *topk_ids, const float *topk_w,
                const int32_t *union_ids, const int32_t *offsets, const int32_t *slots,
                const int32_t *n_union, int32_t act_mode, float *y, void *workspace,
                coli_moe_place_stats *stats, void *place_ws, hipStream_t st, hipStream_t cs)
{
    const int32_t cap = cap_of(L->E, L->k, T);
    const int64_t tk = (int64_t)T * L->k;
    int32_t *packed = static_cast<int32_t *>(place_ws);
    int32_t *sub0 = packed + packed_ints(cap, tk);
    int32_t *sub = sub0 + sub0_ints(cap, tk);
    bind(P, tiers);
    if (P.table_dirty && upload_table(P, tiers, st) != hipSuccess) return COLI_E_DEVICE;

    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, act_mode, L->n_shared);
    LayerDev d{};
    d.H = L->H; d.I = L->I; d.E = L->E; d.k = L->k; d.n_shared = L->n_shared;
    d.router_w = L->router_w; d.router_bias = L->router_bias;
    d.w13 = tiers.slot_w13; d.s13 = tiers.slot_s13; d.w2 = tiers.slot_w2; d.s2 = tiers.slot_s2;
    d.sh_w13 = L->sh_w13; d.sh_s13 = L->sh_s13; d.sh_w2 = L->sh_w2; d.sh_s2 = L->sh_s2;
    ForwardIO io{};
    io.x = x; io.T = T; io.ids = topk_ids; io.w = topk_w; io.y = y;
    io.ws = static_cast<uint8_t *>(workspace); io.lay = lay;
    io.acc_dump = nullptr; io.dump = dump_layout(L->H, L->I, L->k, T, L->n_shared);
    io.combine = false;
    const float *o = reinterpret_cast<const float *>(io.ws + lay.o);
    auto run_pass = [&](const int32_t *n, const int32_t *ent, const int32_t *off,
                        const int32_t *sl, int n_shared) {
        d.n_shared = n_shared;
        io.union_ids = ent; io.offsets = off; io.slots = sl; io.n_union = n;
        return act_mode == COLI_ACT_I8 ? launch_forward_i8(d, io, st, nullptr)
                                       : launch_forward_f32(d, io, st, nullptr);
    };
    auto combine = [&]() {
        return launch_combine(o, topk_ids, topk_w, T, L->k, L->H, L->n_shared, y, st);
    };
    const int32_t *ent0 = sub0 + 4;
    const int32_t *off0 = ent0 + pad4(cap);
    const int32_t *sl0 = off0 + pad4((size_t)cap + 1);

    // 1. split on the device, the packed union to the host, speculative pass 0
    hipLaunchKernelGGL(place_split_kernel, dim3(1), dim3(1024), 0, st, n_union, union_ids,
                       offsets, slots, tiers.slot_table, L->E, cap, (int)tk, packed, sub0);
    if (hipGetLastError() != hipSuccess) return COLI_E_DEVICE;
    if (hipMemcpyAsync(P.stage_in, packed, (3 + 2 * (size_t)cap + tk) * 4, hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipEventRecord(P.packed, st) != hipSuccess)
        return COLI_E_DEVICE;
    const bool spec = L->n_shared == 1;  // pass 0 never empty: launch it before planning
    if (spec) {
        if (run_pass(sub0, ent0, off0, sl0, 1) != hipSuccess) return COLI_E_DEVICE;
        if (hipEventRecord(P.done[0], st) != hipSuccess || combine() != hipSuccess)
            return COLI_E_DEVICE;
    }
    if (hipEventSynchronize(P.packed) != hipSuccess) return COLI_E_DEVICE;

    // 2. plan
    const int32_t U = P.stage_in[0], n0_dev = P.stage_in[1];
    const int32_t *h_uid = P.stage_in + 2;
    const int32_t *h_off = P.stage_in + 2 + cap;
    const int32_t *h_slots = P.stage_in + 3 + 2 * cap;
    if (U < 1 || U > cap) return COLI_E_ARG;  // T >= 1 keeps at least one slot per token
    if (h_off[0] != 0) return COLI_E_ARG;
    for (int32_t u = 0; u < U; ++u)
        if (h_off[u + 1] < h_off[u]) return COLI_E_ARG;
    if (h_off[U] > tk) return COLI_E_ARG;
    for (int32_t i = 0; i < h_off[U]; ++i)
        if (h_slots[i] < 0 || h_slots[i] >= tk) return COLI_E_ARG;
    int32_t counts[3];
    if (int rc = plan_impl(P, h_uid, U, P.chunk, P.entry_slot.data(), P.entry_pass.data(),
                           P.load_entry.data(), P.load_wait.data(), counts))
        return rc;
    // the device split used the same table the plan started from
    if (counts[0] != n0_dev) return COLI_E_DEVICE;
    const int32_t n_pass = counts[2], n_loads = counts[1];
    if (stats) *stats = {U, counts[0], n_loads, n_pass};
    if (!spec) {
        if (counts[0] > 0 && run_pass(sub0, ent0, off0, sl0, 0) != hipSuccess) return COLI_E_DEVICE;
        if (hipEventRecord(P.done[0], st) != hipSuccess) return COLI_E_DEVICE;
    }
    if (n_loads == 0) return (spec || combine() == hipSuccess) ? COLI_OK : COLI_E_DEVICE;

    // 3. sub-unions of passes 1.. (union order within a pass) and the new table
    std::vector<int32_t> cnt(n_pass, 0), rows(n_pass, 0);
    for (int32_t u = 0; u < U; ++u) {
        ++cnt[P.entry_pass[u]];
        rows[P.entry_pass[u]] += h_off[u + 1] - h_off[u];
    }
    std::vector<size_t> base(n_pass, 0);
    size_t q = 0;
    for (int32_t p = 1; p < n_pass; ++p) {
        base[p] = q;
        q += 4 + pad4(cnt[p]) + pad4((size_t)cnt[p] + 1) + pad4(std::max(rows[p], 1));
    }
    if (q > subunion_ints(cap, tk) || q > P.stage_out_ints) return COLI_E_ARG;  // cannot happen
    if (hipEventSynchronize(P.sub) != hipSuccess) return COLI_E_DEVICE;  // stage_out is free
    std::vector<int32_t> fill(n_pass, 0), filled(n_pass, 0);
    for (int32_t p = 1; p < n_pass; ++p) {
        int32_t *b = P.stage_out + base[p];
        b[0] = cnt[p];
        b[1] = b[2] = b[3] = 0;
        b[4 + pad4(cnt[p])] = 0;  // offsets[0]
    }
    for (int32_t u = 0; u < U; ++u) {
        const int32_t p = P.entry_pass[u];
        if (p == 0) continue;
        int32_t *b = P.stage_out + base[p];
        int32_t *ent = b + 4, *off = ent + pad4(cnt[p]), *sl = off + pad4((size_t)cnt[p] + 1);
        const int32_t i = fill[p]++;
        ent[i] = P.entry_slot[u];
        for (int32_t r = h_off[u]; r < h_off[u + 1]; ++r) sl[filled[p]++] = h_slots[r];
        off[i + 1] = filled[p];
    }
    if (hipMemcpyAsync(sub, P.stage_out, q * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipEventRecord(P.sub, st) != hipSuccess)
        return COLI_E_DEVICE;
    if (upload_table(P, tiers, st) != hipSuccess) return COLI_E_DEVICE;

    // 4. copies and passes 1.., then the combine
    int32_t li = 0;
    for (int32_t p = 1; p < n_pass; ++p) {
        for (; li < n_loads && P.entry_pass[P.load_entry[li]] == p; ++li) {
            const int32_t u = P.load_entry[li];
            if (P.load_wait[li] >= 0 &&
                hipStreamWaitEvent(cs, P.done[P.load_wait[li]], 0) != hipSuccess)
                return COLI_E_DEVICE;
            if (copy_expert(P, tiers, h_uid[u], P.entry_slot[u], cs) != hipSuccess)
                return COLI_E_DEVICE;
        }
        if (hipEventRecord(P.ready[p], cs) != hipSuccess ||
            hipStreamWaitEvent(st, P.ready[p], 0) != hipSuccess)
            return COLI_E_DEVICE;
        const int32_t *b = sub + base[p];
        const int32_t *ent = b + 4, *off = ent + pad4(cnt[p]), *sl = off + pad4((size_t)cnt[p] + 1);
        if (run_pass(b, ent, off, sl, 0) != hipSuccess) return COLI_E_DEVICE;
        if (hipEventRecord(P.done[p], st) != hipSuccess) return COLI_E_DEVICE;
    }
    return combine() == hipSuccess ? COLI_OK : COLI_E_DEVICE;
}

}  // namespace

extern "C" {

int coli_moe_placer_create(int32_t H, int32_t I, int32_t E, int32_t k, int32_t n_slots,
                           int32_t T_max, int32_t chunk, coli_moe_placer **out)
{
    if (!out) return COLI_E_ARG;
    if (H < 64 || H > COLI_MAX_H || H % 64 || I < 64 || I > COLI_MAX_I || I % 64) return COLI_E_SHAPE;
    if (E < 1 || E > COLI_MAX_E || k < 1 || k > COLI_MAX_K || k > E) return COLI_E_SHAPE;
    if (T_max < 1 || T_max > COLI_MAX_T) return COLI_E_SHAPE;
    if (n_slots < 1 || n_slots > E) return COLI_E_SHAPE;
    if (chunk < 1 || chunk > n_slots) return COLI_E_ARG;
    coli_moe_placer *P = new (std::nothrow) coli_moe_placer;
    if (!P) return COLI_E_ARG;
    P->H = H; P->I = I; P->E = E; P->k = k; P->n_slots = n_slots; P->T_max = T_max;
    P->chunk = chunk;
    P->cap_max = cap_of(E, k, T_max);
    P->slot_of.assign(E, -1);
    P->expert_in.assign(n_slots, -1);
    P->last_use.assign(n_slots, 0);
    P->slot_pass.assign(n_slots, -1);
    P->entry_slot.assign(E, 0);
    P->entry_pass.assign(E, 0);
    P->load_entry.assign(E, 0);
    P->load_wait.assign(E, 0);
    *out = P;
    return COLI_OK;
}

void coli_moe_placer_destroy(coli_moe_placer *P)
{
    if (!P) return;
    for (hipEvent_t e : P->ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : P->done)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : {P->packed, P->tab, P->sub, P->order[0], P->order[1]})
        if (e) (void)hipEventDestroy(e);
    for (int32_t *p : {P->stage_in, P->stage_out, P->stage_tab})
        if (p) (void)hipHostFree(p);
    delete P;
}

int coli_moe_placer_reset(coli_moe_placer *P)
{
    if (!P) return COLI_E_ARG;
    forget(*P);
    return COLI_OK;
}

int32_t coli_moe_placer_slot_of(const coli_moe_placer *P, int32_t e)
{
    if (!P || e < 0 || e >= P->E) return -1;
    return P->slot_of[e];
}

int coli_moe_place_plan(coli_moe_placer *P, const int32_t *union_ids, int32_t n_union,
                        int32_t *entry_slot, int32_t *entry_pass, int32_t *load_entry,
                        int32_t *load_wait, int32_t *counts)
{
    if (!P || n_union < 0 || !counts) return COLI_E_ARG;
    if (n_union > 0 && (!union_ids || !entry_slot || !entry_pass || !load_entry || !load_wait))
        return COLI_E_ARG;
    const int rc = plan_impl(*P, union_ids, n_union, P->chunk, entry_slot, entry_pass, load_entry,
                             load_wait, counts);
    if (rc == COLI_OK) P->table_dirty = true;  // residency changed outside a placed call
    return rc;
}

size_t coli_moe_place_ws_bytes(int32_t E, int32_t k, int32_t T)
{
    if (E < 1 || E > COLI_MAX_E || k < 1 || k > COLI_MAX_K || k > E) return 0;
    if (T < 0 || T > COLI_MAX_T) return 0;
    const int32_t cap = cap_of(E, k, T);
    const int64_t tk = (int64_t)T * k;
    const size_t b = (packed_ints(cap, tk) + sub0_ints(cap, tk) + subunion_ints(cap, tk)) * 4;
    return (b + 255) & ~size_t(255);
}

int coli_moe_forward_placed(const coli_moe_layer *L, const coli_moe_tiers *tiers,
                            coli_moe_placer *P, const float *x, int32_t T,
                            const int32_t *topk_ids, const float *topk_w,
                            const int32_t *union_ids, const int32_t *offsets,
                            const int32_t *slots, const int32_t *n_union, int32_t act_mode,
                            float *y, void *workspace, size_t workspace_bytes, void *place_ws,
                            size_t place_ws_bytes, coli_moe_place_stats *stats,
                            void *hip_stream, void *copy_stream)
{
    if (!L || !P) return COLI_E_ARG;
    if (L->H != P->H || L->I != P->I || L->E != P->E || L->k != P->k) return COLI_E_SHAPE;
    if (L->n_shared != 0 && L->n_shared != 1) return COLI_E_SHAPE;
    if (T < 0 || T > P->T_max) return COLI_E_SHAPE;
    if (act_mode != COLI_ACT_F32 && act_mode != COLI_ACT_I8) return COLI_E_UNSUPPORTED;
    if (int rc = check_tiers(tiers)) return rc;
    const bool any_sh = L->sh_w13 || L->sh_s13 || L->sh_w2 || L->sh_s2;
    const bool all_sh = L->sh_w13 && L->sh_s13 && L->sh_w2 && L->sh_s2;
    if (L->n_shared ? !all_sh : any_sh) return COLI_E_ARG;
    if (L->n_shared && (!aligned16(L->sh_w13) || !aligned16(L->sh_s13) || !aligned16(L->sh_w2) ||
                        !aligned16(L->sh_s2)))
        return COLI_E_ALIGN;
    if (stats) *stats = {0, 0, 0, 0};
    if (T == 0) return COLI_OK;
    if (!x || !topk_ids || !topk_w || !union_ids || !offsets || !slots || !n_union || !y ||
        !workspace || !place_ws)
        return COLI_E_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(union_ids) ||
        !aligned16(offsets) || !aligned16(slots) || !aligned16(n_union) || !aligned16(y) ||
        !aligned16(workspace) || !aligned16(place_ws))
        return COLI_E_ALIGN;
    const Workspace lay = workspace_layout(L->H, L->I, L->E, L->k, T, act_mode, L->n_shared);
    if (workspace_bytes < lay.forward_end) return COLI_E_WORKSPACE;
    if (place_ws_bytes < coli_moe_place_ws_bytes(L->E, L->k, T)) return COLI_E_WORKSPACE;
    if (int rc = coli_moe_device_check()) return rc;
    if (int rc = ensure_device(*P)) return rc;
    const int rc = placed_impl(L, *tiers, *P, x, T, topk_ids, topk_w, union_ids, offsets, slots,
                               n_union, act_mode, y, workspace, stats, place_ws,
                               static_cast<hipStream_t>(hip_stream),
                               static_cast<hipStream_t>(copy_stream));
    if (rc == COLI_E_DEVICE) forget(*P);
    return rc;
}

int coli_moe_place_prefetch(coli_moe_placer *P, const coli_moe_tiers *tiers,
                            const int32_t *experts, int32_t n, void *hip_stream,
                            void *copy_stream)
{
    if (!P || n < 0 || n > P->n_slots) return COLI_E_ARG;
    if (int rc = check_tiers(tiers)) return rc;
    if (n == 0) return COLI_OK;
    if (!experts) return COLI_E_ARG;
    std::vector<int32_t> ids(experts, experts + n);
    std::sort(ids.begin(), ids.end());
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= P->E || (i > 0 && ids[i] == ids[i - 1])) return COLI_E_ARG;
    if (int rc = coli_moe_device_check()) return rc;
    if (int rc = ensure_device(*P)) return rc;
    bind(*P, *tiers);
    std::vector<int32_t> es(n), ep(n), le(n), lw(n);
    int32_t counts[3];
    if (int rc = plan_impl(*P, ids.data(), n, n, es.data(), ep.data(), le.data(), lw.data(), counts))
        return rc;
    hipStream_t st = static_cast<hipStream_t>(hip_stream), cs = static_cast<hipStream_t>(copy_stream);
    bool ok = hipEventRecord(P->order[0], st) == hipSuccess &&
              hipStreamWaitEvent(cs, P->order[0], 0) == hipSuccess;
    for (int32_t i = 0; ok && i < counts[1]; ++i)
        ok = copy_expert(*P, *tiers, ids[le[i]], es[le[i]], cs) == hipSuccess;
    ok = ok && hipEventRecord(P->order[1], cs) == hipSuccess &&
         hipStreamWaitEvent(st, P->order[1], 0) == hipSuccess;
    ok = ok && upload_table(*P, *tiers, st) == hipSuccess;
    if (!ok) {
        forget(*P);
        return COLI_E_DEVICE;
    }
    return COLI_OK;
}

}  // extern "C"
