// union_wave.h -- batch-union of at most 64 slots by one wave (Colibri
// getting-started page, section "토큰당 처리 경로": experts picked by several
// tokens of a batch are computed once).  Shared by the union kernel for
// small batches and by the top-k kernel that routes and unions a small batch
// in one launch.
#pragma once

#include "common.h"

namespace coli {

// Lane l holds the expert of slot l (slot = t * k + j; -1 for a dropped slot
// or l >= n).  The 64 keys (expert << 6 | slot) are sorted with a bitonic
// network across the wave and the union is read off the sorted order:
// union_ids ascending, offsets of each expert's run of slots, slots grouped
// by expert in ascending slot order, entries past U set to -1 / n_kept.
__device__ __forceinline__ void union_wave(int lane, int id, int E, int cap,
                                           int32_t *__restrict__ union_ids,
                                           int32_t *__restrict__ offsets,
                                           int32_t *__restrict__ slots,
                                           int32_t *__restrict__ n_union)
{
    const bool valid = id >= 0 && id < E;
    uint32_t key = valid ? ((uint32_t)id << 6 | (uint32_t)lane) : 0xFFFFFFFFu;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride >= 1; stride >>= 1) {
            const uint32_t other = __shfl_xor(key, stride, 64);
            const bool ascending = (lane & size) == 0 || size == 64;
            const bool lower = (lane & stride) == 0;
            const uint32_t lo = min(key, other), hi = max(key, other);
            key = (lower == ascending) ? lo : hi;
        }
    }
    const bool has = key != 0xFFFFFFFFu;
    const int sid = has ? (int)(key >> 6) : -1;
    const int prev = __shfl_up(sid, 1, 64);
    const bool first = has && (lane == 0 || prev != sid);
    const uint64_t fm = __ballot(first);
    const int U = __popcll(fm);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int upos = __popcll(fm & lt_mask);
    if (has) slots[lane] = (int32_t)(key & 63u);
    if (first && upos < cap) {
        union_ids[upos] = sid;
        offsets[upos] = lane;
    }
    const int kept = __popcll(__ballot(has));  // slots with an expert
    if (lane >= U && lane < cap) union_ids[lane] = -1;
    if (lane >= U && lane <= cap) offsets[lane] = kept;
    if (lane == 0) {
        n_union[0] = U;
        if (cap == 64) offsets[64] = kept;
    }
}

}  // namespace coli
