// union.hip -- batch-union of the routed experts (Colibri getting-started
// page, section "토큰당 처리 경로": experts picked by several tokens of the
// batch are de-duplicated and computed once).
//
// One workgroup of W waves.  Wave w owns a contiguous range of slots.
//   1. per-wave expert histograms in LDS (integer atomics: order-free),
//   2. a block scan gives each expert its start and its union position, and
//      each wave its private cursor per expert (start + counts of the
//      waves before it),
//   3. each wave walks its range in order, 64 slots at a time: the 64 keys
//      (expert << 6 | lane) are sorted with a bitonic network across the
//      wave, so that equal experts form runs in lane order; a lane's rank in
//      its run plus the wave's cursor of that expert is where its slot goes,
//      and the last lane of a run advances the cursor.
// The result is the stable order (ascending slot) and is deterministic.
// Batches of more than 8,192 slots split the slots over several workgroups
// (union_multi_kernel) with the same result.
#include <algorithm>

#include "common.h"
#include "union_wave.h"

namespace coli {


__device__ void block_exclusive_scan(int32_t *a, int n, int32_t *tmp)
{
    // Hillis-Steele inclusive scan over n <= 2 * blockDim entries, then shift.
    for (int i = threadIdx.x; i < n; i += blockDim.x) tmp[i] = a[i];
    __syncthreads();
    for (int off = 1; off < n; off <<= 1) {
        int32_t v[2];
        int c = 0;
        for (int i = threadIdx.x; i < n; i += blockDim.x, ++c) v[c] = (i >= off) ? tmp[i - off] : 0;
        __syncthreads();
        c = 0;
        for (int i = threadIdx.x; i < n; i += blockDim.x, ++c) tmp[i] += v[c];
        __syncthreads();
    }
    for (int i = threadIdx.x; i < n; i += blockDim.x) a[i] = (i == 0) ? 0 : tmp[i - 1];
    __syncthreads();
}

// Bitonic sort of one key per lane across the wave, ascending by lane.
__device__ __forceinline__ uint32_t wave_sort64(uint32_t key, int lane)
{
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
    return key;
}

template <int W>
__global__ __launch_bounds__(W * 64) void union_kernel(const int32_t *__restrict__ ids,
                                                              int n, int E, int cap,
                                                              int32_t *__restrict__ union_ids,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ slots,
                                                              int32_t *__restrict__ n_union)
{
    extern __shared__ int32_t smem[];
    volatile int32_t *cur = smem;                       // [W][E]
    int32_t *start = smem + W * E;                      // [E]
    int32_t *upos = start + E;                          // [E]
    int32_t *tmp = upos + E;                            // [E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < W * E; i += blockDim.x) cur[i] = 0;
    __syncthreads();

    const int per = ((n + W - 1) / W + 63) & ~63;
    const int r0 = min(n, wave * per), r1 = min(n, r0 + per);
    for (int s = r0 + lane; s < r1; s += 64) {
        int id = ids[s];
        if (id >= 0 && id < E) atomicAdd((int32_t *)&cur[wave * E + id], 1);
    }
    __syncthreads();

    for (int e = tid; e < E; e += blockDim.x) {
        int32_t c = 0;
        for (int w = 0; w < W; ++w) c += cur[w * E + e];
        start[e] = c;
        upos[e] = c > 0 ? 1 : 0;
    }
    __syncthreads();
    // counts -> flags are recovered below from the scanned starts
    for (int e = tid; e < E; e += blockDim.x) tmp[e] = start[e];
    __syncthreads();
    // keep the counts in the first row of a scratch region before scanning
    block_exclusive_scan(start, E, smem + W * E + 3 * E);
    block_exclusive_scan(upos, E, smem + W * E + 4 * E);

    int32_t U = upos[E - 1] + (tmp[E - 1] > 0 ? 1 : 0);
    const int32_t kept = start[E - 1] + tmp[E - 1];  // slots with an expert
    for (int e = tid; e < E; e += blockDim.x) {
        int32_t c = tmp[e];
        if (c > 0) {
            union_ids[upos[e]] = e;
            offsets[upos[e]] = start[e];
        }
        int32_t base = start[e];
        for (int w = 0; w < W; ++w) {
            int32_t v = cur[w * E + e];
            cur[w * E + e] = base;
            base += v;
        }
    }
    for (int u = U + tid; u < cap; u += blockDim.x) union_ids[u] = -1;
    for (int u = U + tid; u <= cap; u += blockDim.x) offsets[u] = kept;
    if (tid == 0) n_union[0] = U;
    __syncthreads();

    for (int b = r0; b < r1; b += 64) {
        const int s = b + lane;
        const int id = (s < r1) ? ids[s] : -1;
        const bool valid = id >= 0 && id < E;
        const uint32_t key = wave_sort64(valid ? ((uint32_t)id << 6 | (uint32_t)lane) : 0xFFFFFFFFu,
                                         lane);
        const bool has = key != 0xFFFFFFFFu;
        const int sid = has ? (int)(key >> 6) : -1;
        const int prev = __shfl_up(sid, 1, 64);
        const int next = __shfl_down(sid, 1, 64);
        const bool head = has && (lane == 0 || prev != sid);
        const bool tail = has && (lane == 63 || next != sid);
        const uint64_t heads = __ballot(head);
        const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1);
        const int rank = lane - (63 - __clzll(heads & upto));  // lane of this run's head
        int32_t base = 0;
        if (has) {
            base = cur[wave * E + sid];
            slots[base + rank] = b + (int)(key & 63u);
        }
        __builtin_amdgcn_wave_barrier();
        if (tail) cur[wave * E + sid] = base + rank + 1;
        __builtin_amdgcn_wave_barrier();
    }
}

// Large batches: the same result from B workgroups, workgroup b taking the
// slots of chunk b.  Every workgroup counts the experts of ALL slots
// (totals: the union, its starts) and of the slots before its chunk, so it
// knows where its chunk's slots of each expert begin without waiting for
// the other workgroups; its waves then scatter the chunk exactly as above.
// Workgroup 0 writes the union, its offsets and its size.
template <int W>
__global__ __launch_bounds__(W * 64) void union_multi_kernel(const int32_t *__restrict__ ids,
                                                            int n, int E, int cap, int chunk,
                                                            int32_t *__restrict__ union_ids,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ slots,
                                                            int32_t *__restrict__ n_union)
{
    extern __shared__ int32_t smem[];
    volatile int32_t *cur = smem;  // [W][E] counts of each wave's range, then its cursors
    int32_t *tot = smem + W * E;   // [E] slots of each expert
    int32_t *bef = tot + E;        // [E] of them before the chunk
    int32_t *start = bef + E;      // [E]
    int32_t *upos = start + E;     // [E]
    int32_t *tmp = upos + E;       // [E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = min(n, (int)blockIdx.x * chunk), c1 = min(n, c0 + chunk);
    const int per = ((c1 - c0 + W - 1) / W + 63) & ~63;
    const int r0 = min(c1, c0 + wave * per), r1 = min(c1, r0 + per);

    for (int i = tid; i < (W + 2) * E; i += blockDim.x) smem[i] = 0;
    __syncthreads();
    auto count = [&](int s, int id) {
        if (id < 0 || id >= E) return;
        atomicAdd(&tot[id], 1);
        if (s < c0) atomicAdd(&bef[id], 1);
        else if (s < c1) atomicAdd((int32_t *)&cur[((s - c0) / per) * E + id], 1);
    };
    // the ids as 16-byte vectors, kBatch loads of a thread in flight before
    // its first count (one memory latency per batch, not per id)
    constexpr int kBatch = 8;
    const bool vec = ((uintptr_t)ids & 15u) == 0;
    const int n4 = vec ? n >> 2 : 0;
    const int4 *ids4 = reinterpret_cast<const int4 *>(ids);
    for (int j0 = tid; j0 < n4; j0 += kBatch * (int)blockDim.x) {
        int4 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int j = j0 + b * (int)blockDim.x;
            v[b] = j < n4 ? ids4[j] : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int s = 4 * (j0 + b * (int)blockDim.x);
            count(s, v[b].x);
            count(s + 1, v[b].y);
            count(s + 2, v[b].z);
            count(s + 3, v[b].w);
        }
    }
    for (int s = 4 * n4 + tid; s < n; s += blockDim.x) count(s, ids[s]);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        start[e] = tot[e];
        upos[e] = tot[e] > 0 ? 1 : 0;
    }
    __syncthreads();
    block_exclusive_scan(start, E, tmp);
    block_exclusive_scan(upos, E, tmp);

    if (blockIdx.x == 0) {
        const int32_t U = upos[E - 1] + (tot[E - 1] > 0 ? 1 : 0);
        const int32_t kept = start[E - 1] + tot[E - 1];
        for (int e = tid; e < E; e += blockDim.x)
            if (tot[e] > 0) {
                union_ids[upos[e]] = e;
                offsets[upos[e]] = start[e];
            }
        for (int u = U + tid; u < cap; u += blockDim.x) union_ids[u] = -1;
        for (int u = U + tid; u <= cap; u += blockDim.x) offsets[u] = kept;
        if (tid == 0) n_union[0] = U;
    }
    for (int e = tid; e < E; e += blockDim.x) {
        int32_t base = start[e] + bef[e];
        for (int w = 0; w < W; ++w) {
            const int32_t v = cur[w * E + e];
            cur[w * E + e] = base;
            base += v;
        }
    }
    __syncthreads();

    for (int b = r0; b < r1; b += 64) {
        const int s = b + lane;
        const int id = (s < r1) ? ids[s] : -1;
        const bool valid = id >= 0 && id < E;
        const uint32_t key = wave_sort64(valid ? ((uint32_t)id << 6 | (uint32_t)lane) : 0xFFFFFFFFu,
                                         lane);
        const bool has = key != 0xFFFFFFFFu;
        const int sid = has ? (int)(key >> 6) : -1;
        const int prev = __shfl_up(sid, 1, 64);
        const int next = __shfl_down(sid, 1, 64);
        const bool head = has && (lane == 0 || prev != sid);
        const bool tail = has && (lane == 63 || next != sid);
        const uint64_t heads = __ballot(head);
        const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1);
        const int rank = lane - (63 - __clzll(heads & upto));
        int32_t base = 0;
        if (has) {
            base = cur[wave * E + sid];
            slots[base + rank] = b + (int)(key & 63u);
        }
        __builtin_amdgcn_wave_barrier();
        if (tail) cur[wave * E + sid] = base + rank + 1;
        __builtin_amdgcn_wave_barrier();
    }
}

// Small batches (T*k <= 64): one wave (union_wave.h).
__global__ __launch_bounds__(64) void union_small_kernel(const int32_t *__restrict__ ids, int n,
                                                         int E, int cap,
                                                         int32_t *__restrict__ union_ids,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ slots,
                                                         int32_t *__restrict__ n_union)
{
    const int lane = threadIdx.x;
    union_wave(lane, lane < n ? ids[lane] : -1, E, cap, union_ids, offsets, slots, n_union);
}

constexpr int kUnionChunk = 2048, kUnionBlocks = 64, kUnionMultiMin = 8192;

hipError_t launch_union(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *union_ids,
                        int32_t *offsets, int32_t *slots, int32_t *n_union, hipStream_t st)
{
    const int n = T * k;
    const int cap = n < E ? n : E;
    if (n <= 64) {
        hipLaunchKernelGGL(union_small_kernel, dim3(1), dim3(64), 0, st, ids, n, E, cap, union_ids,
                           offsets, slots, n_union);
        return hipGetLastError();
    }
    // more than kUnionMultiMin slots: one workgroup per chunk of kUnionChunk
    // slots (at most kUnionBlocks, the chunks growing beyond that).  Below,
    // the single workgroup is as fast (4,096 slots: 17-18 us against 18.7
    // with two chunks; 32,768: 62.4 against 27.2)
    if (n > kUnionMultiMin) {
        const int B = std::min(kUnionBlocks, (n + kUnionChunk - 1) / kUnionChunk);
        const int chunk = (n + B - 1) / B;
        const int nb = (n + chunk - 1) / chunk;
        const size_t lds = (size_t)(8 + 5) * E * sizeof(int32_t);
        hipLaunchKernelGGL(union_multi_kernel<8>, dim3(nb), dim3(8 * 64), lds, st, ids, n, E, cap, chunk,
                           union_ids, offsets, slots, n_union);
        return hipGetLastError();
    }
    // 16 waves while the per-wave histograms fit in 64 KB of LDS, else 8
    if (E <= 512) {
        const size_t lds = (size_t)(16 + 5) * E * sizeof(int32_t);
        hipLaunchKernelGGL(union_kernel<16>, dim3(1), dim3(16 * 64), lds, st, ids, n, E, cap,
                           union_ids, offsets, slots, n_union);
    } else {
        const size_t lds = (size_t)(8 + 5) * E * sizeof(int32_t);
        hipLaunchKernelGGL(union_kernel<8>, dim3(1), dim3(8 * 64), lds, st, ids, n, E, cap,
                           union_ids, offsets, slots, n_union);
    }
    return hipGetLastError();
}

}  // namespace coli
