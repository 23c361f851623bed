// stream.h -- building blocks of the HBM-streaming GEMV kernels (both
// arithmetic families): buffer-resource loads, the per-stage weight loads of
// a register ring, and the split of waves over union entries and row blocks.
#pragma once

#include "common.h"

#include <type_traits>

namespace coli {

// Buffer resource over [p, p + bytes): loads use 32-bit offsets from an
// SGPR base (no 64-bit address arithmetic per lane); out-of-range reads
// return 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint16_t load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

constexpr uint32_t kOOB = 0x40000000u;

// Timeline mark j (0..7) of the calling wave, compiled into the kernels'
// TL variants only (the measurement entry point): the chip-wide 100 MHz
// real-time counter at that point, written by lane 0 to tl[w * 8 + j] (w =
// the wave's index in the grid, recorded while w < cap).
template <bool TL>
__device__ __forceinline__ void tl_mark(uint64_t *tl, int cap, int j)
{
    if constexpr (TL) {
        const int w = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        if ((threadIdx.x & 63) == 0 && w < cap) tl[(size_t)w * 8 + j] = t;
    }
}

struct StageRsrc {
    __amdgpu_buffer_rsrc_t w, s, w0, s0;  // weights, scales, and their empty twins
};

__device__ __forceinline__ StageRsrc stage_rsrc(const uint8_t *wb, const uint16_t *sb, int N,
                                                int rb, int sbs)
{
    StageRsrc R;
    R.w = make_rsrc(wb, (uint32_t)(N * rb));
    R.s = make_rsrc(sb, (uint32_t)(N * sbs * 2));
    R.w0 = make_rsrc(wb, 0);
    R.s0 = make_rsrc(sb, 0);
    return R;
}

template <int NR, int P>
__device__ __forceinline__ void load_stage(const StageRsrc &R, const int (&rows)[NR], bool valid,
                                           int rb, int sbs, const uint32_t (&vw)[P],
                                           const uint32_t (&vs)[P], uint4 (&w)[NR][P],
                                           uint16_t (&s)[NR][P])
{
    const __amdgpu_buffer_rsrc_t rw = valid ? R.w : R.w0, rs = valid ? R.s : R.s0;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            w[r][p] = load16(rw, vw[p], (uint32_t)rows[r] * rb);
            s[r][p] = load2(rs, vs[p], (uint32_t)rows[r] * sbs * 2);
        }
}

template <int P>
__device__ __forceinline__ void lane_offsets(int lane, int C, uint32_t (&vw)[P], uint32_t (&vs)[P])
{
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int c = lane + 64 * p;
        vw[p] = c < C ? (uint32_t)c * 16 : kOOB;
        vs[p] = c < C ? (uint32_t)(c >> 1) * 2 : kOOB;
    }
}


constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

// Work split of one token's streaming kernels: the wpe = waves / entries
// waves of an entry take its row blocks round-robin (wave part p: blocks
// p, p + wpe, ...), so at any moment an entry's waves read one contiguous
// stretch of rows (DRAM page locality) while every wave stays inside one
// entry (its activation chunk is loaded once).
struct T1Split {
    int ue, part, wpe, nsteps;
};

__device__ __forceinline__ T1Split t1_split(int gw, int GW, int ne, int nblocks)
{
    T1Split s;
    s.wpe = ne > 0 ? GW / ne : 0;
    const bool has = s.wpe > 0 && gw < ne * s.wpe;
    s.ue = has ? gw / s.wpe : 0;
    s.part = has ? gw - s.ue * s.wpe : 0;
    s.nsteps = has && s.part < nblocks ? (nblocks - s.part + s.wpe - 1) / s.wpe : 0;
    return s;
}


// f(std::integral_constant<int, c>) for the runtime count 1 <= c <= NMAX
// (NMAX a power of two <= 4): one specialised body per count.
template <int NMAX, class F>
__device__ __forceinline__ void dispatch_count(int c, F &&f)
{
    if (c <= 1) f(std::integral_constant<int, 1>{});
    else if (NMAX >= 2 && c == 2) f(std::integral_constant<int, (NMAX >= 2 ? 2 : 1)>{});
    else if (NMAX >= 4 && c == 3) f(std::integral_constant<int, (NMAX >= 4 ? 3 : 1)>{});
    else if (NMAX >= 4) f(std::integral_constant<int, (NMAX >= 4 ? 4 : 1)>{});
}


}  // namespace coli
