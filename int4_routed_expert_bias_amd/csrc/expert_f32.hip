// expert_f32.hip -- the fp32 arithmetic family of the expert FFN
// ("Colibri 完全ガイド", walk-through "詳細解説" step 3: single-token decode
// computes in f32).  Weights are int4 with one fp16 scale per row per
// 64-group ("colibri: 744B MoE...", section "はじめにとソースが語らないこと":
// the gs64 build).
//
// The matmuls stream every union expert's packed weights once from HBM
// (a GEMV at decode, a few tokens for a verify batch).  Design for CDNA4:
//  - grid = (row blocks, union entries + shared expert); many small
//    workgroups keep ~20 waves per CU with all their weight loads in flight;
//  - a wave owns a few weight rows, loads all of its 16-byte chunks up front
//    (lane l reads chunks l, l+64, ...: 1 KB per wave instruction) through
//    32-bit buffer offsets, and keeps them in registers for every batch of
//    the entry's tokens;
//  - gate/up stages the token rows in LDS; it writes h in a chunk-transposed
//    row layout so that the down matmul's per-lane activation reads are
//    coalesced;
//  - a packed dword w of 8 codes becomes the signed bytes (w << 4) & 0xF0F0F0F0
//    (even elements) and w & 0xF0F0F0F0 (odd elements), each equal to 16 x
//    the code; one sign-extending byte-to-float conversion per weight feeds
//    an fp32 FMA; the 1/16 is folded into the group scale (exact);
//  - lane partials are combined with a reduce-scatter that applies the same
//    xor-butterfly (32, 16, 8, 4, 2, 1) to every value, so the sum of a
//    given (token, row) does not depend on how many values a wave reduces.
// A token's arithmetic is the same whatever the batch and whichever kernel
// variant runs it: a token alone and inside a batch give identical bits.
#include "common.h"

namespace coli {

struct GemvArgs {
    const uint8_t *w;      // routed experts, [E][N][K/2]
    const uint16_t *s;     // [E][N][K/64]
    const uint8_t *sh_w;   // shared expert [N][K/2]
    const uint16_t *sh_s;  // [N][K/64]
    int N, K, I;           // rows, reduction length, I (up-row offset for SwiGLU)
    int upe;               // output units per entry (I for SwiGLU, N otherwise)
    const float *in;       // input rows
    int in_by_slot;        // 0: input row = token; 1: input row = output row
    float *out;            // output rows [R][out_ld]
    int out_ld;
    const int32_t *union_ids, *offsets, *slots, *n_union;
    int T, k, cap, n_shared;
};

constexpr int kRows = 4;  // weight rows a wave computes at a time

// 32 products of one 16-byte chunk (32 int4 codes) with 32 activations,
// fp32, ascending element order.  Returns 16 x the dot product.
__device__ __forceinline__ float chunk_dot16(const uint4 wv, const float *xv)
{
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = (wd[d] << 4) & 0xF0F0F0F0u;  // 16 x even codes
        const uint32_t hi = wd[d] & 0xF0F0F0F0u;         // 16 x odd codes
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            acc = fmaf((float)(int8_t)(lo >> (8 * b)), xv[8 * d + 2 * b], acc);
            acc = fmaf((float)(int8_t)(hi >> (8 * b)), xv[8 * d + 2 * b + 1], acc);
        }
    }
    return acc;
}

// Sum of v[i] over the 64 lanes for V values (V a power of two <= 64):
// halving exchanges over xor 32, 16, ... while more than one value is left,
// then a plain butterfly.  Every value sees the same pairing tree.  On
// return, lane l holds the total of value (l >> (6 - log2 V)) in v[0].
template <int V>
__device__ __forceinline__ float reduce_scatter(float (&v)[V], int lane)
{
    int off = 32;
#pragma unroll
    for (int n = V; n > 1; n >>= 1, off >>= 1) {
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float send = upper ? v[i] : v[i + n / 2];
            const float keep = upper ? v[i + n / 2] : v[i];
            v[i] = keep + __shfl_xor(send, off, 64);
        }
    }
#pragma unroll
    for (; off >= 1; off >>= 1) v[0] += __shfl_xor(v[0], off, 64);
    return v[0];
}

// Value index held by a lane after reduce_scatter<V>.
template <int V>
__device__ __forceinline__ int scatter_index(int lane)
{
    int idx = 0, off = 32;
#pragma unroll
    for (int n = V; n > 1; n >>= 1, off >>= 1) {
        idx = idx * 2 + ((lane & off) ? 1 : 0);
    }
    return idx;
}

// Entry -> (weights, scales, token list).  Returns the token count.
__device__ __forceinline__ int entry_info(const GemvArgs &a, int ue, const uint8_t *&wb,
                                          const uint16_t *&sb, const int32_t *&list)
{
    const int U = a.n_union[0];
    if (ue < U) {
        const int e = a.union_ids[ue];
        wb = a.w + (size_t)e * a.N * (a.K / 2);
        sb = a.s + (size_t)e * a.N * (a.K / 64);
        const int o0 = a.offsets[ue];
        list = a.slots + o0;
        return a.offsets[ue + 1] - o0;
    }
    wb = a.sh_w;
    sb = a.sh_s;
    list = nullptr;
    return a.T;
}

__device__ __forceinline__ void token_rows(const GemvArgs &a, const int32_t *list, int idx,
                                           int &in_row, int &out_row)
{
    const int TK = a.T * a.k;
    if (list) {
        const int s = list[idx];
        out_row = s;
        in_row = a.in_by_slot ? s : s / a.k;
    } else {
        out_row = TK + idx;
        in_row = a.in_by_slot ? TK + idx : idx;
    }
}

// Buffer resource over [p, p + bytes): loads use 32-bit offsets from an
// SGPR base (no 64-bit address arithmetic per lane); out-of-range reads
// return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint16_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Position of element i of an h row in the chunk-transposed layout used
// between the two matmuls: chunk c = i / 32 holds 8 float4 pieces q; piece q
// of every chunk is stored contiguously, so a wave reading piece q of chunks
// lane + 64p reads 1 KB in one instruction.
__device__ __forceinline__ int ht_pos(int i, int chunks)
{
    return (((i & 31) >> 2) * chunks + (i >> 5)) * 4 + (i & 3);
}

// Marks the packed weights as redefined at this point.  The per-token loops
// reuse the same packed codes for every token; without this the compiler
// hoists all the code-to-float conversions out of the loop and keeps
// hundreds of floats live, which collapses occupancy.  Emits no instruction.
template <int R, int P>
__device__ __forceinline__ void opaque_codes(uint4 (&w)[R][P])
{
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < P; ++p)
            asm volatile("" : "+v"(w[r][p].x), "+v"(w[r][p].y), "+v"(w[r][p].z), "+v"(w[r][p].w));
}

// Gate/up matmul + SwiGLU.  Grid: (I / (W * RW / 2), entries).  Wave w of a
// workgroup owns RW/2 units (gate rows i and up rows I + i), keeps their
// P chunks per lane in registers for all of the entry's token batches, and
// stages each batch of NT token rows in LDS.
template <int NT, int P, int W, int RW, bool ONE>
__global__ __launch_bounds__(W * 64) void gateup_f32_kernel(GemvArgs a)
{
    extern __shared__ float xs[];  // [NT][K]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ue = blockIdx.y;
    if (ue < a.cap && ue >= a.n_union[0]) return;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    const int cnt = entry_info(a, ue, wb, sb, list);
    if (cnt <= 0) return;
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, K4 = K / 4;
    const auto rw = make_rsrc(wb, (uint32_t)(a.N * rb));
    const auto rs = make_rsrc(sb, (uint32_t)(a.N * sbs * 2));
    const int u0 = (blockIdx.x * W + wave) * (RW / 2);
    int rows[RW];
#pragma unroll
    for (int r = 0; r < RW / 2; ++r) {
        rows[r] = u0 + r;
        rows[RW / 2 + r] = a.I + u0 + r;
    }
    uint4 wv[RW][P];
    uint16_t sc[RW][P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        // lanes past the row's last chunk read a valid chunk with a zero scale
        const bool live = lane + 64 * p < C;
        const int c = live ? lane + 64 * p : C - 1;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            wv[r][p] = load16(rw, (uint32_t)rows[r] * rb + c * 16);
            sc[r][p] = live ? load2(rs, ((uint32_t)rows[r] * sbs + (c >> 1)) * 2) : (uint16_t)0;
        }
    }
    const int CI = a.I / 32;
    // ONE: every entry has exactly one token (T == 1): straight-line code
    for (int t0 = 0; t0 < (ONE ? 1 : cnt); t0 += NT) {
        const int nt = ONE ? 1 : min(NT, cnt - t0);
        int in_row[NT], out_row[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) token_rows(a, list, t0 + (tt < nt ? tt : 0), in_row[tt], out_row[tt]);
        if (t0 > 0) __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float4 *src = reinterpret_cast<const float4 *>(a.in + (size_t)in_row[tt] * K);
            float4 *dst = reinterpret_cast<float4 *>(xs + tt * K);
            for (int i = threadIdx.x; i < K4; i += blockDim.x) dst[i] = src[i];
        }
        __syncthreads();
        float racc[RW * NT];
#pragma unroll
        for (int i = 0; i < RW * NT; ++i) racc[i] = 0.f;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (!ONE) opaque_codes(wv);  // convert per token: keeps registers low
            if (tt < nt) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int c = min(lane + 64 * p, C - 1);
                    float xv[32];
                    const float4 *xp = reinterpret_cast<const float4 *>(xs + tt * K + c * 32);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float4 v = xp[q];
                        xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y;
                        xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
                    }
#pragma unroll
                    for (int r = 0; r < RW; ++r)
                        racc[r * NT + tt] = fmaf(chunk_dot16(wv[r][p], xv), f16_to_f32(sc[r][p]),
                                                 racc[r * NT + tt]);
                }
            }
        }
        // value v = r * NT + tt; the up row of unit r sits RW/2 * NT values
        // later, i.e. in the lane with bit 5 flipped
        const float tot = reduce_scatter<RW * NT>(racc, lane) * 0.0625f;
        const float up = __shfl_xor(tot, 32, 64);
        const int vi = scatter_index<RW * NT>(lane);
        const int r = vi / NT, tt = vi % NT;
        constexpr int LPV = 64 / (RW * NT);
        if ((lane % LPV) == 0 && r < RW / 2 && tt < nt) {
            const float g = tot;
            a.out[(size_t)out_row[tt] * a.out_ld + ht_pos(rows[r], CI)] = g / (1.0f + expf(-g)) * up;
        }
    }
}

// Down matmul.  Grid: (H / (W * RW), entries).  Wave w owns RW consecutive
// rows (P chunks per lane in registers) and walks the entry's tokens; each
// token's h chunk is read straight from the chunk-transposed h rows
// (coalesced).  Writes o[row][n].
template <int P, int W, int RW, bool ONE>
__global__ __launch_bounds__(W * 64) void down_f32_kernel(GemvArgs a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ue = blockIdx.y;
    if (ue < a.cap && ue >= a.n_union[0]) return;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    const int cnt = entry_info(a, ue, wb, sb, list);
    if (cnt <= 0) return;
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32;
    const auto rw = make_rsrc(wb, (uint32_t)(a.N * rb));
    const auto rs = make_rsrc(sb, (uint32_t)(a.N * sbs * 2));
    const int n0 = (blockIdx.x * W + wave) * RW;
    uint4 wv[RW][P];
    uint16_t sc[RW][P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const bool live = lane + 64 * p < C;
        const int c = live ? lane + 64 * p : C - 1;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            wv[r][p] = load16(rw, (uint32_t)(n0 + r) * rb + c * 16);
            sc[r][p] = live ? load2(rs, ((uint32_t)(n0 + r) * sbs + (c >> 1)) * 2) : (uint16_t)0;
        }
    }
    for (int t = 0; t < (ONE ? 1 : cnt); ++t) {
        int in_row, out_row;
        token_rows(a, list, t, in_row, out_row);
        const float4 *hrow = reinterpret_cast<const float4 *>(a.in + (size_t)in_row * K);
        if (!ONE) opaque_codes(wv);
        float racc[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) racc[r] = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = min(lane + 64 * p, C - 1);  // dead lanes have a zero scale
            float xv[32];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 v = hrow[q * C + c];
                xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y;
                xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int r = 0; r < RW; ++r)
                racc[r] = fmaf(chunk_dot16(wv[r][p], xv), f16_to_f32(sc[r][p]), racc[r]);
        }
        const float tot = reduce_scatter<RW>(racc, lane) * 0.0625f;
        constexpr int LPV = 64 / RW;
        if ((lane % LPV) == 0) a.out[(size_t)out_row * a.out_ld + n0 + lane / LPV] = tot;
    }
}

hipError_t launch_forward_f32(const LayerDev &L, const ForwardIO &io, hipStream_t st, Marks *mk)
{
    const int T = io.T;
    if (T <= 0) return hipSuccess;
    float *h = reinterpret_cast<float *>(io.ws + io.lay.h);
    float *o = reinterpret_cast<float *>(io.ws + io.lay.o);
    GemvArgs a{};
    a.union_ids = io.union_ids; a.offsets = io.offsets; a.slots = io.slots; a.n_union = io.n_union;
    a.T = T; a.k = L.k; a.cap = (int)io.lay.cap; a.n_shared = L.n_shared;
    a.I = L.I;
    const int entries = a.cap + a.n_shared;
    // gate/up + SwiGLU -> h (chunk-transposed rows)
    a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
    a.N = 2 * L.I; a.K = L.H; a.upe = L.I;
    a.in = io.x; a.in_by_slot = 0;
    a.out = h; a.out_ld = L.I;
    if (mk) mk->mark(st);
    {
        constexpr int W = 4, RW = 4;
        const int P = (L.H / 32 + 63) / 64;
        int nt = 65536 / (L.H * 4);  // staged token rows must fit 64 KB of LDS
        nt = T < nt ? T : nt;
        nt = nt >= 2 ? 2 : 1;
        const dim3 grid(L.I / (W * RW / 2), entries), block(W * 64);
        const size_t lds = (size_t)nt * L.H * 4;
        const bool one = T == 1;
#define COLI_GU(NT_, P_) \
        if (nt == NT_ && P == P_) { \
            if (one) hipLaunchKernelGGL((gateup_f32_kernel<NT_, P_, W, RW, true>), grid, block, lds, st, a); \
            else hipLaunchKernelGGL((gateup_f32_kernel<NT_, P_, W, RW, false>), grid, block, lds, st, a); }
        COLI_GU(1, 1) COLI_GU(1, 2) COLI_GU(1, 3) COLI_GU(1, 4)
        COLI_GU(2, 1) COLI_GU(2, 2) COLI_GU(2, 3) COLI_GU(2, 4)
#undef COLI_GU
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // down -> o[row][n]
    a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
    a.N = L.H; a.K = L.I; a.upe = L.H;
    a.in = h; a.in_by_slot = 1;
    a.out = o; a.out_ld = L.H;
    if (mk) mk->mark(st);
    {
        constexpr int W = 4, RW = 8;
        const int P = (L.I / 32 + 63) / 64;
        const dim3 grid(L.H / (W * RW), entries), block(W * 64);
        const bool one = T == 1;
#define COLI_DN(P_) \
        if (P == P_) { \
            if (one) hipLaunchKernelGGL((down_f32_kernel<P_, W, RW, true>), grid, block, 0, st, a); \
            else hipLaunchKernelGGL((down_f32_kernel<P_, W, RW, false>), grid, block, 0, st, a); }
        COLI_DN(1) COLI_DN(2) COLI_DN(3) COLI_DN(4)
#undef COLI_DN
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (mk) mk->mark(st);
    hipError_t err = launch_combine(o, io.w, T, L.k, L.H, L.n_shared, io.y, st);
    if (mk) mk->mark(st);
    return err;
}

}  // namespace coli
