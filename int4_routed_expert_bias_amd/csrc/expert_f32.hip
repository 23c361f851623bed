// expert_f32.hip -- the fp32 arithmetic family of the expert FFN
// ("Colibri 完全ガイド", walk-through "詳細解説" step 3: single-token decode
// computes in f32).  Weights are int4 with one fp16 scale per row per
// 64-group ("colibri: 744B MoE...", section "はじめにとソースが語らないこと":
// the gs64 build).
//
// The matmuls stream every union expert's packed weights once from HBM (a
// GEMV at decode, a few tokens for a verify batch).  On CDNA4 the dequantise
// and multiply work is the VALU bottleneck of this stream, so the chunk
// arithmetic uses only full-rate vector ops:
//  - a lane owns 16-byte chunks (32 codes) of a row, lane l chunk l + 64 p,
//    so one wave instruction reads 1 KB of a row;
//  - a packed dword q of 8 codes gives the biased codes n = code + 8 in
//    [0, 15] of its even elements as the bytes of (q ^ 0x88888888) &
//    0x0F0F0F0F and of its odd elements as the bytes of ((q >> 4) ^
//    0x08080808) & 0x0F0F0F0F (one v_bitop3_b32 each, plus one shift);
//  - v_cvt_pk_f32_fp8 turns two such bytes into fp32 at once (the gate/up
//    streaming kernels; the others convert one byte at a time and run the
//    same chains in units of 1, with bitwise the same results): read as OCP
//    E4M3 numbers, the bytes 0..15 are exactly n * 2^-9 (the exponent-0
//    values are the subnormals), so the chains run in units of 2^-9;
//    v_fmac_f32 accumulates them times x and the chunk sum starts at -K,
//    K = 8 sum(x) 2^-9, which removes the bias: sum (code + 8) x - 8 sum x =
//    sum code * x, times 2^-9, up to fp32 rounding (every product is exact;
//    for integer x and power-of-two scales the whole sum is exact);
//  - one fp16 group scale per chunk, times 2^9, applied with one more FMA.
//    Scaling by powers of two commutes with rounding, so every chain value
//    is exactly 2^-9 times the value of the same chain over the integer
//    codes, and the scaled product equals the unscaled one;
//  - lane partials are combined with permlane swaps and DPP (reduce_values),
//    one fixed pairing sequence for every value, so the sum of a given
//    (token, row) does not depend on how many values a wave reduces.
// A token's arithmetic is the same whatever the batch and whichever kernel
// variant runs it: a token alone and inside a batch give identical bits.
#include "common.h"
#include "stream.h"
#include "route_tokens.h"

#include <algorithm>

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
    uint64_t *tl;          // timeline marks (measurement only; null: none)
    int tl_cap;
};

// U9 selects the units of a kernel's chains: 2^-9 (codes converted in pairs
// by v_cvt_pk_f32_fp8) or 1 (one v_cvt_f32_ubyte per code).  Both give
// bitwise the same results; the gate/up streaming kernels, where the
// conversions are the VALU bottleneck, use 2^-9, the others (more registers
// per code) units of 1.

// K of an activation chunk: 8 sum(v) in the chain units, the sum in
// ascending element order (the scaling is exact).
template <bool U9 = false>
__device__ __forceinline__ float chunk_K(const float (&v)[32])
{
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += v[i];
    return U9 ? 0.015625f * sum : 8.f * sum;
}

// A weight group scale in the inverse chain units.
template <bool U9 = false>
__device__ __forceinline__ float wscale(uint16_t h)
{
    return U9 ? f16_to_f32(h) * 512.0f : f16_to_f32(h);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &w, int d)
{
    return d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w;
}

// Byte b of v as fp32 (one v_cvt_f32_ubyte{b}): chain units of 1.
__device__ __forceinline__ float byte_f32(uint32_t v, int b)
{
    return (float)((v >> (8 * b)) & 0xFFu);
}

// The four bytes n of v (each in [0, 15]) as n * 2^-9: two
// v_cvt_pk_f32_fp8 (chain units of 2^-9).
template <bool U9>
__device__ __forceinline__ void byte_vals(uint32_t v, float (&f)[4])
{
    static_assert(U9, "the pair conversion gives units of 2^-9");
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
}

// out[r][c] = sum_i code_i * x_i over 16-byte chunk w[r][c] of packed codes
// and activation chunk x[c] (see the file comment): every chain starts at
// -K[c] and adds its 32 products in ascending element order.  The NR * NC
// chains are interleaved so that no product waits on the previous one of
// its own chain.
template <int NR, int NC, bool U9 = false>
__device__ __forceinline__ void chunk_dots(const uint4 (&w)[NR][NC], const float (&x)[NC][32],
                                           const float (&K)[NC], float (&out)[NR][NC])
{
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) out[r][c] = -K[c];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (U9) {
            float lo[NR][NC][4], hi[NR][NC][4];
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint32_t q = word_of(w[r][c], d);
                    byte_vals<true>((q ^ 0x88888888u) & 0x0F0F0F0Fu, lo[r][c]);         // even elements
                    byte_vals<true>(((q >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu, hi[r][c]);  // odd elements
                }
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        out[r][c] = fmaf(lo[r][c][b], x[c][8 * d + 2 * b], out[r][c]);
                        out[r][c] = fmaf(hi[r][c][b], x[c][8 * d + 2 * b + 1], out[r][c]);
                    }
        } else {
            uint32_t lo[NR][NC], hi[NR][NC];
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint32_t q = word_of(w[r][c], d);
                    lo[r][c] = (q ^ 0x88888888u) & 0x0F0F0F0Fu;         // even elements
                    hi[r][c] = ((q >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;  // odd elements
                }
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        out[r][c] = fmaf(byte_f32(lo[r][c], b), x[c][8 * d + 2 * b], out[r][c]);
                        out[r][c] = fmaf(byte_f32(hi[r][c], b), x[c][8 * d + 2 * b + 1], out[r][c]);
                    }
        }
    }
}

// ---------------------------------------------------------------------------
// Cross-lane reduction.  reduce_values<V> sums each of V per-lane values over
// the 64 lanes with one fixed pairing sequence: lane bit 5 (v_permlane32_swap),
// bit 4 (v_permlane16_swap), then DPP row_ror:8 (bit 3), row_half_mirror
// (lanes l and 7 - l), quad_perm xor 2 and xor 1.  The two swap levels also
// halve the value count (lanes with the bit set keep the upper half of the
// values), the DPP levels reduce the n = V / 4 (at least 1) values left in
// every lane.  The partial sums of a value meet in the same pairs whatever
// V is, so a (token, row) sum does not depend on how many values a wave
// reduces.  On return v[j], j < reduced_count(V), holds the total of value
// reduced_value(V, j, lane) in every lane.
__device__ __forceinline__ void swap32(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                   false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap16(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                   false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

constexpr int reduced_count(int V) { return V >= 4 ? V / 4 : 1; }

template <int V>
__device__ __forceinline__ int reduced_value(int j, int lane)
{
    const int b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1;
    if (V >= 4) return j + (V / 4) * (b4 + 2 * b5);
    if (V == 2) return b5;
    return 0;
}

template <int V>
__device__ __forceinline__ void reduce_values(float (&v)[V])
{
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    constexpr int N = reduced_count(V);
    if constexpr (V >= 2) {
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            float a = v[i], b = v[i + V / 2];
            swap32(a, b);
            v[i] = a + b;
        }
    } else {
        float a = v[0], b = v[0];
        swap32(a, b);
        v[0] = a + b;
    }
    if constexpr (V >= 4) {
#pragma unroll
        for (int i = 0; i < V / 4; ++i) {
            float a = v[i], b = v[i + V / 4];
            swap16(a, b);
            v[i] = a + b;
        }
    } else {
        float a = v[0], b = v[0];
        swap16(a, b);
        v[0] = a + b;
    }
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = dpp_add<0x128>(v[j]);  // row_ror:8
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = dpp_add<0x141>(v[j]);  // row_half_mirror
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = dpp_add<0x4E>(v[j]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = dpp_add<0xB1>(v[j]);   // quad_perm [1,0,3,2]
}

// The value held by lane l ^ 32 (a gate row's up partner sits V/2 values
// later, i.e. across lane bit 5).
__device__ __forceinline__ float across32(float v)
{
    float a = v, b = v;
    swap32(a, b);
    return (threadIdx.x & 32) ? a : b;
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
// hoists all the code-to-fp16 conversions out of the loop and keeps
// hundreds of values live, which collapses occupancy.  Emits no instruction.
template <int R, int P>
__device__ __forceinline__ void opaque_codes(uint4 (&w)[R][P])
{
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < P; ++p)
            asm volatile("" : "+v"(w[r][p].x), "+v"(w[r][p].y), "+v"(w[r][p].z), "+v"(w[r][p].w));
}

// SwiGLU: h = silu(g) * u = g / (1 + e^-g) * u (fp32).
__device__ __forceinline__ float swiglu(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// Lane that writes reduced value slot j (one lane per value).
template <int V>
__device__ __forceinline__ bool value_writer(int j, int lane)
{
    if (V >= 4) return (lane & 15) == j;
    if (V == 2) return (lane & 31) == 0;
    return lane == 0;
}

// Load an 8-float4 chunk row segment into 32 registers.
__device__ __forceinline__ void load_chunk32(const float4 *src, int stride4, float (&v)[32])
{
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 f = src[q * stride4];
        v[4 * q + 0] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
}

// Gate/up matmul + SwiGLU, any batch.  Grid: (I / (W * RW / 2), entries).
// Wave w of a workgroup owns RW/2 units (gate rows i and up rows I + i),
// keeps their P chunks per lane in registers for all of the entry's token
// batches, and stages each batch of NT token rows (plus the K of every
// chunk) in LDS.
template <int NT, int P, int W, int RW>
__global__ __launch_bounds__(W * 64) void gateup_f32_kernel(GemvArgs a)
{
    constexpr int V = RW * NT, N = reduced_count(V);
    // [NT][K] token rows chunk-transposed (token t, piece q of chunk c at
    // float4 (8 t + q) C + c: conflict-free wave reads), then [NT][K/32] chunk K
    extern __shared__ float xs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ue = blockIdx.y;
    if (ue < a.cap && ue >= a.n_union[0]) return;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    const int cnt = entry_info(a, ue, wb, sb, list);
    if (cnt <= 0) return;
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, K4 = K / 4;
    float *ks = xs + NT * K;
    const float4 *xt = reinterpret_cast<const float4 *>(xs);
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
    for (int t0 = 0; t0 < cnt; t0 += NT) {
        const int nt = min(NT, cnt - t0);
        int in_row[NT], out_row[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) token_rows(a, list, t0 + (tt < nt ? tt : 0), in_row[tt], out_row[tt]);
        if (t0 > 0) __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float4 *src = reinterpret_cast<const float4 *>(a.in + (size_t)in_row[tt] * K);
            float4 *dst = reinterpret_cast<float4 *>(xs);
            for (int i = threadIdx.x; i < K4; i += blockDim.x)
                dst[(8 * tt + (i & 7)) * C + (i >> 3)] = src[i];
        }
        __syncthreads();
        for (int j = threadIdx.x; j < nt * C; j += blockDim.x) {
            const int tt = j / C, c = j - tt * C;
            float v[32];
            load_chunk32(xt + 8 * tt * C + c, C, v);
            ks[tt * C + c] = chunk_K(v);
        }
        __syncthreads();
        float racc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) racc[i] = 0.f;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            opaque_codes(wv);  // convert per token: keeps registers low
            if (tt < nt) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int c = min(lane + 64 * p, C - 1);
                    float xv[1][32], kc[1];
                    load_chunk32(xt + 8 * tt * C + c, C, xv[0]);
                    kc[0] = ks[tt * C + c];
                    uint4 wl[RW][1];
#pragma unroll
                    for (int r = 0; r < RW; ++r) wl[r][0] = wv[r][p];
                    float dots[RW][1];
                    chunk_dots<RW, 1>(wl, xv, kc, dots);
#pragma unroll
                    for (int r = 0; r < RW; ++r)
                        racc[r * NT + tt] = fmaf(dots[r][0], wscale(sc[r][p]), racc[r * NT + tt]);
                }
            }
        }
        // value v = r * NT + tt; the up row of unit r sits V/2 values later
        reduce_values<V>(racc);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float up = across32(racc[j]);
            const int vi = reduced_value<V>(j, lane);
            const int r = vi / NT, tt = vi % NT;
            if (value_writer<V>(j, lane) && r < RW / 2 && tt < nt)
                a.out[(size_t)out_row[tt] * a.out_ld + ht_pos(rows[r], CI)] =
                    swiglu(racc[j], up);
        }
    }
}

// Down matmul, any batch.  Grid: (H / (W * RW), entries).  Wave w owns RW
// consecutive rows (P chunks per lane in registers) and walks the entry's
// tokens; each token's h chunk is read straight from the chunk-transposed
// h rows (coalesced).  Writes o[row][n].
template <int P, int W, int RW>
__global__ __launch_bounds__(W * 64) void down_f32_kernel(GemvArgs a)
{
    constexpr int V = RW, N = reduced_count(V);
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
    for (int t = 0; t < cnt; ++t) {
        int in_row, out_row;
        token_rows(a, list, t, in_row, out_row);
        const float4 *hrow = reinterpret_cast<const float4 *>(a.in + (size_t)in_row * K);
        opaque_codes(wv);
        float racc[V];
#pragma unroll
        for (int r = 0; r < RW; ++r) racc[r] = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = min(lane + 64 * p, C - 1);  // dead lanes have a zero scale
            float xv[1][32], kc[1];
            load_chunk32(hrow + c, C, xv[0]);
            kc[0] = chunk_K(xv[0]);
            uint4 wl[RW][1];
#pragma unroll
            for (int r = 0; r < RW; ++r) wl[r][0] = wv[r][p];
            float dots[RW][1];
            chunk_dots<RW, 1>(wl, xv, kc, dots);
#pragma unroll
            for (int r = 0; r < RW; ++r) racc[r] = fmaf(dots[r][0], wscale(sc[r][p]), racc[r]);
        }
        reduce_values<V>(racc);
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (value_writer<V>(j, lane))
                a.out[(size_t)out_row * a.out_ld + n0 + reduced_value<V>(j, lane)] = racc[j];
    }
}

// ---------------------------------------------------------------------------
// Single-token streaming path (T == 1, the decode step).
//
// A decode step reads every union expert's weights exactly once and has no
// reuse to exploit, so the kernels are built as HBM streams: a fixed grid of
// persistent waves (a few per SIMD), each walking a contiguous share of one
// entry's weight rows through a DEPTH-stage register ring.  The loads of
// stage s + DEPTH are issued as soon as stage s has been consumed, so the
// dequantising FMAs of one stage overlap the HBM latency of the next ones
// inside every wave; the partial sums of M stages are reduced together.
//
// Stage loads: a row's chunk p of lane l sits at voffset (l + 64 p) * 16
// (precomputed per lane) plus the row's byte offset in the scalar soffset,
// so a stage costs no vector address arithmetic.  Every load is issued
// unconditionally (branches around loads make the compiler's wait-count
// analysis fall back to waiting for everything in flight): lanes past the
// row's last chunk get a voffset beyond the buffer, and stages past the end
// of a wave's work use a zero-size buffer resource; both read 0 without
// touching memory.
// Entry ue of the compact entry list (union experts in union order, then the
// shared expert): weight and scale bases and the output row of its token.
__device__ __forceinline__ void t1_entry(const GemvArgs &a, int ue, int U, const uint8_t *&wb,
                                         const uint16_t *&sb, int &out_row)
{
    if (ue < U) {
        const int e = a.union_ids[ue];
        wb = a.w + (size_t)e * a.N * (a.K / 2);
        sb = a.s + (size_t)e * a.N * (a.K / 64);
        out_row = a.slots[a.offsets[ue]];
    } else {
        wb = a.sh_w;
        sb = a.sh_s;
        out_row = a.T * a.k;
    }
}

// Gate/up + SwiGLU for one token.  Unit (row block) = NP gate rows i and
// their up rows I + i.  Each lane reads the x chunks it needs once (staged
// through LDS) and keeps them in registers (XREG) or re-reads them from LDS
// every stage.  h is written chunk-transposed.
// ROUTE: the token routes itself.  Every workgroup first runs the router's
// top-k selection and batch union (route_tokens, the code of the top-k
// kernel) on the token's sigmoid scores, into LDS, and streams its share of
// the selected experts from there; workgroup 0 also writes the selection and
// the union to global memory (for the down kernel and the caller).  The
// selection costs each workgroup a few microseconds before its first weight
// load, against a whole launch of the top-k kernel.  E <= 256.
template <int P, int NP, int M, int DEPTH, bool XREG, bool ROUTE, bool TL = false>
__global__ __launch_bounds__(256) void gateup_t1_kernel(GemvArgs a, RouteSelf r)
{
    static_assert(M % DEPTH == 0, "stage ring must divide the reduction batch");
    constexpr int V = next_pow2(2 * NP * M), N = reduced_count(V);
    static_assert(V <= 64, "at most 64 values per reduction");
    // x chunk-transposed (piece q of chunk c at float4 q C + c: conflict-free
    // wave reads), then [K/32] chunk K
    extern __shared__ float xs[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, CI = a.I / 32;
    tl_mark<TL>(a.tl, a.tl_cap, 0);
    int U;
    // ROUTE: x is loaded into registers before the selection (its latency
    // overlaps the selection's) and staged to LDS after it
    constexpr int XPRE = ROUTE ? COLI_MAX_H_DEV / 4 / 256 : 1;
    uint4 xpre[XPRE];
    if constexpr (ROUTE) {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.in, (uint32_t)K * 4);
#pragma unroll
        for (int j = 0; j < XPRE; ++j) {
            const int i = (int)threadIdx.x + 256 * j;
            xpre[j] = load16(rx, i < K / 4 ? (uint32_t)i * 16 : kOOB);
        }
    }
    if constexpr (ROUTE) {
        __shared__ RouteLds rl;
        route_self<TL>(r, rl, a.tl, a.tl_cap);
        const int nu = rl.n[0];
        a.union_ids = rl.u;
        a.offsets = rl.off;
        a.slots = rl.sl;
        a.n_union = rl.n;
        U = __builtin_amdgcn_readfirstlane(nu);
    } else {
        U = a.n_union[0];
    }
    tl_mark<TL>(a.tl, a.tl_cap, 1);
    const int upe = a.I / NP;
    const T1Split sp = t1_split(blockIdx.x * 4 + wave, gridDim.x * 4, U + a.n_shared, upe);
    const int nsteps = sp.nsteps;
    const uint8_t *wb;
    const uint16_t *sb;
    int orow;
    if constexpr (ROUTE) {
        // (the union is in LDS, read per lane: its values made uniform)
        if (sp.ue < U) {
            const int e = __builtin_amdgcn_readfirstlane(a.union_ids[sp.ue]);
            wb = a.w + (size_t)e * a.N * (a.K / 2);
            sb = a.s + (size_t)e * a.N * (a.K / 64);
            orow = __builtin_amdgcn_readfirstlane(a.slots[a.offsets[sp.ue]]);
        } else {
            wb = a.sh_w;
            sb = a.sh_s;
            orow = a.T * a.k;
        }
    } else {
        t1_entry(a, sp.ue, U, wb, sb, orow);
    }
    const StageRsrc R = stage_rsrc(wb, sb, a.N, rb, sbs);
    uint32_t vw[P], vs[P];
    lane_offsets<P>(lane, C, vw, vs);

    uint4 wv[DEPTH][2 * NP][P];
    uint16_t sv[DEPTH][2 * NP][P];
    auto issue = [&](int d, int step) {
        const int blk = sp.part + step * sp.wpe;
        int rows[2 * NP];
#pragma unroll
        for (int r = 0; r < NP; ++r) {
            rows[r] = blk * NP + r;
            rows[NP + r] = a.I + blk * NP + r;
        }
        load_stage<2 * NP, P>(R, rows, step < nsteps, rb, sbs, vw, vs, wv[d], sv[d]);
    };
    // the first stages go out before x is staged: one memory latency, not two
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, d);
    float *ks = xs + K;
    const float4 *xt = reinterpret_cast<const float4 *>(xs);
    {
        const float4 *src = reinterpret_cast<const float4 *>(a.in);
        float4 *dst = reinterpret_cast<float4 *>(xs);
        if constexpr (ROUTE) {
#pragma unroll
            for (int jj = 0; jj < XPRE; ++jj) {
                const int i = (int)threadIdx.x + 256 * jj;
                if (i < K / 4)
                    dst[(i & 7) * C + (i >> 3)] = make_float4(
                        __uint_as_float(xpre[jj].x), __uint_as_float(xpre[jj].y),
                        __uint_as_float(xpre[jj].z), __uint_as_float(xpre[jj].w));
            }
        } else {
            for (int i = threadIdx.x; i < K / 4; i += blockDim.x) dst[(i & 7) * C + (i >> 3)] = src[i];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < C; c += blockDim.x) {
            float v[32];
            load_chunk32(xt + c, C, v);
            ks[c] = chunk_K<true>(v);
        }
        __syncthreads();
    }
    tl_mark<TL>(a.tl, a.tl_cap, 2);
    if (nsteps == 0) {
        tl_mark<TL>(a.tl, a.tl_cap, 7);
        return;
    }
    float *hrow = a.out + (size_t)orow * a.out_ld;
    float xr[XREG ? P : 1][32], kx[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int c = min(lane + 64 * p, C - 1);  // dead lanes: scale 0
        if constexpr (XREG) load_chunk32(xt + c, C, xr[p]);
        kx[p] = ks[c];
    }

    for (int g0 = 0; g0 < nsteps; g0 += M) {
        float racc[V];  // [gate, up][m][NP], zero padded to a power of two
#pragma unroll
        for (int i = 0; i < V; ++i) racc[i] = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
                float dots[2 * NP][P];
                if constexpr (XREG) {
                    chunk_dots<2 * NP, P, true>(wv[d], xr, kx, dots);
                } else {
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        float xl[1][32], kl[1] = {kx[p]};
                        load_chunk32(xt + min(lane + 64 * p, C - 1), C, xl[0]);
                        uint4 wl[2 * NP][1];
                        float dl[2 * NP][1];
#pragma unroll
                        for (int r = 0; r < 2 * NP; ++r) wl[r][0] = wv[d][r][p];
                        chunk_dots<2 * NP, 1, true>(wl, xl, kl, dl);
#pragma unroll
                        for (int r = 0; r < 2 * NP; ++r) dots[r][p] = dl[r][0];
                    }
                }
#pragma unroll
                for (int r = 0; r < 2 * NP; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int p = 0; p < P; ++p) acc = fmaf(dots[r][p], wscale<true>(sv[d][r][p]), acc);
                    racc[(r / NP) * (V / 2) + m * NP + r % NP] = acc;
                }
            }
            issue(d, g0 + m + DEPTH);
        }
        reduce_values<V>(racc);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float up = across32(racc[j]);
            const int vi = reduced_value<V>(j, lane);
            const int m = vi / NP, i = (sp.part + (g0 + m) * sp.wpe) * NP + vi % NP;
            if (value_writer<V>(j, lane) && vi < NP * M && g0 + m < nsteps)
                hrow[ht_pos(i, CI)] = swiglu(racc[j], up);
        }
        if (g0 == 0) tl_mark<TL>(a.tl, a.tl_cap, 3);
    }
    tl_mark<TL>(a.tl, a.tl_cap, 7);
}

// Rows of one workgroup of the fused down + combine (at most), and its
// waves (at most): a top-8 selection plus the shared expert, one wave each.
constexpr int kDownRowsMax = 64;
constexpr int kDownT1cWaves = 9;

// Down projection for one token.  Unit (row block) = RD rows of one entry.
// A wave loads its entry's h chunk once and keeps it in registers
// while it streams its row blocks (those of sp).  Each output value is also
// stored to so[out row][local index] when so is given (the fused combine).
template <int P, int RD, int M, int DEPTH>
__device__ __forceinline__ void down_t1_rows(const GemvArgs &a, const T1Split &sp, int U, int lane,
                                             float (*so)[kDownRowsMax])
{
    static_assert(M % DEPTH == 0, "stage ring must divide the reduction batch");
    constexpr int V = next_pow2(RD * M), N = reduced_count(V);
    static_assert(V <= 64, "at most 64 values per reduction");
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32;
    const int nsteps = sp.nsteps;
    const uint8_t *wb;
    const uint16_t *sb;
    int orow;
    t1_entry(a, sp.ue, U, wb, sb, orow);
    const StageRsrc R = stage_rsrc(wb, sb, a.N, rb, sbs);
    uint32_t vw[P], vs[P];
    lane_offsets<P>(lane, C, vw, vs);

    // this lane's h chunks (chunk-transposed rows: piece q of chunk
    // c at q*C + c), loaded before the weight ring so the first wait covers them
    float hv[P][32], kh[P];
    {
        const float4 *hrow = reinterpret_cast<const float4 *>(a.in + (size_t)orow * K);
#pragma unroll
        for (int p = 0; p < P; ++p) load_chunk32(hrow + min(lane + 64 * p, C - 1), C, hv[p]);
    }
    uint4 wv[DEPTH][RD][P];
    uint16_t sv[DEPTH][RD][P];
    auto issue = [&](int d, int step) {
        int rows[RD];
#pragma unroll
        for (int r = 0; r < RD; ++r) rows[r] = (sp.part + step * sp.wpe) * RD + r;
        load_stage<RD, P>(R, rows, step < nsteps, rb, sbs, vw, vs, wv[d], sv[d]);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, d);
#pragma unroll
    for (int p = 0; p < P; ++p) kh[p] = chunk_K(hv[p]);
    float *orow_p = a.out + (size_t)orow * a.out_ld;
    for (int g0 = 0; g0 < nsteps; g0 += M) {
        float racc[V];  // [m][RD], zero padded to a power of two
#pragma unroll
        for (int i = 0; i < V; ++i) racc[i] = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
                float dots[RD][P];
                chunk_dots<RD, P>(wv[d], hv, kh, dots);
#pragma unroll
                for (int r = 0; r < RD; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int p = 0; p < P; ++p) acc = fmaf(dots[r][p], wscale(sv[d][r][p]), acc);
                    racc[m * RD + r] = acc;
                }
            }
            issue(d, g0 + m + DEPTH);
        }
        reduce_values<V>(racc);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int vi = reduced_value<V>(j, lane), m = vi / RD;
            if (value_writer<V>(j, lane) && vi < RD * M && g0 + m < nsteps) {
                orow_p[(sp.part + (g0 + m) * sp.wpe) * RD + vi % RD] = racc[j];
                if (so) so[orow][(g0 + m) * RD + vi % RD] = racc[j];
            }
        }
    }
}

template <int P, int RD, int M, int DEPTH>
__global__ __launch_bounds__(256) void down_t1_kernel(GemvArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int U = a.n_union[0];
    const T1Split sp = t1_split(blockIdx.x * 4 + wave, gridDim.x * 4, U + a.n_shared, a.N / RD);
    if (sp.nsteps == 0) return;
    down_t1_rows<P, RD, M, DEPTH>(a, sp, U, lane, nullptr);
}

// Down projection and combine for one token in one launch.  Workgroup g
// owns row blocks g, g + G, g + 2G, ... (G workgroups, at most
// kDownRowsMax / RD blocks each) of EVERY entry: wave v computes entries
// v, v + NW, ... (NW waves) for those rows and leaves the values in LDS as
// well; after a barrier the workgroup forms y of its rows with exactly the
// combine's arithmetic (slots in order, fp32 fma chain, dropped slots
// skipped, then the shared expert added), so y is bitwise that of the
// two-launch form.
template <int P, int RD, int M, int DEPTH, bool TL = false>
// (one chunk per lane: registers for five waves per SIMD, two workgroups per
// CU -- 16.4 us against 17.5 with four waves per SIMD; wider rows keep the
// registers they need)
__global__ __launch_bounds__(64 * kDownT1cWaves, P == 1 ? 5 : 1) void down_t1c_kernel(GemvArgs a, const int32_t *__restrict__ ids,
                                                        const float *__restrict__ w,
                                                        float *__restrict__ y)
{
    __shared__ float so[COLI_MAX_K_DEV + 1][kDownRowsMax];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int NW = blockDim.x >> 6;
    tl_mark<TL>(a.tl, a.tl_cap, 0);
    const int U = a.n_union[0];
    const int nblocks = a.N / RD, G = gridDim.x, g = blockIdx.x;
    T1Split sp;
    sp.part = g;
    sp.wpe = G;
    sp.nsteps = g < nblocks ? (nblocks - g + G - 1) / G : 0;
    for (int ue = wave; ue < U + a.n_shared && sp.nsteps > 0; ue += NW) {
        sp.ue = ue;
        down_t1_rows<P, RD, M, DEPTH>(a, sp, U, lane, so);
        if (ue == wave) tl_mark<TL>(a.tl, a.tl_cap, 1);
    }
    tl_mark<TL>(a.tl, a.tl_cap, 2);
    __syncthreads();
    tl_mark<TL>(a.tl, a.tl_cap, 3);
    const int k = a.k, i = threadIdx.x;
    if (i < sp.nsteps * RD) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            if (ids[j] < 0) continue;
            acc = fmaf(w[j], so[j][i], acc);
        }
        if (a.n_shared) acc += so[k][i];
        y[(g + (i / RD) * G) * RD + i % RD] = acc;
    }
    tl_mark<TL>(a.tl, a.tl_cap, 7);
}

// Small batches (2 <= T <= kStreamTMax, the verify step): the same streams,
// each weight stage applied to every token of the wave's entry (at most
// NTOK: the shared expert takes all T).  x of the T tokens and their chunk
// constants sit in LDS (NTOK token rows do not fit in registers); the
// per-(token, row) arithmetic is the single-token one, value for value, so
// a token's h and o do not depend on its batch.
constexpr int kStreamTMax = 4;

// chunk_dots for CNT activation chunks at once: each code byte is converted
// once and used by every token.  out[r][j] is chain (row r, token j) with
// exactly the arithmetic of chunk_dots (start at -K[j], products in
// ascending element order).
template <int NR, int CNT, int NX, bool U9 = false>
__device__ __forceinline__ void chunk_dots_tok(const uint4 (&w)[NR], const float (&x)[NX][32],
                                               const float (&K)[NX], float (&out)[NR][NX])
{
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int j = 0; j < CNT; ++j) out[r][j] = -K[j];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t lw[NR], hw[NR];
        float lo[NR][4], hi[NR][4];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint32_t q = word_of(w[r], d);
            lw[r] = (q ^ 0x88888888u) & 0x0F0F0F0Fu;
            hw[r] = ((q >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;
            if constexpr (U9) {
                byte_vals<true>(lw[r], lo[r]);
                byte_vals<true>(hw[r], hi[r]);
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float fl = U9 ? lo[r][b] : byte_f32(lw[r], b);
                const float fh = U9 ? hi[r][b] : byte_f32(hw[r], b);
#pragma unroll
                for (int j = 0; j < CNT; ++j) {
                    out[r][j] = fmaf(fl, x[j][8 * d + 2 * b], out[r][j]);
                    out[r][j] = fmaf(fh, x[j][8 * d + 2 * b + 1], out[r][j]);
                }
            }
    }
}

// Work split of the small-batch streaming kernels.  A wave streaming one
// entry is bound by its load latency until its FMAs take longer, which a
// few tokens do: measured on the 4-token verify layer, a stage costs about
// (1 + tokens) / 2 single-token stages.  Entry e, of cost 1 + its token
// count, gets waves [B(e), B(e+1)) with
// B(e) = e + (GW - ne) * (cost of entries before e) / (total cost), so every
// entry has at least one wave.  Within an entry the row blocks go
// round-robin as in t1_split.
// UL: the union lists are in LDS (read per lane): the values read are made
// uniform explicitly.
template <bool UL = false>
__device__ __forceinline__ int rd_union(const int32_t *p, int i)
{
    if constexpr (UL) return __builtin_amdgcn_readfirstlane(p[i]);
    return p[i];
}

// Stage cost of an entry with tok tokens, in units of a quarter of a
// single-token stage: one wave up to two tokens, a wave pair (tokens split
// two and one or two and two) from three.  Measured on the 4-token verify
// layer: 1.2, ~1.8, ~2.2 and 2.56 us per stage for 1-4 tokens.
__device__ __forceinline__ int pair_stage_cost(int tok)
{
    return tok <= 1 ? 4 : tok == 2 ? 6 : tok == 3 ? 7 : 9;
}

template <bool UL = false, bool PAIRS = false>
__device__ __forceinline__ T1Split mt_split(const GemvArgs &a, int gw, int GW, int U,
                                            int nblocks)
{
    T1Split s{0, 0, 0, 0};
    const int ne = U + a.n_shared;
    if (ne <= 0 || GW < ne) return s;
    // one entry per lane (64 at a time): its cost, the exclusive prefix of
    // the costs by a wave scan, its wave range; the wave's entry is the
    // lane whose range holds gw (32-bit: spare * total stays far below 2^31)
    const int lane = threadIdx.x & 63;
    const uint32_t spare = (uint32_t)(GW - ne);
    auto cost = [&](int e) {
        const int tok = e < U ? a.offsets[e + 1] - a.offsets[e] : a.T;
        return PAIRS ? pair_stage_cost(tok) : 1 + tok;
    };
    uint32_t total = 0;
    for (int base = 0; base < ne; base += 64) {
        int c = base + lane < ne ? cost(base + lane) : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
        total += (uint32_t)c;
    }
    int before = 0;
    for (int base = 0; base < ne; base += 64) {
        const int e = base + lane;
        const int cnt = e < ne ? cost(e) : 0;
        int inc = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off, 64);
            if (lane >= off) inc += o;
        }
        const uint32_t bef = (uint32_t)(before + inc - cnt);
        const int b0 = e + (int)(spare * bef / total);
        const int b1 = e + 1 + (int)(spare * (bef + (uint32_t)cnt) / total);
        const uint64_t hit = __ballot(e < ne && gw >= b0 && gw < b1);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            const int b0l = __builtin_amdgcn_readlane(b0, l), b1l = __builtin_amdgcn_readlane(b1, l);
            s.ue = base + l;
            s.part = gw - b0l;
            s.wpe = b1l - b0l;
            s.nsteps = s.part < nblocks ? (nblocks - s.part + s.wpe - 1) / s.wpe : 0;
            return s;
        }
        before += __builtin_amdgcn_readlane(inc, 63);
    }
    return s;
}

// ROUTE: the tokens route themselves first (route_self, as the
// single-token kernel), and the union is read from LDS.
// WPB = 8: wave pairs.  Waves w and w + 4 of a workgroup (one SIMD) stream
// the same row blocks of the same entry; an entry of three or four tokens
// splits them (w the even ones, w + 4 the odd ones), so the number of DRAM
// streams is that of four waves while two waves per SIMD share the VALU
// work (a wave alone issues a VALU instruction only about every other
// slot; the second wave's weight loads mostly hit the cache).  Entries of
// one or two tokens run on wave w alone (a pair was measured slower there:
// 2.17 us a stage against ~1.8).
template <int P, int M, int DEPTH, int NTOK, int WPB, bool ROUTE, bool TL = false>
__global__ __launch_bounds__(WPB * 64) void gateup_mt_kernel(GemvArgs a, RouteSelf r)
{
    static_assert(M % DEPTH == 0, "stage ring must divide the reduction batch");
    // route_self: one token per wave of the first four (T <= 4)
    static_assert(WPB == 4 || (WPB == 8 && NTOK == 4), "four waves, or four pairs of up to two tokens each");
    constexpr bool PAIRS = WPB == 8;
    constexpr int NW = PAIRS ? NTOK / 2 : NTOK;  // tokens per wave
    constexpr int V = next_pow2(2 * M * NW), N = reduced_count(V);
    static_assert(V <= 64, "at most 64 values per reduction");
    // x of the T tokens chunk-transposed (token t, piece q of chunk c at
    // float4 (8 t + q) C + c: the lanes of a wave read consecutive float4s,
    // free of bank conflicts), then [T][K/32] chunk K
    extern __shared__ float xs[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, CI = a.I / 32;
    tl_mark<TL>(a.tl, a.tl_cap, 0);
    // x of the batch: every load issued at once, before the selection (its
    // latency overlaps the selection's); staged to LDS after it
    constexpr int XPRE = (NTOK * (COLI_MAX_H_DEV / 4) + WPB * 64 - 1) / (WPB * 64);
    uint4 xpre[XPRE];
    {
        const int nx = a.T * (K / 4);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.in, (uint32_t)nx * 16);
#pragma unroll
        for (int j = 0; j < XPRE; ++j) {
            const int i = (int)threadIdx.x + WPB * 64 * j;
            xpre[j] = load16(rx, i < nx ? (uint32_t)i * 16 : kOOB);
        }
    }
    int U;
    if constexpr (ROUTE) {
        __shared__ RouteLds rl;
        route_self<TL>(r, rl, a.tl, a.tl_cap);
        a.union_ids = rl.u;
        a.offsets = rl.off;
        a.slots = rl.sl;
        a.n_union = rl.n;
        U = __builtin_amdgcn_readfirstlane(rl.n[0]);
    } else {
        U = a.n_union[0];
    }
    tl_mark<TL>(a.tl, a.tl_cap, 1);
    const int hh = PAIRS ? (wave >> 2) : 0;  // wave pair half: its tokens hh, hh + 2, ...
    const T1Split sp = mt_split<ROUTE, PAIRS>(a, blockIdx.x * 4 + (wave & 3), gridDim.x * 4, U, a.I);
    const int nsteps = sp.nsteps;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    int cnt;
    if constexpr (ROUTE) {
        if (sp.ue < U) {
            const int e = rd_union<true>(a.union_ids, sp.ue);
            wb = a.w + (size_t)e * a.N * (a.K / 2);
            sb = a.s + (size_t)e * a.N * (a.K / 64);
            const int o0 = rd_union<true>(a.offsets, sp.ue);
            list = a.slots + o0;
            cnt = rd_union<true>(a.offsets, sp.ue + 1) - o0;
        } else {
            wb = a.sh_w;
            sb = a.sh_s;
            list = nullptr;
            cnt = a.T;
        }
        cnt = min(cnt, NTOK);
    } else {
        cnt = min(entry_info(a, sp.ue, wb, sb, list), NTOK);
    }
    const StageRsrc R = stage_rsrc(wb, sb, a.N, rb, sbs);
    uint32_t vw[P], vs[P];
    lane_offsets<P>(lane, C, vw, vs);

    uint4 wv[DEPTH][2][P];
    uint16_t sv[DEPTH][2][P];
    auto issue = [&](int d, int step) {
        const int blk = sp.part + step * sp.wpe;
        const int rows[2] = {blk, a.I + blk};
        load_stage<2, P>(R, rows, step < nsteps, rb, sbs, vw, vs, wv[d], sv[d]);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, d);
    float *ks = xs + a.T * K;
    const float4 *xt = reinterpret_cast<const float4 *>(xs);
    {
        float4 *dst = reinterpret_cast<float4 *>(xs);
#pragma unroll
        for (int j = 0; j < XPRE; ++j) {
            const int i = (int)threadIdx.x + WPB * 64 * j;
            if (i < a.T * (K / 4)) {
                const int t = i / (K / 4), r = i - t * (K / 4), c = r >> 3, q = r & 7;
                dst[(8 * t + q) * C + c] = make_float4(__uint_as_float(xpre[j].x), __uint_as_float(xpre[j].y),
                                                       __uint_as_float(xpre[j].z), __uint_as_float(xpre[j].w));
            }
        }
        __syncthreads();
        for (int tc = threadIdx.x; tc < a.T * C; tc += blockDim.x) {
            const int t = tc / C, c = tc - t * C;
            float v[32];
            load_chunk32(xt + 8 * t * C + c, C, v);
            ks[tc] = chunk_K<true>(v);
        }
        __syncthreads();
    }
    tl_mark<TL>(a.tl, a.tl_cap, 2);
    // this wave's tokens: entry tokens hh + 2 j (a pair splitting three or
    // four) or j
    const bool split = PAIRS && cnt > 2;
    const int cntw = split ? (cnt - hh + 1) / 2 : hh == 0 ? cnt : 0;
    if (nsteps == 0 || cntw <= 0) {
        tl_mark<TL>(a.tl, a.tl_cap, 7);
        return;
    }
    int tok[NW], orow[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        int in_row = 0, out_row = 0;
        if (j < cntw) token_rows(a, list, split ? hh + 2 * j : j, in_row, out_row);
        tok[j] = in_row;
        orow[j] = out_row;
    }

    for (int g0 = 0; g0 < nsteps; g0 += M) {
        float racc[V];  // [gate, up][token][m], zero padded to a power of two
#pragma unroll
        for (int i = 0; i < V; ++i) racc[i] = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
                // per-lane sums over the P chunks (p ascending) for every token
                auto stage = [&](auto cnt_c) {
                    constexpr int CNT = decltype(cnt_c)::value;
                    float acc[2][NW];
#pragma unroll
                    for (int j = 0; j < CNT; ++j) acc[0][j] = acc[1][j] = 0.f;
                    if constexpr (CNT == 1 && !PAIRS) {
                        // one token: all P chunks at once, 2 * P interleaved chains
                        float xl[P][32], kl[P], dots[2][P];
#pragma unroll
                        for (int p = 0; p < P; ++p) {
                            const int c = min(lane + 64 * p, C - 1);
                            kl[p] = ks[tok[0] * C + c];
                            load_chunk32(xt + 8 * tok[0] * C + c, C, xl[p]);
                        }
                        chunk_dots<2, P, true>(wv[d], xl, kl, dots);
#pragma unroll
                        for (int p = 0; p < P; ++p) {
                            acc[0][0] = fmaf(dots[0][p], wscale<true>(sv[d][0][p]), acc[0][0]);
                            acc[1][0] = fmaf(dots[1][p], wscale<true>(sv[d][1][p]), acc[1][0]);
                        }
                    } else {
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        const int c = min(lane + 64 * p, C - 1);  // dead lanes: scale 0
                        float xl[NW][32], kl[NW];
#pragma unroll
                        for (int j = 0; j < CNT; ++j) {
                            kl[j] = ks[tok[j] * C + c];
                            load_chunk32(xt + 8 * tok[j] * C + c, C, xl[j]);
                        }
                        const uint4 wl[2] = {wv[d][0][p], wv[d][1][p]};
                        float dl[2][NW];
                        chunk_dots_tok<2, CNT, NW, true>(wl, xl, kl, dl);
                        const float s0 = wscale<true>(sv[d][0][p]), s1 = wscale<true>(sv[d][1][p]);
#pragma unroll
                        for (int j = 0; j < CNT; ++j) {
                            acc[0][j] = fmaf(dl[0][j], s0, acc[0][j]);
                            acc[1][j] = fmaf(dl[1][j], s1, acc[1][j]);
                        }
                    }
                    }
#pragma unroll
                    for (int j = 0; j < CNT; ++j) {
                        racc[j * M + m] = acc[0][j];
                        racc[V / 2 + j * M + m] = acc[1][j];
                    }
                };
                dispatch_count<NW>(cntw, stage);
            }
            issue(d, g0 + m + DEPTH);
        }
        reduce_values<V>(racc);
#pragma unroll
        for (int jj = 0; jj < N; ++jj) {
            const float up = across32(racc[jj]);
            const int vi = reduced_value<V>(jj, lane);
            const int j = vi / M, m = vi % M;
            const int i = sp.part + (g0 + m) * sp.wpe;
            if (value_writer<V>(jj, lane) && vi < NW * M && j < cntw && g0 + m < nsteps)
                a.out[(size_t)orow[j] * a.out_ld + ht_pos(i, CI)] = swiglu(racc[jj], up);
        }
        if (g0 == 0) tl_mark<TL>(a.tl, a.tl_cap, 3);
    }
    tl_mark<TL>(a.tl, a.tl_cap, 7);
}

template <int P, int RD, int M, int DEPTH, int NTOK, bool TL = false>
__global__ __launch_bounds__(256) void down_mt_kernel(GemvArgs a)
{
    static_assert(M % DEPTH == 0, "stage ring must divide the reduction batch");
    constexpr int V = next_pow2(RD * M * NTOK), N = reduced_count(V);
    static_assert(V <= 64, "at most 64 values per reduction");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32;
    tl_mark<TL>(a.tl, a.tl_cap, 0);
    const int U = a.n_union[0];
    const T1Split sp = mt_split(a, blockIdx.x * 4 + wave, gridDim.x * 4, U, a.N / RD);
    const int nsteps = sp.nsteps;
    if (nsteps == 0) {
        tl_mark<TL>(a.tl, a.tl_cap, 7);
        return;
    }
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    const int cnt = min(entry_info(a, sp.ue, wb, sb, list), NTOK);
    if (cnt <= 0) {
        tl_mark<TL>(a.tl, a.tl_cap, 7);
        return;
    }
    const StageRsrc R = stage_rsrc(wb, sb, a.N, rb, sbs);
    uint32_t vw[P], vs[P];
    lane_offsets<P>(lane, C, vw, vs);

    // the h chunks of the entry's tokens (chunk-transposed rows), in registers
    float hv[NTOK][P][32], kh[NTOK][P];
    int orow[NTOK];
#pragma unroll
    for (int j = 0; j < NTOK; ++j) {
        int in_row = 0, out_row = 0;
        if (j < cnt) token_rows(a, list, j, in_row, out_row);
        orow[j] = out_row;
        const float4 *hrow = reinterpret_cast<const float4 *>(a.in + (size_t)in_row * K);
#pragma unroll
        for (int p = 0; p < P; ++p) load_chunk32(hrow + min(lane + 64 * p, C - 1), C, hv[j][p]);
    }
    uint4 wv[DEPTH][RD][P];
    uint16_t sv[DEPTH][RD][P];
    auto issue = [&](int d, int step) {
        int rows[RD];
#pragma unroll
        for (int r = 0; r < RD; ++r) rows[r] = (sp.part + step * sp.wpe) * RD + r;
        load_stage<RD, P>(R, rows, step < nsteps, rb, sbs, vw, vs, wv[d], sv[d]);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, d);
#pragma unroll
    for (int j = 0; j < NTOK; ++j)
#pragma unroll
        for (int p = 0; p < P; ++p) kh[j][p] = chunk_K(hv[j][p]);
    for (int g0 = 0; g0 < nsteps; g0 += M) {
        float racc[V];  // [token][m][RD], zero padded to a power of two
#pragma unroll
        for (int i = 0; i < V; ++i) racc[i] = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
                auto stage = [&](auto cnt_c) {
                    constexpr int CNT = decltype(cnt_c)::value;
                    float acc[RD][NTOK];
#pragma unroll
                    for (int r = 0; r < RD; ++r)
#pragma unroll
                        for (int j = 0; j < CNT; ++j) acc[r][j] = 0.f;
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        float xl[NTOK][32], kl[NTOK];
#pragma unroll
                        for (int j = 0; j < CNT; ++j) {
                            kl[j] = kh[j][p];
#pragma unroll
                            for (int i = 0; i < 32; ++i) xl[j][i] = hv[j][p][i];
                        }
                        uint4 wl[RD];
#pragma unroll
                        for (int r = 0; r < RD; ++r) wl[r] = wv[d][r][p];
                        float dl[RD][NTOK];
                        chunk_dots_tok<RD, CNT, NTOK>(wl, xl, kl, dl);
#pragma unroll
                        for (int r = 0; r < RD; ++r) {
                            const float sc = wscale(sv[d][r][p]);
#pragma unroll
                            for (int j = 0; j < CNT; ++j) acc[r][j] = fmaf(dl[r][j], sc, acc[r][j]);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < RD; ++r)
#pragma unroll
                        for (int j = 0; j < CNT; ++j) racc[(j * M + m) * RD + r] = acc[r][j];
                };
                dispatch_count<NTOK>(cnt, stage);
            }
            issue(d, g0 + m + DEPTH);
        }
        reduce_values<V>(racc);
#pragma unroll
        for (int jj = 0; jj < N; ++jj) {
            const int vi = reduced_value<V>(jj, lane);
            const int j = vi / (M * RD), m = (vi / RD) % M, r = vi % RD;
            if (value_writer<V>(jj, lane) && vi < NTOK * M * RD && j < cnt && g0 + m < nsteps)
                a.out[(size_t)orow[j] * a.out_ld + (sp.part + (g0 + m) * sp.wpe) * RD + r] =
                    racc[jj];
        }
    }
    tl_mark<TL>(a.tl, a.tl_cap, 7);
}

// Workgroups of a kernel resident on one CU at once (at least 1).
template <typename Kern>
static int resident_per_cu(Kern kernel, int block)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

template <int NTOK>
static hipError_t launch_f32_mt(const LayerDev &L, const ForwardIO &io, GemvArgs a, float *h,
                                float *o, hipStream_t st, Marks *mk, const RouteSelf *rt = nullptr)
{
    const int entries = a.cap + a.n_shared;
    const int cus = device_cu_count();
    a.tl_cap = mk ? mk->tl_cap : 0;
    {
        a.tl = mk ? mk->tl_next() : nullptr;
        // one workgroup per CU: four streams (eight streaming waves measured
        // slower: more concurrent streams lose DRAM locality), each run by
        // a wave pair that splits the tokens; reductions over M = 2 stages
        // (M = 4 measured 6% slower: twice the code per token count and
        // more live registers)
        constexpr int M = 2, DEPTH = 2, WPB = NTOK == 4 ? 8 : 4;
        a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
        a.N = 2 * L.I; a.K = L.H; a.upe = L.I;
        a.in = io.x; a.in_by_slot = 0;
        a.out = h; a.out_ld = L.I;
        const int P = (L.H / 32 + 63) / 64;
        const dim3 grid(std::max(cus, (entries + 3) / 4)), block(WPB * 64);
        const size_t lds = (size_t)io.T * (L.H + L.H / 32) * 4;
#define COLI_GUM(P_) \
        if (P == P_) { \
            if (rt && a.tl) launch(mk, (gateup_mt_kernel<P_, M, DEPTH, NTOK, WPB, true, true>), grid, block, lds, st, a, *rt); \
            else if (rt) launch(mk, (gateup_mt_kernel<P_, M, DEPTH, NTOK, WPB, true>), grid, block, lds, st, a, *rt); \
            else launch(mk, (gateup_mt_kernel<P_, M, DEPTH, NTOK, WPB, false>), grid, block, lds, st, a, \
                        RouteSelf{}); \
        }
        COLI_GUM(1) COLI_GUM(2) COLI_GUM(3) COLI_GUM(4)
#undef COLI_GUM
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        constexpr int RD = 4, M = (NTOK >= 4 ? 2 : 4), DEPTH = 2;
        a.tl = mk ? mk->tl_next() : nullptr;
        a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
        a.N = L.H; a.K = L.I; a.upe = L.H;
        a.in = h; a.in_by_slot = 1;
        a.out = o; a.out_ld = L.H;
        const int P = (L.I / 32 + 63) / 64;
        // as many workgroups as the CUs hold at once (its registers allow
        // two per CU at the benchmark's shape): a second round of
        // workgroups would start only as the first ones finish
#define COLI_DNM(P_) \
        if (P == P_) { \
            static const int occ = resident_per_cu(down_mt_kernel<P_, RD, M, DEPTH, NTOK>, 256); \
            const dim3 grid(std::max(occ * cus, (entries + 3) / 4)), block(256); \
            if (a.tl) launch(mk, (down_mt_kernel<P_, RD, M, DEPTH, NTOK, true>), grid, block, 0, st, a); \
            else launch(mk, (down_mt_kernel<P_, RD, M, DEPTH, NTOK>), grid, block, 0, st, a); \
        }
        COLI_DNM(1) COLI_DNM(2) COLI_DNM(3) COLI_DNM(4)
#undef COLI_DNM
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t err = io.combine
        ? launch_combine(o, io.ids, io.w, io.T, L.k, L.H, L.n_shared, io.y, st, mk)
        : hipSuccess;
    return err;
}

// Workgroups of NW waves of the fused down + combine kernel (variant P)
// resident on one CU at once (at least 1), cached per device.
// T == 1: the streaming kernels.  Launch shapes measured on MI355X with the
// decode layer (H 6144, I 2048, 9 entries): gate/up runs one 4-wave
// workgroup per CU (its register ring plus the x chunks allow two waves per
// SIMD, and more waves lose DRAM locality), down runs four per CU.
static hipError_t launch_f32_t1(const LayerDev &L, const ForwardIO &io, GemvArgs a, float *h,
                                float *o, hipStream_t st, Marks *mk, const RouteSelf *rt = nullptr)
{
    const int entries = a.cap + a.n_shared;
    const int cus = device_cu_count();
    a.tl_cap = mk ? mk->tl_cap : 0;
    {
        a.tl = mk ? mk->tl_next() : nullptr;
        constexpr int NP = 1, M = 8, DEPTH = 2;
        a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
        a.N = 2 * L.I; a.K = L.H; a.upe = L.I;
        a.in = io.x; a.in_by_slot = 0;
        a.out = h; a.out_ld = L.I;
        const int P = (L.H / 32 + 63) / 64;
        const int units = entries * (L.I / NP);
        const dim3 grid(std::min(cus, (units + 3) / 4)), block(256);
        const size_t lds = (size_t)(L.H + L.H / 32) * 4;
#define COLI_GU1(P_) \
        if (P == P_) { \
            if (rt && a.tl) launch(mk, (gateup_t1_kernel<P_, NP, M, DEPTH, true, true, true>), grid, block, lds, st, a, *rt); \
            else if (rt) launch(mk, (gateup_t1_kernel<P_, NP, M, DEPTH, true, true>), grid, block, lds, st, a, *rt); \
            else launch(mk, (gateup_t1_kernel<P_, NP, M, DEPTH, true, false>), grid, block, lds, st, a, \
                        RouteSelf{}); \
        }
        COLI_GU1(1) COLI_GU1(2) COLI_GU1(3) COLI_GU1(4)
#undef COLI_GU1
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        constexpr int RD = 4, M = 4, DEPTH = 2;
        a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
        a.N = L.H; a.K = L.I; a.upe = L.H;
        a.in = h; a.in_by_slot = 1;
        a.out = o; a.out_ld = L.H;
        a.tl = mk ? mk->tl_next() : nullptr;
        const int P = (L.I / 32 + 63) / 64;
        if (io.combine) {
            // (2 rows per stage and reductions over 2 stages: 16.4 us, against
            // 17.5 for 4 rows and 19.9 for 2 rows over 4 stages)
            constexpr int RD = 2, M = 2, DEPTH = 2;
            // fused with the combine: NW waves per workgroup cover the entries;
            // one workgroup per CU (one round: the traces show one of these
            // 9-wave workgroups resident per CU, and 256 workgroups beat 512),
            // each with at most kDownRowsMax rows
            const int nblocks = L.H / RD, NW = std::min(entries, kDownT1cWaves);
            const dim3 block(64 * NW);
#define COLI_DN1C(P_) \
            if (P == P_) { \
                const auto kern = down_t1c_kernel<P_, RD, M, DEPTH>; \
                const int G = std::min(nblocks, std::max(cus, (nblocks * RD + kDownRowsMax - 1) / kDownRowsMax)); \
                if (a.tl) launch(mk, (down_t1c_kernel<P_, RD, M, DEPTH, true>), dim3(G), block, 0, st, a, \
                                 io.ids, io.w, io.y); \
                else launch(mk, kern, dim3(G), block, 0, st, a, io.ids, io.w, io.y); \
            }
            COLI_DN1C(1) COLI_DN1C(2) COLI_DN1C(3) COLI_DN1C(4)
#undef COLI_DN1C
            return hipGetLastError();
        }
        const dim3 grid(std::max(4 * cus, (entries + 3) / 4)), block(256);
#define COLI_DN1(P_) \
        if (P == P_) launch(mk, (down_t1_kernel<P_, RD, M, DEPTH>), grid, block, 0, st, a);
        COLI_DN1(1) COLI_DN1(2) COLI_DN1(3) COLI_DN1(4)
#undef COLI_DN1
        return hipGetLastError();
    }
}

hipError_t launch_route_forward_small(const LayerDev &L, const ForwardIO &io, int act_mode,
                                      float top_p, hipStream_t st, Marks *mk)
{
    const int T = io.T;
    float *scores = reinterpret_cast<float *>(io.ws + io.lay.scores);
    hipError_t err = launch_scores(L, io.x, T, scores, st, mk);
    if (err != hipSuccess) return err;
    RouteSelf rt{};
    rt.scores = scores; rt.bias = L.router_bias;
    rt.T = T; rt.E = L.E; rt.k = L.k; rt.cap = (int)io.lay.cap; rt.top_p = top_p;
    rt.ids = const_cast<int32_t *>(io.ids); rt.w = const_cast<float *>(io.w);
    rt.union_ids = const_cast<int32_t *>(io.union_ids); rt.offsets = const_cast<int32_t *>(io.offsets);
    rt.slots = const_cast<int32_t *>(io.slots); rt.n_union = const_cast<int32_t *>(io.n_union);
    if (act_mode != 0) {
        ForwardIO ri = io;
        ri.route = &rt;
        return launch_forward_i8(L, ri, st, mk);
    }
    float *h = reinterpret_cast<float *>(io.ws + io.lay.h);
    float *o = reinterpret_cast<float *>(io.ws + io.lay.o);
    GemvArgs a{};
    a.union_ids = io.union_ids; a.offsets = io.offsets; a.slots = io.slots; a.n_union = io.n_union;
    a.T = T; a.k = L.k; a.cap = (int)io.lay.cap; a.n_shared = L.n_shared;
    a.I = L.I;
    if (T == 1) return launch_f32_t1(L, io, a, h, o, st, mk, &rt);
    if (T == 2) return launch_f32_mt<2>(L, io, a, h, o, st, mk, &rt);
    return launch_f32_mt<4>(L, io, a, h, o, st, mk, &rt);
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
    if (T == 1) return launch_f32_t1(L, io, a, h, o, st, mk);
    // the streaming kernels hold every token's x in LDS: at most
    // 4 * (8192 + 256) * 4 = 132 KB of the 160 KB a workgroup may use
    static_assert(kStreamTMax * (COLI_MAX_H_DEV + COLI_MAX_H_DEV / 32) * 4 <= 160 * 1024, "LDS");
    if (T <= kStreamTMax) {
        if (T == 2) return launch_f32_mt<2>(L, io, a, h, o, st, mk);
        return launch_f32_mt<4>(L, io, a, h, o, st, mk);
    }
    // gate/up + SwiGLU -> h (chunk-transposed rows)
    a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
    a.N = 2 * L.I; a.K = L.H; a.upe = L.I;
    a.in = io.x; a.in_by_slot = 0;
    a.out = h; a.out_ld = L.I;
    {
        constexpr int W = 4, RW = 4;
        const int P = (L.H / 32 + 63) / 64;
        // staged token rows and their chunk constants must fit 64 KB of LDS
        int nt = 65536 / ((L.H + L.H / 32) * 4);
        nt = T < nt ? T : nt;
        nt = nt >= 2 ? 2 : 1;
        const dim3 grid(L.I / (W * RW / 2), entries), block(W * 64);
        const size_t lds = (size_t)nt * (L.H + L.H / 32) * 4;
#define COLI_GU(NT_, P_) \
        if (nt == NT_ && P == P_) \
            launch(mk, (gateup_f32_kernel<NT_, P_, W, RW>), grid, block, lds, st, a);
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
    {
        constexpr int W = 4, RW = 8;
        const int P = (L.I / 32 + 63) / 64;
        const dim3 grid(L.H / (W * RW), entries), block(W * 64);
#define COLI_DN(P_) \
        if (P == P_) launch(mk, (down_f32_kernel<P_, W, RW>), grid, block, 0, st, a);
        COLI_DN(1) COLI_DN(2) COLI_DN(3) COLI_DN(4)
#undef COLI_DN
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t err = io.combine
        ? launch_combine(o, io.ids, io.w, T, L.k, L.H, L.n_shared, io.y, st, mk)
        : hipSuccess;
    return err;
}

}  // namespace coli
