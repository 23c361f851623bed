// route.hip -- DeepSeek-V3 style sigmoid router with a selection bias
// ("Colibri" skill page, "コアアーキテクチャ" item 1; "Colibri 完全ガイド",
// table "コア技術のハイライト"), top-k per token ("colibri解説", section
// "なぜ25GBで動くのか": each MoE layer picks its top 8).
//
// logits = x . Wr^T accumulated in fp64 and rounded once to fp32, so the
// selection does not depend on summation order at fp32 precision.
//   small T: one workgroup per expert row streams Wr once (HBM-bound) and
//            writes the expert's sigmoid score;
//   large T: fp64 MFMA GEMM split over K, partials added by the top-k kernel.
// top-k: one wave per token; lane l holds experts l, l+64, ...; the k-th
// largest key by a bitwise radix select, ties by lower expert.
#include "common.h"
#include "route_tokens.h"

namespace coli {

// --- small T: grid = E workgroups of 256 threads (4 waves split H) -------
// Each workgroup writes the score of its expert (the logit rounded to fp32,
// then its sigmoid), so the top-k kernel starts from scores.
// A lane owns the float4 columns lane, lane + 64, ... of its wave's quarter
// (at most kGemvCols of them); all of its weight loads, and then a token's
// activation loads, are issued before the first product, so the kernel pays
// one memory latency per token instead of one per column.  The products are
// accumulated in ascending column order per lane, as in a plain loop.
constexpr int kGemvCols = COLI_MAX_H_DEV / 4 / 4 / 64;  // float4 columns per lane, at most

template <int NT, bool TL = false>
__global__ __launch_bounds__(256) void logits_gemv_kernel(const float *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          int T, int H, int E,
                                                          float *__restrict__ logits,
                                                          uint64_t *tl, int tl_cap)
{
    tl_mark<TL>(tl, tl_cap, 0);
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ double part[4][NT];
    const int H4 = H >> 2;
    const int per = (H4 + 3) / 4;  // float4 columns per wave
    const int c0 = wave * per, c1 = min(H4, c0 + per);
    // buffer loads: columns outside the wave's quarter get an offset past
    // the row and read 0 without touching memory
    uint32_t off[kGemvCols];
#pragma unroll
    for (int i = 0; i < kGemvCols; ++i) {
        const int c = c0 + lane + 64 * i;
        off[i] = c < c1 ? (uint32_t)c * 16 : kOOB;
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(Wr + (size_t)e * H, (uint32_t)H * 4);
    uint4 wv[kGemvCols];
#pragma unroll
    for (int i = 0; i < kGemvCols; ++i) wv[i] = load16(rw, off[i]);
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc[t] = 0.0;
        if (t < T) {
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)t * H, (uint32_t)H * 4);
            uint4 xv[kGemvCols];
#pragma unroll
            for (int i = 0; i < kGemvCols; ++i) xv[i] = load16(rx, off[i]);
            // (a column outside the quarter adds 0 * 0: acc starts at +0 and
            // never becomes -0, so acc + 0 is acc, bit for bit)
#pragma unroll
            for (int i = 0; i < kGemvCols; ++i) {
                acc[t] = fma((double)__uint_as_float(xv[i].x), (double)__uint_as_float(wv[i].x), acc[t]);
                acc[t] = fma((double)__uint_as_float(xv[i].y), (double)__uint_as_float(wv[i].y), acc[t]);
                acc[t] = fma((double)__uint_as_float(xv[i].z), (double)__uint_as_float(wv[i].z), acc[t]);
                acc[t] = fma((double)__uint_as_float(xv[i].w), (double)__uint_as_float(wv[i].w), acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double s = wave_sum_f64(acc[t]);
        if (lane == 0) part[wave][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < NT && (int)threadIdx.x < T) {
        int t = threadIdx.x;
        double s = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
        logits[(size_t)t * E + e] = sigmoid_fp64((float)s);
    }
    tl_mark<TL>(tl, tl_cap, 7);
}

// --- large T: fp64 MFMA GEMM, split over K -------------------------------
// v_mfma_f64_16x16x4f64: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// receives D[4v + l/16][l%16] in its v-th register pair, v < 4 (rows are
// interleaved across the lane quarters, unlike the fp32 16x16x4 form).  The fp32 operands are widened to fp64
// (exact) and each product is exact in fp64.  The K index assigned to a
// lane's quarter is free as long as A and B agree: in a k-block of 16, lane
// quarter q loads the float4 at k0+4q of its row and the m-th MFMA uses its
// m-th element, so every load is a 16-byte vector.
// Workgroup: 64 tokens x 64 experts, 2 x 2 waves of 32 x 32 (2 x 2 MFMA
// tiles); split s covers k-blocks [s*bps, (s+1)*bps) and writes its fp64
// partial sums to part[s][t][e].  Operands come straight from global memory:
// a wave needs 4 KB per 16 MFMAs, which L2 serves.
typedef double coli_d4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4_at(const float4 &v, int m)
{
    return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

__global__ __launch_bounds__(256) void logits_mfma_kernel(const float *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          int T, int H, int E, int tilesE, int S,
                                                          int bps, int nwg,
                                                          double *__restrict__ part)
{
    // The dispatcher deals workgroups to the 8 XCDs round-robin; remap so
    // that consecutive logical ids (the expert tiles of one token tile and
    // split, which read the same x) run on one XCD and share its L2.
    const int G = gridDim.x;  // a multiple of 8
    const int L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (L >= nwg) return;
    const int te = L % tilesE;
    const int r = L / tilesE;
    const int s = r % S;
    const int tt = r / S;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int i = lane & 15, q = lane >> 4;
    const int nb = H >> 4;
    const int b0 = s * bps, b1 = min(nb, b0 + bps);
    const float *ap[2], *bp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int t = min(tt * kLogitTile + wm * 32 + mt * 16 + i, T - 1);
        ap[mt] = x + (size_t)t * H + 16 * b0 + 4 * q;
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int e = min(te * kLogitTile + wn * 32 + nt * 16 + i, E - 1);
        bp[nt] = Wr + (size_t)e * H + 16 * b0 + 4 * q;
    }
    coli_d4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = coli_d4{0.0, 0.0, 0.0, 0.0};
    // Two register buffers: the loads of block n+1 are in flight while the
    // MFMAs of block n run.  Past the split's end the loads re-read the
    // split's last block (in bounds) and are not used.
    float4 a0[2], b0v[2], a1[2], b1v[2];
    auto load = [&](float4 *a, float4 *b, int blk) {
        const int off = 16 * (min(blk, b1 - 1) - b0);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) a[mt] = *reinterpret_cast<const float4 *>(ap[mt] + off);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) b[nt] = *reinterpret_cast<const float4 *>(bp[nt] + off);
    };
    auto mma = [&](const float4 *a, const float4 *b) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                        (double)f4_at(a[mt], m), (double)f4_at(b[nt], m), acc[mt][nt], 0, 0, 0);
    };
    if (b0 >= b1) return;  // no empty split is ever launched
    load(a0, b0v, b0);
    int blk = b0;
    for (; blk + 1 < b1; blk += 2) {
        load(a1, b1v, blk + 1);
        mma(a0, b0v);
        load(a0, b0v, blk + 2);
        mma(a1, b1v);
    }
    if (blk < b1) mma(a0, b0v);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = tt * kLogitTile + wm * 32 + mt * 16 + 4 * v + q;
                const int e = te * kLogitTile + wn * 32 + nt * 16 + i;
                if (t < T && e < E) part[((size_t)s * T + t) * E + e] = acc[mt][nt][v];
            }
}

// --- top-k: one wave per token, 4 tokens per workgroup -------------------
// UNION: a single workgroup also forms the batch-union of its tokens.
template <int KPL, bool UNION = false>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   const double *__restrict__ part, int S,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, float top_p, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, UnionOut uo = {})
{
    route_tokens<KPL, UNION>(logits, part, S, bias, T, E, k, top_p, ids, w, uo, blockIdx.x * 4);
}

hipError_t launch_scores(const LayerDev &L, const float *x, int32_t T, float *scores,
                         hipStream_t st, Marks *mk)
{
    const dim3 grid(L.E), block(256);
    uint64_t *tl = mk ? mk->tl_next() : nullptr;
    const int cap = mk ? mk->tl_cap : 0;
#define COLI_SC(NT_) \
    (tl ? launch(mk, logits_gemv_kernel<NT_, true>, grid, block, 0, st, x, L.router_w, T, L.H, L.E, scores, tl, cap) \
        : launch(mk, logits_gemv_kernel<NT_, false>, grid, block, 0, st, x, L.router_w, T, L.H, L.E, scores, tl, cap))
    if (T <= 1) COLI_SC(1);
    else if (T <= 2) COLI_SC(2);
    else if (T <= 4) COLI_SC(4);
    else COLI_SC(8);
#undef COLI_SC
    return hipGetLastError();
}

hipError_t launch_route(const LayerDev &L, const RouteIO &io, hipStream_t st, const UnionIO *un)
{
    const int T = io.T, H = L.H, E = L.E;
    if (T <= 0) return hipSuccess;
    const RouteSplit rs = route_split(T, H, E);
    const int S = rs.S;
    const double *part = reinterpret_cast<const double *>(io.logits);
    if (S == 0) {
        dim3 grid(E), block(256);
#define COLI_GEMV_CASE(N) \
    case N: hipLaunchKernelGGL(logits_gemv_kernel<N>, grid, block, 0, st, io.x, L.router_w, T, H, E, io.logits, \
                               nullptr, 0); break;
        switch (T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8) {
            COLI_GEMV_CASE(1)
            COLI_GEMV_CASE(2)
            COLI_GEMV_CASE(4)
            COLI_GEMV_CASE(8)
        }
#undef COLI_GEMV_CASE
    } else {
        const int bps = rs.bps;
        const int tilesT = (T + kLogitTile - 1) / kLogitTile, tilesE = (E + kLogitTile - 1) / kLogitTile;
        const int nwg = tilesT * tilesE * S;
        const int G = (nwg + 7) & ~7;
        hipLaunchKernelGGL(logits_mfma_kernel, dim3(G), dim3(256), 0, st, io.x, L.router_w, T, H, E,
                           tilesE, S, bps, nwg, reinterpret_cast<double *>(io.logits));
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int kpl = (E + 63) / 64;
    // a batch of at most 4 tokens is one top-k workgroup: it also forms the union
    const bool fuse = un && T <= 4;
    UnionOut uo{};
    if (un) {
        uo.union_ids = un->union_ids; uo.offsets = un->offsets; uo.slots = un->slots;
        uo.n_union = un->n_union;
        const int n = T * L.k;
        uo.cap = n < E ? n : E;
    }
#define COLI_TOPK(N) \
    if (kpl <= N) { \
        if (fuse) hipLaunchKernelGGL((topk_kernel<N, true>), dim3(1), dim3(256), 0, st, io.logits, part, S, \
                                     L.router_bias, T, E, L.k, io.top_p, io.ids, io.w, uo); \
        else hipLaunchKernelGGL((topk_kernel<N, false>), dim3((T + 3) / 4), dim3(256), 0, st, io.logits, \
                                part, S, L.router_bias, T, E, L.k, io.top_p, io.ids, io.w, uo); \
        err = hipGetLastError(); \
        if (err != hipSuccess || !un || fuse) return err; \
        return launch_union(io.ids, T, L.k, E, un->union_ids, un->offsets, un->slots, un->n_union, st); \
    }
    COLI_TOPK(1)
    COLI_TOPK(2)
    COLI_TOPK(4)
    COLI_TOPK(8)
    COLI_TOPK(16)
#undef COLI_TOPK
    return hipErrorInvalidValue;
}

}  // namespace coli
