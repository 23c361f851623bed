// route.hip -- DeepSeek-V3 style sigmoid router with a selection bias
// ("Colibri" skill page, "コアアーキテクチャ" item 1; "Colibri 完全ガイド",
// table "コア技術のハイライト"), top-k per token ("colibri解説", section
// "なぜ25GBで動くのか": each MoE layer picks its top 8).
//
// logits = x . Wr^T accumulated in fp64 and rounded once to fp32, so the
// selection does not depend on summation order at fp32 precision.
//   small T: one workgroup per expert row streams Wr once (HBM-bound);
//   large T: LDS-tiled fp64 GEMM.
// top-k: one wave per token; lane l holds experts l, l+64, ...; k rounds of
// a wave-wide argmax on (key desc, expert asc).
#include "common.h"

namespace coli {

constexpr int kGemvTMax = 8;

// --- small T: grid = E workgroups of 256 threads (4 waves split H) -------
template <int NT>
__global__ __launch_bounds__(256) void logits_gemv_kernel(const float *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          int T, int H, int E,
                                                          float *__restrict__ logits)
{
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ double part[4][NT];
    const int H4 = H >> 2;
    const int per = (H4 + 3) / 4;  // float4 columns per wave
    const int c0 = wave * per, c1 = min(H4, c0 + per);
    const float4 *w4 = reinterpret_cast<const float4 *>(Wr + (size_t)e * H);
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
    for (int c = c0 + lane; c < c1; c += 64) {
        float4 wv = w4[c];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < T) {
                float4 xv = reinterpret_cast<const float4 *>(x + (size_t)t * H)[c];
                acc[t] = fma((double)xv.x, (double)wv.x, acc[t]);
                acc[t] = fma((double)xv.y, (double)wv.y, acc[t]);
                acc[t] = fma((double)xv.z, (double)wv.z, acc[t]);
                acc[t] = fma((double)xv.w, (double)wv.w, acc[t]);
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
        logits[(size_t)t * E + e] = (float)s;
    }
}

// --- large T: 64 tokens x 64 experts per workgroup, 4x4 per thread -------
constexpr int kLT = 64, kLE = 64, kLK = 16;

__global__ __launch_bounds__(256) void logits_gemm_kernel(const float *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          int T, int H, int E,
                                                          float *__restrict__ logits)
{
    __shared__ double xs[kLK][kLT + 1];
    __shared__ double ws[kLK][kLE + 1];
    const int t0 = blockIdx.y * kLT, e0 = blockIdx.x * kLE;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;  // thread owns experts e0+tx+16j, tokens t0+ty+16i
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    // loader mapping: 256 threads x float4 = 64 rows x 16 columns
    const int lr = tid >> 2, lc = (tid & 3) * 4;
    for (int k0 = 0; k0 < H; k0 += kLK) {
        {
            int t = t0 + lr;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < T) v = *reinterpret_cast<const float4 *>(x + (size_t)t * H + k0 + lc);
            xs[lc + 0][lr] = v.x; xs[lc + 1][lr] = v.y; xs[lc + 2][lr] = v.z; xs[lc + 3][lr] = v.w;
            int e = e0 + lr;
            float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) u = *reinterpret_cast<const float4 *>(Wr + (size_t)e * H + k0 + lc);
            ws[lc + 0][lr] = u.x; ws[lc + 1][lr] = u.y; ws[lc + 2][lr] = u.z; ws[lc + 3][lr] = u.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kLK; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
            if (t < T && e < E) logits[(size_t)t * E + e] = (float)acc[i][j];
        }
}

// --- top-k: one wave per token, 4 tokens per workgroup -------------------
// Radix select: the k-th largest key is found bit by bit with wave ballots
// (32 rounds, no shuffles); keys equal to it are taken in expert order; the
// k winners are then ordered by (key desc, expert asc) through LDS.
__device__ __forceinline__ float sigmoid_fp64(float l)
{
    return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// Monotone map of an fp32 key to uint32 (larger float -> larger integer);
// -0 is folded into +0 first so that equal keys compare equal.
__device__ __forceinline__ uint32_t order_bits(float z)
{
    const uint32_t u = __float_as_uint(z + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w)
{
    __shared__ uint32_t sk[4][COLI_MAX_K_DEV];
    __shared__ int32_t se[4][COLI_MAX_K_DEV];
    __shared__ float ss[4][COLI_MAX_K_DEV];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    const bool live = t < T;
    const float *lrow = logits + (size_t)(live ? t : 0) * E;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (live && e < E) ? order_bits(sigmoid_fp64(lrow[e]) + bias[e]) : 0u;
    }
    // largest tau with #{key >= tau} >= k  (valid keys are >= 1)
    uint32_t tau = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = tau | (1u << b);
        int c = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) c += __popcll(__ballot(key[i] >= cand));
        if (c >= k) tau = cand;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) gt += __popcll(__ballot(key[i] > tau));
    const int need = k - gt;  // keys equal to tau to take, lowest experts first
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t eqm = __ballot(key[i] == tau);
        const bool is_eq = key[i] == tau;
        const bool sel = key[i] > tau || (is_eq && eq_before + __popcll(eqm & lt_mask) < need);
        const uint64_t selm = __ballot(sel);
        if (sel && live && sel_before + __popcll(selm & lt_mask) < k) {
            const int pos = sel_before + __popcll(selm & lt_mask);
            sk[wv][pos] = key[i];
            se[wv][pos] = lane + 64 * i;
        }
        eq_before += __popcll(eqm);
        sel_before += __popcll(selm);
    }
    __syncthreads();
    // lane j < k: rank of winner j among the winners, then its weight
    uint32_t mk = 0;
    int me = 0, rank = 0;
    if (live && lane < k) {
        mk = sk[wv][lane];
        me = se[wv][lane];
        for (int j = 0; j < k; ++j) {
            const uint32_t ok = sk[wv][j];
            const int oe = se[wv][j];
            rank += (ok > mk || (ok == mk && oe < me)) ? 1 : 0;
        }
    }
    __syncthreads();
    float sj = 0.f;
    if (live && lane < k) {
        sj = sigmoid_fp64(lrow[me]);
        ss[wv][rank] = sj;
    }
    __syncthreads();
    if (live && lane < k) {
        float sum = 0.f;
        for (int j = 0; j < k; ++j) sum += ss[wv][j];  // fp32, selection order
        ids[(size_t)t * k + rank] = me;
        w[(size_t)t * k + rank] = sj / sum;
    }
}

hipError_t launch_route(const LayerDev &L, const RouteIO &io, hipStream_t st)
{
    const int T = io.T, H = L.H, E = L.E;
    if (T <= 0) return hipSuccess;
    if (T <= kGemvTMax) {
        dim3 grid(E), block(256);
#define COLI_GEMV_CASE(N) \
    case N: hipLaunchKernelGGL(logits_gemv_kernel<N>, grid, block, 0, st, io.x, L.router_w, T, H, E, io.logits); break;
        switch (T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8) {
            COLI_GEMV_CASE(1)
            COLI_GEMV_CASE(2)
            COLI_GEMV_CASE(4)
            COLI_GEMV_CASE(8)
        }
#undef COLI_GEMV_CASE
    } else {
        dim3 grid((E + kLE - 1) / kLE, (T + kLT - 1) / kLT), block(256);
        hipLaunchKernelGGL(logits_gemm_kernel, grid, block, 0, st, io.x, L.router_w, T, H, E,
                           io.logits);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int kpl = (E + 63) / 64;
#define COLI_TOPK(N) \
    if (kpl <= N) { hipLaunchKernelGGL(topk_kernel<N>, dim3((T + 3) / 4), dim3(256), 0, st, io.logits, \
                                       L.router_bias, T, E, L.k, io.ids, io.w); return hipGetLastError(); }
    COLI_TOPK(1)
    COLI_TOPK(2)
    COLI_TOPK(4)
    COLI_TOPK(8)
    COLI_TOPK(16)
#undef COLI_TOPK
    return hipErrorInvalidValue;
}

}  // namespace coli
