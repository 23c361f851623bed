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
constexpr int kMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb)
{
    return ka > kb || (ka == kb && ea < eb);
}

__device__ __forceinline__ float sigmoid_fp64(float l)
{
    return (float)(1.0 / (1.0 + exp(-(double)l)));
}

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *lrow = logits + (size_t)t * E;
    float key[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? sigmoid_fp64(lrow[e]) + bias[e] : 0.f;
    }
    uint32_t taken = 0;
    int sel = 0;  // lane j < k keeps the j-th selected expert
    for (int j = 0; j < k; ++j) {
        // lane-local best among the lane's untaken experts
        float bk = 0.f;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && (be == 0x7fffffff || better(key[i], e, bk, be))) {
                bk = key[i];
                be = e;
            }
        }
        // wave argmax on (key desc, expert asc); be == INT_MAX marks "none"
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ok = __shfl_xor(bk, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oe != 0x7fffffff && (be == 0x7fffffff || better(ok, oe, bk, be))) {
                bk = ok;
                be = oe;
            }
        }
        if (lane == j) sel = be;
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
    }
    // weights: the selected scores, recomputed exactly as in the keys,
    // normalised with an fp32 sum in selection order
    const float sj = (lane < k) ? sigmoid_fp64(lrow[sel]) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += __shfl(sj, j, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = sel;
        w[(size_t)t * k + lane] = sj / sum;
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
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, io.logits, L.router_bias,
                       T, E, L.k, io.ids, io.w);
    return hipGetLastError();
}

}  // namespace coli
