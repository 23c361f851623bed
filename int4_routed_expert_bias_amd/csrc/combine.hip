// combine.hip -- weighted combine of the routed expert outputs plus the
// ungated shared expert (the router comes with shared experts: "Colibri
// 完全ガイド", table "コア技術のハイライト"; the shared expert belongs to the
// always-resident dense part: getting-started page, "프로젝트 설명"), and the
// glue for stacking layers (unit-gain RMS pre-norm, residual add).
#include "common.h"

namespace coli {

// y[t][n] = sum_j w[t][j] * o[t*k + j][n]  (j ascending, fp32 fma chain,
//           slots dropped by the top-p router -- id -1 -- skipped)
//           + o[T*k + t][n]                (shared expert, if present)
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ w, int T, int k,
                                                      int H, int n_shared, float *__restrict__ y)
{
    const int t = blockIdx.y;
    const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (n4 >= H / 4) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        if (ids[(size_t)t * k + j] < 0) continue;
        const float wj = w[(size_t)t * k + j];
        const float4 v = reinterpret_cast<const float4 *>(o + ((size_t)t * k + j) * H)[n4];
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    if (n_shared) {
        const float4 v = reinterpret_cast<const float4 *>(o + ((size_t)T * k + t) * H)[n4];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4 *>(y + (size_t)t * H)[n4] = acc;
}

hipError_t launch_combine(const float *o, const int32_t *ids, const float *w, int32_t T, int32_t k,
                          int32_t H, int32_t n_shared, float *y, hipStream_t st, Marks *mk)
{
    if (T <= 0) return hipSuccess;
    dim3 grid((H / 4 + 255) / 256, T), block(256);
    launch(mk, combine_kernel, grid, block, 0, st, o, ids, w, T, k, H, n_shared, y);
    return hipGetLastError();
}

// xhat = x / sqrt(mean(x^2) + eps): sum of squares in fp64 (fixed tree),
// scale in fp64, one rounding per element.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x,
                                                      float *__restrict__ xhat, int H, float eps)
{
    __shared__ double part[4];
    const float *r = x + (size_t)blockIdx.x * H;
    double ss = 0.0;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ss = fma((double)r[i], (double)r[i], ss);
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    const double inv = 1.0 / sqrt(tot / (double)H + (double)eps);
    for (int i = threadIdx.x; i < H; i += blockDim.x)
        xhat[(size_t)blockIdx.x * H + i] = (float)((double)r[i] * inv);
}

// x += y, then xhat = rmsnorm(x), one row per workgroup: every element of
// the sum is formed once (fp32 add), written back and kept in registers for
// the norm, whose sum of squares runs over the same elements in the same
// order as rmsnorm_kernel's -- so x and xhat are bitwise those of add_kernel
// followed by rmsnorm_kernel, with one pass over x fewer.
constexpr int kNormPer = COLI_MAX_H_DEV / 256;  // elements per thread, at most

__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float *__restrict__ x,
                                                          const float *__restrict__ y,
                                                          float *__restrict__ xhat, int H, float eps)
{
    __shared__ double part[4];
    float *r = x + (size_t)blockIdx.x * H;
    const float *d = y + (size_t)blockIdx.x * H;
    float v[kNormPer];
#pragma unroll
    for (int c = 0; c < kNormPer; ++c) {
        const int i = threadIdx.x + 256 * c;
        v[c] = i < H ? r[i] + d[i] : 0.f;
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kNormPer; ++c) {
        const int i = threadIdx.x + 256 * c;
        if (i < H) {
            r[i] = v[c];
            ss = fma((double)v[c], (double)v[c], ss);
        }
    }
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    const double inv = 1.0 / sqrt(tot / (double)H + (double)eps);
#pragma unroll
    for (int c = 0; c < kNormPer; ++c) {
        const int i = threadIdx.x + 256 * c;
        if (i < H) xhat[(size_t)blockIdx.x * H + i] = (float)((double)v[c] * inv);
    }
}

hipError_t launch_add_rmsnorm(float *x, const float *y, float *xhat, int32_t T, int32_t H,
                              float eps, hipStream_t st)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(T), dim3(256), 0, st, x, y, xhat, H, eps);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *x, float *xhat, int32_t T, int32_t H, float eps,
                          hipStream_t st)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, st, x, xhat, H, eps);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void add_kernel(float *__restrict__ x, const float *__restrict__ y,
                                                  int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride) x[j] += y[j];
}

hipError_t launch_add(float *x, const float *y, int64_t n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(add_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, y, n);
    return hipGetLastError();
}

}  // namespace coli
