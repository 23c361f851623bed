// probe.hip -- coli_stream_read: the plain HBM read rate with the load
// pattern of the streaming expert kernels (buffer loads of 16 bytes per
// lane, a wave reading 1 KB per instruction, several loads in flight per
// wave), for measurement only: it is the practical ceiling the streaming
// kernels are compared against.
#include "common.h"
#include "stream.h"

namespace coli {

// Workgroup b's four waves read 1 KB blocks w, w + W, ... (w the global wave
// index, W the number of waves), kDepth blocks in flight per wave; the XOR
// of everything read is written to out[b] so that no load is dead.
constexpr int kProbeDepth = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t *__restrict__ buf,
                                                          uint32_t nblk, uint32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const uint32_t w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint32_t W = gridDim.x * 4;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, nblk * 1024u);
    uint32_t acc = 0;
    for (uint32_t b0 = w; b0 < nblk; b0 += W * kProbeDepth) {
        uint4 v[kProbeDepth];
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d) {
            const uint32_t b = b0 + (uint32_t)d * W;
            v[d] = load16(r, b < nblk ? b * 1024u + lane * 16u : 0x80000000u);  // past: 0
        }
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    __shared__ uint32_t red[4];
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
    if (lane == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Issue sharing of one SIMD between the matrix core and the vector ALU,
// the quantity that sets the int8 GEMM's ceiling: workgroups of 8 waves (two
// per SIMD) run ITERS iterations of
//   mode 0: 4 independent v_mfma_i32_16x16x64_i8 per wave,
//   mode 1: 16 independent fp32 FMAs per wave,
//   mode 2: waves 0-3 the MFMAs of mode 0, waves 4-7 the FMAs of mode 1
//           (so each SIMD holds one wave of each kind),
//   mode 3: every wave both, interleaved;
//   mode 4: the FMAs of mode 1 in waves 0-3 only (one wave per SIMD: the
//           rate of a single wave's VALU issue);
//   mode 5: 16 independent three-source fp32 FMAs per wave, every source a
//           distinct VGPR (v_fma_f32 in its VOP3 form, as in the int8 GEMM's
//           epilogue; mode 1's compile to the two-source-plus-constant form);
// ticks[b] = workgroup b's duration in wall-clock (100 MHz) ticks.  If the
// two units issued in parallel, modes 2 and 3 would take about as long as
// the longer of modes 0 and 1 (halved for mode 2); serialised, as long as
// their sum.
constexpr int kIssueIters = 2048;
typedef int v4i_p __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(512) void issue_probe_kernel(uint64_t *__restrict__ ticks, int seed,
                                                          int *__restrict__ sink)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const v4i_p a = {seed + lane, 1, 2, 3}, b = {3, seed, 1, lane};
    v4i_p c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    float f[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = (float)(lane + i) * 1e-3f;
    const float m = 1.0001f + seed * 1e-9f, ad = 1e-7f;
    const bool mfma = MODE == 0 || (MODE == 2 && wave < 4);
    const bool valu = MODE == 1 || (MODE == 2 && wave >= 4) || (MODE == 4 && wave < 4);
    float g[16], h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        g[i] = (float)(lane - i) * 1e-3f;
        h[i] = (float)(i + 1) * 1e-4f;
    }
    __syncthreads();
    const uint64_t t0 = wall_clock64();
    if (MODE == 5) {
        for (int it = 0; it < kIssueIters; ++it) {
#pragma unroll
            for (int i = 0; i < 16; ++i)  // f = g * h + f, all three in VGPRs, f not the destination
                asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(g[i]) : "v"(g[i]), "v"(h[i]), "v"(f[i]));
        }
    } else if (MODE == 3) {
        for (int it = 0; it < kIssueIters; ++it) {
            c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = fmaf(f[i], m, ad);
            c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c1, 0, 0, 0);
#pragma unroll
            for (int i = 4; i < 8; ++i) f[i] = fmaf(f[i], m, ad);
            c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c2, 0, 0, 0);
#pragma unroll
            for (int i = 8; i < 12; ++i) f[i] = fmaf(f[i], m, ad);
            c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c3, 0, 0, 0);
#pragma unroll
            for (int i = 12; i < 16; ++i) f[i] = fmaf(f[i], m, ad);
        }
    } else {
        if (mfma)
            for (int it = 0; it < kIssueIters; ++it) {
                c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c3, 0, 0, 0);
            }
        if (valu)
            for (int it = 0; it < kIssueIters; ++it) {
#pragma unroll
                for (int i = 0; i < 16; ++i) f[i] = fmaf(f[i], m, ad);
            }
    }
    __syncthreads();
    const uint64_t t1 = wall_clock64();
    float fs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) fs += f[i] + g[i];
    if (c0[0] + c1[1] + c2[2] + c3[3] == 0x7fffffff || fs == 12345.f) sink[0] = 1;  // keeps the work
    if (threadIdx.x == 0) ticks[blockIdx.x] = t1 - t0;
}

}  // namespace coli

extern "C" int coli_issue_probe(int32_t mode, int32_t n_groups, uint64_t *ticks, int32_t *sink,
                                void *hip_stream)
{
    if (!ticks || !sink || n_groups < 1 || n_groups > 65536) return COLI_E_ARG;
    if (mode < 0 || mode > 5) return COLI_E_ARG;
    if (((uintptr_t)ticks & 7u) || ((uintptr_t)sink & 3u)) return COLI_E_ALIGN;
    if (int st = coli_moe_device_check()) return st;
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    switch (mode) {
    case 0: hipLaunchKernelGGL(coli::issue_probe_kernel<0>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    case 1: hipLaunchKernelGGL(coli::issue_probe_kernel<1>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    case 2: hipLaunchKernelGGL(coli::issue_probe_kernel<2>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    case 3: hipLaunchKernelGGL(coli::issue_probe_kernel<3>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    case 4: hipLaunchKernelGGL(coli::issue_probe_kernel<4>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    default: hipLaunchKernelGGL(coli::issue_probe_kernel<5>, dim3(n_groups), dim3(512), 0, s, ticks, 1, sink); break;
    }
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_E_DEVICE;
}

extern "C" int coli_stream_read(const void *buf, size_t bytes, uint32_t *out, int32_t n_groups,
                                void *hip_stream)
{
    if (!buf || !out || n_groups < 1 || n_groups > 65536) return COLI_E_ARG;
    if (bytes == 0 || bytes % 1024 || bytes > ((size_t)1 << 30)) return COLI_E_SHAPE;
    if (((uintptr_t)buf & 15u) || ((uintptr_t)out & 3u)) return COLI_E_ALIGN;
    if (int st = coli_moe_device_check()) return st;
    hipLaunchKernelGGL(coli::stream_read_kernel, dim3((unsigned)n_groups), dim3(256), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const uint8_t *>(buf),
                       (uint32_t)(bytes / 1024), out);
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_E_DEVICE;
}
