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

}  // namespace coli

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
