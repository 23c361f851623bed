// expert_f32.hip -- the fp32 arithmetic family of the expert FFN
// ("Colibri 完全ガイド", walk-through "詳細解説" step 3: single-token decode
// computes in f32).  Weights are int4 with one fp16 scale per row per
// 64-group ("colibri: 744B MoE...", section "はじめにとソースが語らないこと":
// the gs64 build).
//
// One kernel streams the packed weights of every union expert once from HBM
// and multiplies them with that expert's tokens (a GEMV for decode, a few
// tokens for a verify batch):
//  - workgroup = 4 waves; each wave owns 4 weight rows (two gate/up row
//    pairs for the SwiGLU matmul, four consecutive rows for the down one);
//  - lane l reads 16-byte chunks l, l+64, ... of each row (coalesced 1 KB
//    per wave instruction); the matching 32 activations come from LDS, where
//    the workgroup staged the tokens' input rows;
//  - per chunk: codes are biased to unsigned (xor 0x8), split into even and
//    odd bytes, converted with byte-to-float conversions and fused into the
//    dot product; the bias is removed with the chunk's activation sum
//    (sum q x = sum u x - 8 sum x) and the group scale applied once per chunk;
//  - lane partials are reduced with a fixed butterfly.
// A token's arithmetic is the same whatever the batch, so a token computed
// alone and inside a batch give bitwise identical results.
#include "common.h"

namespace coli {

struct GemvArgs {
    const uint8_t *w;      // routed experts, [E][N][K/2]
    const uint16_t *s;     // [E][N][K/64]
    const uint8_t *sh_w;   // shared expert [N][K/2]
    const uint16_t *sh_s;  // [N][K/64]
    int N, K, I;           // rows, reduction length, I (up-row offset for SwiGLU)
    const float *in;       // input rows
    int in_by_slot;        // 0: input row = token; 1: input row = output row
    float *out;            // output rows [R][out_ld]
    int out_ld;
    const int32_t *union_ids, *offsets, *slots, *n_union;
    int T, k, cap, n_shared;
};

constexpr int kRowsPerWave = 4;
constexpr int kGemvWaves = 4;

template <int NT, bool SWIGLU>
__global__ __launch_bounds__(256) void gemv_int4_kernel(GemvArgs a)
{
    extern __shared__ float xs[];  // [NT][K]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ue = blockIdx.y;
    const uint8_t *wbase;
    const uint16_t *sbase;
    int cnt;
    const int32_t *list = nullptr;
    if (ue < a.cap) {
        if (ue >= a.n_union[0]) return;
        const int e = a.union_ids[ue];
        wbase = a.w + (size_t)e * a.N * (a.K / 2);
        sbase = a.s + (size_t)e * a.N * (a.K / 64);
        const int o0 = a.offsets[ue];
        cnt = a.offsets[ue + 1] - o0;
        list = a.slots + o0;
    } else {
        wbase = a.sh_w;
        sbase = a.sh_s;
        cnt = a.T;
    }
    if (cnt <= 0) return;

    int rows[kRowsPerWave];
    if (SWIGLU) {
        const int i0 = (blockIdx.x * kGemvWaves + wave) * 2;
        rows[0] = i0; rows[1] = i0 + 1; rows[2] = a.I + i0; rows[3] = a.I + i0 + 1;
    } else {
        const int n0 = (blockIdx.x * kGemvWaves + wave) * kRowsPerWave;
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) rows[r] = n0 + r;
    }
    const int rb = a.K / 2, sb = a.K / 64, C = a.K / 32;
    const int K4 = a.K / 4;
    const int TK = a.T * a.k;

    for (int b0 = 0; b0 < cnt; b0 += NT) {
        const int nt = min(NT, cnt - b0);
        int in_row[NT], out_row[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            int idx = b0 + (tt < nt ? tt : 0);
            if (list) {
                int s = list[idx];
                out_row[tt] = s;
                in_row[tt] = a.in_by_slot ? s : s / a.k;
            } else {
                out_row[tt] = TK + idx;
                in_row[tt] = a.in_by_slot ? TK + idx : idx;
            }
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float4 *src = reinterpret_cast<const float4 *>(a.in + (size_t)in_row[tt] * a.K);
            float4 *dst = reinterpret_cast<float4 *>(xs + tt * a.K);
            for (int i = threadIdx.x; i < K4; i += blockDim.x) dst[i] = src[i];
        }
        __syncthreads();

        float racc[kRowsPerWave][NT];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) racc[r][tt] = 0.f;

        for (int c = lane; c < C; c += 64) {
            uint4 wv[kRowsPerWave];
            float sc[kRowsPerWave];
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
                wv[r] = *reinterpret_cast<const uint4 *>(wbase + (size_t)rows[r] * rb + c * 16);
                sc[r] = f16_to_f32(sbase[(size_t)rows[r] * sb + (c >> 1)]);
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (tt < nt) {
                    float xv[32];
                    const float4 *xp = reinterpret_cast<const float4 *>(xs + tt * a.K + c * 32);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        float4 v = xp[q];
                        xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y;
                        xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
                    }
                    float xsum = 0.f;
#pragma unroll
                    for (int q = 0; q < 32; ++q) xsum += xv[q];
#pragma unroll
                    for (int r = 0; r < kRowsPerWave; ++r) {
                        const uint32_t wd[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
                        float acc = 0.f;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const uint32_t u = wd[d] ^ 0x88888888u;
                            const uint32_t lo = u & 0x0F0F0F0Fu;
                            const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                acc = fmaf((float)((lo >> (8 * b)) & 0xFFu), xv[8 * d + 2 * b], acc);
                                acc = fmaf((float)((hi >> (8 * b)) & 0xFFu), xv[8 * d + 2 * b + 1], acc);
                            }
                        }
                        const float part = fmaf(-8.0f, xsum, acc);
                        racc[r][tt] = fmaf(part, sc[r], racc[r][tt]);
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) racc[r][tt] = wave_sum(racc[r][tt]);

        if (lane == 0) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (tt >= nt) continue;
                float *orow = a.out + (size_t)out_row[tt] * a.out_ld;
                if (SWIGLU) {
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const float g = racc[p][tt], u = racc[2 + p][tt];
                        orow[rows[p]] = g / (1.0f + expf(-g)) * u;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < kRowsPerWave; ++r) orow[rows[r]] = racc[r][tt];
                }
            }
        }
    }
}

template <bool SWIGLU>
static hipError_t launch_gemv(const GemvArgs &a, int max_tokens, hipStream_t st)
{
    // tokens per batch limited so the staged inputs fit 64 KB of LDS
    int nt_lds = 65536 / (a.K * 4);
    int nt = max_tokens < nt_lds ? max_tokens : nt_lds;
    nt = nt >= 4 ? 4 : nt >= 2 ? 2 : 1;
    const int rows_per_wg = SWIGLU ? kGemvWaves * 2 : kGemvWaves * kRowsPerWave;
    const int units = SWIGLU ? a.I : a.N;
    dim3 grid((units + rows_per_wg - 1) / rows_per_wg, a.cap + a.n_shared), block(256);
    const size_t lds = (size_t)nt * a.K * sizeof(float);
    switch (nt) {
    case 1: hipLaunchKernelGGL((gemv_int4_kernel<1, SWIGLU>), grid, block, lds, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_int4_kernel<2, SWIGLU>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((gemv_int4_kernel<4, SWIGLU>), grid, block, lds, st, a); break;
    }
    return hipGetLastError();
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
    // gate/up + SwiGLU: h[row][i]
    a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
    a.N = 2 * L.I; a.K = L.H;
    a.in = io.x; a.in_by_slot = 0;
    a.out = h; a.out_ld = L.I;
    if (mk) mk->mark(st);
    hipError_t err = launch_gemv<true>(a, T, st);
    if (err != hipSuccess) return err;
    // down: o[row][n]
    a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
    a.N = L.H; a.K = L.I;
    a.in = h; a.in_by_slot = 1;
    a.out = o; a.out_ld = L.H;
    if (mk) mk->mark(st);
    err = launch_gemv<false>(a, T, st);
    if (err != hipSuccess) return err;
    if (mk) mk->mark(st);
    err = launch_combine(o, io.w, T, L.k, L.H, L.n_shared, io.y, st);
    if (mk) mk->mark(st);
    return err;
}

}  // namespace coli
