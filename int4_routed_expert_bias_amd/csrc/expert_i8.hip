// expert_i8.hip -- the integer arithmetic family of the expert FFN
// ("Colibri 完全ガイド": table "コア技術のハイライト", int8 x packed-int4 integer
// dot kernels; walk-through "詳細解説" step 3, batched prefill on the integer
// kernel).  Rebuilt for CDNA4 matrix cores:
//
//  quant:    per token per 64-group, scale = amax / 127 (IEEE divide),
//            q = clamp(rint(v / scale), -127, 127); codes are stored in the
//            permuted order [0,2,4,6,1,3,5,7] inside every 8-element block.
//  schedule: one thread per union expert turns its slot count into 16-row
//            tiles (device side: the union size never leaves the GPU).
//  gemm:     v_mfma_i32_16x16x64_i8, one MFMA per 64-group, so the exact
//            int32 group accumulator comes straight out of the matrix core.
//            A = 16 token rows of int8 codes, B = 16 weight rows.  A packed
//            int4 dword w splits into (w << 4) & 0xF0F0F0F0 (even elements)
//            and w & 0xF0F0F0F0 (odd elements): signed bytes equal to 16 x
//            the code, so the MFMA yields 16 x acc exactly (|16 acc| < 2^21)
//            and the activation layout above matches that byte order.
//            Epilogue per group: out += float(acc) * act_scale * w_scale.
//  gate/up:  each wave owns 64 gate rows and the matching 64 up rows, so the
//            SwiGLU and the int8 quantisation of h (one 64-group) stay in
//            registers; the down GEMM reads the quantised h.
#include "common.h"

namespace coli {

typedef int v4i __attribute__((ext_vector_type(4)));

// --- activation quantisation ---------------------------------------------
// rows [nrows][K] fp32 -> q [nrows][K] int8 (permuted), s [nrows][K/64]
__global__ __launch_bounds__(256) void quant_rows_kernel(const float *__restrict__ x, int64_t ngroups,
                                                         int K, int8_t *__restrict__ q,
                                                         float *__restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= ngroups) return;
    const int G = K / 64;
    const int64_t row = g / G;
    const int gi = (int)(g % G);
    const float v = x[row * K + gi * 64 + lane];
    const float amax = wave_max(fabsf(v));
    int8_t code = 0;
    float sc = 0.f;
    if (amax > 0.f) {
        sc = amax / 127.0f;
        float r = rintf(v / sc);
        r = fminf(fmaxf(r, -127.f), 127.f);
        code = (int8_t)r;
    }
    q[row * K + perm8_pos(gi * 64 + lane)] = code;
    if (lane == 0) s[row * G + gi] = sc;
}

// --- tile schedule ---------------------------------------------------------
// tiles[i] = (entry, first row) for i < count; count stored at tiles[max].x
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ offsets,
                                                        const int32_t *__restrict__ n_union,
                                                        int cap, int T, int n_shared,
                                                        int2 *__restrict__ tiles, int max_tiles)
{
    __shared__ int32_t cnt[COLI_MAX_E_DEV + 1];
    __shared__ int32_t scan[COLI_MAX_E_DEV + 2];  // entries cap + shared, plus the total
    const int tid = threadIdx.x;
    const int U = n_union[0];
    const int nent = cap + n_shared;  // entry cap = the shared expert
    for (int e = tid; e < nent; e += blockDim.x) {
        int n = 0;
        if (e < cap) {
            if (e < U) n = offsets[e + 1] - offsets[e];
        } else {
            n = T;
        }
        cnt[e] = (n + kTileM - 1) / kTileM;
    }
    __syncthreads();
    if (tid < 64) {
        // single-wave exclusive scan over nent <= 1025 entries
        int32_t carry = 0;
        for (int base = 0; base < nent; base += 64) {
            int e = base + tid;
            int32_t v = e < nent ? cnt[e] : 0;
            int32_t incl = v;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int32_t o = __shfl_up(incl, off, 64);
                if (tid >= off) incl += o;
            }
            if (e < nent) scan[e] = carry + incl - v;
            carry += __shfl(incl, 63, 64);
        }
        if (tid == 0) scan[nent] = carry;
    }
    __syncthreads();
    for (int e = tid; e < nent; e += blockDim.x) {
        int32_t b = scan[e];
        for (int m = 0; m < cnt[e]; ++m) tiles[b + m] = make_int2(e, m * kTileM);
    }
    if (tid == 0) tiles[max_tiles] = make_int2(min(scan[nent], max_tiles), 0);
}

// --- shared tile bookkeeping ---------------------------------------------
struct I8Args {
    const int8_t *qin;        // activation codes (permuted) [rows][K]
    const float *sin;         // activation scales [rows][K/64]
    int in_by_slot;           // 0: input row = token, 1: input row = output row
    const uint8_t *w; const uint16_t *s;        // routed [E][N][K/2], [E][N][K/64]
    const uint8_t *sh_w; const uint16_t *sh_s;  // shared
    int N, K, I, H;
    const int32_t *union_ids, *offsets, *slots;
    const int2 *tiles;
    int max_tiles;
    int T, k, cap;
    // outputs
    int8_t *qh; float *sh;    // gate/up: quantised h (permuted) and scales
    float *o;                 // down: [R][H]
    int32_t *dump_acc;        // [R][N][K/64] or null
    int8_t *dump_qh; float *dump_sh;
};

__device__ __forceinline__ v4i unpack_b(uint2 w)
{
    v4i r;
    r[0] = (int)((w.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)(w.x & 0xF0F0F0F0u);
    r[2] = (int)((w.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)(w.y & 0xF0F0F0F0u);
    return r;
}

// Resolve the tile: entry, weight base, rows.  Returns false if past count.
__device__ __forceinline__ bool tile_rows(const I8Args &a, int tile, int lane_m, int &mt,
                                          int &in_row, int &out_row, const uint8_t *&wb,
                                          const uint16_t *&sb)
{
    const int count = a.tiles[a.max_tiles].x;
    if (tile >= count) return false;
    const int2 td = a.tiles[tile];
    const int ue = td.x, m0 = td.y;
    const int TK = a.T * a.k;
    if (ue < a.cap) {
        const int e = a.union_ids[ue];
        const int o0 = a.offsets[ue];
        const int n = a.offsets[ue + 1] - o0;
        mt = min(kTileM, n - m0);
        wb = a.w + (size_t)e * a.N * (a.K / 2);
        sb = a.s + (size_t)e * a.N * (a.K / 64);
        const int m = min(lane_m, mt - 1);
        const int sl = a.slots[o0 + m0 + m];
        out_row = sl;
        in_row = a.in_by_slot ? sl : sl / a.k;
    } else {
        mt = min(kTileM, a.T - m0);
        wb = a.sh_w;
        sb = a.sh_s;
        const int t = m0 + min(lane_m, mt - 1);
        out_row = TK + t;
        in_row = a.in_by_slot ? TK + t : t;
    }
    return true;
}

// --- gate/up GEMM + SwiGLU + quantisation of h ---------------------------
// grid: (ceil(I / 256), max_tiles); 4 waves, wave w owns i in [i0, i0 + 64)
__global__ __launch_bounds__(256) void ggemm_gateup_kernel(I8Args a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int i0 = (blockIdx.x * 4 + wave) * 64;
    if (i0 >= a.I) return;
    int mt, a_in, a_out;
    const uint8_t *wb;
    const uint16_t *sb;
    // A-operand row (token m = lane & 15)
    if (!tile_rows(a, blockIdx.y, n, mt, a_in, a_out, wb, sb)) return;
    const bool a_valid = n < mt;
    // C rows owned by this lane: m = 4q + i
    int c_in[4], c_out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int mt2, wi, wo;
        const uint8_t *wb2;
        const uint16_t *sb2;
        tile_rows(a, blockIdx.y, 4 * q + i, mt2, wi, wo, wb2, sb2);
        c_in[i] = wi;
        c_out[i] = wo;
    }
    const int K = a.K, G = K / 64, rb = K / 2;
    const int8_t *arow = a.qin + (size_t)a_in * K + 16 * q;
    const uint8_t *brow[8];
    const uint16_t *srow[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int r = (b < 4) ? (i0 + 16 * b + n) : (a.I + i0 + 16 * (b - 4) + n);
        brow[b] = wb + (size_t)r * rb + 8 * q;
        srow[b] = sb + (size_t)r * G;
    }
    float out[8][4];
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[b][i] = 0.f;
    const v4i zero = {0, 0, 0, 0};

    for (int g = 0; g < G; ++g) {
        v4i av = zero;
        if (a_valid) av = *reinterpret_cast<const v4i *>(arow + 64 * g);
        float sx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[i] = a.sin[(size_t)c_in[i] * G + g];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint2 wv = *reinterpret_cast<const uint2 *>(brow[b] + 32 * g);
            const v4i bv = unpack_b(wv);
            const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, zero, 0, 0, 0);
            const float sw = f16_to_f32(srow[b][g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int iacc = acc[i] >> 4;
                if (a.dump_acc && 4 * q + i < mt) {
                    const int r = (b < 4) ? (i0 + 16 * b + n) : (a.I + i0 + 16 * (b - 4) + n);
                    a.dump_acc[((size_t)c_out[i] * a.N + r) * G + g] = iacc;
                }
                const float p = (float)iacc * sx[i];
                out[b][i] = fmaf(p, sw, out[b][i]);
            }
        }
    }

    // SwiGLU and int8 quantisation of the 64-wide h group [i0, i0 + 64)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float hv[4];
        float amax = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float gg = out[b][i], uu = out[b + 4][i];
            hv[b] = gg / (1.0f + expf(-gg)) * uu;
            amax = fmaxf(amax, fabsf(hv[b]));
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const bool valid = 4 * q + i < mt;
        float sc = 0.f;
        if (amax > 0.f) sc = amax / 127.0f;
        if (valid) {
            int8_t *qrow = a.qh + (size_t)c_out[i] * a.I;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = i0 + 16 * b + n;
                int8_t code = 0;
                if (amax > 0.f) {
                    float r = rintf(hv[b] / sc);
                    r = fminf(fmaxf(r, -127.f), 127.f);
                    code = (int8_t)r;
                }
                qrow[perm8_pos(col)] = code;
                if (a.dump_qh) a.dump_qh[(size_t)c_out[i] * a.I + col] = code;
            }
            if (n == 0) {
                a.sh[(size_t)c_out[i] * (a.I / 64) + i0 / 64] = sc;
                if (a.dump_sh) a.dump_sh[(size_t)c_out[i] * (a.I / 64) + i0 / 64] = sc;
            }
        }
    }
}

// --- down GEMM -------------------------------------------------------------
// grid: (ceil(H / 256), max_tiles); wave w owns rows [n0, n0 + 64)
__global__ __launch_bounds__(256) void ggemm_down_kernel(I8Args a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int n0 = (blockIdx.x * 4 + wave) * 64;
    if (n0 >= a.N) return;
    int mt, a_in, a_out;
    const uint8_t *wb;
    const uint16_t *sb;
    if (!tile_rows(a, blockIdx.y, n, mt, a_in, a_out, wb, sb)) return;
    const bool a_valid = n < mt;
    int c_in[4], c_out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int mt2, wi, wo;
        const uint8_t *wb2;
        const uint16_t *sb2;
        tile_rows(a, blockIdx.y, 4 * q + i, mt2, wi, wo, wb2, sb2);
        c_in[i] = wi;
        c_out[i] = wo;
    }
    const int K = a.K, G = K / 64, rb = K / 2;
    const int8_t *arow = a.qin + (size_t)a_in * K + 16 * q;
    const uint8_t *brow[4];
    const uint16_t *srow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int r = n0 + 16 * b + n;
        brow[b] = wb + (size_t)r * rb + 8 * q;
        srow[b] = sb + (size_t)r * G;
    }
    float out[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[b][i] = 0.f;
    const v4i zero = {0, 0, 0, 0};
    for (int g = 0; g < G; ++g) {
        v4i av = zero;
        if (a_valid) av = *reinterpret_cast<const v4i *>(arow + 64 * g);
        float sx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[i] = a.sin[(size_t)c_in[i] * G + g];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint2 wv = *reinterpret_cast<const uint2 *>(brow[b] + 32 * g);
            const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, unpack_b(wv), zero, 0, 0, 0);
            const float sw = f16_to_f32(srow[b][g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int iacc = acc[i] >> 4;
                if (a.dump_acc && 4 * q + i < mt)
                    a.dump_acc[((size_t)c_out[i] * a.N + n0 + 16 * b + n) * G + g] = iacc;
                out[b][i] = fmaf((float)iacc * sx[i], sw, out[b][i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (4 * q + i >= mt) continue;
        float *orow = a.o + (size_t)c_out[i] * a.H;
#pragma unroll
        for (int b = 0; b < 4; ++b) orow[n0 + 16 * b + n] = out[b][i];
    }
}

hipError_t launch_forward_i8(const LayerDev &L, const ForwardIO &io, hipStream_t st, Marks *mk)
{
    const int T = io.T;
    if (T <= 0) return hipSuccess;
    const Workspace &lay = io.lay;
    int8_t *qx = reinterpret_cast<int8_t *>(io.ws + lay.qx);
    float *sx = reinterpret_cast<float *>(io.ws + lay.sx);
    int8_t *qh = reinterpret_cast<int8_t *>(io.ws + lay.qh);
    float *sh = reinterpret_cast<float *>(io.ws + lay.sh);
    float *o = reinterpret_cast<float *>(io.ws + lay.o);
    int2 *tiles = reinterpret_cast<int2 *>(io.ws + lay.tiles);

    const int64_t ng = (int64_t)T * (L.H / 64);
    if (mk) mk->mark(st);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((ng + 3) / 4)), dim3(256), 0, st, io.x, ng,
                       L.H, qx, sx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mk) mk->mark(st);
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, st, io.offsets, io.n_union,
                       (int)lay.cap, T, L.n_shared, tiles, (int)lay.max_tiles);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    I8Args a{};
    a.union_ids = io.union_ids; a.offsets = io.offsets; a.slots = io.slots;
    a.tiles = tiles; a.max_tiles = (int)lay.max_tiles;
    a.T = T; a.k = L.k; a.cap = (int)lay.cap; a.I = L.I; a.H = L.H;
    a.qh = qh; a.sh = sh; a.o = o;
    int32_t *dump = io.acc_dump;
    uint8_t *dump_b = reinterpret_cast<uint8_t *>(dump);
    // gate/up
    a.qin = qx; a.sin = sx; a.in_by_slot = 0;
    a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
    a.N = 2 * L.I; a.K = L.H;
    a.dump_acc = dump ? reinterpret_cast<int32_t *>(dump_b + io.dump.acc13) : nullptr;
    a.dump_qh = dump ? reinterpret_cast<int8_t *>(dump_b + io.dump.qh) : nullptr;
    a.dump_sh = dump ? reinterpret_cast<float *>(dump_b + io.dump.sh) : nullptr;
    if (mk) mk->mark(st);
    hipLaunchKernelGGL(ggemm_gateup_kernel, dim3((L.I + 255) / 256, (unsigned)lay.max_tiles),
                       dim3(256), 0, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // down
    a.qin = qh; a.sin = sh; a.in_by_slot = 1;
    a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
    a.N = L.H; a.K = L.I;
    a.dump_acc = dump ? reinterpret_cast<int32_t *>(dump_b + io.dump.acc2) : nullptr;
    a.dump_qh = nullptr; a.dump_sh = nullptr;
    if (mk) mk->mark(st);
    hipLaunchKernelGGL(ggemm_down_kernel, dim3((L.H + 255) / 256, (unsigned)lay.max_tiles),
                       dim3(256), 0, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (mk) mk->mark(st);
    err = launch_combine(o, io.w, T, L.k, L.H, L.n_shared, io.y, st);
    if (mk) mk->mark(st);
    return err;
}

}  // namespace coli
