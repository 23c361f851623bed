// mla.hip -- decode attention over the compressed (MLA) KV cache
// (C ABI in include/coli_mla.h).
//
// mcpfield.com "Colibri", section "コアアーキテクチャ" item 5, and the
// dashen-tech.com guide, table "コア技術のハイライト": the KV cache keeps 576
// floats per token.  Read as latent (512) + rotary key (64); queries arrive
// absorbed (576 floats per head), so every head attends the same cache rows:
// the keys are shared by all heads of a query, as in multi-query attention.
//
// mla_attn_kernel: one workgroup = 8 waves for 64 heads of one query and
// one range of its keys; the two waves of a pair share 16 heads and split
// the work in halves (score dims 0..287 / 288..575, output dims 0..255 /
// 256..511).  Keys are staged 16 at a time through three LDS buffers (the
// next tile's loads are in flight during the current tile, one barrier per
// tile).  Everything is computed transposed, with the heads as the MFMA
// columns: a wave forms its half of S^T = K Q^T (v_mfma_f32_16x16x4_f32, 72
// per tile; its query half lives in 72 registers as B operands), the pair
// adds the halves through LDS (the same sum in both waves), both run the same
// online base-2 softmax per head (column), and each accumulates
// O^T += V^T P^T into its 16 output tiles.  In that orientation the
// probabilities are already where the next MFMA wants its B operand (key
// 4k + s of k-step s sits in register s of the lanes of k-slot k), and the
// rescale of a head's accumulators is lane-local.  The cached row serves as
// key (576 dims) and value (first 512).  Partial (max, sum, unnormalised
// output) per head and key range go to the workspace; mla_merge_kernel
// combines the ranges in a fixed order.
#include "../../include/coli_mla.h"

#include <hip/hip_runtime.h>

#include <math.h>

#include "common.h"

namespace coli {
namespace {

constexpr int kD = 576, kDv = 512;
constexpr int kKT = 16;        // keys per staged tile
constexpr int kStr = kD + 4;   // LDS row stride in floats (conflict-free b128 reads)
// partial record: O[512], m, l, padding to whole 128-byte lines (records of
// different workgroups never share a cache line)
constexpr int kRec = kDv + 32;
constexpr int kHeadsPerBlock = 64;

using v4f = __attribute__((__vector_size__(4 * sizeof(float)))) float;

struct MlaArgs {
    const float *q, *kv;
    const int32_t *lens, *idx;
    float *part;  // [B][S][H][kRec]
    int B, H, T, n_sel, S, kps, HG, G;
    float sl2;    // scale * log2(e)
};

struct MlaLds {
    float kt[3][kKT][kStr];  // 111,360 B
    float4 sx[2][8][64];     // score halves, by tile parity, 16,384 B
};

// Output dim of tile c = 4u + i (u < 4), column n, within a half:
// 16n + 4 sigma(u, n) + i.  The rotation sigma puts the lanes that read
// their value segments in one LDS pass (8 lanes of 16 bytes on 32 banks,
// 16 lanes on 64) on distinct banks.
__device__ __forceinline__ int vseg(int u, int n)
{
    return 16 * n + 4 * ((u + (n >> 1) + (n >> 3)) & 3);
}

// LIST: the keys of a query are the rows of its key list, else its prefix.
template <bool LIST>
__global__ __launch_bounds__(512, 1) void mla_attn_kernel(MlaArgs a)
{
    __shared__ MlaLds sm;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, q4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = wave >> 1, half = wave & 1;
    // XCD-aware order: blocks p and p + 8 run on one XCD; consecutive L
    // (the head groups of one key range) share that XCD's L2
    const int p = blockIdx.x;
    const int L = (p & 7) * ((int)gridDim.x >> 3) + (p >> 3);
    if (L >= a.G) return;
    const int hg = L % a.HG;
    const int split = (L / a.HG) % a.S;
    const int b = L / (a.HG * a.S);
    int nkeys;
    if constexpr (LIST) nkeys = a.n_sel;
    else nkeys = min(max(a.lens[b], 0), a.T);
    const int k0 = split * a.kps;
    const int k1 = min(nkeys, k0 + a.kps);
    const int ntiles = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;
    const int h0 = hg * kHeadsPerBlock + hb * 16;
    const bool live = h0 < a.H;  // uniform over the wave pair

    // staging: thread tid moves float4s e = it * 512 + tid of the 16 x 144 tile
    constexpr int kTile4 = kKT * (kD / 4);          // 2,304
    constexpr int kPer = (kTile4 + 511) / 512;      // 5
    float4 stage[kPer];
    // cache row of key position pos, -1 if none.  Loads are unconditional
    // (positions clamped into the range) so that they all stay in flight.
    auto key_row = [&](int pos) -> int {
        if constexpr (LIST) {
            const int t = a.idx[(size_t)b * a.n_sel + min(pos, k1 - 1)];
            return (pos < k1 && t >= 0 && t < a.T) ? t : -1;
        } else {
            return pos < k1 ? pos : -1;
        }
    };
    auto load_tile = [&](int tile) {
        const int kk = k0 + tile * kKT;
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int e = it * 512 + tid;
            const int r = e / (kD / 4), c = e % (kD / 4);
            const int t = e < kTile4 ? key_row(kk + r) : -1;
            const float4 v = reinterpret_cast<const float4 *>(a.kv + (size_t)max(t, 0) * kD)[c];
            stage[it] = t >= 0 ? v : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int e = it * 512 + tid;
            const int r = e / (kD / 4), c = e % (kD / 4);
            if (e < kTile4) *reinterpret_cast<float4 *>(&sm.kt[buf][r][4 * c]) = stage[it];
        }
    };

    v4f o[16];  // O^T tiles: o[4u + i][v] = O[head h0 + n][dim of row 4 q4 + v]
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = v4f{0.f, 0.f, 0.f, 0.f};
    float mcol = -INFINITY, lpart = 0.f;  // softmax state of head h0 + n

    // the first key tile's loads go out before the query's
    if (ntiles > 0) load_tile(0);
    // this wave's half of the query of head h0 + n as MFMA B operands:
    // qa[4m + i] holds dim 16 (18 half + m) + 4 q4 + i
    float qa[72];
    {
        const int hr = h0 + n;
        const bool ok = live && hr < a.H;
        const float4 *qr = reinterpret_cast<const float4 *>(
            a.q + ((size_t)b * a.H + (ok ? hr : 0)) * kD) + 72 * half;
#pragma unroll
        for (int m = 0; m < 18; ++m) {
            const float4 v = qr[4 * m + q4];  // row 0 stands in for a missing head
            qa[4 * m + 0] = ok ? v.x : 0.f; qa[4 * m + 1] = ok ? v.y : 0.f;
            qa[4 * m + 2] = ok ? v.z : 0.f; qa[4 * m + 3] = ok ? v.w : 0.f;
        }
    }

    // this half of S^T[key 4 q4 + v][head n] for the tile in buffer buf
    auto scores = [&](int buf) -> v4f {
        v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        const float *kr = &sm.kt[buf][n][4 * q4 + 288 * half];
#pragma unroll
        for (int m = 0; m < 18; ++m) {
            const float4 kb = *reinterpret_cast<const float4 *>(kr + 16 * m);
            v4f &acc = (m & 1) ? s1 : s0;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.x, qa[4 * m + 0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.y, qa[4 * m + 1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.z, qa[4 * m + 2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.w, qa[4 * m + 3], acc, 0, 0, 0);
        }
        // keep two operand reads in flight ahead of the matrix-core ops
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        return s0 + s1;
    };

    // Software pipeline: iteration t runs the softmax of tile t, the scores
    // of tile t + 1 and the P x V of tile t (independent matrix-core work
    // around the softmax), stores tile t + 2 into the buffer tile t - 1 left,
    // and ends with the one barrier that publishes both.
    if (ntiles > 0) {
        store_tile(0);
        if (ntiles > 1) load_tile(1);
    }
    __syncthreads();
    v4f sh = {0.f, 0.f, 0.f, 0.f};
    if (ntiles > 0) {
        if (live) sh = scores(0);
        if (ntiles > 1) store_tile(1);
        if (live) sm.sx[0][wave][lane] = make_float4(sh[0], sh[1], sh[2], sh[3]);
        __syncthreads();
        if (ntiles > 2) load_tile(2);
    }
    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile % 3;
        const bool more = tile + 1 < ntiles;  // uniform
        v4f sn = {0.f, 0.f, 0.f, 0.f};
        if (live) {
            // both waves of the pair form the same sum: low half + high half
            const float4 ot = sm.sx[tile & 1][wave ^ 1][lane];
            const v4f ov = {ot.x, ot.y, ot.z, ot.w};
            const v4f full = half == 0 ? sh + ov : ov + sh;
            const int kp = k0 + tile * kKT + 4 * q4;
            float sv[4];
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                sv[v] = key_row(kp + v) >= 0 ? full[v] * a.sl2 : -INFINITY;
                mx = fmaxf(mx, sv[v]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(mcol, mx);
            const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mcol - mn);
            float pv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) pv[v] = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[v] - mn);
            lpart = lpart * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
            mcol = mn;
            if (more) sn = scores((tile + 1) % 3);
            // the accumulators change only when some head's running max rose
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int c = 0; c < 16; ++c) o[c] *= alpha;
            }
            // O^T += V^T P^T; k-step s takes key 4k + s in k-slot k
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float *vr = &sm.kt[buf][4 * q4 + s][256 * half];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float4 vb = *reinterpret_cast<const float4 *>(vr + vseg(u, n));
                    o[4 * u + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.x, pv[s], o[4 * u + 0], 0, 0, 0);
                    o[4 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.y, pv[s], o[4 * u + 1], 0, 0, 0);
                    o[4 * u + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.z, pv[s], o[4 * u + 2], 0, 0, 0);
                    o[4 * u + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.w, pv[s], o[4 * u + 3], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int g = 0; g < 14; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        if (more) {
            if (tile + 2 < ntiles) store_tile((tile + 2) % 3);
            if (live) sm.sx[(tile + 1) & 1][wave][lane] = make_float4(sn[0], sn[1], sn[2], sn[3]);
            __syncthreads();
            if (tile + 3 < ntiles) load_tile(tile + 3);
            sh = sn;
        }
    }

    // partial record of head h0 + n: O (this half), m and l (low half)
    if (!live) return;
    float l = lpart;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int h = h0 + n;
    if (h >= a.H) return;
    float *rec = a.part + (((size_t)b * a.S + split) * a.H + h) * kRec + 256 * half;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<float4 *>(rec + vseg(u, 4 * q4 + v)) =
                make_float4(o[4 * u + 0][v], o[4 * u + 1][v], o[4 * u + 2][v], o[4 * u + 3][v]);
    if (half == 0 && q4 == 0) {
        rec[kDv] = mcol;
        rec[kDv + 1] = l;
    }
}

// out[b][h] = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max m); zeros
// when no range saw a key.  Block (b h, quarter): 8 groups of 32 threads,
// group g sums the ranges s = g mod 8 for 128 output dims, then the groups
// are added in ascending order (a fixed order: bitwise reproducible).
__global__ __launch_bounds__(256) void mla_merge_kernel(const float *__restrict__ part, int S, int H,
                                                        float *__restrict__ out)
{
    __shared__ float red[8];
    __shared__ float4 acc_g[8][32];
    const int bh = blockIdx.x >> 2, quarter = blockIdx.x & 3;
    const int tid = threadIdx.x, g = tid >> 5, t = tid & 31;
    const int b = bh / H, h = bh % H;
    const size_t rs = (size_t)H * kRec;  // from one key range to the next
    const float *pr = part + ((size_t)b * S * H + h) * kRec;
    // max and denominator over all ranges (block reductions)
    float m = -INFINITY;
    for (int s = tid; s < S; s += 256) m = fmaxf(m, pr[(size_t)s * rs + kDv]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float d = 0.f;
    if (M != -INFINITY)
        for (int s = tid; s < S; s += 256) {
            const float ms = pr[(size_t)s * rs + kDv];
            if (ms != -INFINITY) d += __builtin_amdgcn_exp2f(ms - M) * pr[(size_t)s * rs + kDv + 1];
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = d;
    // this group's ranges, eight records in flight at a time (a range that
    // saw no key has m = -inf and O = 0: weight 0)
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
        for (int s0 = g; s0 < S; s0 += 64) {
            float ms[8];
            float4 ov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = s0 + 8 * j;
                ms[j] = s < S ? pr[(size_t)s * rs + kDv] : -INFINITY;
                ov[j] = s < S ? reinterpret_cast<const float4 *>(pr + (size_t)s * rs)[quarter * 32 + t]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float w = ms[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[j] - M);
                acc.x += w * ov[j].x; acc.y += w * ov[j].y; acc.z += w * ov[j].z; acc.w += w * ov[j].w;
            }
        }
    }
    acc_g[g][t] = acc;
    __syncthreads();
    if (g == 0) {
        const float den = (red[4] + red[5]) + (red[6] + red[7]);
        float4 sum = acc_g[0][t];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            const float4 v = acc_g[j][t];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        reinterpret_cast<float4 *>(out + (size_t)bh * kDv)[quarter * 32 + t] =
            make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    }
}

struct MlaPlan {
    int HG, S, kps, G;
};

// Key ranges: enough (b, head group, range) blocks to give every compute
// unit one, at least 16 keys per range.
MlaPlan mla_plan(int B, int H, int T, int n_sel, bool list, int cus)
{
    MlaPlan p{};
    p.HG = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int nk = list ? n_sel : T;
    const int units = B * p.HG;
    int S = (cus + units - 1) / units;
    const int max_s = (nk + kKT - 1) / kKT;
    S = S < 1 ? 1 : (S > max_s ? max_s : S);
    const int per = (nk + S - 1) / S;
    p.kps = (per + kKT - 1) / kKT * kKT;
    p.S = (nk + p.kps - 1) / p.kps;
    p.G = B * p.HG * p.S;
    return p;
}

int check_args(const float *q, int32_t B, int32_t n_heads, const float *kv, int32_t T,
               const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale, float *out,
               void *workspace)
{
    if (B < 1 || B > COLI_MLA_MAX_B || n_heads < 1 || n_heads > COLI_MLA_MAX_HEADS) return COLI_E_SHAPE;
    if (T < 1 || T > COLI_MLA_MAX_T) return COLI_E_SHAPE;
    if (idx && (n_sel < 1 || n_sel > COLI_MLA_MAX_T)) return COLI_E_SHAPE;
    if (!__builtin_isfinite(scale)) return COLI_E_ARG;
    if (!q || !kv || !out || !workspace || (!idx && !lens)) return COLI_E_ARG;
    auto al = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    if (!al(q) || !al(kv) || !al(out) || !al(workspace) || (lens && !al(lens)) || (idx && !al(idx)))
        return COLI_E_ALIGN;
    return COLI_OK;
}

int mla_impl(const float *q, int32_t B, int32_t n_heads, const float *kv, int32_t T,
             const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale, float *out,
             void *workspace, size_t workspace_bytes, Marks *mk, void *hip_stream)
{
    if (int st = check_args(q, B, n_heads, kv, T, lens, idx, n_sel, scale, out, workspace)) return st;
    if (workspace_bytes < coli_mla_workspace_bytes(B, n_heads, T, idx ? n_sel : 0))
        return COLI_E_WORKSPACE;
    if (int st = coli_moe_device_check()) return st;
    const MlaPlan pl = mla_plan(B, n_heads, T, n_sel, idx != nullptr, device_cu_count());
    MlaArgs a{};
    a.q = q; a.kv = kv; a.lens = lens; a.idx = idx;
    a.part = static_cast<float *>(workspace);
    a.B = B; a.H = n_heads; a.T = T; a.n_sel = idx ? n_sel : 0;
    a.S = pl.S; a.kps = pl.kps; a.HG = pl.HG; a.G = pl.G;
    a.sl2 = scale * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const unsigned grid = (unsigned)((pl.G + 7) / 8 * 8);
    if (idx) launch(mk, mla_attn_kernel<true>, dim3(grid), dim3(512), 0, st, a);
    else launch(mk, mla_attn_kernel<false>, dim3(grid), dim3(512), 0, st, a);
    if (hipGetLastError() != hipSuccess) return COLI_E_DEVICE;
    launch(mk, mla_merge_kernel, dim3((unsigned)(B * n_heads * 4)), dim3(256), 0, st,
           (const float *)a.part, pl.S, n_heads, out);
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_E_DEVICE;
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" {

size_t coli_mla_workspace_bytes(int32_t B, int32_t n_heads, int32_t T, int32_t n_sel)
{
    if (B < 1 || B > COLI_MLA_MAX_B || n_heads < 1 || n_heads > COLI_MLA_MAX_HEADS) return 0;
    if (T < 1 || T > COLI_MLA_MAX_T || n_sel < 0 || n_sel > COLI_MLA_MAX_T) return 0;
    // the plan with the most ranges any device may choose (1024 compute units)
    size_t most = 0;
    for (int cus : {device_cu_count(), 1024}) {
        const MlaPlan p = mla_plan(B, n_heads, T, n_sel, n_sel > 0, cus);
        const size_t b = (size_t)B * n_heads * p.S * kRec * 4;
        most = b > most ? b : most;
    }
    return (most + 255) & ~size_t(255);
}

int coli_mla_decode(const float *q, int32_t B, int32_t n_heads, const float *kv, int32_t T,
                    const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale,
                    float *out, void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return mla_impl(q, B, n_heads, kv, T, lens, idx, n_sel, scale, out, workspace,
                    workspace_bytes, nullptr, hip_stream);
}

int coli_mla_decode_profiled(const float *q, int32_t B, int32_t n_heads, const float *kv,
                             int32_t T, const int32_t *lens, const int32_t *idx, int32_t n_sel,
                             float scale, float *out, void *workspace, size_t workspace_bytes,
                             void **events, int32_t n_events, void *hip_stream)
{
    if (!events || n_events < 4) return COLI_E_ARG;
    for (int i = 0; i < 4; ++i)
        if (!events[i]) return COLI_E_ARG;
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    return mla_impl(q, B, n_heads, kv, T, lens, idx, n_sel, scale, out, workspace,
                    workspace_bytes, &mk, hip_stream);
}

}  // extern "C"
