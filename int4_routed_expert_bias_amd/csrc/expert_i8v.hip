// expert_i8v.hip -- the integer arithmetic family for small batches
// (1 <= T <= kI8StreamTMax: decode, draft and verify steps).  The pages run
// decode in f32 and batches on the integer kernel ("Colibri 完全ガイド",
// walk-through "詳細解説" step 3) and note that the two round differently
// ("colibri解説", "使えるかどうかの判定材料"); this path gives small batches the
// integer family's function, so a token's output is the same whether it is
// decoded alone, verified with a few others or prefilled in a large batch.
//
// Same arithmetic as the grouped GEMM (expert_i8.hip), value for value:
//   acc_g  = exact int32 sum over the 64-group g of (int8 activation code) x
//            (16 x int4 code), here from v_dot4_i32_i8 instead of the MFMA;
//   out    = 0; for g ascending: out = fma(float(acc_g) * act_scale_g,
//            w_scale_g / 16, out)    (fp32, one chain per output), the
//            activation scale rounded to 22 significant bits
//            (epi_act_scale);
//   h      = g / (1 + exp(-g)) * u, quantised per 64-group of I with
//            scale = amax / 127, code = clamp(rint(h / scale), +-127).
// Only the work split differs: the weights are streamed once by persistent
// waves through a register ring (as in the fp32 streaming kernels), each
// lane forms the integer partial of one 32-element chunk per row, lane pairs
// add the two halves of a group (exact), and the group terms go through LDS
// to one lane per output that adds them in group order.  The dequantising
// FMAs of the fp32 family are replaced by 0.6 integer instructions per
// weight; the serial group chain per output through LDS is the part that
// keeps these kernels from the weight stream's rate.
#include "common.h"
#include "stream.h"
#include "route_tokens.h"

namespace coli {

struct I8vArgs {
    const uint8_t *w; const uint16_t *s;        // routed [E][N][K/2], [E][N][K/64]
    const uint8_t *sh_w; const uint16_t *sh_s;  // shared expert [N][K/2], [N][K/64]
    int N, K, I;                 // rows, reduction length, up-row offset (gate/up)
    const int8_t *qx; const float *sx;  // gate/up input: codes [T][K] (permuted), scales [T][K/64]
    const float *h;              // down input: SwiGLU outputs [R][K] (natural order)
    float *out; int out_ld;      // gate/up: h [R][I]; down: o [R][H]
    const int32_t *union_ids, *offsets, *slots, *n_union;
    int T, k, n_shared;
    // tests only (DUMP kernels): exact group accumulators [R][N][K/64]
    // (gate/up: acc13, down: acc2) and the down kernel's int8 codes of h
    // [R][I] (natural order) and their scales [R][I/64]
    int32_t *dump_acc;
    int8_t *dump_qh;
    float *dump_sh;
};

// Entry ue (union experts in union order, then the shared expert): weight
// and scale bases and its slot list; returns its token count.
__device__ __forceinline__ int i8v_entry(const I8vArgs &a, int ue, int U, const uint8_t *&wb,
                                         const uint16_t *&sb, const int32_t *&list)
{
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

// Token j of an entry: its token index and its row of h / o (the slot, or
// T*k + t for the shared expert).
__device__ __forceinline__ void i8v_token(const I8vArgs &a, const int32_t *list, int j, int &tok,
                                          int &row)
{
    if (list) {
        const int s = list[j];
        tok = s / a.k;
        row = s;
    } else {
        tok = j;
        row = a.T * a.k + j;
    }
}

// 16 x the exact dot product of a 16-byte chunk of packed int4 codes (32
// elements) with the 32 activation codes of the same elements in the
// permuted order (dword 2d: elements 8d, 8d+2, 8d+4, 8d+6; dword 2d+1: the
// odd ones).  (w << 4) & 0xF0F0F0F0 puts 16 x the even elements' codes in
// signed bytes, w & 0xF0F0F0F0 the odd ones.
__device__ __forceinline__ int dot_chunk_i8(const uint4 &w, const uint32_t (&xq)[8])
{
    int acc = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t q = d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w;
        acc = __builtin_amdgcn_sdot4((int)((q << 4) & 0xF0F0F0F0u), (int)xq[2 * d], acc, false);
        acc = __builtin_amdgcn_sdot4((int)(q & 0xF0F0F0F0u), (int)xq[2 * d + 1], acc, false);
    }
    return acc;
}

// The value of lane l ^ 1 (the other half of a 64-group: chunks 2g, 2g + 1).
__device__ __forceinline__ int pair_lane(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}

__device__ __forceinline__ float pair_lane_f(float v)
{
    return __int_as_float(pair_lane(__float_as_int(v)));
}

// Per-wave LDS of the group terms: t[slot][g] = float(acc_g) * act_scale_g
// for slot = (m * NTOK + token) * NR + r, and ws[m * NR + r][g] = the weight
// scale / 16; rows padded to G + 1 floats (conflict-free column walks).
template <int M, int NTOK, int NR>
struct TermLds {
    float *t, *ws;
    int gs;
    __device__ TermLds(float *base, int G) : gs(G + 1)
    {
        t = base;
        ws = base + M * NTOK * NR * gs;
    }
    static constexpr int rows() { return M * NTOK * NR + M * NR; }
};

// One output: the fp32 chain over the groups in ascending order.
__device__ __forceinline__ float group_chain(const float *t, const float *ws, int G)
{
    float out = 0.f;
    for (int g = 0; g < G; ++g) out = fmaf(t[g], ws[g], out);
    return out;
}

// Gate/up + SwiGLU.  Unit = gate row i and up row I + i of one entry; the
// waves of an entry take its units round-robin (t1_split).  Writes h rows
// (natural order) for every token of the entry.
// ROUTE (one token): the workgroup first selects the token's experts and
// forms the union itself from its sigmoid scores (route_self, as the fp32
// single-token gate/up kernel), then reads the union from LDS.
template <int P, int M, int DEPTH, int NTOK, bool ROUTE, bool DUMP = false>
__global__ __launch_bounds__(256) void gateup_i8v_kernel(I8vArgs a, RouteSelf r)
{
    static_assert(M % DEPTH == 0, "stage ring must divide the batch");
    static_assert(!ROUTE || NTOK == 1, "a routing gate/up kernel serves one token");
    extern __shared__ float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, G = K / 64;
    // this lane's activation codes and scales for every token of the entry
    // (ROUTE: the one token's, loaded before the selection so that their
    // latency overlaps it)
    uint32_t xq[NTOK][P][8];
    float xs[NTOK][P];
    auto load_x = [&](int j, int tok) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = min(lane + 64 * p, C - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(a.qx + (size_t)tok * K + 32 * c);
            const uint4 lo = src[0], hi = src[1];
            xq[j][p][0] = lo.x; xq[j][p][1] = lo.y; xq[j][p][2] = lo.z; xq[j][p][3] = lo.w;
            xq[j][p][4] = hi.x; xq[j][p][5] = hi.y; xq[j][p][6] = hi.z; xq[j][p][7] = hi.w;
            xs[j][p] = epi_act_scale(a.sx[(size_t)tok * G + (c >> 1)]);
        }
    };
    if constexpr (ROUTE) load_x(0, 0);
    int U;
    if constexpr (ROUTE) {
        __shared__ RouteLds rl;
        route_self(r, rl);
        a.union_ids = rl.u;
        a.offsets = rl.off;
        a.slots = rl.sl;
        a.n_union = rl.n;
        U = __builtin_amdgcn_readfirstlane(rl.n[0]);
    } else {
        U = a.n_union[0];
    }
    const T1Split sp = t1_split(blockIdx.x * 4 + wave, gridDim.x * 4, U + a.n_shared, a.I);
    const int nsteps = sp.nsteps;
    if (nsteps == 0) return;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    int cnt;
    if constexpr (ROUTE) {
        // (the union is in LDS, read per lane: its values made uniform)
        if (sp.ue < U) {
            const int e = __builtin_amdgcn_readfirstlane(a.union_ids[sp.ue]);
            wb = a.w + (size_t)e * a.N * (a.K / 2);
            sb = a.s + (size_t)e * a.N * (a.K / 64);
            const int o0 = __builtin_amdgcn_readfirstlane(a.offsets[sp.ue]);
            list = a.slots + o0;
            cnt = __builtin_amdgcn_readfirstlane(a.offsets[sp.ue + 1]) - o0;
        } else {
            wb = a.sh_w;
            sb = a.sh_s;
            list = nullptr;
            cnt = a.T;
        }
        cnt = min(cnt, NTOK);
    } else {
        cnt = min(i8v_entry(a, sp.ue, U, wb, sb, list), NTOK);
    }
    if (cnt <= 0) return;
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

    int orow[NTOK];
#pragma unroll
    for (int j = 0; j < NTOK; ++j) {
        int tok = 0, row = 0;
        if (j < cnt) i8v_token(a, list, j, tok, row);
        orow[j] = row;
        if constexpr (!ROUTE) load_x(j, tok);
    }
    using Lds = TermLds<M, NTOK, 2>;
    Lds tl(lds + (size_t)wave * Lds::rows() * (G + 1), G);
    const bool writer = (lane & 1) == 0;

    for (int g0 = 0; g0 < nsteps; g0 += M) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        const int c = lane + 64 * p, g = c >> 1;
                        if (writer && c < C)
                            tl.ws[(m * 2 + r) * tl.gs + g] = f16_to_f32(sv[d][r][p]) * 0.0625f;
                    }
                auto stage = [&](auto cnt_c) {
                    constexpr int CNT = decltype(cnt_c)::value;
#pragma unroll
                    for (int j = 0; j < CNT; ++j)
#pragma unroll
                        for (int r = 0; r < 2; ++r)
#pragma unroll
                            for (int p = 0; p < P; ++p) {
                                int acc = dot_chunk_i8(wv[d][r][p], xq[j][p]);
                                acc += pair_lane(acc);
                                const int c = lane + 64 * p, g = c >> 1;
                                if (writer && c < C) {
                                    tl.t[((m * NTOK + j) * 2 + r) * tl.gs + g] = (float)acc * xs[j][p];
                                    if constexpr (DUMP) {
                                        const int blk = sp.part + (g0 + m) * sp.wpe;
                                        const int row = r == 0 ? blk : a.I + blk;
                                        a.dump_acc[((size_t)orow[j] * a.N + row) * G + g] = acc >> 4;
                                    }
                                }
                            }
                };
                dispatch_count<NTOK>(cnt, stage);
            }
            issue(d, g0 + m + DEPTH);
        }
        __builtin_amdgcn_wave_barrier();
        // one lane per (token, unit): gate and up chains, then SwiGLU
        const int j = lane / M, m = lane % M;
        if (lane < M * cnt && g0 + m < nsteps) {
            const float gg = group_chain(tl.t + ((m * NTOK + j) * 2 + 0) * tl.gs, tl.ws + (m * 2 + 0) * tl.gs, G);
            const float uu = group_chain(tl.t + ((m * NTOK + j) * 2 + 1) * tl.gs, tl.ws + (m * 2 + 1) * tl.gs, G);
            const int i = sp.part + (g0 + m) * sp.wpe;
            a.out[(size_t)orow[j] * a.out_ld + i] = gg / (1.0f + expf(-gg)) * uu;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Down.  Unit = RD rows of one entry.  Each wave quantises the h rows of its
// entry's tokens itself (per 64-group, the gate/up GEMM epilogue's
// arithmetic) into registers, then streams its rows.
template <int P, int RD, int M, int DEPTH, int NTOK, bool DUMP = false>
__global__ __launch_bounds__(256) void down_i8v_kernel(I8vArgs a)
{
    static_assert(M % DEPTH == 0, "stage ring must divide the batch");
    extern __shared__ float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int K = a.K, rb = K / 2, sbs = K / 64, C = K / 32, G = K / 64;
    const int U = a.n_union[0];
    const T1Split sp = t1_split(blockIdx.x * 4 + wave, gridDim.x * 4, U + a.n_shared, a.N / RD);
    const int nsteps = sp.nsteps;
    if (nsteps == 0) return;
    const uint8_t *wb;
    const uint16_t *sb;
    const int32_t *list;
    const int cnt = min(i8v_entry(a, sp.ue, U, wb, sb, list), NTOK);
    if (cnt <= 0) return;
    const StageRsrc R = stage_rsrc(wb, sb, a.N, rb, sbs);
    uint32_t vw[P], vs[P];
    lane_offsets<P>(lane, C, vw, vs);

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

    // quantise this lane's chunk of every token's h row: the group's amax
    // comes from the lane pair holding its two chunks
    uint32_t xq[NTOK][P][8];
    float xs[NTOK][P];
    int orow[NTOK];
#pragma unroll
    for (int j = 0; j < NTOK; ++j) {
        int tok = 0, row = 0;
        if (j < cnt) i8v_token(a, list, j, tok, row);
        orow[j] = row;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = min(lane + 64 * p, C - 1);
            const float4 *src = reinterpret_cast<const float4 *>(a.h + (size_t)row * K + 32 * c);
            float v[32];
#pragma unroll
            for (int qd = 0; qd < 8; ++qd) {
                const float4 f = src[qd];
                v[4 * qd] = f.x; v[4 * qd + 1] = f.y; v[4 * qd + 2] = f.z; v[4 * qd + 3] = f.w;
            }
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
            amax = fmaxf(amax, pair_lane_f(amax));
            const float sc = amax > 0.f ? amax / 127.0f : 0.f;
            xs[j][p] = epi_act_scale(sc);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                uint32_t ev = 0, od = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    int ce = 0, co = 0;
                    if (amax > 0.f) {
                        ce = (int)fminf(fmaxf(rintf(v[8 * blk + 2 * b] / sc), -127.f), 127.f);
                        co = (int)fminf(fmaxf(rintf(v[8 * blk + 2 * b + 1] / sc), -127.f), 127.f);
                    }
                    ev |= ((uint32_t)ce & 0xFFu) << (8 * b);
                    od |= ((uint32_t)co & 0xFFu) << (8 * b);
                }
                xq[j][p][2 * blk] = ev;
                xq[j][p][2 * blk + 1] = od;
                if constexpr (DUMP) {
                    // every wave of the entry holds the same codes: the one
                    // with the first row block writes them in natural order
                    if (sp.part == 0 && j < cnt && lane + 64 * p < C) {
                        uint32_t *dq = reinterpret_cast<uint32_t *>(
                            a.dump_qh + (size_t)row * K + 32 * (lane + 64 * p) + 8 * blk);
                        dq[0] = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // e0 o0 e1 o1
                        dq[1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // e2 o2 e3 o3
                    }
                }
            }
            if constexpr (DUMP) {
                if (sp.part == 0 && j < cnt && (lane & 1) == 0 && lane + 64 * p < C)
                    a.dump_sh[(size_t)row * G + ((lane + 64 * p) >> 1)] = sc;
            }
        }
    }
    using Lds = TermLds<M, NTOK, RD>;
    Lds tl(lds + (size_t)wave * Lds::rows() * (G + 1), G);
    const bool writer = (lane & 1) == 0;

    for (int g0 = 0; g0 < nsteps; g0 += M) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int d = m % DEPTH;
            if (g0 + m < nsteps) {
#pragma unroll
                for (int r = 0; r < RD; ++r)
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        const int c = lane + 64 * p, g = c >> 1;
                        if (writer && c < C)
                            tl.ws[(m * RD + r) * tl.gs + g] = f16_to_f32(sv[d][r][p]) * 0.0625f;
                    }
                auto stage = [&](auto cnt_c) {
                    constexpr int CNT = decltype(cnt_c)::value;
#pragma unroll
                    for (int j = 0; j < CNT; ++j)
#pragma unroll
                        for (int r = 0; r < RD; ++r)
#pragma unroll
                            for (int p = 0; p < P; ++p) {
                                int acc = dot_chunk_i8(wv[d][r][p], xq[j][p]);
                                acc += pair_lane(acc);
                                const int c = lane + 64 * p, g = c >> 1;
                                if (writer && c < C) {
                                    tl.t[((m * NTOK + j) * RD + r) * tl.gs + g] = (float)acc * xs[j][p];
                                    if constexpr (DUMP) {
                                        const int row = (sp.part + (g0 + m) * sp.wpe) * RD + r;
                                        a.dump_acc[((size_t)orow[j] * a.N + row) * G + g] = acc >> 4;
                                    }
                                }
                            }
                };
                dispatch_count<NTOK>(cnt, stage);
            }
            issue(d, g0 + m + DEPTH);
        }
        __builtin_amdgcn_wave_barrier();
        // one lane per (token, row)
        const int j = lane / (M * RD), m = (lane / RD) % M, r = lane % RD;
        if (lane < M * RD * cnt && g0 + m < nsteps) {
            const float o = group_chain(tl.t + ((m * NTOK + j) * RD + r) * tl.gs, tl.ws + (m * RD + r) * tl.gs, G);
            a.out[(size_t)orow[j] * a.out_ld + (sp.part + (g0 + m) * sp.wpe) * RD + r] = o;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <int NTOK>
static hipError_t launch_i8v(const LayerDev &L, const ForwardIO &io, I8vArgs a, float *h, float *o,
                             hipStream_t st, Marks *mk)
{
    const int cus = device_cu_count();
    const int entries = (int)io.lay.cap + L.n_shared;
    uint8_t *dump = reinterpret_cast<uint8_t *>(io.acc_dump);  // tests only
    {
        // measured on MI355X with the decode layer: one token streams best with
        // two workgroups per CU and a three-stage ring (28.6 us vs 32.2 for one
        // workgroup and two stages); several tokens keep one workgroup per CU
        // (their term buffers in LDS)
        constexpr int M = NTOK == 1 ? 6 : 4, DEPTH = NTOK == 1 ? 3 : 2;
        using Lds = TermLds<M, NTOK, 2>;
        a.w = L.w13; a.s = L.s13; a.sh_w = L.sh_w13; a.sh_s = L.sh_s13;
        a.N = 2 * L.I; a.K = L.H;
        a.out = h; a.out_ld = L.I;
        a.dump_acc = dump ? reinterpret_cast<int32_t *>(dump + io.dump.acc13) : nullptr;
        const int P = (L.H / 32 + 63) / 64;
        const size_t lds = (size_t)4 * Lds::rows() * (L.H / 64 + 1) * 4;
        const dim3 grid(std::max((NTOK == 1 ? 2 : 1) * cus, (entries + 3) / 4)), block(256);
#define COLI_GUV(P_) \
        if (P == P_) { \
            if (NTOK == 1 && io.route) \
                launch(mk, (gateup_i8v_kernel<P_, M, DEPTH, NTOK, NTOK == 1>), grid, block, lds, st, a, \
                       *io.route); \
            else if (dump) \
                launch(mk, (gateup_i8v_kernel<P_, M, DEPTH, NTOK, false, true>), grid, block, lds, st, \
                       a, RouteSelf{}); \
            else launch(mk, (gateup_i8v_kernel<P_, M, DEPTH, NTOK, false>), grid, block, lds, st, a, \
                        RouteSelf{}); \
        }
        COLI_GUV(1) COLI_GUV(2) COLI_GUV(3) COLI_GUV(4)
#undef COLI_GUV
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        // one token: RD 4, M 8, a four-stage ring, two workgroups per CU
        // (15.4 us vs 16.7 for four workgroups and two stages)
        constexpr int RD = 4, M = NTOK == 1 ? 8 : (NTOK >= 4 ? 2 : 4), DEPTH = NTOK == 1 ? 4 : 2;
        using Lds = TermLds<M, NTOK, RD>;
        a.w = L.w2; a.s = L.s2; a.sh_w = L.sh_w2; a.sh_s = L.sh_s2;
        a.N = L.H; a.K = L.I;
        a.h = h;
        a.out = o; a.out_ld = L.H;
        a.dump_acc = dump ? reinterpret_cast<int32_t *>(dump + io.dump.acc2) : nullptr;
        a.dump_qh = dump ? reinterpret_cast<int8_t *>(dump + io.dump.qh) : nullptr;
        a.dump_sh = dump ? reinterpret_cast<float *>(dump + io.dump.sh) : nullptr;
        const int P = (L.I / 32 + 63) / 64;
        const size_t lds = (size_t)4 * Lds::rows() * (L.I / 64 + 1) * 4;
        const dim3 grid(std::max((NTOK == 1 ? 2 : 4) * cus, (entries + 3) / 4)), block(256);
#define COLI_DNV(P_) \
        if (P == P_) { \
            if (dump) launch(mk, (down_i8v_kernel<P_, RD, M, DEPTH, NTOK, true>), grid, block, lds, st, a); \
            else launch(mk, (down_i8v_kernel<P_, RD, M, DEPTH, NTOK>), grid, block, lds, st, a); \
        }
        COLI_DNV(1) COLI_DNV(2) COLI_DNV(3) COLI_DNV(4)
#undef COLI_DNV
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t err = io.combine
        ? launch_combine(o, io.ids, io.w, io.T, L.k, L.H, L.n_shared, io.y, st, mk)
        : hipSuccess;
    return err;
}

// Gate/up and down of the integer family for 1 <= T <= kI8StreamTMax, after
// the activation quantiser (qx, sx); h is an fp32 [R][I] workspace region.
hipError_t launch_forward_i8_small(const LayerDev &L, const ForwardIO &io, const int8_t *qx,
                                   const float *sx, float *h, float *o, hipStream_t st, Marks *mk)
{
    I8vArgs a{};
    a.I = L.I;
    a.qx = qx; a.sx = sx;
    a.union_ids = io.union_ids; a.offsets = io.offsets; a.slots = io.slots; a.n_union = io.n_union;
    a.T = io.T; a.k = L.k; a.n_shared = L.n_shared;
    if (io.T == 1) return launch_i8v<1>(L, io, a, h, o, st, mk);
    if (io.T == 2) return launch_i8v<2>(L, io, a, h, o, st, mk);
    return launch_i8v<4>(L, io, a, h, o, st, mk);
}

}  // namespace coli
