// route_tokens.h -- top-k selection of routed tokens by the waves of one
// workgroup: DeepSeek-V3 style sigmoid scores plus a selection bias
// ("Colibri" skill page, "コアアーキテクチャ" item 1; "Colibri 完全ガイド",
// table "コア技術のハイライト"), the top k per token ("colibri解説", section
// "なぜ25GBで動くのか"), optionally the adaptive top-p prefix, and for a
// batch that fits the workgroup the batch union.  Used by the router's top-k
// kernel and by the streaming gate/up kernels of batches of at most 4 tokens
// that route their tokens themselves (route_self).
#pragma once

#include "common.h"
#include "stream.h"
#include "union_wave.h"

namespace coli {

// Router score of a logit: sigmoid in fp64 of the fp32 logit, rounded to fp32.
__device__ __forceinline__ float sigmoid_fp64(float l)
{
    return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// --- top-k: one wave per token, 4 tokens per workgroup -------------------
// Radix select: the k-th largest key is found two bits at a time with wave
// ballots (16 rounds, no shuffles); keys equal to it are taken in expert order; the
// k winners are then ordered by (key desc, expert asc) through LDS.

// Monotone map of an fp32 key to uint32 (larger float -> larger integer);
// -0 is folded into +0 first so that equal keys compare equal.
__device__ __forceinline__ uint32_t order_bits(float z)
{
    const uint32_t u = __float_as_uint(z + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Logit of (t, e) for S >= 1: the fp64 partials of the S K-splits added in
// split order and rounded once to fp32 (S == 0: the stored value).
__device__ __forceinline__ float logit_at(const float *__restrict__ logits,
                                          const double *__restrict__ part, int S, int T, int E,
                                          int t, int e)
{
    if (S == 0) return logits[(size_t)t * E + e];
    const size_t stride = (size_t)T * E;
    const double *p = part + (size_t)t * E + e;
    double acc = p[0];
    int s = 1;
    for (; s + 4 <= S; s += 4) {  // four loads in flight, added in split order
        const double v0 = p[s * stride], v1 = p[(s + 1) * stride];
        const double v2 = p[(s + 2) * stride], v3 = p[(s + 3) * stride];
        acc += v0; acc += v1; acc += v2; acc += v3;
    }
    for (; s < S; ++s) acc += p[s * stride];
    return (float)acc;
}

// Union outputs of a routed batch, written by the top-k kernel itself when
// the batch fits one workgroup (T <= 4, so T * k <= 64).
struct UnionOut {
    int32_t *union_ids, *offsets, *slots, *n_union;
    int cap;
};

// Tokens t0 .. t0 + 3 (one per wave; waves past T only take part in the
// barriers, so every wave of the 256-thread workgroup must call this).
// ids / w are indexed by token (t * k + rank); with UNION the workgroup's
// tokens (T <= 4, t0 = 0) also form the batch union into uo.
// TL: timeline marks 4 (keys loaded), 5 (threshold found), 6 (selection
// and union written) into tl (measurement variants only).
template <int KPL, bool UNION, bool TL = false>
__device__ __forceinline__ void route_tokens(const float *__restrict__ logits,
                                             const double *__restrict__ part, int S,
                                             const float *__restrict__ bias, int T, int E, int k,
                                             float top_p, int32_t *__restrict__ ids,
                                             float *__restrict__ w, const UnionOut &uo, int t0,
                                             uint64_t *tl = nullptr, int tl_cap = 0)
{
    __shared__ int32_t sid[64];  // the batch's selections (UNION)
    __shared__ uint32_t sk[4][COLI_MAX_K_DEV];
    __shared__ int32_t se[4][COLI_MAX_K_DEV];
    __shared__ float ss[4][COLI_MAX_K_DEV];
    __shared__ float sg[4][64 * KPL];  // each expert's sigmoid score, per wave
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int t = t0 + wv;
    const bool live = t < T;
    const int tr = live ? t : 0;
    // the token's scores (S == 0: written by the GEMV) or logits, and the
    // biases: every load issued before the first use (buffer loads; experts
    // past E read 0 and are not keys)
    float lg[KPL], bs[KPL];
    {
        uint32_t off[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) off[i] = lane + 64 * i < E ? (uint32_t)(lane + 64 * i) * 4 : kOOB;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, (uint32_t)E * 4);
        if (S == 0) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(logits + (size_t)tr * E, (uint32_t)E * 4);
#pragma unroll
            for (int i = 0; i < KPL; ++i)
                lg[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, off[i], 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < KPL; ++i)
                lg[i] = lane + 64 * i < E ? logit_at(logits, part, S, T, E, tr, lane + 64 * i) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            bs[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, off[i], 0, 0));
        // all values present here (one wait for every load), so that no
        // load is sunk into the conditional code below
#pragma unroll
        for (int i = 0; i < KPL; ++i) asm volatile("" : "+v"(lg[i]), "+v"(bs[i]));
    }
    tl_mark<TL>(tl, tl_cap, 4);
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        const float sgm = S == 0 ? lg[i] : sigmoid_fp64(lg[i]);
        sg[wv][e] = sgm;
        key[i] = (live && e < E) ? order_bits(sgm + bs[i]) : 0u;
    }
    // largest tau with #{key >= tau} >= k  (valid keys are >= 1), two bits
    // per round: the counts of the three candidates of a round are
    // independent (their ballots overlap, where one bit per round would wait
    // for each count before the next compare)
    uint32_t tau = 0;
    for (int b = 30; b >= 0; b -= 2) {
        const uint32_t c1 = tau | (1u << b), c2 = tau | (2u << b), c3 = tau | (3u << b);
        int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            n1 += __popcll(__ballot(key[i] >= c1));
            n2 += __popcll(__ballot(key[i] >= c2));
            n3 += __popcll(__ballot(key[i] >= c3));
        }
        tau = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : tau;
    }
    tl_mark<TL>(tl, tl_cap, 5);
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
        // all COLI_MAX_K_DEV entries read at once (one LDS round trip; the
        // ones past k are not counted)
#pragma unroll
        for (int j = 0; j < COLI_MAX_K_DEV; ++j) {
            const uint32_t ok = sk[wv][j];
            const int oe = se[wv][j];
            rank += (j < k && (ok > mk || (ok == mk && oe < me))) ? 1 : 0;
        }
    }
    __syncthreads();
    float sj = 0.f;
    if (live && lane < k) {
        sj = sg[wv][me];
        ss[wv][rank] = sj;
    }
    __syncthreads();
    if (live && lane < k) {
        float sv[COLI_MAX_K_DEV];
#pragma unroll
        for (int j = 0; j < COLI_MAX_K_DEV; ++j) sv[j] = ss[wv][j];
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < COLI_MAX_K_DEV; ++j)
            if (j < k) sum += sv[j];  // fp32, selection order
        // adaptive top-p: keep the shortest prefix of the selection whose
        // weights reach top_p (fp32, in order), renormalised over the kept
        int kp = k;
        if (top_p < 1.0f) {
            float c = 0.f;
            for (int m = 1; m <= k; ++m) {
                c += ss[wv][m - 1] / sum;
                if (c >= top_p) {
                    kp = m;
                    break;
                }
            }
            sum = 0.f;
            for (int j = 0; j < kp; ++j) sum += ss[wv][j];
        }
        ids[(size_t)t * k + rank] = rank < kp ? me : -1;
        w[(size_t)t * k + rank] = rank < kp ? sj / sum : 0.f;
        if constexpr (UNION) sid[t * k + rank] = rank < kp ? me : -1;
    }
    if constexpr (UNION) {
        __syncthreads();
        if (wv == 0) {
            if (T == 1) {
                // one token: its kept experts are distinct, so the union is
                // the kept slots ordered by expert (rank by counting): the
                // lists union_wave forms, without its sorting network
                const int id = lane < k ? sid[lane] : -1;
                const bool valid = id >= 0 && id < E;
                int pos = 0;
#pragma unroll
                for (int i = 0; i < COLI_MAX_K_DEV; ++i) {
                    const int o = sid[i];
                    pos += (i < k && o >= 0 && o < E && o < id) ? 1 : 0;
                }
                const int kept = __popcll(__ballot(valid));
                if (valid) {
                    uo.union_ids[pos] = id;
                    uo.offsets[pos] = pos;
                    uo.slots[pos] = lane;
                }
                if (lane >= kept && lane < uo.cap) uo.union_ids[lane] = -1;
                if (lane >= kept && lane <= uo.cap) uo.offsets[lane] = kept;
                if (lane == 0) {
                    uo.n_union[0] = kept;
                    if (uo.cap == 64) uo.offsets[64] = kept;
                }
            } else {
                const int n = T * k;
                union_wave(lane, lane < n ? sid[lane] : -1, E, uo.cap, uo.union_ids, uo.offsets,
                           uo.slots, uo.n_union);
            }
        }
    }
    tl_mark<TL>(tl, tl_cap, 6);
}

// The selection lists of at most 4 tokens in LDS (T * k <= 64).
struct RouteLds {
    int32_t ids[64], u[64], sl[64];
    int32_t off[65], n[1];
    float w[64];
};

// The tokens (r.T <= 4, one per wave) select their top k and form their
// union into l (every thread of the 256-thread workgroup calls this);
// workgroup 0 also writes the global contents the top-k kernel leaves
// (slots past the kept ones untouched).
template <bool TL = false>
__device__ __forceinline__ void route_self(const RouteSelf &r, RouteLds &l, uint64_t *tl = nullptr,
                                           int tl_cap = 0)
{
    const UnionOut uo{l.u, l.off, l.sl, l.n, r.cap};
    route_tokens<4, true, TL>(r.scores, nullptr, 0, r.bias, r.T, r.E, r.k, r.top_p, l.ids, l.w, uo,
                              0, tl, tl_cap);
    __syncthreads();
    if (blockIdx.x == 0) {
        const int i = threadIdx.x, nu = l.n[0], kept = l.off[nu];
        if (i < r.T * r.k) {
            r.ids[i] = l.ids[i];
            r.w[i] = l.w[i];
        }
        if (i < kept) r.slots[i] = l.sl[i];
        if (i < r.cap) r.union_ids[i] = l.u[i];
        if (i <= r.cap) r.offsets[i] = l.off[i];
        if (i == 0) r.n_union[0] = nu;
    }
}

}  // namespace coli
