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
// k rounds of a wave maximum: each round takes the largest key left, the
// lowest expert among equal keys (a ballot), so the winners come out in
// selection order (key desc, expert asc) without a ranking step.

// Monotone map of an fp32 key to uint32 (larger float -> larger integer);
// -0 is folded into +0 first so that equal keys compare equal.
__device__ __forceinline__ uint32_t order_bits(float z)
{
    const uint32_t u = __float_as_uint(z + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest v over the wave, in every lane: DPP steps inside the 16-lane rows
// (neighbour, pair of neighbours, half-row mirror, row mirror), then the
// four row maxima read out.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
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

// Tokens t0 .. t0 + 3 (one per wave of the first four; later waves, and
// waves past T, only take part in the barriers, so every wave of the
// workgroup must call this).
// ids / w are indexed by token (t * k + rank); with UNION the workgroup's
// tokens (T <= 4, t0 = 0) also form the batch union into uo.
// TL: timeline marks 4 (keys loaded), 5 (selection found), 6 (selection
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
    float sgm[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        sgm[i] = S == 0 ? lg[i] : sigmoid_fp64(lg[i]);
        key[i] = (live && e < E) ? order_bits(sgm[i] + bs[i]) : 0u;
    }
    // The k winners in selection order: round j takes the largest key left
    // (the lowest expert among equal keys) and removes it.  Lane j keeps
    // winner j's expert and score; the scores add up in selection order.
    int my_e = 0;
    float my_s = 0.f, sum = 0.f;
    if (live) {
        for (int j = 0; j < k; ++j) {
            uint32_t m = key[0];
#pragma unroll
            for (int i = 1; i < KPL; ++i) m = max(m, key[i]);
            m = wave_max_u32(m);
            int e = -1;
            float sc = 0.f;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                if (e < 0) {
                    const uint64_t b = __ballot(key[i] == m);
                    if (b) {
                        const int l = __builtin_ctzll(b);
                        e = 64 * i + l;
                        sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sgm[i]), l));
                        if (lane == l) key[i] = 0u;
                    }
                }
            }
            if (lane == j) {
                my_e = e;
                my_s = sc;
            }
            sum += sc;  // fp32, selection order
        }
    }
    tl_mark<TL>(tl, tl_cap, 5);
    if (live && lane < k) {
        // adaptive top-p: keep the shortest prefix of the selection whose
        // weights reach top_p (fp32, in order), renormalised over the kept
        int kp = k;
        if (top_p < 1.0f) {
            float c = 0.f;
            for (int m = 1; m <= k; ++m) {
                c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), m - 1)) / sum;
                if (c >= top_p) {
                    kp = m;
                    break;
                }
            }
            sum = 0.f;
            for (int j = 0; j < kp; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
        }
        const int rank = lane;
        ids[(size_t)t * k + rank] = rank < kp ? my_e : -1;
        w[(size_t)t * k + rank] = rank < kp ? my_s / sum : 0.f;
        if constexpr (UNION) sid[t * k + rank] = rank < kp ? my_e : -1;
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
// union into l (every thread of the workgroup calls this: 4 or 8 waves);
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
