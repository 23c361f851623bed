/*
 * coli_oracle.c -- the reference definition of the int4 routed-expert MoE
 * layer, written as plainly as possible: single-threaded C99, double
 * precision accumulation, no blocking, no fusion, no reordering.
 *
 * TEST INFRASTRUCTURE ONLY (see coli_oracle.h).  Build with
 *   gcc -std=c99 -O2 -ffp-contract=off   (never -ffast-math)
 *
 * Sources (web pages about the Colibri engine), cited by title and section:
 *   [Skill]  "Colibri" (mcpfield.com skill page), section "コアアーキテクチャ".
 *   [Guide]  "Colibri 完全ガイド — 25GB のメモリで 744B パラメータの大規模モデルを
 *            動かす" (dashen-tech.com), table "コア技術のハイライト" and the
 *            numbered walk-through "詳細解説：Colibri はどう動いているのか".
 *   [Hysen]  "colibri: 744B MoEをストレージから推論するCエンジン"
 *            (hysenlabs.com), sections "トークンごとの5ステップパスとデュアルSSD
 *            ミラー", "エンドツーエンドの測定で地位を獲得する技術" and
 *            "はじめにとソースが語らないこと".
 *   [Start]  Colibri getting-started page (cti.vibequant.cc), section
 *            "토큰당 처리 경로 (The Per-Token Path)".
 *   [Heart]  "colibri解説｜GLM-5.2（744B MoE）を25GB RAMで動かす純Cランタイムの
 *            実測速度" (ai-heartland.com), section "なぜ25GBで動くのか".
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function; every such reading is listed in the design notes.
 * Parity of a function is pinned in tests/test_oracle_pins.py unless its
 * comment says "parity unpinned".
 */
#include "coli_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Encodings                                                                 */

/* IEEE binary16 -> binary32 (exact).  Scales are stored as fp16 bit
 * patterns, one per weight row per 64-wide group along the reduction axis
 * ([Hysen] "はじめにとソースが語らないこと": the model is the gs64 build). */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                   /* zero / subnormal */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25);     /* 1.man * 2^(exp-15) */
    return (float)(sign ? -v : v);
}

/* The int4 code of element kk of a packed row: byte kk/2, low nibble for
 * even kk, high nibble for odd kk, two's complement in [-8, 7]
 * ([Guide] "コア技術のハイライト": packed int4 integer dot kernels; the nibble
 * order and the signed code are the readings taken for the container). */
int orc_int4(const uint8_t *row, int64_t kk)
{
    int byte = row[kk >> 1];
    int nib = (kk & 1) ? (byte >> 4) & 0xF : byte & 0xF;
    return nib < 8 ? nib : nib - 16;
}

/* Dequantised weight: code times its group's scale (decoded scales of the
 * row in fsrow).  Exact in fp32: a 4-bit code times an 11-bit significand
 * needs at most 15 bits. */
static float wdeq(const uint8_t *row, const float *fsrow, int64_t kk)
{
    return (float)orc_int4(row, kk) * fsrow[kk / 64];
}

static void decode_scales(const uint16_t *srow, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(srow[i]);
}

/* ------------------------------------------------------------------------ */
/* Route ([Skill] "コアアーキテクチャ" item 1 and [Guide] "コア技術のハイライト":
 * a DeepSeek-V3 style sigmoid router; [Heart] "なぜ25GBで動くのか": each MoE
 * layer picks its top 8 experts per token).                                  */

/* logits[t][e] = fp32( sum_h x[t][h] * Wr[e][h] ), products and the running
 * sum in double, ascending h, one rounding at the end (reading: the pages
 * give no precision for the router; fp64 makes the selection reproducible). */
void orc_logits(const orc_layer *L, const float *x, int32_t T, float *logits)
{
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < L->E; ++e) {
            const float *xr = x + (size_t)t * L->H;
            const float *wr = L->router_w + (size_t)e * L->H;
            double acc = 0.0;
            for (int32_t h = 0; h < L->H; ++h) acc += (double)xr[h] * (double)wr[h];
            logits[(size_t)t * L->E + e] = (float)acc;
        }
}

typedef struct { float key; int32_t e; } orc_cand;

/* order: larger key first; equal keys -> lower expert index first */
static int cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->e > b->e) - (a->e < b->e);
}

/* DeepSeek-V3 selection (the router the pages name):
 *   s[e] = sigmoid(l[e]) computed in double and rounded once to fp32,
 *   key[e] = s[e] + b[e] (fp32 add): the bias steers selection only,
 *   ids = the k largest keys, ties to the lower expert index, listed in
 *         selection order (largest key first),
 *   w[j] = s[ids[j]] / sum_j' s[ids[j']], sum in fp32 in j order.
 * No group-limited routing and no extra scaling factor (neither appears on
 * the pages).  `scores` (optional) receives s [T][E]. */
void orc_select(int32_t E, int32_t k, int32_t T, const float *logits, const float *bias,
                int32_t *ids, float *w, float *scores)
{
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)E);
    float *s = (float *)malloc(sizeof(float) * (size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double l = (double)logits[(size_t)t * E + e];
            s[e] = (float)(1.0 / (1.0 + exp(-l)));
            c[e].key = s[e] + bias[e];
            c[e].e = e;
            if (scores) scores[(size_t)t * E + e] = s[e];
        }
        qsort(c, (size_t)E, sizeof(orc_cand), cand_cmp);
        float sum = 0.0f;
        for (int32_t j = 0; j < k; ++j) sum += s[c[j].e];
        for (int32_t j = 0; j < k; ++j) {
            ids[(size_t)t * k + j] = c[j].e;
            w[(size_t)t * k + j] = s[c[j].e] / sum;
        }
    }
    free(s);
    free(c);
}

/* Adaptive expert top-p ([Heart] "速度を稼ぐ実用ノブ" knob list: an
 * adaptive expert top-p, `--topp 0.7`, that reads 30-40% fewer expert bytes;
 * the pages give no formula).  Reading: after the top-k selection above,
 * keep the shortest prefix of the selection order whose routing weights add
 * up to at least p (fp32, in selection order), drop the rest (id -1, weight
 * 0) and renormalise the kept weights over the kept experts:
 *   c_m = w[0] + ... + w[m-1]  (fp32, j ascending),
 *   k'  = the least m in [1, k] with c_m >= p, or k if there is none,
 *   w'[j] = s[ids[j]] / (s[ids[0]] + ... + s[ids[k'-1]])  for j < k'.
 * p >= 1 keeps all k (no pruning).  ids and w are updated in place. */
void orc_prune_topp(int32_t E, int32_t k, int32_t T, float p, const float *scores, int32_t *ids,
                    float *w)
{
    (void)E;
    if (!(p < 1.0f)) return;
    for (int32_t t = 0; t < T; ++t) {
        int32_t *it = ids + (size_t)t * k;
        float *wt = w + (size_t)t * k;
        int32_t kp = k;
        float c = 0.0f;
        for (int32_t m = 1; m <= k; ++m) {
            c += wt[m - 1];
            if (c >= p) {
                kp = m;
                break;
            }
        }
        float sum = 0.0f;
        for (int32_t j = 0; j < kp; ++j) sum += scores[(size_t)t * E + it[j]];
        for (int32_t j = 0; j < k; ++j) {
            if (j < kp) {
                wt[j] = scores[(size_t)t * E + it[j]] / sum;
            } else {
                it[j] = -1;
                wt[j] = 0.0f;
            }
        }
    }
}

void orc_route(const orc_layer *L, const float *x, int32_t T, int32_t *ids, float *w,
               float *logits, float *scores)
{
    float *lg = logits ? logits : (float *)malloc(sizeof(float) * (size_t)T * (size_t)L->E);
    orc_logits(L, x, T, lg);
    orc_select(L->E, L->k, T, lg, L->router_b, ids, w, scores);
    if (!logits) free(lg);
}

/* ------------------------------------------------------------------------ */
/* Union ([Start] "토큰당 처리 경로": experts chosen by several tokens of a
 * batch are de-duplicated; [Hysen] lists the batched expert union).
 *   union_ids[u]  ascending distinct experts of ids[T*k], u < U = *n_union,
 *   offsets[u]    exclusive prefix sum of the per-expert slot counts,
 *                 offsets[U] = n_kept, the number of slots with an expert
 *                 (T*k unless the top-p router dropped some: id -1),
 *   slots[...]    for each union expert in order, its slots s = t*k + j in
 *                 ascending s.
 * Positions past U in union_ids are -1 and in offsets are n_kept, up to the
 * buffers' capacity min(E, T*k) (+1 for offsets). */
void orc_union(int32_t T, int32_t k, int32_t E, const int32_t *ids, int32_t *union_ids,
               int32_t *offsets, int32_t *slots, int32_t *n_union)
{
    int32_t n = T * k;
    int32_t cap = n < E ? n : E;
    int32_t *count = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *start = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int32_t s = 0; s < n; ++s)
        if (ids[s] >= 0) count[ids[s]] += 1;
    int32_t U = 0, run = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (count[e] == 0) continue;
        union_ids[U] = e;
        offsets[U] = run;
        start[e] = run;
        run += count[e];
        ++U;
    }
    for (int32_t u = U; u < cap; ++u) union_ids[u] = -1;
    for (int32_t u = U; u <= cap; ++u) offsets[u] = run;
    for (int32_t s = 0; s < n; ++s)
        if (ids[s] >= 0) slots[start[ids[s]]++] = s;
    *n_union = U;
    free(start);
    free(count);
}

/* ------------------------------------------------------------------------ */
/* Activation quantisation for the integer kernel family ([Guide]
 * "詳細解説" step 3: batched prefill runs the integer kernel; "コア技術の
 * ハイライト": int8 x packed-int4 dot kernels).  Reading: symmetric int8 per
 * 64-wide group of one token, scale = amax / 127 (IEEE fp32 divide),
 * q = clamp(rint(x / scale), -127, 127) with an IEEE divide and
 * round-half-to-even; an all-zero group has scale 0 and codes 0.
 * n must be a multiple of 64; s receives n/64 scales. */
void orc_quant_i8(int64_t n, const float *x, int8_t *q, float *s)
{
    for (int64_t g = 0; g < n / 64; ++g) {
        const float *xg = x + g * 64;
        float amax = 0.0f;
        for (int i = 0; i < 64; ++i) {
            float a = fabsf(xg[i]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            s[g] = 0.0f;
            for (int i = 0; i < 64; ++i) q[g * 64 + i] = 0;
            continue;
        }
        float sc = amax / 127.0f;
        s[g] = sc;
        for (int i = 0; i < 64; ++i) {
            float r = rintf(xg[i] / sc);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[g * 64 + i] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert FFN.  Reading: a SwiGLU expert (gate and up rows in w13, down rows
 * in w2), which with H = 6144, I = 2048 gives the ~19 MB int4 expert of
 * [Guide] "Colibri とは？" and [Heart] "なぜ25GBで動くのか".
 *   silu(g) * u  computed in fp32 as  g / (1 + expf(-g)) * u.                */

static float swiglu(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

float orc_swiglu(float g, float u) { return swiglu(g, u); }

/* fp32 family ([Guide] "詳細解説" step 3: single-token decode computes in
 * f32).  g, u: double dot products of dequantised weights and x, rounded
 * once to fp32; h = swiglu(g, u) in fp32; o[n] = double dot of dequantised
 * down weights and h (kept in double for the combine).  g/u/h may be NULL. */
void orc_expert_f32(int32_t H, int32_t I, const uint8_t *w13, const uint16_t *s13,
                    const uint8_t *w2, const uint16_t *s2, const float *x,
                    float *g, float *u, float *h, double *o)
{
    float *hv = (float *)malloc(sizeof(float) * (size_t)I);
    const int64_t rb13 = H / 2, rs13 = H / 64, rb2 = I / 2, rs2 = I / 64;
    float *sg = (float *)malloc(sizeof(float) * (size_t)rs13);
    float *su = (float *)malloc(sizeof(float) * (size_t)rs13);
    float *sd = (float *)malloc(sizeof(float) * (size_t)rs2);
    for (int32_t i = 0; i < I; ++i) {
        double ag = 0.0, au = 0.0;
        const uint8_t *rg = w13 + (size_t)i * rb13, *ru = w13 + (size_t)(I + i) * rb13;
        decode_scales(s13 + (size_t)i * rs13, rs13, sg);
        decode_scales(s13 + (size_t)(I + i) * rs13, rs13, su);
        for (int64_t kk = 0; kk < H; ++kk) {
            ag += (double)wdeq(rg, sg, kk) * (double)x[kk];
            au += (double)wdeq(ru, su, kk) * (double)x[kk];
        }
        float gf = (float)ag, uf = (float)au;
        if (g) g[i] = gf;
        if (u) u[i] = uf;
        hv[i] = swiglu(gf, uf);
        if (h) h[i] = hv[i];
    }
    for (int32_t n = 0; n < H; ++n) {
        const uint8_t *r = w2 + (size_t)n * rb2;
        decode_scales(s2 + (size_t)n * rs2, rs2, sd);
        double acc = 0.0;
        for (int64_t kk = 0; kk < I; ++kk) acc += (double)wdeq(r, sd, kk) * (double)hv[kk];
        o[n] = acc;
    }
    free(sd);
    free(su);
    free(sg);
    free(hv);
}

/* Integer group accumulator: exact int32 sum over one 64-group of
 * int8 activation codes times int4 weight codes (|acc| <= 64*127*8). */
static int32_t group_dot(const int8_t *q, const uint8_t *row, int64_t g)
{
    int32_t acc = 0;
    for (int64_t kk = g * 64; kk < g * 64 + 64; ++kk) acc += (int32_t)q[kk] * orc_int4(row, kk);
    return acc;
}

/* Down-projection accumulators from given int8 codes qh [I]:
 * acc2[n][g] = group_dot(qh, w2 row n, g). */
void orc_down_acc_i8(int32_t H, int32_t I, const uint8_t *w2, const int8_t *qh, int32_t *acc2)
{
    const int64_t rb2 = I / 2, G = I / 64;
    for (int32_t n = 0; n < H; ++n)
        for (int64_t g = 0; g < G; ++g)
            acc2[(size_t)n * G + g] = group_dot(qh, w2 + (size_t)n * rb2, g);
}

/* Down projection of the integer family from given int8 codes of h (qh [I],
 * natural order) and their scales (sh [I/64]):
 *   o[n] = sum_g (double)acc2[n][g] * sh[g] * s2[n][g]   (double),
 *   acc2[n][g] = group_dot(qh, w2 row n, g).
 * The same down stage as orc_expert_i8, for operands that come from
 * elsewhere: the accumulators are exact given the codes, while the codes of
 * h themselves depend on how g and u were rounded (a code may differ by one
 * at a rounding boundary), so a GPU down projection is compared with the
 * oracle on the GPU's own codes. */
void orc_down_i8(int32_t H, int32_t I, const uint8_t *w2, const uint16_t *s2, const int8_t *qh,
                 const float *sh, double *o)
{
    const int64_t rb2 = I / 2, G2 = I / 64;
    for (int32_t n = 0; n < H; ++n) {
        const uint8_t *row = w2 + (size_t)n * rb2;
        const uint16_t *srow = s2 + (size_t)n * G2;
        double acc = 0.0;
        for (int64_t gg = 0; gg < G2; ++gg)
            acc += (double)group_dot(qh, row, gg) * (double)sh[gg] * (double)orc_f16_to_f32(srow[gg]);
        o[n] = acc;
    }
}

/* Integer family ([Guide] "詳細解説" step 3 and "コア技術のハイライト").
 *   qx, sx = quant(x);  acc13[r][g] = group_dot(qx, w13 row r, g);
 *   g/u[r] = fp32( sum_g (double)acc13[r][g] * sx[g] * s13[r][g] );
 *   h = swiglu(g, u) in fp32;  qh, sh = quant(h);
 *   acc2[n][g] = group_dot(qh, w2 row n, g);
 *   o[n] = sum_g (double)acc2[n][g] * sh[g] * s2[n][g]   (double).
 * Each product acc*sx*sw is exact in double (17 + 24 + 11 bits).  Every
 * output pointer except o may be NULL. */
void orc_expert_i8(int32_t H, int32_t I, const uint8_t *w13, const uint16_t *s13,
                   const uint8_t *w2, const uint16_t *s2, const float *x,
                   int32_t *acc13, float *g, float *u, float *h, int8_t *qh, float *sh,
                   int32_t *acc2, double *o)
{
    const int64_t rb13 = H / 2, G13 = H / 64, rb2 = I / 2, G2 = I / 64;
    int8_t *qx = (int8_t *)malloc((size_t)H);
    float *sx = (float *)malloc(sizeof(float) * (size_t)G13);
    float *hv = (float *)malloc(sizeof(float) * (size_t)I);
    int8_t *qhv = (int8_t *)malloc((size_t)I);
    float *shv = (float *)malloc(sizeof(float) * (size_t)G2);
    orc_quant_i8(H, x, qx, sx);
    for (int32_t i = 0; i < I; ++i) {
        double val[2];
        for (int half = 0; half < 2; ++half) {
            int64_t r = (int64_t)half * I + i;
            const uint8_t *row = w13 + (size_t)r * rb13;
            const uint16_t *srow = s13 + (size_t)r * G13;
            double acc = 0.0;
            for (int64_t gg = 0; gg < G13; ++gg) {
                int32_t a = group_dot(qx, row, gg);
                if (acc13) acc13[(size_t)r * G13 + gg] = a;
                acc += (double)a * (double)sx[gg] * (double)orc_f16_to_f32(srow[gg]);
            }
            val[half] = acc;
        }
        float gf = (float)val[0], uf = (float)val[1];
        if (g) g[i] = gf;
        if (u) u[i] = uf;
        hv[i] = swiglu(gf, uf);
        if (h) h[i] = hv[i];
    }
    orc_quant_i8(I, hv, qhv, shv);
    if (qh) memcpy(qh, qhv, (size_t)I);
    if (sh) memcpy(sh, shv, sizeof(float) * (size_t)G2);
    for (int32_t n = 0; n < H; ++n) {
        const uint8_t *row = w2 + (size_t)n * rb2;
        const uint16_t *srow = s2 + (size_t)n * G2;
        double acc = 0.0;
        for (int64_t gg = 0; gg < G2; ++gg) {
            int32_t a = group_dot(qhv, row, gg);
            if (acc2) acc2[(size_t)n * G2 + gg] = a;
            acc += (double)a * (double)shv[gg] * (double)orc_f16_to_f32(srow[gg]);
        }
        o[n] = acc;
    }
    free(shv);
    free(qhv);
    free(hv);
    free(sx);
    free(qx);
}

/* ------------------------------------------------------------------------ */
/* Combine: one token's layer output
 *   y = fp32( sum_{j=0..k-1} w[j] * o_{ids[j]}  +  o_shared ),
 * summed in double in j order with the shared expert last.  The shared
 * expert is ungated (weight 1): [Guide] "コア技術のハイライト" (the router
 * comes with shared experts) and [Start] project description (shared experts
 * belong to the always-resident dense part).  Placement never enters: the
 * result depends only on x, the routing and the weights ([Hysen] "トークンご
 * との5ステップパス": placement decides speed, never semantics). */
void orc_token_forward(const orc_layer *L, const float *x_t, const int32_t *ids_t,
                       const float *w_t, int32_t act_mode, float *y_t)
{
    const int32_t H = L->H, I = L->I;
    const size_t e13 = (size_t)2 * I * (H / 2), es13 = (size_t)2 * I * (H / 64);
    const size_t e2 = (size_t)H * (I / 2), es2 = (size_t)H * (I / 64);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *acc = (double *)calloc((size_t)H, sizeof(double));
    for (int32_t j = 0; j <= L->k; ++j) {
        const uint8_t *w13, *w2;
        const uint16_t *s13, *s2;
        double wj;
        if (j < L->k) {
            int32_t e = ids_t[j];
            if (e < 0) continue;  /* dropped by the top-p router */
            w13 = L->w13 + e * e13; s13 = L->s13 + e * es13;
            w2 = L->w2 + e * e2; s2 = L->s2 + e * es2;
            wj = (double)w_t[j];
        } else {
            if (!L->n_shared) break;
            w13 = L->sh_w13; s13 = L->sh_s13; w2 = L->sh_w2; s2 = L->sh_s2;
            wj = 1.0;
        }
        if (act_mode == ORC_ACT_I8)
            orc_expert_i8(H, I, w13, s13, w2, s2, x_t, NULL, NULL, NULL, NULL, NULL, NULL,
                          NULL, o);
        else
            orc_expert_f32(H, I, w13, s13, w2, s2, x_t, NULL, NULL, NULL, o);
        if (j < L->k)
            for (int32_t n = 0; n < H; ++n) acc[n] += wj * o[n];
        else
            for (int32_t n = 0; n < H; ++n) acc[n] += o[n];
    }
    for (int32_t n = 0; n < H; ++n) y_t[n] = (float)acc[n];
    free(acc);
    free(o);
}

void orc_forward(const orc_layer *L, const float *x, int32_t T, const int32_t *ids,
                 const float *w, int32_t act_mode, float *y)
{
    for (int32_t t = 0; t < T; ++t)
        orc_token_forward(L, x + (size_t)t * L->H, ids + (size_t)t * L->k,
                          w + (size_t)t * L->k, act_mode, y + (size_t)t * L->H);
}

/* The layer output for a selection of tokens only (tokens are independent,
 * so this equals the matching rows of orc_forward). */
void orc_forward_rows(const orc_layer *L, const float *x, const int32_t *ids, const float *w,
                      int32_t act_mode, int32_t n_sel, const int32_t *sel, float *y_sel)
{
    for (int32_t i = 0; i < n_sel; ++i) {
        int32_t t = sel[i];
        orc_token_forward(L, x + (size_t)t * L->H, ids + (size_t)t * L->k,
                          w + (size_t)t * L->k, act_mode, y_sel + (size_t)i * L->H);
    }
}

/* ------------------------------------------------------------------------ */
/* Pre-norm between stacked layers (reading: the pages do not describe the
 * blocks around the MoE layer; a unit-gain RMSNorm with eps = 1e-6, as in a
 * GLM-style pre-norm block, keeps a stack of synthetic layers finite).
 *   xhat = fp32( x / sqrt(mean(x^2) + 1e-6) ), computed in double.          */
void orc_rmsnorm(int32_t T, int32_t H, const float *x, float *xhat)
{
    for (int32_t t = 0; t < T; ++t) {
        const float *r = x + (size_t)t * H;
        double ss = 0.0;
        for (int32_t h = 0; h < H; ++h) ss += (double)r[h] * (double)r[h];
        double inv = 1.0 / sqrt(ss / (double)H + 1e-6);
        for (int32_t h = 0; h < H; ++h) xhat[(size_t)t * H + h] = (float)((double)r[h] * inv);
    }
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the compressed (MLA) KV cache, in its absorbed form.
 * The Colibri pages (mcpfield.com "Colibri", section "コアアーキテクチャ",
 * item 5; dashen-tech.com guide, table "コア技術のハイライト"; getting-started
 * page, section "압축 KV 상태") state that MLA keeps 576 floats per token in
 * the KV cache instead of 32,768.  Reading: the 576 floats are the 512-wide
 * latent c_t followed by the 64-wide rotary key k_t; a query head arrives
 * already absorbed as 576 floats (its latent query, then its rotary query),
 * so that for head h of query b
 *   s_t  = scale * sum_{d<576} q[b][h][d] * kv[t][d]          (double)
 *   p_t  = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
 *   o    = fp32( sum_t p_t * kv[t][0..512) )
 * over the keys t of query b: t < lens[b] (the cached prefix), or, with a
 * key list idx (the sparse top-k selection the pages' DSA indexer makes),
 * the listed rows idx[b][j] that lie in [0, T).  A query with no key gets
 * o = 0. */
void orc_mla_decode(int32_t B, int32_t n_heads, const float *q, int32_t T, const float *kv,
                    const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale,
                    float *out)
{
    const int32_t D = 576, DV = 512;
    const int32_t n_max = idx ? n_sel : T;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n_max > 0 ? n_max : 1));
    int32_t *row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_max > 0 ? n_max : 1));
    double *o = (double *)malloc(sizeof(double) * DV);
    for (int32_t b = 0; b < B; ++b) {
        /* the keys of query b */
        int32_t nk = 0;
        if (idx) {
            for (int32_t j = 0; j < n_sel; ++j) {
                int32_t t = idx[(size_t)b * n_sel + j];
                if (t >= 0 && t < T) row[nk++] = t;
            }
        } else {
            int32_t len = lens[b] < 0 ? 0 : (lens[b] > T ? T : lens[b]);
            for (int32_t t = 0; t < len; ++t) row[nk++] = t;
        }
        for (int32_t h = 0; h < n_heads; ++h) {
            const float *qv = q + ((size_t)b * n_heads + h) * D;
            float *ov = out + ((size_t)b * n_heads + h) * DV;
            double m = -INFINITY;
            for (int32_t j = 0; j < nk; ++j) {
                const float *kr = kv + (size_t)row[j] * D;
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) acc += (double)qv[d] * (double)kr[d];
                s[j] = (double)scale * acc;
                if (s[j] > m) m = s[j];
            }
            double den = 0.0;
            for (int32_t d = 0; d < DV; ++d) o[d] = 0.0;
            for (int32_t j = 0; j < nk; ++j) {
                const float *vr = kv + (size_t)row[j] * D;
                double p = exp(s[j] - m);
                den += p;
                for (int32_t d = 0; d < DV; ++d) o[d] += p * (double)vr[d];
            }
            for (int32_t d = 0; d < DV; ++d) ov[d] = den > 0.0 ? (float)(o[d] / den) : 0.0f;
        }
    }
    free(s);
    free(row);
    free(o);
}
