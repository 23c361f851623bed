/*
 * coli_oracle.h -- plain, slow, single-threaded CPU oracle of the int4
 * routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the GPU library.
 *
 * All pointers are host memory.  Layouts are row-major:
 *   router_w [E][H] f32, router_b [E] f32,
 *   w13 [E][2I][H/2] packed int4 (rows [0,I) gate, [I,2I) up; byte b of a row
 *       holds k = 2b in its low nibble and k = 2b+1 in its high nibble; codes
 *       are two's complement in [-8, 7]),
 *   s13 [E][2I][H/64] fp16 bit patterns (one scale per row per 64-wide group
 *       along k), w2 [E][H][I/2], s2 [E][H][I/64], shared expert without E.
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t H, I, E, k, n_shared;
    const float *router_w;
    const float *router_b;
    const uint8_t *w13;
    const uint16_t *s13;
    const uint8_t *w2;
    const uint16_t *s2;
    const uint8_t *sh_w13;
    const uint16_t *sh_s13;
    const uint8_t *sh_w2;
    const uint16_t *sh_s2;
} orc_layer;

enum { ORC_ACT_F32 = 0, ORC_ACT_I8 = 1 };

float orc_f16_to_f32(uint16_t h);
int orc_int4(const uint8_t *row, int64_t kk);

void orc_logits(const orc_layer *L, const float *x, int32_t T, float *logits);
void orc_select(int32_t E, int32_t k, int32_t T, const float *logits, const float *bias,
                int32_t *ids, float *w, float *scores);
void orc_route(const orc_layer *L, const float *x, int32_t T, int32_t *ids, float *w,
               float *logits, float *scores);
void orc_prune_topp(int32_t E, int32_t k, int32_t T, float p, const float *scores, int32_t *ids,
                    float *w);
void orc_union(int32_t T, int32_t k, int32_t E, const int32_t *ids, int32_t *union_ids,
               int32_t *offsets, int32_t *slots, int32_t *n_union);

float orc_swiglu(float g, float u);
void orc_quant_i8(int64_t n, const float *x, int8_t *q, float *s);

void orc_expert_f32(int32_t H, int32_t I, const uint8_t *w13, const uint16_t *s13,
                    const uint8_t *w2, const uint16_t *s2, const float *x,
                    float *g, float *u, float *h, double *o);
void orc_expert_i8(int32_t H, int32_t I, const uint8_t *w13, const uint16_t *s13,
                   const uint8_t *w2, const uint16_t *s2, const float *x,
                   int32_t *acc13, float *g, float *u, float *h, int8_t *qh, float *sh,
                   int32_t *acc2, double *o);
void orc_down_acc_i8(int32_t H, int32_t I, const uint8_t *w2, const int8_t *qh, int32_t *acc2);
void orc_down_i8(int32_t H, int32_t I, const uint8_t *w2, const uint16_t *s2, const int8_t *qh,
                 const float *sh, double *o);

void orc_token_forward(const orc_layer *L, const float *x_t, const int32_t *ids_t,
                       const float *w_t, int32_t act_mode, float *y_t);
void orc_forward(const orc_layer *L, const float *x, int32_t T, const int32_t *ids,
                 const float *w, int32_t act_mode, float *y);
void orc_forward_rows(const orc_layer *L, const float *x, const int32_t *ids, const float *w,
                      int32_t act_mode, int32_t n_sel, const int32_t *sel, float *y_sel);

void orc_rmsnorm(int32_t T, int32_t H, const float *x, float *xhat);

/* Decode attention over the compressed (MLA) KV cache, absorbed form:
 * q [B][n_heads][576], kv [T][576] (latent 512 then rotary key 64),
 * keys of query b: t < lens[b] (idx NULL) or the rows idx[b][0..n_sel) in
 * [0, T); out [B][n_heads][512] = softmax(scale * q.kv_t) weighted sum of
 * kv_t[0..512), computed in double, 0 when a query has no key. */
void orc_mla_decode(int32_t B, int32_t n_heads, const float *q, int32_t T, const float *kv,
                    const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale,
                    float *out);

#ifdef __cplusplus
}
#endif
#endif
