/*
 * coli_mla.h -- decode attention over the compressed (MLA) KV cache, on
 * AMD Instinct MI355X (gfx950).  Part of libcoli_moe.so.
 *
 * What the pages describe:
 *   [Skill]  "Colibri" (mcpfield.com), section "コアアーキテクチャ", item 5:
 *            MLA attention over a compressed KV cache of 576 floats per
 *            token (32,768 for dense attention, 57 times smaller), with
 *            q/kv low-rank projections and interleaved partial RoPE.
 *   [Guide]  "Colibri 完全ガイド" (dashen-tech.com), table "コア技術のハイライト"
 *            (MLA with a 576 floats/token KV cache; DSA sparse attention that
 *            keeps the top-2048 causal keys per layer).
 *   [Start]  Colibri getting-started page (cti.vibequant.cc), section
 *            "압축 KV 상태".
 * The pages give no formula.  This library's reading: the 576 floats of a
 * cached token are its 512-wide latent c_t followed by its 64-wide rotary key
 * k_t (RoPE already applied); a query head arrives absorbed (its latent
 * query, i.e. the no-position query times the key up-projection, then its
 * rotary query), so that attention needs the cache only:
 *   s_t      = scale * sum_{d<576} q[b][h][d] * kv[t][d]
 *   out[b][h] = sum_t softmax_t(s)_t * kv[t][0..512)
 * The caller applies the value up-projection to out.  Conventions of
 * coli_moe.h apply (caller-owned device memory, 16-byte alignment, host-side
 * checks before any HIP call, COLI_* status codes, no synchronisation).
 */
#ifndef COLI_MLA_H
#define COLI_MLA_H

#include <stddef.h>
#include <stdint.h>

#include "coli_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_MLA_DIM 576        /* floats per cached token: latent 512 + rotary 64 */
#define COLI_MLA_LATENT 512     /* value width (the latent part)                   */
#define COLI_MLA_MAX_HEADS 128  /* 1 <= n_heads <= COLI_MLA_MAX_HEADS             */
#define COLI_MLA_MAX_B 256      /* 1 <= B <= COLI_MLA_MAX_B                       */
#define COLI_MLA_MAX_T (1 << 24) /* 1 <= T <= COLI_MLA_MAX_T                      */

/* Bytes of device workspace coli_mla_decode needs (0 if invalid).  n_sel is
 * the key-list width when a key list is used, else 0. */
size_t coli_mla_workspace_bytes(int32_t B, int32_t n_heads, int32_t T, int32_t n_sel);

/* Decode attention for B query tokens over one cache.
 *   q    [B][n_heads][576] fp32   absorbed queries
 *   kv   [T][576] fp32            the compressed cache
 *   keys of query b: with idx == NULL the cached prefix t < lens[b]
 *        (lens [B] int32, device; values outside [0, T] are clamped); with
 *        idx [B][n_sel] int32 (device) the listed rows, entries outside
 *        [0, T) skipped (the sparse selection of the pages' DSA indexer;
 *        each listed row counts once per listing)
 *   out  [B][n_heads][512] fp32   written; a query with no key gets zeros
 * Scores and the weighted sum use fp32 matrix-core products with fp32
 * accumulation and a max-shifted, base-2 softmax; the keys are split over
 * workgroups and the partial results merged in a second kernel, in a fixed
 * order (results are bitwise reproducible).  Requires n_sel >= 1 when idx
 * is given, a finite scale, workspace_bytes >= coli_mla_workspace_bytes. */
int coli_mla_decode(const float *q, int32_t B, int32_t n_heads, const float *kv, int32_t T,
                    const int32_t *lens, const int32_t *idx, int32_t n_sel, float scale,
                    float *out, void *workspace, size_t workspace_bytes, void *hip_stream);

/* coli_mla_decode that also records, through each kernel's own dispatch,
 * events[0] / events[1] at the start / end of the attention kernel and
 * events[2] / events[3] around the merge kernel (n_events >= 4, hipEvent_t
 * values created by the caller with timing).  For measurement only. */
int coli_mla_decode_profiled(const float *q, int32_t B, int32_t n_heads, const float *kv,
                             int32_t T, const int32_t *lens, const int32_t *idx, int32_t n_sel,
                             float scale, float *out, void *workspace, size_t workspace_bytes,
                             void **events, int32_t n_events, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_MLA_H */
