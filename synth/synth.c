/*
 * synth.c -- seeded, counter-based generator of the synthetic inputs of the
 * int4 routed-expert MoE layer (activations, router weights and bias, packed
 * int4 expert weights and their fp16 group scales).
 *
 * This module is shared by the CPU oracle and by the GPU path: both consume
 * the very same host bytes it writes.  It holds no arithmetic of the layer
 * itself -- only random-number generation, the distributions that shape the
 * inputs, and the fp16 encoding of the scales.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based generator: the
 * i-th draw of stream `key` is the SplitMix64 output after i+1 increments of
 * the golden-gamma counter, so any index range can be produced independently
 * (and in parallel) with identical results.
 * Normals: Box-Muller (cosine branch), one normal per pair of uniforms.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_at(uint64_t key, uint64_t i)
{
    return sm_mix(key + (i + 1) * SYNTH_GAMMA);
}

uint64_t synth_key(uint64_t seed, uint64_t stream)
{
    return sm_mix(sm_mix(seed ^ 0x5851F42D4C957F2DULL) ^ (stream * SYNTH_GAMMA));
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i)
{
    return sm_at(synth_key(seed, stream), i);
}

/* uniform double in (0, 1): 53 random bits, centred in their cell */
static inline double u01(uint64_t r) { return ((double)(r >> 11) + 0.5) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t i)
{
    double u1 = u01(sm_at(key, 2 * i));
    double u2 = u01(sm_at(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t i)
{
    return normal_at(synth_key(seed, stream), i);
}

/* IEEE binary16 encoding of a double, round-to-nearest-even, with
 * subnormals and overflow to infinity. */
uint16_t synth_f16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return 0x7E00u;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {
        double r = nearbyint(a * 0x1p24); /* units of the smallest subnormal */
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e;
    double m = frexp(a, &e);         /* a = m * 2^e, m in [0.5, 1) */
    double r = nearbyint(m * 2048.0); /* 11 significant bits */
    int be = e - 1 + 15;
    if (r == 2048.0) { r = 1024.0; be += 1; }
    if (be >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(be << 10) | (uint16_t)((int)r - 1024));
}

/* ---------------------------------------------------------------------- */
/* threaded fill helpers                                                   */

enum { FILL_BYTES, FILL_NORMAL_F32, FILL_LOGNORMAL_F16 };

typedef struct {
    int kind;
    uint64_t key;
    void *dst;
    uint64_t begin, end; /* element range of dst handled by this job */
    uint64_t offset;     /* index of dst[0] in the stream */
    double a, b;         /* distribution parameters */
} fill_job;

static void run_fill(const fill_job *j)
{
    if (j->kind == FILL_BYTES) {
        uint8_t *d = (uint8_t *)j->dst;
        for (uint64_t i = j->begin; i < j->end; ++i) {
            uint64_t g = j->offset + i;
            d[i] = (uint8_t)(sm_at(j->key, g >> 3) >> (8 * (g & 7)));
        }
    } else if (j->kind == FILL_NORMAL_F32) {
        float *d = (float *)j->dst;
        for (uint64_t i = j->begin; i < j->end; ++i)
            d[i] = (float)(j->a + j->b * normal_at(j->key, j->offset + i));
    } else {
        uint16_t *d = (uint16_t *)j->dst;
        for (uint64_t i = j->begin; i < j->end; ++i)
            d[i] = synth_f16_from_double(exp(j->a + j->b * normal_at(j->key, j->offset + i)));
    }
}

static void *fill_thread(void *p)
{
    run_fill((const fill_job *)p);
    return NULL;
}

#define SYNTH_MAX_THREADS 64

static void parallel_fill(fill_job base, uint64_t n, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > SYNTH_MAX_THREADS) threads = SYNTH_MAX_THREADS;
    if (n < (1u << 16)) threads = 1;
    fill_job jobs[SYNTH_MAX_THREADS];
    pthread_t tid[SYNTH_MAX_THREADS];
    int started[SYNTH_MAX_THREADS];
    uint64_t per = (n + (uint64_t)threads - 1) / (uint64_t)threads;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].begin = (uint64_t)t * per < n ? (uint64_t)t * per : n;
        jobs[t].end = jobs[t].begin + per < n ? jobs[t].begin + per : n;
        started[t] = 0;
        if (t > 0 && jobs[t].begin < jobs[t].end)
            started[t] = pthread_create(&tid[t], NULL, fill_thread, &jobs[t]) == 0;
        if (t > 0 && !started[t]) run_fill(&jobs[t]);
    }
    run_fill(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
}

/* dst[i] = byte (offset+i) of the stream's little-endian 64-bit draws.
 * Used for packed int4 weights: every nibble is uniform on 0..15, i.e. the
 * two's-complement code is uniform on [-8, 7]. */
void synth_fill_bytes(uint64_t seed, uint64_t stream, uint8_t *dst, uint64_t n,
                      uint64_t offset, int threads)
{
    fill_job j = {FILL_BYTES, synth_key(seed, stream), dst, 0, n, offset, 0.0, 0.0};
    parallel_fill(j, n, threads);
}

/* dst[i] = fp32(mean + std * N_{offset+i}) */
void synth_fill_normal_f32(uint64_t seed, uint64_t stream, float *dst, uint64_t n,
                           uint64_t offset, double mean, double std, int threads)
{
    fill_job j = {FILL_NORMAL_F32, synth_key(seed, stream), dst, 0, n, offset, mean, std};
    parallel_fill(j, n, threads);
}

/* dst[i] = fp16(exp(mu + sigma * N_{offset+i})), RNE */
void synth_fill_lognormal_f16(uint64_t seed, uint64_t stream, uint16_t *dst, uint64_t n,
                              uint64_t offset, double mu, double sigma, int threads)
{
    fill_job j = {FILL_LOGNORMAL_F16, synth_key(seed, stream), dst, 0, n, offset, mu, sigma};
    parallel_fill(j, n, threads);
}

/* Overlapping-token activations: x[t][h] = fp32((s[h] + 0.5 z[t][h]) / sqrt(1.25))
 * with s (stream_s, index h) and z (stream_z, index t*H+h) iid N(0,1); every
 * element is N(0,1), tokens share the s component. */
void synth_fill_overlap_x(uint64_t seed, uint64_t stream_s, uint64_t stream_z, float *dst,
                          int32_t T, int32_t H)
{
    uint64_t ks = synth_key(seed, stream_s), kz = synth_key(seed, stream_z);
    double inv = 1.0 / sqrt(1.25);
    for (int32_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double s = normal_at(ks, (uint64_t)h);
            double z = normal_at(kz, (uint64_t)t * (uint64_t)H + (uint64_t)h);
            dst[(size_t)t * H + h] = (float)((s + 0.5 * z) * inv);
        }
}

/* Seeded permutation of 0..n-1 (Fisher-Yates; the index in [0, i] comes from
 * a 64x64->128-bit multiply-shift of one draw, bias below i * 2^-64). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t *perm)
{
    uint64_t key = synth_key(seed, stream);
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    for (int32_t i = n - 1; i > 0; --i) {
        unsigned __int128 m = (unsigned __int128)sm_at(key, (uint64_t)i) * (uint64_t)(i + 1);
        int32_t j = (int32_t)(m >> 64);
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}

/* Zipf(s) popularity expressed as a router bias:
 *   p_r = r^-s / sum_{r'=1..E} r'^-s,  b_e = fp32(tau * ln p_{rank(e)}),
 * where rank(e) = perm[e] + 1 and perm is the seeded permutation above. */
void synth_zipf_bias(uint64_t seed, uint64_t stream, int32_t E, double s, double tau,
                     float *dst)
{
    if (E <= 0) return;
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!perm) return;
    synth_permutation(seed, stream, E, perm);
    double z = 0.0;
    for (int32_t r = 1; r <= E; ++r) z += pow((double)r, -s);
    for (int32_t e = 0; e < E; ++e) {
        double p = pow((double)(perm[e] + 1), -s) / z;
        dst[e] = (float)(tau * log(p));
    }
    free(perm);
}
