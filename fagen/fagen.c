/*
 * fagen.c - seeded, counter-based input generator for the flash-attention
 * training forward workloads.
 *
 * This file holds none of the attention arithmetic: it only produces input
 * tensors (bf16 bit patterns and an f32 additive mask) from a 64-bit seed, so
 * that the CPU oracle and the GPU path can be fed identical bytes.
 *
 * Construction (all public definitions):
 *   - word(seed, stream, i): the SplitMix64 output function (Steele, Lea and
 *     Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
 *     applied to the Weyl sequence  base + (i + 1) * 0x9E3779B97F4A7C15,
 *     where base = mix64(seed ^ ((stream + 1) * 0x9E3779B97F4A7C15)).
 *     Every element is a pure function of (seed, stream, i), so the tensor can
 *     be split across threads without changing a single bit.
 *   - uniforms: the top 53 bits of a word scaled by 2^-53.
 *   - normals: the Box-Muller transform (Box and Muller, 1958) on the pair of
 *     words (2j, 2j+1): r = sqrt(-2 ln u1), z0 = r cos(2 pi u2),
 *     z1 = r sin(2 pi u2), u1 in (0,1], u2 in [0,1); computed in double,
 *     multiplied by sigma, cast to float, then rounded to bf16 with
 *     round-to-nearest-even on the f32 bit pattern.
 *   - mask: each entry is -inf with probability p (uniform < p), else 0; then
 *     for every (b,h) a partial Fisher-Yates shuffle of the query rows picks
 *     n_full distinct rows that are set entirely to -inf.
 *   - the method's own test inputs (fagen_lcg_*): the 64-bit linear
 *     congruential generator of its test page ("mlx-native 0.9.0",
 *     tests/test_flash_attn_train.rs, section "Test helpers",
 *     pseudo_random_f32): state <- state * 6364136223846793005 +
 *     1442695040888963407 (mod 2^64), starting from the seed; each value is
 *     the top 31 bits of the new state, converted to f32 (round to nearest),
 *     divided by the f32 value of 2^32 - 1 (which is 2^32) and lowered by 0.5,
 *     all in f32. The values lie in [-0.5, 0): the top 31 bits are below 2^31.
 *     Sequential by construction (one stream per seed).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t stream)
{
    return mix64(seed ^ (((uint64_t)stream + 1u) * GOLDEN));
}

uint64_t fagen_word(uint64_t seed, uint32_t stream, uint64_t i)
{
    return mix64(stream_base(seed, stream) + (i + 1u) * GOLDEN);
}

static inline double unit_open0(uint64_t w) /* (0, 1] */
{
    return ((double)(w >> 11) + 1.0) * 0x1.0p-53;
}

static inline double unit_closed0(uint64_t w) /* [0, 1) */
{
    return (double)(w >> 11) * 0x1.0p-53;
}

static inline uint16_t f32_to_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN (never produced) */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    uint64_t base;
    double sigma;
    uint16_t *out;
    uint64_t n;
    uint64_t pair_begin, pair_end;
} normal_job;

static void *normal_worker(void *arg)
{
    const normal_job *j = (const normal_job *)arg;
    const double two_pi = 6.283185307179586476925286766559;
    for (uint64_t p = j->pair_begin; p < j->pair_end; ++p) {
        uint64_t i0 = 2 * p, i1 = 2 * p + 1;
        double u1 = unit_open0(mix64(j->base + (i0 + 1u) * GOLDEN));
        double u2 = unit_closed0(mix64(j->base + (i1 + 1u) * GOLDEN));
        double r = sqrt(-2.0 * log(u1));
        double z0 = r * cos(two_pi * u2);
        double z1 = r * sin(two_pi * u2);
        j->out[i0] = f32_to_bf16_rne((float)(j->sigma * z0));
        if (i1 < j->n)
            j->out[i1] = f32_to_bf16_rne((float)(j->sigma * z1));
    }
    return NULL;
}

/* n iid N(0, sigma^2) values rounded to bf16, written as raw bf16 bits. */
int fagen_normal_bf16(uint64_t seed, uint32_t stream, double sigma, uint16_t *out,
                      uint64_t n, int n_threads)
{
    if (!out && n)
        return 1;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    uint64_t pairs = (n + 1) / 2;
    if (pairs < (uint64_t)n_threads * 4096u)
        n_threads = 1;
    pthread_t tid[256];
    normal_job jobs[256];
    uint64_t base = stream_base(seed, stream);
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].base = base;
        jobs[t].sigma = sigma;
        jobs[t].out = out;
        jobs[t].n = n;
        jobs[t].pair_begin = pairs * (uint64_t)t / (uint64_t)n_threads;
        jobs[t].pair_end = pairs * (uint64_t)(t + 1) / (uint64_t)n_threads;
    }
    if (n_threads == 1) {
        normal_worker(&jobs[0]);
        return 0;
    }
    for (int t = 0; t < n_threads; ++t)
        if (pthread_create(&tid[t], NULL, normal_worker, &jobs[t]) != 0)
            return 2;
    for (int t = 0; t < n_threads; ++t)
        pthread_join(tid[t], NULL);
    return 0;
}

/*
 * Additive mask [B,H,ql,kl] (f32): entry -inf with probability p_masked,
 * else 0 (stream `stream_bern`, counter = flat index); then n_full distinct
 * rows per (b,h), picked by a partial Fisher-Yates shuffle of 0..ql-1 driven
 * by stream `stream_rows` (counter = (b*H+h)*n_full + t), are set to -inf.
 * The picked row indices are written to rows_out [B*H*n_full] if non-NULL.
 */
int fagen_mask_f32(uint64_t seed, uint32_t stream_bern, uint32_t stream_rows,
                   double p_masked, int n_full, int64_t B, int64_t H, int64_t ql,
                   int64_t kl, float *out, int32_t *rows_out)
{
    if (B < 0 || H < 0 || ql < 0 || kl < 0 || n_full < 0 || n_full > ql)
        return 1;
    uint64_t total = (uint64_t)B * H * ql * kl;
    if (total && !out)
        return 1;
    uint64_t bbase = stream_base(seed, stream_bern);
    for (uint64_t i = 0; i < total; ++i) {
        double u = unit_closed0(mix64(bbase + (i + 1u) * GOLDEN));
        out[i] = (u < p_masked) ? -INFINITY : 0.0f;
    }
    if (n_full == 0 || ql == 0)
        return 0;
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)ql);
    if (!perm)
        return 2;
    uint64_t rbase = stream_base(seed, stream_rows);
    for (int64_t bh = 0; bh < B * H; ++bh) {
        for (int64_t r = 0; r < ql; ++r)
            perm[r] = (int32_t)r;
        for (int t = 0; t < n_full; ++t) {
            uint64_t w = mix64(rbase + ((uint64_t)bh * n_full + t + 1u) * GOLDEN);
            uint64_t span = (uint64_t)(ql - t);
            uint64_t pick = (uint64_t)(((unsigned __int128)w * span) >> 64);
            int32_t tmp = perm[t];
            perm[t] = perm[t + pick];
            perm[t + pick] = tmp;
            int64_t row = perm[t];
            float *dst = out + ((uint64_t)bh * ql + row) * kl;
            for (int64_t j = 0; j < kl; ++j)
                dst[j] = -INFINITY;
            if (rows_out)
                rows_out[bh * n_full + t] = (int32_t)row;
        }
    }
    free(perm);
    return 0;
}

/* n values of the test page's LCG from `seed` (f32, in [-0.5, 0)). */
void fagen_lcg_f32(uint64_t seed, uint64_t n, float *out)
{
    uint64_t state = seed;
    const float denom = (float)UINT32_MAX; /* rounds to 2^32 */
    for (uint64_t i = 0; i < n; ++i) {
        state = state * 6364136223846793005ULL + 1442695040888963407ULL;
        out[i] = (float)(state >> 33) / denom - 0.5f;
    }
}

/* The same values rounded to bf16 (round to nearest even), as raw bits. */
void fagen_lcg_bf16(uint64_t seed, uint64_t n, uint16_t *out)
{
    uint64_t state = seed;
    const float denom = (float)UINT32_MAX;
    for (uint64_t i = 0; i < n; ++i) {
        state = state * 6364136223846793005ULL + 1442695040888963407ULL;
        out[i] = f32_to_bf16_rne((float)(state >> 33) / denom - 0.5f);
    }
}
