/* Host half of the synthetic gradient generator; definition in synth.h. */
#include "synth.h"

#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

uint64_t synth_sm64(uint64_t x)
{
    uint64_t z = x + GOLDEN;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint32_t stream, uint32_t replica, uint32_t param)
{
    uint64_t k = synth_sm64(seed);
    k = synth_sm64(k ^ (uint64_t)stream);
    k = synth_sm64(k ^ (uint64_t)replica);
    return synth_sm64(k ^ (uint64_t)param);
}

float synth_normal_scale(double sigma)
{
    return (float)(sigma * 0.86602540378443864676);
}

static float unit24(uint64_t h)
{
    /* top 24 bits as an integer, times 2^-23, minus one: every step exact */
    float k = (float)(uint32_t)(h >> 40);
    float t = k * 0x1p-23f;
    return t - 1.0f;
}

float synth_value(uint64_t key, int dist, float scale, int64_t i)
{
    if (dist == SYNTH_UNIFORM)
        return unit24(synth_sm64(key + (uint64_t)i * GOLDEN));
    uint64_t h1 = synth_sm64(key + (uint64_t)(2 * i) * GOLDEN);
    uint64_t h2 = synth_sm64(key + (uint64_t)(2 * i + 1) * GOLDEN);
    float a = unit24(h1) + unit24(h1 << 24);
    float b = unit24(h2) + unit24(h2 << 24);
    float s = a + b;
    return s * scale;
}

static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int synth_fill_f32_host(float *dst, int64_t n, uint64_t key, int dist, float scale, int64_t first)
{
    if (n < 0 || (n > 0 && !dst)) return -1;
    for (int64_t j = 0; j < n; ++j) dst[j] = synth_value(key, dist, scale, first + j);
    return 0;
}

int synth_fill_bf16_host(uint16_t *dst, int64_t n, uint64_t key, int dist, float scale, int64_t first)
{
    if (n < 0 || (n > 0 && !dst)) return -1;
    for (int64_t j = 0; j < n; ++j) dst[j] = to_bf16(synth_value(key, dist, scale, first + j));
    return 0;
}

int synth_gather_f32_host(float *dst, const int64_t *idx, int64_t m, uint64_t key, int dist, float scale)
{
    if (m < 0 || (m > 0 && (!dst || !idx))) return -1;
    for (int64_t j = 0; j < m; ++j) dst[j] = synth_value(key, dist, scale, idx[j]);
    return 0;
}

int synth_gather_bf16_host(uint16_t *dst, const int64_t *idx, int64_t m, uint64_t key, int dist, float scale)
{
    if (m < 0 || (m > 0 && (!dst || !idx))) return -1;
    for (int64_t j = 0; j < m; ++j) dst[j] = to_bf16(synth_value(key, dist, scale, idx[j]));
    return 0;
}
