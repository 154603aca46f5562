/* O3 / O5 — the mean over W replicas that a ring all-reduce leaves in a bucket.
 *
 * TEST INFRASTRUCTURE ONLY: called by tests/, smoke() and the CPU-baseline
 * leg of bench.py; never linked by the GPU library. Built with gcc -O2
 * -ffp-contract=off (IEEE binary32, round to nearest even, no FMA, no FTZ).
 *
 * What the pages fix:
 *   - every replica scales its gradient by 1/W while copying it into the
 *     bucket, then the buckets are summed, so the result is the mean
 *     [DDP-ch17 §17.1, §17.9; MegatronDDP §3 (gradient_scaling_factor)];
 *   - bf16 weight gradients are accumulated into an fp32 main_grad and the
 *     reduction runs in fp32 [MegatronDDP §1];
 *   - the ring all-reduce cuts the buffer into W chunks; in the reduce-scatter
 *     phase each rank adds the chunk it receives from its neighbour to its
 *     own copy, W-1 times, after which each rank owns one fully reduced
 *     chunk; the all-gather phase passes those chunks around the ring
 *     [DDP-ch17 §17.4].
 *
 * Readings (where the pages are silent):
 *   - chunk size q = ceil(n / W); chunk c covers [c*q, min((c+1)*q, n));
 *   - at reduce-scatter step s, rank r sends chunk (r - s) mod W to rank r+1,
 *     so chunk c is accumulated starting from replica c, then c+1, ...,
 *     c+W-1 (mod W): acc = (((t_c + t_{c+1}) + t_{c+2}) + ... );
 *   - the scale is s = fp32(1/W) applied by one fp32 multiply per element;
 *   - bf16 accumulate: y = main + fp32(wgrad) (exact widening), t = y * s.
 * Each output is the same value on every replica (the all-gather copies it),
 * so one array is returned per bucket.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MAX_W 1024

static float widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* t[w] holds replica w's scaled value of one element of chunk c */
static float ring_fold(int W, int c, const float *t)
{
    float acc = t[c];
    for (int k = 1; k < W; ++k) acc = acc + t[(c + k) % W];
    return acc;
}

static int64_t chunk_len(int W, int64_t n)
{
    return (n + W - 1) / W;
}

/* ---- whole bucket, fp32 gradients ---- */
static void reduce_range_f32(int W, int64_t n, const float *const *x, float *out, int64_t e0, int64_t e1)
{
    const float s = 1.0f / (float)W;
    const int64_t q = chunk_len(W, n);
    float t[MAX_W];
    for (int64_t e = e0; e < e1; ++e) {
        for (int w = 0; w < W; ++w) t[w] = x[w][e] * s;
        out[e] = ring_fold(W, (int)(e / q), t);
    }
}

/* ---- whole bucket, bf16 wgrad accumulated into fp32 main_grad ---- */
static void reduce_range_bf16acc(int W, int64_t n, const float *const *main_, const uint16_t *const *wg,
                                 float *out, int64_t e0, int64_t e1)
{
    const float s = 1.0f / (float)W;
    const int64_t q = chunk_len(W, n);
    float t[MAX_W];
    for (int64_t e = e0; e < e1; ++e) {
        for (int w = 0; w < W; ++w) {
            float y = main_[w][e] + widen_bf16(wg[w][e]);
            t[w] = y * s;
        }
        out[e] = ring_fold(W, (int)(e / q), t);
    }
}

int oracle_reduce_f32(int W, int64_t n, const float *const *x, float *out)
{
    if (W < 1 || W > MAX_W || n < 0) return -1;
    reduce_range_f32(W, n, x, out, 0, n);
    return 0;
}

int oracle_reduce_bf16acc(int W, int64_t n, const float *const *main_, const uint16_t *const *wg, float *out)
{
    if (W < 1 || W > MAX_W || n < 0) return -1;
    reduce_range_bf16acc(W, n, main_, wg, out, 0, n);
    return 0;
}

/* ---- selected elements of a bucket of n elements ----
 * vals[j*W + w] is replica w's unscaled gradient at bucket element e[j]. */
int oracle_reduce_at_f32(int W, int64_t n, const int64_t *e, int64_t m, const float *vals, float *out)
{
    if (W < 1 || W > MAX_W || n < 0 || m < 0) return -1;
    const float s = 1.0f / (float)W;
    const int64_t q = chunk_len(W, n);
    float t[MAX_W];
    for (int64_t j = 0; j < m; ++j) {
        if (e[j] < 0 || e[j] >= n) return -1;
        for (int w = 0; w < W; ++w) t[w] = vals[j * W + w] * s;
        out[j] = ring_fold(W, (int)(e[j] / q), t);
    }
    return 0;
}

int oracle_reduce_at_bf16acc(int W, int64_t n, const int64_t *e, int64_t m, const float *main_vals,
                             const uint16_t *wg_vals, float *out)
{
    if (W < 1 || W > MAX_W || n < 0 || m < 0) return -1;
    const float s = 1.0f / (float)W;
    const int64_t q = chunk_len(W, n);
    float t[MAX_W];
    for (int64_t j = 0; j < m; ++j) {
        if (e[j] < 0 || e[j] >= n) return -1;
        for (int w = 0; w < W; ++w) {
            float y = main_vals[j * W + w] + widen_bf16(wg_vals[j * W + w]);
            t[w] = y * s;
        }
        out[j] = ring_fold(W, (int)(e[j] / q), t);
    }
    return 0;
}

/* ---- O5: the whole-bucket fp32 fold split over host threads ----
 * Threads own disjoint element ranges; each element is folded exactly as in
 * oracle_reduce_f32, so the bits are identical. */
typedef struct {
    int W;
    int64_t n;
    const float *const *x;
    const float *const *main_;
    const uint16_t *const *wg;
    float *out;
    int64_t e0, e1;
} job_t;

static void *run_f32(void *arg)
{
    job_t *j = (job_t *)arg;
    reduce_range_f32(j->W, j->n, j->x, j->out, j->e0, j->e1);
    return NULL;
}

static void *run_bf16acc(void *arg)
{
    job_t *j = (job_t *)arg;
    reduce_range_bf16acc(j->W, j->n, j->main_, j->wg, j->out, j->e0, j->e1);
    return NULL;
}

static int run_threads(int nthreads, job_t *proto, void *(*fn)(void *))
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int created[256];
    job_t jobs[256];
    int64_t n = proto->n;
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *proto;
        jobs[i].e0 = n * i / nthreads;
        jobs[i].e1 = n * (i + 1) / nthreads;
        created[i] = pthread_create(&th[i], NULL, fn, &jobs[i]) == 0;
        if (!created[i]) fn(&jobs[i]);   /* run inline if a thread cannot be started */
    }
    for (int i = 0; i < nthreads; ++i)
        if (created[i]) rc |= pthread_join(th[i], NULL);
    return rc ? -1 : 0;
}

int oracle_reduce_f32_mt(int W, int64_t n, const float *const *x, float *out, int nthreads)
{
    if (W < 1 || W > MAX_W || n < 0) return -1;
    job_t proto = {W, n, x, NULL, NULL, out, 0, n};
    return run_threads(nthreads, &proto, run_f32);
}

int oracle_reduce_bf16acc_mt(int W, int64_t n, const float *const *main_, const uint16_t *const *wg, float *out,
                             int nthreads)
{
    if (W < 1 || W > MAX_W || n < 0) return -1;
    job_t proto = {W, n, NULL, main_, wg, out, 0, n};
    return run_threads(nthreads, &proto, run_bf16acc);
}
