/* synth.h — seeded synthetic gradient generator and workload stand-ins.
 *
 * This module creates inputs only. It contains none of the bucketed
 * reduction's arithmetic; both the CPU oracle (through the host half) and the
 * GPU path (through the device half) take their gradients from it.
 *
 * Generator (a counter-based SplitMix64, Steele, Lea & Flood, OOPSLA 2014,
 * output function as published by S. Vigna):
 *
 *   sm64(x):  z = x + 0x9E3779B97F4A7C15
 *             z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *             z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *             return z ^ (z >> 31)                      (all mod 2^64)
 *
 *   key(seed, stream, replica, param)
 *       = sm64(sm64(sm64(sm64(seed) ^ stream) ^ replica) ^ param)
 *   draw(key, n) = sm64(key + n * 0x9E3779B97F4A7C15)
 *
 *   unit(h) = fp32(h >> 40) * 2^-23 - 1        exact, in [-1, 1)
 *
 *   UNIFORM  element i:  unit(draw(key, i))
 *   NORMAL   element i:  h1 = draw(key, 2i), h2 = draw(key, 2i+1)
 *                        u1 = unit(h1), u2 = unit(h1 << 24),
 *                        u3 = unit(h2), u4 = unit(h2 << 24)
 *                        z  = ((u1 + u2) + (u3 + u4)) * c,
 *                        c  = fp32(sigma * sqrt(3) / 2)
 *            (Irwin-Hall sum of four uniforms: zero mean, standard deviation
 *             sigma; every step is one correctly rounded fp32 + or *, in this
 *             order, so host and device agree bit for bit)
 *   BF16 element: round-to-nearest-even of the fp32 draw to its top 16 bits.
 *
 * All functions return 0 on success, a negative value on error.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SYNTH_UNIFORM = 0, SYNTH_NORMAL = 1 };

/* ---- host half (libsynth_host.so, plain C) ---- */
uint64_t synth_sm64(uint64_t x);
uint64_t synth_key(uint64_t seed, uint32_t stream, uint32_t replica, uint32_t param);
float    synth_normal_scale(double sigma);
/* element i of a stream, as fp32 */
float    synth_value(uint64_t key, int dist, float scale, int64_t i);
/* dst[j] = element (first + j), j in [0, n) */
int synth_fill_f32_host(float *dst, int64_t n, uint64_t key, int dist, float scale, int64_t first);
/* dst[j] = bf16 bits of element (first + j) */
int synth_fill_bf16_host(uint16_t *dst, int64_t n, uint64_t key, int dist, float scale, int64_t first);
/* dst[j] = element idx[j] */
int synth_gather_f32_host(float *dst, const int64_t *idx, int64_t m, uint64_t key, int dist, float scale);
int synth_gather_bf16_host(uint16_t *dst, const int64_t *idx, int64_t m, uint64_t key, int dist, float scale);

/* ---- device half (libsynth_dev.so, HIP for gfx950) ---- */
typedef struct {
    void    *dst;      /* device pointer, fp32 or bf16 elements              */
    int64_t  n;        /* elements to write                                 */
    uint64_t key;      /* synth_key(...) of the tensor                      */
} synth_entry;

/* Fill every entry (all fp32 when out_bf16 == 0, all bf16 otherwise) in one
 * launch on `stream` (a hipStream_t; NULL = default stream). Blocks until the
 * fill has completed. */
int synth_fill_dev(const synth_entry *entries, int32_t n_entries, int dist, float scale,
                   int32_t out_bf16, void *stream);
/* Plain 16-byte vector copy of `bytes` (a multiple of 16) between 16-byte
 * aligned device buffers; a known-size kernel for calibrating HBM counters. */
int synth_copy_dev(void *dst, const void *src, int64_t bytes, void *stream);
/* HBM-rate probe over `world` (1, 2, 4, 8, 16 or 32) equal-sized buffers whose
 * device pointers sit in the device tables src_table / dst_table: `tiles`
 * workgroups of 256 threads, each moving one 4 KiB tile of every buffer
 * (every buffer holds tiles * 4096 bytes, 16-byte aligned). kind 0 reads the
 * sources (sink: a device array of 256 uint32 that is written only if a
 * loaded word pattern is all ones), 1 writes the destinations, 2 copies
 * source k to destination k, 3 reads the sources and the 16-bit buffers of
 * aux_table (tiles * 2048 bytes each, 8-byte aligned) and writes the sources
 * back in place: the byte pattern of accumulating bf16 wgrads into fp32
 * main_grad. Tables a kind does not use may be NULL. workgroups_per_cu
 * (0..8; 0 = no cap) bounds the workgroups resident per CU the way the
 * reduction does, with reserved LDS. Enqueued on `stream`; returns -1 on bad
 * arguments or a launch error. */
int synth_stream_probe_dev(int kind, int32_t world, const void *src_table, const void *dst_table,
                           const void *aux_table, void *sink, int64_t tiles, int32_t workgroups_per_cu, void *stream);
/* One workgroup that waits `microseconds` of wall-clock time on the device
 * (at most 10 s); a stand-in for a slice of backward compute. */
int synth_spin_dev(double microseconds, void *stream);
const char *synth_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
