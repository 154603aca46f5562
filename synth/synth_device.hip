// Device half of the synthetic gradient generator (definition in synth.h),
// plus workload stand-ins used around the reduction: a plain vector copy of
// known size (to calibrate HBM byte counters), a wall-clock wait that stands
// in for a slice of backward compute, and probes of the HBM rate of W
// equal-offset streams (data movement only).
#include "synth.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(const char *what, hipError_t e)
{
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return -1;
}

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;
constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int64_t kBlockElems = int64_t(kThreads) * kPerThread;

__device__ __forceinline__ uint64_t sm64(uint64_t x)
{
    uint64_t z = x + kGolden;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float unit24(uint64_t h)
{
    float k = static_cast<float>(static_cast<uint32_t>(h >> 40));
    return __fsub_rn(__fmul_rn(k, 0x1p-23f), 1.0f);
}

__device__ __forceinline__ float value(uint64_t key, int dist, float scale, int64_t i)
{
    if (dist == SYNTH_UNIFORM) return unit24(sm64(key + static_cast<uint64_t>(i) * kGolden));
    uint64_t h1 = sm64(key + static_cast<uint64_t>(2 * i) * kGolden);
    uint64_t h2 = sm64(key + static_cast<uint64_t>(2 * i + 1) * kGolden);
    float a = __fadd_rn(unit24(h1), unit24(h1 << 24));
    float b = __fadd_rn(unit24(h2), unit24(h2 << 24));
    return __fmul_rn(__fadd_rn(a, b), scale);
}

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

struct BlockRef {
    int32_t entry;
    int32_t pad;
    int64_t first;   // first element of the entry this block writes
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void fill_kernel(const synth_entry *__restrict__ entries,
                                                        const BlockRef *__restrict__ blocks,
                                                        int dist, float scale)
{
    const BlockRef br = blocks[blockIdx.x];
    const synth_entry en = entries[br.entry];
    for (int k = 0; k < kPerThread; ++k) {
        int64_t i = br.first + int64_t(k) * kThreads + threadIdx.x;
        if (i < en.n) {
            float v = value(en.key, dist, scale, i);
            if (BF16)
                static_cast<uint16_t *>(en.dst)[i] = to_bf16(v);
            else
                static_cast<float *>(en.dst)[i] = v;
        }
    }
}

__global__ __launch_bounds__(256) void copy_kernel(float4 *__restrict__ dst, const float4 *__restrict__ src,
                                                   int64_t n16)
{
    int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// One 4 KiB tile of every one of W buffers per 256-thread workgroup, the
// reduction's launch shape. KIND 0 reads the W sources (the loaded words are
// OR-ed and compared with a pattern the probe's fill never produces, so the
// loads stay live; nothing is stored), KIND 1 writes a constant to the W
// destinations, KIND 2 copies source k to destination k, KIND 3 is the
// byte pattern of accumulating bf16 wgrads into fp32 main_grad: it reads a
// 2 KiB tile of W 16-bit buffers (aux, kept live like KIND 0) and the W fp32
// sources, and writes the fp32 values back in place. Nontemporal loads and
// stores, as in the reduction.
typedef float probe_f4 __attribute__((ext_vector_type(4)));
typedef unsigned probe_u4 __attribute__((ext_vector_type(4)));
typedef unsigned probe_u2 __attribute__((ext_vector_type(2)));
#define PROBE_GLOBAL __attribute__((address_space(1)))   // global-memory instructions, as the reduction uses

template <class T>
__device__ __forceinline__ T probe_ld(const T *p)
{
    return __builtin_nontemporal_load((const PROBE_GLOBAL T *)(p));
}

template <class T>
__device__ __forceinline__ void probe_st(T v, T *p)
{
    __builtin_nontemporal_store(v, (PROBE_GLOBAL T *)(p));
}

template <int W, int KIND>
__global__ __launch_bounds__(256) void stream_probe_kernel(const probe_f4 *const *__restrict__ src,
                                                           probe_f4 *const *__restrict__ dst,
                                                           const probe_u2 *const *__restrict__ aux,
                                                           unsigned *__restrict__ sink)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (KIND == 3) {
        probe_f4 v[W];
        probe_u2 h[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            v[k] = probe_ld(src[k] + i);
            h[k] = probe_ld(aux[k] + i);
        }
        unsigned bits = 0;
#pragma unroll
        for (int k = 0; k < W; ++k) bits |= h[k].x & h[k].y;
        if (bits == 0xFFFFFFFFu) sink[threadIdx.x] = bits;
#pragma unroll
        for (int k = 0; k < W; ++k) {
            // an empty asm that claims to change v[k]: without it the
            // compiler may drop the store of a value just loaded from the
            // same address, and the probe would write nothing
            asm volatile("" : "+v"(v[k]));
            probe_st(v[k], const_cast<probe_f4 *>(src[k]) + i);
        }
        return;
    }
    if (KIND == 1) {
        const probe_f4 c = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int k = 0; k < W; ++k) probe_st(c, dst[k] + i);
        return;
    }
    probe_f4 v[W];
#pragma unroll
    for (int k = 0; k < W; ++k) v[k] = probe_ld(src[k] + i);
    if (KIND == 2) {
#pragma unroll
        for (int k = 0; k < W; ++k) probe_st(v[k], dst[k] + i);
        return;
    }
    probe_u4 bits = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < W; ++k) bits |= __builtin_bit_cast(probe_u4, v[k]);
    if ((bits.x & bits.y & bits.z & bits.w) == 0xFFFFFFFFu) sink[threadIdx.x] = bits.x;
}

template <int W>
hipError_t launch_probe(int kind, const void *src, const void *dst, const void *aux, void *sink, unsigned grid,
                        unsigned lds, hipStream_t st)
{
    const auto *s = static_cast<const probe_f4 *const *>(src);
    auto *d = static_cast<probe_f4 *const *>(const_cast<void *>(dst));
    const auto *a = static_cast<const probe_u2 *const *>(aux);
    auto *k = static_cast<unsigned *>(sink);
    if (kind == 0) hipLaunchKernelGGL((stream_probe_kernel<W, 0>), dim3(grid), dim3(256), lds, st, s, d, a, k);
    else if (kind == 1) hipLaunchKernelGGL((stream_probe_kernel<W, 1>), dim3(grid), dim3(256), lds, st, s, d, a, k);
    else if (kind == 2) hipLaunchKernelGGL((stream_probe_kernel<W, 2>), dim3(grid), dim3(256), lds, st, s, d, a, k);
    else hipLaunchKernelGGL((stream_probe_kernel<W, 3>), dim3(grid), dim3(256), lds, st, s, d, a, k);
    return hipGetLastError();
}

__global__ void spin_kernel(uint64_t ticks, uint64_t max_iter)
{
    uint64_t t0 = wall_clock64();
    for (uint64_t it = 0; it < max_iter; ++it) {
        if (wall_clock64() - t0 >= ticks) break;
        __builtin_amdgcn_s_sleep(8);
    }
}

}  // namespace

extern "C" {

const char *synth_last_error(void) { return g_err.c_str(); }

int synth_fill_dev(const synth_entry *entries, int32_t n_entries, int dist, float scale, int32_t out_bf16,
                   void *stream)
{
    if (n_entries < 0 || (n_entries > 0 && !entries)) {
        g_err = "synth_fill_dev: bad entry list";
        return -1;
    }
    std::vector<BlockRef> blocks;
    for (int32_t e = 0; e < n_entries; ++e) {
        if (entries[e].n < 0 || (entries[e].n > 0 && !entries[e].dst)) {
            g_err = "synth_fill_dev: bad entry " + std::to_string(e);
            return -1;
        }
        for (int64_t f = 0; f < entries[e].n; f += kBlockElems) blocks.push_back(BlockRef{e, 0, f});
    }
    if (blocks.empty()) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    synth_entry *d_entries = nullptr;
    BlockRef *d_blocks = nullptr;
    hipError_t err = hipMalloc(&d_entries, sizeof(synth_entry) * n_entries);
    if (err != hipSuccess) return fail("hipMalloc", err);
    err = hipMalloc(&d_blocks, sizeof(BlockRef) * blocks.size());
    if (err != hipSuccess) {
        (void)hipFree(d_entries);
        return fail("hipMalloc", err);
    }
    int rc = 0;
    err = hipMemcpy(d_entries, entries, sizeof(synth_entry) * n_entries, hipMemcpyHostToDevice);
    if (err == hipSuccess)
        err = hipMemcpy(d_blocks, blocks.data(), sizeof(BlockRef) * blocks.size(), hipMemcpyHostToDevice);
    if (err != hipSuccess) {
        rc = fail("hipMemcpy", err);
    } else {
        // one launch covers at most 2^30 blocks; larger jobs are split
        const size_t max_grid = size_t(1) << 30;
        for (size_t b0 = 0; b0 < blocks.size() && rc == 0; b0 += max_grid) {
            unsigned grid = unsigned(std::min(max_grid, blocks.size() - b0));
            if (out_bf16)
                hipLaunchKernelGGL(fill_kernel<true>, dim3(grid), dim3(kThreads), 0, s, d_entries,
                                   d_blocks + b0, dist, scale);
            else
                hipLaunchKernelGGL(fill_kernel<false>, dim3(grid), dim3(kThreads), 0, s, d_entries,
                                   d_blocks + b0, dist, scale);
            err = hipGetLastError();
            if (err != hipSuccess) rc = fail("fill launch", err);
        }
        err = hipStreamSynchronize(s);
        if (err != hipSuccess && rc == 0) rc = fail("hipStreamSynchronize", err);
    }
    (void)hipFree(d_blocks);
    (void)hipFree(d_entries);
    return rc;
}

int synth_copy_dev(void *dst, const void *src, int64_t bytes, void *stream)
{
    if (bytes < 0 || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16 ||
        reinterpret_cast<uintptr_t>(src) % 16) {
        g_err = "synth_copy_dev: size and pointers must be multiples of 16 bytes";
        return -1;
    }
    int64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    int64_t want = (n16 + 255) / 256;
    unsigned grid = unsigned(std::min<int64_t>(want, 256 * 64));
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<float4 *>(dst), static_cast<const float4 *>(src), n16);
    hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : fail("copy launch", err);
}

int synth_stream_probe_dev(int kind, int32_t world, const void *src_table, const void *dst_table,
                           const void *aux_table, void *sink, int64_t tiles, int32_t workgroups_per_cu, void *stream)
{
    if (kind < 0 || kind > 3 || tiles < 0 || tiles > int64_t(0x7FFFFFFF) || workgroups_per_cu < 0 ||
        workgroups_per_cu > 8 || (kind != 1 && (!src_table || !sink)) || ((kind == 1 || kind == 2) && !dst_table) ||
        (kind == 3 && !aux_table)) {
        g_err = "synth_stream_probe_dev: bad kind, tile count, cap or table";
        return -1;
    }
    if (tiles == 0) return 0;
    // the occupancy cap as the reduction sets it: LDS reserved so that at
    // most workgroups_per_cu workgroups fit on a CU (0: no cap)
    unsigned lds = 0;
    if (workgroups_per_cu > 0) {
        int dev = 0, per_cu = 0, per_block = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (err == hipSuccess) err = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (err != hipSuccess) return fail("LDS sizes", err);
        int bytes = per_cu / (workgroups_per_cu + 1) + 2048;
        bytes = (bytes + 255) / 256 * 256;
        lds = unsigned(std::min(bytes, per_block));
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned grid = unsigned(tiles);
    hipError_t err;
    switch (world) {
    case 1: err = launch_probe<1>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    case 2: err = launch_probe<2>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    case 4: err = launch_probe<4>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    case 8: err = launch_probe<8>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    case 16: err = launch_probe<16>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    case 32: err = launch_probe<32>(kind, src_table, dst_table, aux_table, sink, grid, lds, st); break;
    default:
        g_err = "synth_stream_probe_dev: world must be 1, 2, 4, 8, 16 or 32";
        return -1;
    }
    return err == hipSuccess ? 0 : fail("stream probe launch", err);
}

int synth_spin_dev(double microseconds, void *stream)
{
    if (!(microseconds >= 0.0) || microseconds > 10e6) {
        g_err = "synth_spin_dev: duration must be in [0, 10 s]";
        return -1;
    }
    int dev = 0, khz = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (err != hipSuccess) return fail("wall clock rate", err);
    if (khz <= 0) {
        g_err = "synth_spin_dev: device reports no wall clock rate";
        return -1;
    }
    uint64_t ticks = uint64_t(microseconds * double(khz) / 1000.0);
    // one iteration (a clock read plus a 512-cycle sleep) lasts far longer than
    // one tick, so this bound never cuts a real wait short, yet still ends the
    // loop if the clock were to stop advancing
    uint64_t max_iter = ticks + 1024;
    hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks, max_iter);
    err = hipGetLastError();
    return err == hipSuccess ? 0 : fail("spin launch", err);
}

}  // extern "C"
