// Device templates of the bucket reduction, shared by the translation units
// that instantiate them (bucket_reduce.hip: the fp32 mean; bucket_bf16_hook.hip
// and bucket_fp16_hook.hip: the compression hooks). Not part of the C ABI.
//
// One launch reduces a range of tiles over W replicas resident in HBM: for
// every element it reads the W replicas' values, forms each replica's term,
// sums the terms in the ring all-reduce's order for the element's chunk and
// writes the sum to all W flat buffers (or to the chunk owner's only). This
// fuses three steps of the pages' design into a single pass over HBM: the
// copy of each gradient into its bucket with its scaling [DDP-ch17 §17.9,
// §17.12], the reduce-scatter half of the ring and its all-gather half
// [DDP-ch17 §17.4]; in bf16 mode the accumulation of the bf16 weight
// gradient into the fp32 main_grad is fused in as well [MegatronDDP §1].
//
// Terms and sums per hook:
//   mean:            t = y * fp32(1/W);            acc = acc + t
//   bf16/fp16 hook:  t = R(R(y) / W);              acc = R(acc + t)
// with y the replica's gradient (or main_grad + wgrad), R the round-to-
// nearest-even conversion to the 16-bit wire format (kept widened in fp32
// registers) and every operation rounded on its own (no contraction), so the
// results equal the CPU oracle bit for bit. The compression hooks cast, then
// divide by W, and round each hop's sum to the wire format [DDP-ch17 §17.9];
// the decompressed result is the widened wire value.
//
// It is a streaming reduction (a few ALU operations per element against 8 or
// 10 bytes of HBM traffic per element and replica), far below the fp32 ridge
// point, so it runs on the vector ALUs; the design aims only at HBM:
//   * the host cuts each bucket into segments that lie inside one gradient
//     tensor and one ring chunk, so a workgroup has one source tensor and one
//     fold order (wave-uniform addresses in scalar registers, no per-lane
//     branching on the chunk);
//   * the fold order is fixed by loading replica (c + k) mod W into register
//     slot k, so the order is a plain slot-0..W-1 sum; W is a compile-time
//     constant for W = 1..8, 16, 32, and W = 9..31 run the 16- or 32-slot
//     instance with the slots past W switched off;
//   * 16-byte vector loads and stores (8-byte for bf16), every load of a
//     thread issued before the first add, non-temporal hints on the streamed
//     data so it does not evict other lines from L2 / MALL.
// The reduce-scatter variant (ZeRO-1 [MegatronDDP §3]) folds the same way but
// stores chunk c only to replica c's flat buffer. With unused-parameter
// detection, a replica that did not use a gradient contributes a zero-filled
// slice (its source is not read), and a gradient no replica used is left
// untouched [DDP-ch17 §17.33].
#pragma once

#include "internal.h"

#include <hip/hip_runtime.h>

namespace ddp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

enum { MODE_COPY = 0, MODE_VIEW = 1, MODE_BF16 = 2 };
enum { HOOK_MEAN = 0, HOOK_BF16 = 1, HOOK_FP16 = 2 };

__device__ __forceinline__ float widen(unsigned short b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// R: round to the wire format, returned widened. Both use gfx950's
// conversion instructions (v_cvt_pk_bf16_f32, v_cvt_f16_f32) under the
// default mode: round to nearest even, overflow to inf, subnormals kept
// (the kernels run with fp32 and fp16 denormals enabled), NaN stays NaN.
// The empty asm pins v as an fp32 register value: without it the compiler
// merges the fp32 multiply or add that produced v with the conversion into
// one mixed-precision FMA (v_fma_mix*_f16 with a +0 addend), which rounds
// once instead of twice and turns a -0 product into +0.
template <int HOOK>
__device__ __forceinline__ float wire(float v)
{
    if (HOOK == HOOK_BF16) return static_cast<float>(static_cast<__bf16>(v));
    if (HOOK == HOOK_FP16) {
        asm volatile("" : "+v"(v));
        return static_cast<float>(static_cast<_Float16>(v));
    }
    return v;
}

// Every buffer the kernels touch is device (global) memory; saying so lets
// the compiler emit global_* rather than flat_* memory instructions, which
// only count against the vector-memory counter.
#define GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ f32x4 ld4(const float *p)
{
    return __builtin_nontemporal_load((const GLOBAL f32x4 *)(p));
}

__device__ __forceinline__ u16x4 ld4h(const unsigned short *p)
{
    return __builtin_nontemporal_load((const GLOBAL u16x4 *)(p));
}

// Masked loads through a buffer resource (a base address and a byte range):
// a load at an offset outside the range returns zero without touching
// memory, so a replica that did not use a gradient gets range 0 and its
// loads cost no memory traffic, with no branch and no address select. The
// third dword is the gfx9 default (32-bit data format, untyped access); the
// aux operand 2 is the nontemporal hint the global loads use.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_of(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ f32x4 ld4_in(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, kLoadNT));
}

__device__ __forceinline__ u16x4 ld4h_in(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(u16x4, __builtin_amdgcn_raw_buffer_load_b64(r, int(byte_off), 0, kLoadNT));
}

// Stores of the instances that write through the L2: a buffer store with
// the nontemporal hint at device scope (aux bits nt | sc1). The L2 of each
// XCD is not coherent with the others, so a device-scope store goes on to
// memory instead of lingering as a dirty line the next reduction has to
// evict; an offset past the range drops the store.
constexpr int kStoreThrough = 2 | 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st4_in(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(byte_off), 0, kStoreThrough);
}

// The instances that store through the L2 (all-reduce at 8, 16 and 32
// replicas; measured: +1.5-4% for ResNet-50 and BERT-large, +2% for the
// W = 16 and W = 32 sweeps; not kept where it lost, as for the reduce-scatter
// and W = 4).
constexpr bool writes_through(int W, bool rs, bool partial)
{
    return !rs && !partial && (W == 8 || W == 16 || W == 32);
}
static_assert(!writes_through(16, false, true), "partial instances keep their global stores");

__device__ __forceinline__ void st4(float *p, f32x4 v)
{
    __builtin_nontemporal_store(v, (GLOBAL f32x4 *)(p));
}

__device__ __forceinline__ float ld1(const float *p)
{
    return *(const GLOBAL float *)(p);
}

__device__ __forceinline__ unsigned short ld1h(const unsigned short *p)
{
    return *(const GLOBAL unsigned short *)(p);
}

__device__ __forceinline__ void st1(float *p, float v)
{
    *(GLOBAL float *)(p) = v;
}

// How a compression hook divides by W: DIV_MUL multiplies by s = fp32(1/W)
// (W a power of two: the same quotient as a division), DIV_TRUE divides,
// DIV_RUNTIME reads the choice from the Scale (W only known at run time).
enum { DIV_MUL = 0, DIV_TRUE = 1, DIV_RUNTIME = 2 };

constexpr int div_for(int W)
{
    return (W & (W - 1)) == 0 ? DIV_MUL : DIV_TRUE;
}

// One replica's term. y = x, or main + wgrad in bf16 mode; the mean scales
// by s = fp32(1/W); a compression hook casts, divides by W and casts.
template <int MODE, int HOOK, int DIV>
__device__ __forceinline__ float term1(float x, unsigned short g, const Scale &sc)
{
    const float y = MODE == MODE_BF16 ? __fadd_rn(x, widen(g)) : x;
    if (HOOK == HOOK_MEAN) return __fmul_rn(y, sc.s);
    const float h = wire<HOOK>(y);
    const bool divide = DIV == DIV_TRUE || (DIV == DIV_RUNTIME && sc.divide);
    return wire<HOOK>(divide ? __fdiv_rn(h, sc.w) : __fmul_rn(h, sc.s));
}

template <int HOOK>
__device__ __forceinline__ float add1(float a, float b)
{
    return wire<HOOK>(__fadd_rn(a, b));
}

template <int MODE, int HOOK, int DIV>
__device__ __forceinline__ f32x4 term4(f32x4 x, u16x4 g, const Scale &sc)
{
    return f32x4{term1<MODE, HOOK, DIV>(x.x, g.x, sc), term1<MODE, HOOK, DIV>(x.y, g.y, sc),
                 term1<MODE, HOOK, DIV>(x.z, g.z, sc), term1<MODE, HOOK, DIV>(x.w, g.w, sc)};
}

template <int HOOK>
__device__ __forceinline__ f32x4 add4(f32x4 a, f32x4 b)
{
    return f32x4{add1<HOOK>(a.x, b.x), add1<HOOK>(a.y, b.y), add1<HOOK>(a.z, b.z), add1<HOOK>(a.w, b.w)};
}

__device__ __forceinline__ int slot_replica(int chunk, int k, int W)
{
    int r = chunk + k;
    return r >= W ? r - W : r;
}

// Source of replica r for a segment: the gradient tensor (COPY, bf16 wgrad)
// or the flat buffer itself (VIEW).
template <int MODE>
__device__ __forceinline__ const float *src_f32(const KernelTables &T, const DeviceSeg &sg, int r)
{
    if (MODE == MODE_COPY) return static_cast<const float *>(T.grads[int64_t(r) * T.n_params + sg.param]) + sg.src;
    return T.flat[r] + sg.flat;   // VIEW input and bf16-mode main_grad live in the flat buffer
}

__device__ __forceinline__ const unsigned short *src_bf16(const KernelTables &T, const DeviceSeg &sg, int r)
{
    return static_cast<const unsigned short *>(T.grads[int64_t(r) * T.n_params + sg.param]) + sg.src;
}

// Whether replica r contributes under mask m. Masks exist for W <= 64 only;
// replicas past 64 (W > 64, no masks) always contribute, and the shift stays
// below 64.
__device__ __forceinline__ bool replica_on(uint64_t m, int r)
{
    return r >= 64 || ((m >> r) & 1);
}

// One element, any W: used for unaligned heads and tails and for segments
// whose pointers do not allow 16-byte vectors.
template <int MODE, int HOOK>
__device__ void fold_scalar(const KernelTables &T, const DeviceSeg &sg, uint64_t m, int64_t e, const Scale &sc, int W,
                            bool rs)
{
    float acc = 0.0f;
    for (int k = 0; k < W; ++k) {
        const int r = slot_replica(sg.chunk, k, W);
        float t = 0.0f;
        if (replica_on(m, r)) {
            float x = ld1(src_f32<MODE>(T, sg, r) + e);
            unsigned short g = MODE == MODE_BF16 ? ld1h(src_bf16(T, sg, r) + e) : 0;
            t = term1<MODE, HOOK, DIV_RUNTIME>(x, g, sc);
        }
        acc = k == 0 ? t : add1<HOOK>(acc, t);
    }
    if (rs) {
        st1(T.flat[sg.chunk] + sg.flat + e, acc);
        return;
    }
    for (int w = 0; w < W; ++w) st1(T.flat[w] + sg.flat + e, acc);
}

// Heads, tails and scalar-only segments of a tile.
template <int MODE, int HOOK>
__device__ __forceinline__ void scalar_parts(const KernelTables &T, const DeviceSeg &sg, uint64_t m, int64_t tin,
                                             int64_t tile, const Scale &sc, int W, bool rs)
{
    const int tid = threadIdx.x;
    if (sg.head >= 0) {
        if (tin != 0) return;
        const int64_t body = (sg.len - sg.head) / 4 * 4;
        const int64_t tail = sg.len - sg.head - body;
        if (tid < sg.head) fold_scalar<MODE, HOOK>(T, sg, m, tid, sc, W, rs);
        if (tid >= 64 && tid < 64 + tail) fold_scalar<MODE, HOOK>(T, sg, m, sg.head + body + (tid - 64), sc, W, rs);
        return;
    }
    const int64_t base = tin * tile;
    for (int64_t j = tid; j < tile; j += kThreads) {
        const int64_t e = base + j;
        if (e < sg.len) fold_scalar<MODE, HOOK>(T, sg, m, e, sc, W, rs);
    }
}

// Replica slots of a kernel instance: W of them at compile time. With
// PARTIAL the replica count n (n <= W) is known only at run time, and slots
// k >= n are absent: not read, not added (adding a zero would turn a -0 sum
// into +0) and not written. Such instances serve the replica counts without
// an instance of their own, with the fixed instances' single pass (every
// load before the first add) instead of the generic kernel's groups of eight.
template <int W, bool PARTIAL>
struct Slots {
    int n;
    __device__ __forceinline__ bool has(int k) const { return !PARTIAL || k < n; }
    __device__ __forceinline__ int count() const { return PARTIAL ? n : W; }
};

// The division rule of an instance: fixed by W, or read from the Scale when
// the replica count is only known at run time.
template <int W, bool PARTIAL>
constexpr int div_of()
{
    return PARTIAL ? DIV_RUNTIME : div_for(W);
}

// One element from hoisted pointers; the sum goes to the NOUT destinations
// (all replicas, or the chunk's owner).
template <int W, int NOUT, int MODE, int HOOK, bool USED, bool PARTIAL>
__device__ __forceinline__ void fold_scalar_fixed(const float *const (&xs)[W], const unsigned short *const (&gs)[W],
                                                  float *const (&ds)[NOUT], uint64_t on, int64_t e,
                                                  const Scale &sc, Slots<W, PARTIAL> slots, bool write)
{
    float t[W];
#pragma unroll
    for (int k = 0; k < W; ++k) {
        if (slots.has(k) && (!USED || ((on >> k) & 1)))
            t[k] = term1<MODE, HOOK, div_of<W, PARTIAL>()>(ld1(xs[k] + e), MODE == MODE_BF16 ? ld1h(gs[k] + e) : 0,
                                                          sc);
        else
            t[k] = 0.0f;
    }
    float acc = t[0];
#pragma unroll
    for (int k = 1; k < W; ++k)
        if (slots.has(k)) acc = add1<HOOK>(acc, t[k]);
    if (!write) return;
#pragma unroll
    for (int w = 0; w < NOUT; ++w)
        if (NOUT == 1 || slots.has(w)) st1(ds[w] + e, acc);
}

// The 16-byte-vector part of one tile: U groups of 4 elements per thread.
// CHECK = false: the whole tile lies inside the segment body (the common
// case), so the block is straight-line code: all W*U loads, then the folds,
// then all stores. CHECK = true: the segment's last tile, with per-lane
// bounds; out-of-range lanes load an in-bounds vector (value unused) and skip
// their stores.
//
// With USED the loads go through buffer resources over this tile of each
// replica's source: a replica that did not use the gradient gets range 0,
// so its loads return the zero-filled slice its term is defined by (a +0
// input) and read nothing, with no branch; an out-of-range lane of the last
// tile gets an offset past every range and reads nothing either. The
// instances that write through the L2 store the same way, over this tile of
// each destination.
//
// The part is split in three steps (the lanes' offsets, the loads, the folds
// and stores) so that a workgroup holding two tiles can issue both tiles'
// loads before its first store.
template <int U>
struct TileLanes {
    int64_t t0;          // the tile's first element
    int64_t e[U];        // element of vector group u
    int64_t el[U];       // the element a lane loads (in bounds also for lanes past the segment)
    uint32_t rel[U];     // element offset from t0 (buffer loads and stores)
    bool ok[U];          // vector group u lies inside the segment
    uint32_t span;       // elements of the tile inside the segment
};

template <int U, bool CHECK>
__device__ __forceinline__ TileLanes<U> tile_lanes(const DeviceSeg &sg, int64_t tin)
{
    constexpr int64_t TILE = int64_t(kThreads) * 4 * U;
    constexpr uint32_t kPast = 0x3FFFFFF0u;   // an element offset past every range (x4 bytes still fits)
    const int tid = int(threadIdx.x);
    TileLanes<U> L;
    L.t0 = sg.head + tin * TILE;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t r = int64_t(u * kThreads + tid) * 4;
        L.e[u] = L.t0 + r;
        L.ok[u] = !CHECK || L.e[u] + 4 <= sg.len;
        L.el[u] = L.ok[u] ? L.e[u] : int64_t(sg.head);   // the segment's first vector: in bounds
        L.rel[u] = L.ok[u] ? uint32_t(r) : kPast;
    }
    // elements of this tile inside the segment (the last tile may hold fewer,
    // or none past its head: t0 can exceed len by less than one vector group)
    L.span = CHECK ? uint32_t(sg.len > L.t0 ? (sg.len - L.t0 < TILE ? sg.len - L.t0 : TILE) : 0) : uint32_t(TILE);
    return L;
}

template <int W, int U, int MODE, bool USED, bool PARTIAL>
__device__ __forceinline__ void vector_load(const float *const (&xs)[W], const unsigned short *const (&gs)[W],
                                            uint64_t on, const TileLanes<U> &L, Slots<W, PARTIAL> slots,
                                            f32x4 (&v)[U][W], u16x4 (&g)[U][W])
{
#pragma unroll
    for (int k = 0; k < W; ++k) {
        if (!slots.has(k)) {   // an absent slot: nothing to read
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v[u][k] = f32x4{0, 0, 0, 0};
                g[u][k] = u16x4{0, 0, 0, 0};
            }
            continue;
        }
        if (USED) {
            const bool use = (on >> k) & 1;
            const __amdgpu_buffer_rsrc_t rx = range_of(xs[k] + L.t0, use ? 4 * L.span : 0);
#pragma unroll
            for (int u = 0; u < U; ++u) v[u][k] = ld4_in(rx, 4 * L.rel[u]);
            if (MODE == MODE_BF16) {
                const __amdgpu_buffer_rsrc_t rg = range_of(gs[k] + L.t0, use ? 2 * L.span : 0);
#pragma unroll
                for (int u = 0; u < U; ++u) g[u][k] = ld4h_in(rg, 2 * L.rel[u]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) g[u][k] = u16x4{0, 0, 0, 0};
            }
            continue;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u][k] = ld4(xs[k] + L.el[u]);
            g[u][k] = MODE == MODE_BF16 ? ld4h(gs[k] + L.el[u]) : u16x4{0, 0, 0, 0};
        }
    }
}

template <int W, int NOUT, int U, int MODE, int HOOK, bool RS, bool PARTIAL>
__device__ __forceinline__ void vector_fold_store(const f32x4 (&v)[U][W], const u16x4 (&g)[U][W],
                                                  float *const (&ds)[NOUT], const TileLanes<U> &L,
                                                  const Scale &sc, Slots<W, PARTIAL> slots, bool write)
{
    constexpr int DIV = div_of<W, PARTIAL>();
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        acc[u] = term4<MODE, HOOK, DIV>(v[u][0], g[u][0], sc);
#pragma unroll
        for (int k = 1; k < W; ++k)
            if (slots.has(k)) acc[u] = add4<HOOK>(acc[u], term4<MODE, HOOK, DIV>(v[u][k], g[u][k], sc));
    }
    if constexpr (writes_through(W, RS, PARTIAL)) {
        // through a buffer resource over this tile of each destination: the
        // lanes past the segment (offset past the range) and a gradient no
        // replica used (range 0) store nothing
        const uint32_t range = write ? 4 * L.span : 0;
#pragma unroll
        for (int w = 0; w < NOUT; ++w) {
            if (!(NOUT == 1 || slots.has(w))) continue;   // an absent slot has no destination
            const __amdgpu_buffer_rsrc_t rd = range_of(ds[w] + L.t0, range);
#pragma unroll
            for (int u = 0; u < U; ++u) st4_in(rd, 4 * L.rel[u], acc[u]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (L.ok[u] && write) {
#pragma unroll
                for (int w = 0; w < NOUT; ++w)
                    if (NOUT == 1 || slots.has(w)) st4(ds[w] + L.e[u], acc[u]);
            }
    }
}

template <int W, int NOUT, int MODE, int HOOK, bool RS, bool CHECK, bool USED, bool PARTIAL>
__device__ __forceinline__ void vector_tile(const float *const (&xs)[W], const unsigned short *const (&gs)[W],
                                            float *const (&ds)[NOUT], uint64_t on, const DeviceSeg &sg,
                                            int64_t tin, const Scale &sc, Slots<W, PARTIAL> slots, bool write)
{
    constexpr int U = PARTIAL ? 1 : unroll_for(W, RS, MODE == MODE_BF16);
    const TileLanes<U> L = tile_lanes<U, CHECK>(sg, tin);
    f32x4 v[U][W];
    u16x4 g[U][W];
    vector_load<W, U, MODE, USED, PARTIAL>(xs, gs, on, L, slots, v, g);
    vector_fold_store<W, NOUT, U, MODE, HOOK, RS, PARTIAL>(v, g, ds, L, sc, slots, write);
}

// Everything one tile needs before its first memory access: its segment, its
// index inside it, the hoisted source and destination pointers, and the slot
// mask. All table reads (segment, source and destination pointers) happen
// here, before the first store, so they stay in scalar registers; a table
// read after a store would have to go through the vector memory path and wait
// for every outstanding store.
template <int W, int NOUT>
struct TileRefs {
    DeviceSeg sg;
    int64_t tin;
    const float *xs[W];
    const unsigned short *gs[W];
    float *ds[NOUT];
    uint64_t on;   // bit k: slot k contributes
    bool write;    // false: no replica used the gradient, leave it untouched
};

template <int W, int NOUT, int MODE, bool RS, bool USED, bool PARTIAL>
__device__ __forceinline__ void tile_refs(const KernelTables &T, int32_t tile, Slots<W, PARTIAL> slots,
                                          TileRefs<W, NOUT> &t)
{
    const int nrep = slots.count();
    t.sg = T.segs[T.tile_seg[tile]];
    const DeviceSeg &sg = t.sg;
    const uint64_t m = USED ? sg.used : ~uint64_t(0);
    t.tin = int64_t(tile - sg.tile0);

    // slot k holds replica (chunk + k) mod nrep, so the fold is slot 0, 1, ...
#pragma unroll
    for (int k = 0; k < W; ++k) {
        t.xs[k] = nullptr;
        t.gs[k] = nullptr;
        if (!slots.has(k)) continue;
        const int r = slot_replica(sg.chunk, k, nrep);
        t.xs[k] = src_f32<MODE>(T, sg, r);
        t.gs[k] = MODE == MODE_BF16 ? src_bf16(T, sg, r) : nullptr;
    }
    if (MODE != MODE_COPY) {
        // The sources are the flat buffers themselves (VIEW input, bf16-mode
        // main_grad). Slot k reads replica (chunk + k) mod n, so slot 0 is the
        // chunk's owner and the slots cover every replica once: the stores go
        // through the source pointers, and no second set of W pointers takes
        // scalar registers.
#pragma unroll
        for (int w = 0; w < NOUT; ++w) t.ds[w] = slots.has(w) ? const_cast<float *>(t.xs[w]) : nullptr;
    } else if (RS) {
        t.ds[0] = T.flat[sg.chunk] + sg.flat;   // chunk c belongs to replica c
    } else {
#pragma unroll
        for (int w = 0; w < NOUT; ++w) t.ds[w] = slots.has(w) ? T.flat[w] + sg.flat : nullptr;
    }

    // No early exit when no replica used the gradient: a branch on the mask
    // ahead of the loads lets the compiler fetch the mask chain first and the
    // segment chain only after it (two more round trips per tile). With every
    // replica's range empty nothing is read; the stores are skipped.
    // Slot bits: bit k is set when slot k's replica, (chunk + k) mod n, used
    // the gradient: the replica mask rotated into fold order (n <= 32 here).
    // One 64-bit value instead of a flag per slot, which would take a scalar
    // register pair each.
    t.on = ~uint64_t(0);
    t.write = true;
    if (USED) {
        t.write = m != 0;
        const uint64_t full = (uint64_t(1) << nrep) - 1;
        const uint64_t mm = m & full;
        const int c = sg.chunk;
        t.on = ((mm >> c) | (mm << (nrep - c))) & full;
    }
}

// One tile: the vector body (whole or last tile of the segment), the first
// tile's scalar head and tail, or a segment folded one element per lane.
template <int W, int NOUT, int MODE, int HOOK, bool RS, bool USED, bool PARTIAL>
__device__ __forceinline__ void run_tile(const TileRefs<W, NOUT> &t, const Scale &sc, Slots<W, PARTIAL> slots)
{
    constexpr int64_t TILE = PARTIAL ? int64_t(kThreads) * 4 : tile_elems(W, RS, MODE == MODE_BF16);
    const DeviceSeg &sg = t.sg;
    const int64_t tin = t.tin;
    const int tid = int(threadIdx.x);
    if (sg.head >= 0) {
        if (sg.head + (tin + 1) * TILE <= sg.len)
            vector_tile<W, NOUT, MODE, HOOK, RS, false, USED, PARTIAL>(t.xs, t.gs, t.ds, t.on, sg, tin, sc, slots,
                                                                       t.write);
        else if (sg.len - sg.head >= 4)
            vector_tile<W, NOUT, MODE, HOOK, RS, true, USED, PARTIAL>(t.xs, t.gs, t.ds, t.on, sg, tin, sc, slots,
                                                                      t.write);
        if (tin == 0) {
            const int64_t body = (sg.len - sg.head) / 4 * 4;
            const int64_t tail = sg.len - sg.head - body;
            if (tid < sg.head)
                fold_scalar_fixed<W, NOUT, MODE, HOOK, USED, PARTIAL>(t.xs, t.gs, t.ds, t.on, tid, sc, slots,
                                                                      t.write);
            if (tid >= 64 && tid < 64 + tail)
                fold_scalar_fixed<W, NOUT, MODE, HOOK, USED, PARTIAL>(t.xs, t.gs, t.ds, t.on,
                                                                      sg.head + body + (tid - 64), sc, slots, t.write);
        }
        return;
    }
    for (int64_t j = tid; j < TILE; j += kThreads) {
        const int64_t e = tin * TILE + j;
        if (e < sg.len)
            fold_scalar_fixed<W, NOUT, MODE, HOOK, USED, PARTIAL>(t.xs, t.gs, t.ds, t.on, e, sc, slots, t.write);
    }
}

// W slots at compile time: fully unrolled over replicas and vector groups.
// With PARTIAL, n replicas (n <= W, known at run time) fill the first n
// slots and the tiles are 4 elements per thread (the host's tiling for every
// replica count these instances serve).
//
// Waves per SIMD an instance is compiled for: the most the automatic cap
// lets share a SIMD. The 32-slot instances run at most two workgroups per CU
// (two waves per SIMD); saying so lets the compiler keep all 32 loads of a
// group in flight before the first add, where aiming at more waves it holds
// back the later loads until earlier ones return (measured: +4% for
// reduce-scatter and +2% with unused masks at W = 32, no change at W = 16).
// The all-reduce of bf16 wgrads into fp32 main_grad at 16 replicas runs one
// workgroup per CU (one wave per SIMD), so its 64 loads per thread may use
// the whole register file (measured in one process on one set of buffers:
// 5691-5694 against 5605-5651 GB/s on the Megatron Llama-1B workload).
template <int W, int MODE, bool RS, bool PARTIAL>
constexpr int max_waves_per_simd()
{
    if (W == 16 && MODE == MODE_BF16 && !RS && !PARTIAL) return 1;
    return W >= 32 ? 2 : 8;
}

template <int W, int MODE, int HOOK, bool RS, bool USED, bool PARTIAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, max_waves_per_simd<W, MODE, RS, PARTIAL>())))
void reduce_fixed(
    KernelTables T, int32_t tile_begin, Scale sc, int n)
{
    constexpr int NOUT = RS ? 1 : W;
    const Slots<W, PARTIAL> slots{n};
    TileRefs<W, NOUT> t;
    tile_refs<W, NOUT, MODE, RS, USED, PARTIAL>(T, tile_begin + int32_t(blockIdx.x), slots, t);
    run_tile<W, NOUT, MODE, HOOK, RS, USED, PARTIAL>(t, sc, slots);
}

// Two consecutive tiles per workgroup, for launches that run one workgroup
// per CU with a small-tile instance (beside a running backward): the same
// bytes in flight per CU as two single-tile workgroups, in half as many
// workgroups, which leaves the backward's kernels more room. Both tiles'
// tables are read first; when both tiles are whole vector tiles (the common
// case), the second tile's loads go out before the first tile's stores, else
// the two run one after the other. tile_end bounds the launch: the last
// workgroup of an odd count holds one tile.
template <int W, int MODE, int HOOK, bool USED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 8)))
void reduce_pair(KernelTables T, int32_t tile_begin, int32_t tile_end, Scale sc)
{
    static_assert(pairs_tiles(W, false, false, MODE == MODE_BF16), "no two-tile form");
    constexpr int U = 1;
    constexpr int64_t TILE = tile_elems(W, false, MODE == MODE_BF16);
    const Slots<W, false> slots{W};
    const int32_t first = tile_begin + 2 * int32_t(blockIdx.x);
    const bool two = first + 1 < tile_end;
    TileRefs<W, W> a, b;
    tile_refs<W, W, MODE, false, USED, false>(T, first, slots, a);
    if (two) tile_refs<W, W, MODE, false, USED, false>(T, first + 1, slots, b);
    // a whole vector tile with no scalar head or tail to fold
    auto whole = [](const TileRefs<W, W> &t) {
        return t.sg.head >= 0 && t.tin != 0 && t.sg.head + (t.tin + 1) * TILE <= t.sg.len;
    };
    if (two && whole(a) && whole(b)) {
        const TileLanes<U> la = tile_lanes<U, false>(a.sg, a.tin);
        const TileLanes<U> lb = tile_lanes<U, false>(b.sg, b.tin);
        f32x4 va[U][W], vb[U][W];
        u16x4 ga[U][W], gb[U][W];
        vector_load<W, U, MODE, USED, false>(a.xs, a.gs, a.on, la, slots, va, ga);
        vector_load<W, U, MODE, USED, false>(b.xs, b.gs, b.on, lb, slots, vb, gb);
        vector_fold_store<W, W, U, MODE, HOOK, false, false>(va, ga, a.ds, la, sc, slots, a.write);
        vector_fold_store<W, W, U, MODE, HOOK, false, false>(vb, gb, b.ds, lb, sc, slots, b.write);
        return;
    }
    run_tile<W, W, MODE, HOOK, false, USED, false>(a, sc, slots);
    if (two) run_tile<W, W, MODE, HOOK, false, USED, false>(b, sc, slots);
}

// Any W the fixed and partial instances do not serve (above 32): replicas are
// taken eight at a time, in fold order. It walks its tile with any tiling.
template <int MODE, int HOOK>
__global__ __launch_bounds__(kThreads) void reduce_generic(KernelTables T, int32_t tile_begin, Scale sc, int W,
                                                           int rs)
{
    const int64_t TILE = tile_elems(W, rs != 0, MODE == MODE_BF16);
    const int32_t tile = tile_begin + int32_t(blockIdx.x);
    const DeviceSeg sg = T.segs[T.tile_seg[tile]];
    const int64_t tin = int64_t(tile - sg.tile0);
    const uint64_t m = sg.used;   // all ones without unused detection
    if (m == 0) return;   // no replica used this gradient: leave it untouched

    if (sg.head >= 0) {
        for (int64_t e = sg.head + tin * TILE + int64_t(threadIdx.x) * 4; e < sg.head + (tin + 1) * TILE;
             e += int64_t(kThreads) * 4) {
            if (e + 4 > sg.len) break;
            f32x4 acc = f32x4{0, 0, 0, 0};
            for (int k0 = 0; k0 < W; k0 += 8) {
                f32x4 v[8];
                u16x4 g[8];
                bool on[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    on[j] = false;
                    if (k0 + j < W) {
                        const int r = slot_replica(sg.chunk, k0 + j, W);
                        on[j] = replica_on(m, r);
                        if (on[j]) {
                            v[j] = ld4(src_f32<MODE>(T, sg, r) + e);
                            g[j] = MODE == MODE_BF16 ? ld4h(src_bf16(T, sg, r) + e) : u16x4{0, 0, 0, 0};
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (k0 + j < W) {
                        const f32x4 t = on[j] ? term4<MODE, HOOK, DIV_RUNTIME>(v[j], g[j], sc) : f32x4{0, 0, 0, 0};
                        acc = (k0 + j == 0) ? t : add4<HOOK>(acc, t);
                    }
                }
            }
            if (rs) {
                st4(T.flat[sg.chunk] + sg.flat + e, acc);
            } else {
                for (int w = 0; w < W; ++w) st4(T.flat[w] + sg.flat + e, acc);
            }
        }
    }
    scalar_parts<MODE, HOOK>(T, sg, m, tin, TILE, sc, W, rs != 0);
}

// n: the replica count (at most W; below W only with PARTIAL). pair: two
// tiles per workgroup where the instance has that form (pairs_tiles), else
// ignored.
template <int W, int MODE, int HOOK, bool PARTIAL>
hipError_t launch_fixed(const KernelTables &t, int32_t tile_begin, int32_t n_tiles, const Scale &sc, bool rs,
                        unsigned lds, hipStream_t st, int n, bool pair)
{
    const dim3 b(kThreads);
    if constexpr (pairs_tiles(W, false, PARTIAL, MODE == MODE_BF16)) {
        if (pair && !rs) {
            const dim3 g2((unsigned(n_tiles) + 1) / 2);
            const int32_t tile_end = tile_begin + n_tiles;
            if (t.masked)
                hipLaunchKernelGGL((reduce_pair<W, MODE, HOOK, true>), g2, b, lds, st, t, tile_begin, tile_end, sc);
            else
                hipLaunchKernelGGL((reduce_pair<W, MODE, HOOK, false>), g2, b, lds, st, t, tile_begin, tile_end, sc);
            return hipGetLastError();
        }
    }
    const dim3 g(n_tiles);
    if (t.masked) {
        if (rs)
            hipLaunchKernelGGL((reduce_fixed<W, MODE, HOOK, true, true, PARTIAL>), g, b, lds, st, t, tile_begin, sc, n);
        else
            hipLaunchKernelGGL((reduce_fixed<W, MODE, HOOK, false, true, PARTIAL>), g, b, lds, st, t, tile_begin, sc,
                               n);
    } else {
        if (rs)
            hipLaunchKernelGGL((reduce_fixed<W, MODE, HOOK, true, false, PARTIAL>), g, b, lds, st, t, tile_begin, sc,
                               n);
        else
            hipLaunchKernelGGL((reduce_fixed<W, MODE, HOOK, false, false, PARTIAL>), g, b, lds, st, t, tile_begin,
                               sc, n);
    }
    return hipGetLastError();
}

template <int MODE, int HOOK>
hipError_t dispatch_w(int W, bool rs, const KernelTables &t, int32_t tile_begin, int32_t n_tiles, const Scale &sc,
                      unsigned lds, hipStream_t st, bool pair)
{
    switch (W) {
    case 1: return launch_fixed<1, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 2: return launch_fixed<2, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 3: return launch_fixed<3, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 4: return launch_fixed<4, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 5: return launch_fixed<5, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 6: return launch_fixed<6, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 7: return launch_fixed<7, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 8: return launch_fixed<8, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 16: return launch_fixed<16, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    case 32: return launch_fixed<32, MODE, HOOK, false>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
    default:
        // the partial instances tile 4 elements per thread, as the host does
        // for every replica count between 9 and 31 (checked, so that a change
        // of the tiling rule falls back to the generic kernel)
        if (W > 8 && W < 16 && unroll_for(W, rs, MODE == MODE_BF16) == 1)
            return launch_fixed<16, MODE, HOOK, true>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
        if (W > 16 && W < 32 && unroll_for(W, rs, MODE == MODE_BF16) == 1)
            return launch_fixed<32, MODE, HOOK, true>(t, tile_begin, n_tiles, sc, rs, lds, st, W, pair);
        hipLaunchKernelGGL((reduce_generic<MODE, HOOK>), dim3(n_tiles), dim3(kThreads), lds, st, t, tile_begin, sc,
                           W, rs ? 1 : 0);
        return hipGetLastError();
    }
}

template <int HOOK>
hipError_t dispatch_mode(int mode, int W, bool rs, const KernelTables &t, int32_t tile_begin, int32_t n_tiles,
                         const Scale &sc, unsigned lds, hipStream_t st, bool pair)
{
    switch (mode) {
    case MODE_COPY: return dispatch_w<MODE_COPY, HOOK>(W, rs, t, tile_begin, n_tiles, sc, lds, st, pair);
    case MODE_VIEW: return dispatch_w<MODE_VIEW, HOOK>(W, rs, t, tile_begin, n_tiles, sc, lds, st, pair);
    case MODE_BF16: return dispatch_w<MODE_BF16, HOOK>(W, rs, t, tile_begin, n_tiles, sc, lds, st, pair);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ddp
