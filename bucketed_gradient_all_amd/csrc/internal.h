// Internal types shared by the host reducer (reducer.cpp) and the bucket
// reduction kernels (reduce_kernels.h and the .hip files that instantiate
// them). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace ddp {

constexpr int kThreads = 256;   // one workgroup = four wave64s

// Vector groups (of 4 elements) each thread carries per replica: the tile is
// kThreads * 4 * U elements and a thread holds W * U 16-byte loads in flight.
// Chosen by measurement together with the workgroups per CU each launch
// allows (the host's occupancy rule). For the
// all-reduce of fp32 gradients (W read and W write streams), small tiles with
// two workgroups per CU beat large tiles with one from W = 5 up (one
// workgroup's stores overlap the other's loads), and W = 2 runs small tiles
// uncapped; W = 1, 3 and 4 keep four groups. Accumulating bf16 wgrads into
// fp32 main_grad at W = 16 does better with two groups and one workgroup per
// CU (at W = 8 both shapes measured the same; the generic kernel, W = 9..15,
// loses with larger tiles, which only add serial passes; W = 32 would spill
// registers). The reduce-scatter (W reads, one write) keeps the larger tiles
// up to W = 8.
// bf16_accum: input mode DDP_IN_BF16_ACCUM_F32.
constexpr int unroll_for(int W, bool reduce_scatter, bool bf16_accum)
{
    if (reduce_scatter) return W <= 4 ? 4 : (W <= 8 ? 2 : 1);
    if (bf16_accum && W == 16) return 2;
    return (W == 2 || W >= 5) ? 1 : 4;
}

// Whether an instance has a two-tile form (two consecutive tiles per
// workgroup): the all-reduce instances with small tiles (one vector group per
// thread) that the automatic cap runs two per CU, W = 5 to 8.
constexpr bool pairs_tiles(int W, bool reduce_scatter, bool partial, bool bf16_accum)
{
    return !reduce_scatter && !partial && W >= 5 && W <= 8 && unroll_for(W, reduce_scatter, bf16_accum) == 1;
}

// Elements one workgroup covers (one tile).
constexpr int64_t tile_elems(int W, bool reduce_scatter, bool bf16_accum)
{
    return int64_t(kThreads) * 4 * unroll_for(W, reduce_scatter, bf16_accum);
}

// A run of bucket elements that lies inside one gradient tensor and one ring
// chunk, so every element in it has the same source tensor and the same fold
// order.
struct DeviceSeg {
    int64_t flat;    // first element in the flat buffers
    int64_t src;     // first element inside the source gradient (COPY, BF16_ACCUM)
    int64_t len;     // elements
    int32_t param;   // source gradient (COPY, BF16_ACCUM); -1 for VIEW
    int32_t chunk;   // ring chunk c: the fold starts at replica c
    int32_t tile0;   // first tile of this segment
    int32_t head;    // scalar elements (0..63) before the aligned vector body,
                     // or -1: the segment is processed one element per lane
    uint64_t used;   // bit w: replica w contributes the segment's gradient (unused
                     // detection; all ones otherwise). Part of the record so that a
                     // tile fetches its segment and its mask in one round trip.
};
static_assert(sizeof(DeviceSeg) == 48, "segment records are three 16-byte loads");

struct KernelTables {
    const DeviceSeg *segs;
    const int32_t *tile_seg;       // tile -> segment
    const void *const *grads;      // [W*P] replica-major source pointers (COPY, BF16_ACCUM)
    float *const *flat;            // [W] flat buffers
    int32_t masked;                // unused detection: the segments' replica masks apply
    int32_t n_params;
};

// Scaling of one replica's term. The mean multiplies by s = fp32(1/W); the
// compression hooks divide by w = W, or multiply by s when divide is 0 (W a
// power of two, where both give the same quotient).
struct Scale {
    float s;
    float w;
    int32_t divide;
};

// Each enqueues tiles [tile_begin, tile_begin + n_tiles) of the table on
// stream s: all-reduce (the sum stored to every replica) or reduce-scatter
// (chunk c stored to replica c only), and returns hipSuccess or the launch
// error. With t.masked set (unused detection), a replica whose bit in the
// segment's mask is clear contributes a zero-filled slice (its source is not
// read) and a gradient no replica used is not written at all.
//   launch_mean:       the fp32 mean (no communication hook)
//   launch_bf16_hook:  through the bf16 compression hook
//   launch_fp16_hook:  through the fp16 compression hook
// lds_bytes: LDS each workgroup reserves (unused by the kernel; it bounds the
// workgroups resident per CU). pair: two consecutive tiles per workgroup, for
// launches that run one workgroup per CU; only the instances that have that
// form use it (pairs_tiles), the others ignore it.
hipError_t launch_mean(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                       int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s);
hipError_t launch_bf16_hook(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                            int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s);
hipError_t launch_fp16_hook(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                            int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s);

}  // namespace ddp
