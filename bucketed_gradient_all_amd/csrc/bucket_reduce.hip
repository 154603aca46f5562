// Bucket reduction to the fp32 mean (the reducer's default path, no
// communication hook): every replica's term is its gradient times fp32(1/W)
// [DDP-ch17 §17.9, §17.12], summed in the ring order of its chunk
// [DDP-ch17 §17.4]. The kernels themselves are in reduce_kernels.h.
#include "reduce_kernels.h"

namespace ddp {

hipError_t launch_mean(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                       int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s)
{
    if (n_tiles <= 0) return hipSuccess;
    return dispatch_mode<HOOK_MEAN>(mode, W, reduce_scatter, t, tile_begin, n_tiles, sc, lds_bytes, s, pair);
}

}  // namespace ddp
