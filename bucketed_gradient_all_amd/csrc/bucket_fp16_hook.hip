// Bucket reduction through the fp16 compression hook [DDP-ch17 §17.9]: as
// the bf16 hook, with IEEE binary16 as the wire format (division by W before
// the sum keeps it in range; a gradient beyond fp16's range becomes inf).
// The kernels themselves are in reduce_kernels.h.
#include "reduce_kernels.h"

namespace ddp {

hipError_t launch_fp16_hook(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                            int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s)
{
    if (n_tiles <= 0) return hipSuccess;
    return dispatch_mode<HOOK_FP16>(mode, W, reduce_scatter, t, tile_begin, n_tiles, sc, lds_bytes, s, pair);
}

}  // namespace ddp
