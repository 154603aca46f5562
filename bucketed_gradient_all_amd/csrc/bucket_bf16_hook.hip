// Bucket reduction through the bf16 compression hook [DDP-ch17 §17.9]:
// each replica's bucket is cast to bf16 and divided by W, the sum of every
// ring hop is rounded to bf16, and the result is widened into the fp32
// buckets. The kernels themselves are in reduce_kernels.h.
#include "reduce_kernels.h"

namespace ddp {

hipError_t launch_bf16_hook(int mode, int W, bool reduce_scatter, const Scale &sc, const KernelTables &t,
                            int32_t tile_begin, int32_t n_tiles, unsigned lds_bytes, bool pair, hipStream_t s)
{
    if (n_tiles <= 0) return hipSuccess;
    return dispatch_mode<HOOK_BF16>(mode, W, reduce_scatter, t, tile_begin, n_tiles, sc, lds_bytes, s, pair);
}

}  // namespace ddp
