// K3 / K4, MXFP8: one launch per GEMM stage.  A workgroup is 8 waves, one per
// CU (persistent grid): first the LDS-staged tiles (experts with more than 128
// rows; only when K is a multiple of 128) with all 8 waves, then the streaming
// tiles with its two 4-wave halves as independent workers.  Both designs follow
// the same arithmetic contract (gemm_mxfp8_stream.h).  W4: MXFP4 weights
// (E2M1 B format) in both designs.
#include <hip/hip_ext.h>

#include "gemm_mxfp8_lds.h"
#include "gemm_mxfp8_stream.h"

namespace moe {

template <bool FC1, bool W4>
__global__ void __launch_bounds__(512, 1) gemm_mxfp8_kernel(MxGemmArgs g)
{
    if (!g.stream_big) mx_lds_tiles<FC1, W4>(g);
    // the two halves of a workgroup are workers b and b + grid: consecutive
    // tiles (the N tiles of one M tile) go to different CUs
    mx_stream_tiles<FC1, W4>(g, blockIdx.x + (threadIdx.x >> 8) * gridDim.x, 2 * gridDim.x, (threadIdx.x >> 6) & 3);
}

// t0 / t1 (optional): events that receive the launch's own start and end
// (recorded by the dispatch itself, no separate marker in the stream)
hipError_t launch_gemm_mxfp8(bool fc1, bool w4, const MxGemmArgs& g, int num_cu, hipStream_t s,
                             hipEvent_t t0, hipEvent_t t1)
{
    if (!g.stream_big && g.K % 128 != 0) return hipErrorInvalidValue;
    dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8)), block(512);
    auto go = [&](auto kernel) {
        if (t0 || t1)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, g);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, s, g);
    };
    if (w4) {
        if (fc1) go(gemm_mxfp8_kernel<true, true>);
        else go(gemm_mxfp8_kernel<false, true>);
    } else {
        if (fc1) go(gemm_mxfp8_kernel<true, false>);
        else go(gemm_mxfp8_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace moe
