// K3 / K4, bf16: one launch per GEMM stage.  A workgroup is 8 waves, one per
// CU (persistent grid): first the LDS-staged tiles (experts with more than 128
// rows) with all 8 waves, then the streaming tiles (the other experts) with
// its two 4-wave halves as independent workers.  Both designs follow the same
// arithmetic contract (gemm_bf16_stream.h), so which one computes a row never
// changes its bits.
#include "gemm_bf16_lds.h"
#include "gemm_bf16_stream.h"

namespace moe {

template <bool FC1>
__global__ void __launch_bounds__(512, 1) gemm_bf16_kernel(GemmArgs g)
{
    lds_tiles<FC1>(g);
    // the two halves of a workgroup are workers b and b + grid: consecutive
    // tiles (the N tiles of one M tile) go to different CUs
    stream_tiles<FC1>(g, blockIdx.x + (threadIdx.x >> 8) * gridDim.x, 2 * gridDim.x, (threadIdx.x >> 6) & 3);
}

hipError_t launch_gemm_bf16(bool fc1, const GemmArgs& g, int num_cu, hipStream_t s)
{
    // a multiple of 8 workgroups: the LDS-staged loop splits its tiles over the 8 XCDs
    dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8)), block(512);
    if (fc1)
        hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, block, 0, s, g);
    else
        hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, block, 0, s, g);
    return hipGetLastError();
}

}  // namespace moe
