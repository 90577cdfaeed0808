// K3 / K4, bf16: one launch per GEMM stage.  A workgroup is 8 waves, one per
// CU (persistent grid): first the 256-row tiles (experts with more than 128
// rows), then the 64-row x 512-column tiles (the other experts), both staged
// through one LDS buffer.  Both designs follow the same arithmetic contract
// (gemm_bf16_small.h), so which one computes a row never changes its bits.
#include "gemm_bf16_lds.h"
#include "gemm_bf16_small.h"

namespace moe {

template <bool FC1>
__global__ void __launch_bounds__(512, 1) gemm_bf16_kernel(GemmArgs g)
{
    static_assert(kSmallLds >= kRing * kStageBytes, "one LDS buffer serves both tile designs");
    __shared__ __attribute__((aligned(1024))) char smem[kSmallLds];
    lds_tiles<FC1>(g, smem);
    small_tiles<FC1>(g, smem);
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
