// K3 / K4, bf16: one launch per GEMM stage.  A workgroup is 8 waves, one per
// CU (persistent grid): first the 256-row tiles (experts with more than 128
// rows), then the 64-row x 512-column tiles (the other experts), both staged
// through one LDS buffer.  Both designs follow the same arithmetic contract
// (gemm_bf16_small.h), so which one computes a row never changes its bits.
#include <hip/hip_ext.h>

#include "gemm_bf16_lds.h"
#include "gemm_bf16_small.h"

namespace moe {

template <bool FC1>
__global__ void __launch_bounds__(512, 1) gemm_bf16_kernel(GemmArgs g)
{
    static_assert(kSmallLds >= kRing * kStageBytes, "one LDS buffer serves both tile designs");
    __shared__ __attribute__((aligned(1024))) char smem[kSmallLds];
    // both tile counts in one scalar load, and the first 64-row tile's table
    // entry fetched beside them (its index clamped into the table; unused when
    // the tile does not exist), so the first weight loads wait for one round trip
    const int n_big = ld_const(&g.hdr->n_tiles_big);
    const int n_small = ld_const(&g.hdr->n_tiles);
    const int* te0 = (const int*)(g.tiles + min((int)blockIdx.x / small_col_tiles(g), g.max_tiles - 1));
    const int e0 = ld_const(te0), row00 = ld_const(te0 + 1);
    asm volatile("" : : "s"(n_big), "s"(n_small), "s"(e0), "s"(row00));   // one round trip for all four
    lds_tiles<FC1>(g, smem, n_big);
    small_tiles<FC1>(g, smem, n_small, e0, row00);
}

// t0 / t1 (optional): events that receive the launch's own start and end
// (recorded by the dispatch itself, no separate marker in the stream)
hipError_t launch_gemm_bf16(bool fc1, const GemmArgs& g, int num_cu, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1)
{
    // a multiple of 8 workgroups: the LDS-staged loop splits its tiles over the 8 XCDs
    dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8)), block(512);
    auto go = [&](auto kernel) {
        if (t0 || t1)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, g);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, s, g);
    };
    if (fc1) go(gemm_bf16_kernel<true>);
    else go(gemm_bf16_kernel<false>);
    return hipGetLastError();
}

}  // namespace moe
