// K3 / K4, MXFP8 / MXFP4.  A workgroup is 8 waves, one per CU (persistent
// grid).  MXFP8: one launch per GEMM stage, first the LDS-staged 256-row tiles
// (experts with more than 128 rows; only when K is a multiple of 128) with all
// 8 waves, then the streaming 64-row tiles with its two 4-wave halves as
// independent workers.  MXFP4 (W4, E2M1 B format): the same, except that with
// K a multiple of 128 the 64-row tiles run in a launch of their own
// (gemm_mx4_small.h), which at token capacities up to 1024 also takes the
// 256-row tiles (then the stage is that one launch).  All designs follow the
// same arithmetic contract (gemm_mxfp8_stream.h).
#include <hip/hip_ext.h>

#include "gemm_mxfp8_lds.h"
#include "gemm_mxfp8_stream.h"
#include "gemm_mx4_small.h"

namespace moe {

// PROB: FC1 with the routes' probabilities applied to the SwiGLU rows (a
// compile-time variant; the default epilogues carry no probability loads)
template <bool FC1, bool W4, bool PROB>
__global__ void __launch_bounds__(512, 1) gemm_mxfp8_kernel(MxGemmArgs g)
{
    if (!g.stream_big) mx_lds_tiles<FC1, W4, PROB>(g);
    if (g.lds_small) return;          // the 64-row tiles have a launch of their own
    // the two halves of a workgroup are workers f and f + grid (f: the
    // workgroup's XCD-contiguous first tile): consecutive tiles (the N tiles of
    // one M tile) go to different CUs of one XCD
    mx_stream_tiles<FC1, W4, PROB>(g, xcd_first_tile() + (threadIdx.x >> 8) * gridDim.x, 2 * gridDim.x,
                                   (threadIdx.x >> 6) & 3);
}

// MXFP4, the LDS-staged 64-row tiles (gemm_mx4_small.h)
template <bool FC1, bool PROB>
__global__ void __launch_bounds__(512, 1) gemm_mx4_small_kernel(MxGemmArgs g)
{
    __shared__ __attribute__((aligned(1024))) char w0[kMx4SlotAll];
    __shared__ __attribute__((aligned(1024))) char w1[kMx4SlotAll];
    __shared__ __attribute__((aligned(1024))) char w2[kMx4SlotAll];
    __shared__ __attribute__((aligned(1024))) char q0[kMx4ASlot];
    __shared__ __attribute__((aligned(1024))) char q1[kMx4ASlot];
    __shared__ __attribute__((aligned(1024))) char q2[kMx4ASlot];
    mx4_small_tiles<FC1, PROB>(g, Mx4Ring{w0, w1, w2, q0, q1, q2});
}

// t0 / t1 (optional): events that receive the launch's own start and end
// (recorded by the dispatch itself, no separate marker in the stream)
hipError_t launch_gemm_mxfp8(bool fc1, bool w4, const MxGemmArgs& g, int num_cu, hipStream_t s,
                             hipEvent_t t0, hipEvent_t t1)
{
    if (!g.stream_big && g.K % 128 != 0) return hipErrorInvalidValue;
    dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8)), block(512);
    auto go = [&](auto kernel, hipEvent_t e0, hipEvent_t e1, const MxGemmArgs& a) {
        if (e0 || e1)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, a);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
    };
    MxGemmArgs a = g;
    a.lds_small = 0;
    // MXFP4 with K a multiple of 128 and 32-bit buffer offsets: the 64-row
    // tiles go to the LDS-staged kernel, after the 256-row tiles' launch, or
    // alone (taking the 256-row tiles too) at decode-sized batches
    const bool mx4_lds = w4 && !g.stream_big && g.a_bytes < ((int64_t)1 << 31) &&
                         (int64_t)g.N * g.K / 2 < ((int64_t)1 << 31);
    const bool prob = fc1 && g.row_prob != nullptr;
    if (mx4_lds) {
        a.lds_small = g.small_batch ? 2 : 1;
        if (a.lds_small == 1) {
            if (prob) go(gemm_mxfp8_kernel<true, true, true>, t0, nullptr, a);
            else if (fc1) go(gemm_mxfp8_kernel<true, true, false>, t0, nullptr, a);
            else go(gemm_mxfp8_kernel<false, true, false>, t0, nullptr, a);
        }
        hipEvent_t e0 = a.lds_small == 2 ? t0 : nullptr;
        if (prob) go(gemm_mx4_small_kernel<true, true>, e0, t1, a);
        else if (fc1) go(gemm_mx4_small_kernel<true, false>, e0, t1, a);
        else go(gemm_mx4_small_kernel<false, false>, e0, t1, a);
        return hipGetLastError();
    }
    if (w4) {
        if (prob) go(gemm_mxfp8_kernel<true, true, true>, t0, t1, a);
        else if (fc1) go(gemm_mxfp8_kernel<true, true, false>, t0, t1, a);
        else go(gemm_mxfp8_kernel<false, true, false>, t0, t1, a);
    } else {
        if (prob) go(gemm_mxfp8_kernel<true, false, true>, t0, t1, a);
        else if (fc1) go(gemm_mxfp8_kernel<true, false, false>, t0, t1, a);
        else go(gemm_mxfp8_kernel<false, false, false>, t0, t1, a);
    }
    return hipGetLastError();
}

}  // namespace moe
