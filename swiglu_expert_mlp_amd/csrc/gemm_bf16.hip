// K3 / K4, bf16.  Two designs obey one arithmetic contract (gemm_bf16_small.h),
// so which one computes a row never changes its bits:
//   gemm_bf16_small_kernel  8 waves per CU, 64-row x 512-column tiles that
//                           stream the weights (experts with at most 128 rows);
//   gemm_bf16_big_kernel    8 waves per CU, 256 x 256 tiles staged through LDS
//                           (experts with more than 128 rows).
// Token capacities up to 1024 run one launch per GEMM stage: the 64-row kernel
// takes every tile, a 256-row tile as four 64-row tiles; so do shapes whose K
// is not a multiple of 64 (the 256-row design's stage) or whose operand
// offsets would not fit its 32-bit buffer offsets.  Otherwise the stage runs
// the 256-row launch, then the 64-row launch.  The choice depends on shapes
// and the capacity only, never on the live count.
#include <hip/hip_ext.h>

#include "gemm_bf16_big.h"
#include "gemm_bf16_small.h"

namespace moe {

// PROB: FC1 with the routes' probabilities applied to the SwiGLU rows (a
// compile-time variant; the default epilogues carry no probability loads)
template <bool FC1, bool PROB>
__global__ void __launch_bounds__(512, 1) gemm_bf16_small_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(1024))) char smem[kSmallLds];
    // both tile counts in one scalar load, and the first 64-row tile's table
    // entry fetched beside them (its index clamped into the table; unused when
    // the tile does not exist), so the first weight loads wait for one round trip
    const int n_big = g.small_takes_big ? ld_const(&g.hdr->n_tiles_big) : 0;
    const int n_small = ld_const(&g.hdr->n_tiles);
    const int multi = ld_const(&g.hdr->multi_tile);
    const int* te0 = (const int*)(g.tiles + min(xcd_first_tile() / small_col_tiles(g), g.max_tiles - 1));
    const int e0 = ld_const(te0), row00 = ld_const(te0 + 1);
    asm volatile("" : : "s"(n_big), "s"(n_small), "s"(multi), "s"(e0), "s"(row00));   // one round trip
    if (multi) small_tiles<FC1, PROB, 0, 0>(g, smem, n_small, n_big, e0, row00);
    else small_tiles<FC1, PROB, 0, kNonTemporal>(g, smem, n_small, n_big, e0, row00);
}

template <bool FC1, bool PROB>
__global__ void __launch_bounds__(512, 1) gemm_bf16_big_kernel(GemmArgs g)
{
    big_tiles<FC1, PROB>(g, ld_const(&g.hdr->n_tiles_big));
}

// The single-launch FFN: FC1 then FC2 in one persistent launch of the 64-row
// design (it takes every tile, a 256-row tile as four 64-row tiles), FC2
// tiles waiting on per-M-tile readiness counters instead of the launch
// boundary (gemm_bf16_small.h).  The grid is at most one workgroup per CU, so
// every workgroup is resident and every FC1 tile is taken.  FIN: the FC2
// tiles also run the finalize (small_finalize: the last FC2 tile of a token's
// 512-column block combines it).
template <bool PROB, bool FIN>
__global__ void __launch_bounds__(512, 1) gemm_bf16_fused_kernel(GemmArgs g1, GemmArgs g2)
{
    __shared__ __attribute__((aligned(1024))) char smem[kSmallLds];
    __shared__ SmallFinLds fin_lds;
    constexpr int F2 = FIN ? 3 : 2;
    const int n_big = ld_const(&g1.hdr->n_tiles_big);
    const int n_small = ld_const(&g1.hdr->n_tiles);
    const int multi = ld_const(&g1.hdr->multi_tile);
    const int* te0 = (const int*)(g1.tiles + min(xcd_first_tile() / small_col_tiles(g1), g1.max_tiles - 1));
    const int e0 = ld_const(te0), row00 = ld_const(te0 + 1);
    asm volatile("" : : "s"(n_big), "s"(n_small), "s"(multi), "s"(e0), "s"(row00));
    const int* te1 = (const int*)(g2.tiles + min(xcd_first_tile() / small_col_tiles(g2), g2.max_tiles - 1));
    if (multi) {
        small_tiles<true, PROB, 1, 0>(g1, smem, n_small, n_big, e0, row00);
        small_tiles<false, false, F2, 0>(g2, smem, n_small, n_big, ld_const(te1), ld_const(te1 + 1),
                                         small_col_tiles(g1), &fin_lds);
    } else {
        small_tiles<true, PROB, 1, kNonTemporal>(g1, smem, n_small, n_big, e0, row00);
        small_tiles<false, false, F2, kNonTemporal>(g2, smem, n_small, n_big, ld_const(te1),
                                                    ld_const(te1 + 1), small_col_tiles(g1), &fin_lds);
    }
}

hipError_t launch_gemm_bf16_fused(const GemmArgs& g1, const GemmArgs& g2, int num_cu, hipStream_t s,
                                  hipEvent_t t0, hipEvent_t t1)
{
    if (!g1.small_takes_big || !g2.small_takes_big || !g1.ready || !g1.err) return hipErrorInvalidValue;
    const bool fin = g2.fin_cnt != nullptr;
    if (fin && (!g2.fin_route || !g2.fin_dst || !g2.fin_out || g2.fin_mode < 0 || g2.fin_mode > 2 ||
                g2.topk < 1 || g2.topk > kMaxTopk))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8)), block(512);
    const bool prob = g1.row_prob != nullptr;
    auto go = [&](auto kernel) {
        if (t0 || t1)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, g1, g2);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, s, g1, g2);
    };
    if (fin) {
        if (prob) go(gemm_bf16_fused_kernel<true, true>);
        else go(gemm_bf16_fused_kernel<false, true>);
    } else {
        if (prob) go(gemm_bf16_fused_kernel<true, false>);
        else go(gemm_bf16_fused_kernel<false, false>);
    }
    return hipGetLastError();
}

// t0 / t1 (optional): events that receive the stage's start (the first
// launch's) and end (the last launch's), recorded by the dispatches themselves
// (no separate marker in the stream).  s_small (optional): the stream of the
// 64-row launch when the stage has two launches (the caller orders it).
hipError_t launch_gemm_bf16(bool fc1, const GemmArgs& g, int num_cu, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1, hipStream_t s_small)
{
    // a multiple of 8 workgroups: the 256-row loop splits its tiles over the 8 XCDs
    const dim3 grid((unsigned)(num_cu >= 8 ? num_cu / 8 * 8 : 8));
    auto go = [&](auto kernel, int threads, hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
        if (e0 || e1)
            hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, st, e0, e1, 0, g);
        else
            hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, st, g);
    };
    const bool prob = fc1 && g.row_prob != nullptr;
    hipEvent_t small_start = t0;
    hipStream_t ss = s;
    if (!g.small_takes_big) {
        if (prob) go(gemm_bf16_big_kernel<true, true>, 512, t0, nullptr, s);
        else if (fc1) go(gemm_bf16_big_kernel<true, false>, 512, t0, nullptr, s);
        else go(gemm_bf16_big_kernel<false, false>, 512, t0, nullptr, s);
        small_start = nullptr;
        if (s_small) ss = s_small;
    }
    if (prob) go(gemm_bf16_small_kernel<true, true>, 512, small_start, t1, ss);
    else if (fc1) go(gemm_bf16_small_kernel<true, false>, 512, small_start, t1, ss);
    else go(gemm_bf16_small_kernel<false, false>, 512, small_start, t1, ss);
    return hipGetLastError();
}

}  // namespace moe
