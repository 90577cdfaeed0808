// K5: finalize = per-token, fixed-order fp32 combine of the routes' FC2 rows.
//
// Megatron-LM PR #7798, "What is changed": a token's routes are added as fp32
// fused multiply-adds of probability and row, starting from zero, in the
// listed order; Megatron-LM PR #7830, "1. Mega backend for generation": the
// listed order is the canonical (ascending expert id) one.  Megatron-LM
// PR #8367, "Problem": the result stays fp32 (no bf16 downcast) and only the
// live tokens are touched.
//
// out[t][m] = fma(p_{k-1}, O[dst[t,k-1]][m], ... fma(p_0, O[dst[t,0]][m], +0.0f))
// A route with dst < 0 (an invalid expert id) adds nothing.  Rows >= live are
// neither read nor written.  One workgroup (512 threads) walks tokens; 4
// columns per thread.
#include "common.h"

namespace moe {

__global__ void __launch_bounds__(512) finalize_kernel(
    const float* __restrict__ O, const int32_t* __restrict__ dst,
    const float* __restrict__ sorted_probs, int64_t T_cap, const int32_t* __restrict__ live_ptr,
    int k, int H, float* __restrict__ out)
{
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    const int H4 = H >> 2;    // H is a multiple of 32
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        int32_t d[kMaxTopk];
        float p[kMaxTopk];
        for (int j = 0; j < k; ++j) {
            d[j] = dst[t * k + j];
            p[j] = sorted_probs[t * k + j];
        }
        for (int c = threadIdx.x; c < H4; c += blockDim.x) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int j = 0; j < k; ++j) {
                if (d[j] < 0) continue;
                float4 o = *((const float4*)(O + (int64_t)d[j] * H) + c);
                acc.x = __builtin_fmaf(p[j], o.x, acc.x);
                acc.y = __builtin_fmaf(p[j], o.y, acc.y);
                acc.z = __builtin_fmaf(p[j], o.z, acc.z);
                acc.w = __builtin_fmaf(p[j], o.w, acc.w);
            }
            *((float4*)(out + t * H) + c) = acc;
        }
    }
}

hipError_t launch_finalize(const float* O, const int32_t* dst, const float* sorted_probs,
                           int64_t T_cap, const int32_t* live, int k, int H, float* out, int num_cu,
                           hipStream_t s)
{
    int64_t blocks = T_cap < (int64_t)num_cu * 8 ? T_cap : (int64_t)num_cu * 8;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)blocks), dim3(512), 0, s, O, dst,
                       sorted_probs, T_cap, live, k, H, out);
    return hipGetLastError();
}

}  // namespace moe
