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

// K (the top-k) is a template parameter so that a token's k row loads are all
// in flight before the chain starts (a runtime loop put a memory round trip
// between consecutive routes).  The FC2 rows are read and the output written
// with non-temporal accesses: each byte is touched once (measured 15 % faster
// at 16K tokens than with the default cache policy).
template <int K>
__global__ void __launch_bounds__(512) finalize_kernel(
    const float* __restrict__ O, const int32_t* __restrict__ dst,
    const float* __restrict__ sorted_probs, int64_t T_cap, const int32_t* __restrict__ live_ptr,
    int H, float* __restrict__ out)
{
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    const int H4 = H >> 2;    // H is a multiple of 32
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        int32_t d[K];
        float p[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            d[j] = dst[t * K + j];
            p[j] = sorted_probs[t * K + j];
        }
        for (int c = threadIdx.x; c < H4; c += blockDim.x) {
            float4 o[K];
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (d[j] >= 0) {
                    typedef float f4v __attribute__((ext_vector_type(4)));
                    f4v v = __builtin_nontemporal_load((const f4v*)(O + (int64_t)d[j] * H) + c);
                    o[j] = make_float4(v.x, v.y, v.z, v.w);
                } else {
                    o[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if (d[j] < 0) continue;    // a dropped route adds nothing (not even +0)
                acc.x = __builtin_fmaf(p[j], o[j].x, acc.x);
                acc.y = __builtin_fmaf(p[j], o[j].y, acc.y);
                acc.z = __builtin_fmaf(p[j], o[j].z, acc.z);
                acc.w = __builtin_fmaf(p[j], o[j].w, acc.w);
            }
            {
                typedef float f4v __attribute__((ext_vector_type(4)));
                f4v v = {acc.x, acc.y, acc.z, acc.w};
                __builtin_nontemporal_store(v, (f4v*)(out + t * H) + c);
            }
        }
    }
}

hipError_t launch_finalize(const float* O, const int32_t* dst, const float* sorted_probs,
                           int64_t T_cap, const int32_t* live, int k, int H, float* out, int num_cu,
                           hipStream_t s)
{
    int64_t blocks = T_cap < (int64_t)num_cu * 8 ? T_cap : (int64_t)num_cu * 8;
    if (blocks < 1) blocks = 1;
    const dim3 g((unsigned)blocks), b(512);
#define FIN_CASE(KK)                                                                         \
    case KK:                                                                                 \
        hipLaunchKernelGGL(finalize_kernel<KK>, g, b, 0, s, O, dst, sorted_probs, T_cap, live, H, \
                           out);                                                             \
        break;
    switch (k) {
        FIN_CASE(1) FIN_CASE(2) FIN_CASE(3) FIN_CASE(4) FIN_CASE(5) FIN_CASE(6) FIN_CASE(7)
        FIN_CASE(8) FIN_CASE(9) FIN_CASE(10) FIN_CASE(11) FIN_CASE(12) FIN_CASE(13) FIN_CASE(14)
        FIN_CASE(15) FIN_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef FIN_CASE
    return hipGetLastError();
}

}  // namespace moe
