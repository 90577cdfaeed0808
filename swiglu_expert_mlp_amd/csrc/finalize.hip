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
// neither read nor written.  A workgroup (512 threads) takes a token at a
// time (one token, or a strided run of tokens: launch_finalize); 4 columns
// per thread.
//
// With sorted_probs == nullptr (the probabilities were applied inside FC1, the
// MoeEp apply_topk_in_fc1 option of cudnn-frontend PR #448) every p_j is 1:
// the chain adds the already weighted rows, fma(1, o, acc) = acc + o exactly.
//
// Two more combines (the value pass of Megatron-LM PR #7798, "What is
// changed"):
//   bf16: the same fp32 chain rounded to bf16 (round to nearest even), which
//     is one rank of its BF16_RANK_PARTIALS unpermute and what FlashInfer's
//     finalize returns; out bf16 [T_cap][H].
//   rows: every route through the finalize as a top-1 token with probability
//     1.0, so each route's expert output comes back unscaled:
//     out[t][j][m] = fma(1, O[dst[t,j]][m], +0.0f) (-0 becomes +0; a dropped
//     route gives +0); out fp32 [T_cap][k][H].
#include "common.h"

namespace moe {

// K (the top-k) is a template parameter so that a token's k row loads are all
// in flight before the chain starts (a runtime loop put a memory round trip
// between consecutive routes).  The FC2 rows are read and the output written
// with non-temporal accesses: each byte is touched once (measured 15 % faster
// at 16K tokens than with the default cache policy).  MODE: 0 fp32 combine,
// 1 bf16 combine, 2 rows.
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

template <int K, int MODE>
__global__ void __launch_bounds__(512) finalize_kernel(
    const float* __restrict__ O, const int32_t* __restrict__ dst,
    const float* __restrict__ sorted_probs, int64_t T_cap, const int32_t* __restrict__ live_ptr,
    int H, void* __restrict__ out)
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
            p[j] = (MODE == 2 || !sorted_probs) ? 1.0f : sorted_probs[t * K + j];
        }
        for (int c = threadIdx.x; c < H4; c += blockDim.x) {
            f4v o[K];
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (d[j] >= 0)
                    o[j] = __builtin_nontemporal_load((const f4v*)(O + (int64_t)d[j] * H) + c);
                else
                    o[j] = f4v{0.f, 0.f, 0.f, 0.f};
            if constexpr (MODE == 2) {
                // each route alone: one fma from +0 (a dropped route stays +0)
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    f4v r = {0.f, 0.f, 0.f, 0.f};
                    if (d[j] >= 0) {
                        r.x = __builtin_fmaf(p[j], o[j].x, 0.0f);
                        r.y = __builtin_fmaf(p[j], o[j].y, 0.0f);
                        r.z = __builtin_fmaf(p[j], o[j].z, 0.0f);
                        r.w = __builtin_fmaf(p[j], o[j].w, 0.0f);
                    }
                    __builtin_nontemporal_store(r, (f4v*)((float*)out + (t * K + j) * H) + c);
                }
            } else {
                f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    if (d[j] < 0) continue;    // a dropped route adds nothing (not even +0)
                    acc.x = __builtin_fmaf(p[j], o[j].x, acc.x);
                    acc.y = __builtin_fmaf(p[j], o[j].y, acc.y);
                    acc.z = __builtin_fmaf(p[j], o[j].z, acc.z);
                    acc.w = __builtin_fmaf(p[j], o[j].w, acc.w);
                }
                if constexpr (MODE == 0) {
                    __builtin_nontemporal_store(acc, (f4v*)((float*)out + t * H) + c);
                } else {
                    const u2v v = {(unsigned)f32_to_bf16_bits(acc.x) | ((unsigned)f32_to_bf16_bits(acc.y) << 16),
                                   (unsigned)f32_to_bf16_bits(acc.z) | ((unsigned)f32_to_bf16_bits(acc.w) << 16)};
                    __builtin_nontemporal_store(v, (u2v*)((uint16_t*)out + t * H) + c);
                }
            }
        }
    }
}

hipError_t launch_finalize(const float* O, const int32_t* dst, const float* sorted_probs,
                           int64_t T_cap, const int32_t* live, int k, int H, int mode, void* out,
                           int num_cu, hipStream_t s)
{
    // Two launch shapes, chosen by the capacity (never the live count):
    //  * capacity above 16 and up to 64 tokens per CU: a workgroup per token,
    //    at most two resident per CU (the launch asks for 56 KB of dynamic
    //    LDS, which the kernel does not use, so that only two fit in a CU's
    //    160 KB);
    //  * otherwise at most 8 workgroups per CU, each looping over tokens, as
    //    many resident as the registers allow.
    // A/B on one MI355X (hidden 2048, us): 16K tokens, top-8: 226.5 -> 206.7
    // (bf16 FC2 rows; MXFP8 233.6 -> 215); 4,096 tokens 47.2 -> 49.1; a
    // 65,536-token capacity with 512 live 10.0 -> 16.3 (the 16,384 workgroups
    // past the live tokens still start and exit, two per CU at a time), which
    // is why the larger capacities keep the looping grid.
    const bool per_token = T_cap > (int64_t)num_cu * 16 && T_cap <= (int64_t)num_cu * 64;
    int64_t blocks = per_token ? T_cap : (T_cap < (int64_t)num_cu * 8 ? T_cap : (int64_t)num_cu * 8);
    if (blocks < 1) blocks = 1;
    const dim3 g((unsigned)blocks), b(512);
    const unsigned occupancy_lds = per_token ? 56 * 1024 : 0;
    if (mode < 0 || mode > 2) return hipErrorInvalidValue;
#define FIN_MODE(KK, MM)                                                                     \
    hipLaunchKernelGGL((finalize_kernel<KK, MM>), g, b, occupancy_lds, s, O, dst, sorted_probs, \
                       T_cap, live, H, out)
#define FIN_CASE(KK)                                                                         \
    case KK:                                                                                 \
        if (mode == 0) FIN_MODE(KK, 0);                                                      \
        else if (mode == 1) FIN_MODE(KK, 1);                                                 \
        else FIN_MODE(KK, 2);                                                                \
        break;
    switch (k) {
        FIN_CASE(1) FIN_CASE(2) FIN_CASE(3) FIN_CASE(4) FIN_CASE(5) FIN_CASE(6) FIN_CASE(7)
        FIN_CASE(8) FIN_CASE(9) FIN_CASE(10) FIN_CASE(11) FIN_CASE(12) FIN_CASE(13) FIN_CASE(14)
        FIN_CASE(15) FIN_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef FIN_CASE
#undef FIN_MODE
    return hipGetLastError();
}

}  // namespace moe
