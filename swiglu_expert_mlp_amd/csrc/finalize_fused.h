// Finalize fused into the FC2 epilogue.
//
// Megatron-LM PR #7798, "What is changed": a token's routes are added as fp32
// fused multiply-adds of probability and row, from zero, in the listed order;
// Megatron-LM PR #7830, "1. Mega backend for generation": the listed order is
// ascending expert id.  Megatron-LM PR #8367, "Problem": fp32 result, only
// live tokens.
//
// The k FC2 rows of a token come from k different expert tiles.  Each FC2
// workgroup, after storing its unweighted fp32 rows for one 256-column slice,
// counts one arrival per row on (token, slice); the workgroup whose arrival
// completes the token's count publishes nothing more and sums the token's
// rows for that slice itself:
//   out[t][c] = fma(p_{k-1}, O[dst[t,k-1]][c], ... fma(p_0, O[dst[t,0]][c], +0.0f))
// The atomics only decide WHO sums; the sum is always the same fixed-order
// chain, so the result bits do not depend on the arrival order.
//
// Visibility across XCDs (each XCD has its own L2): after storing its FC2
// rows the workgroup issues one device-scope release fence (the XCD's L2
// writes its dirty lines back) before its arrivals, and the summing workgroup
// reads the rows with device-scope atomic loads, which do not return lines
// cached in its own L2.  No L2 invalidation is needed, so the other
// workgroups of the XCD keep their cached GEMM operands.
#pragma once

#include "common.h"

namespace moe {

struct FinArgs {
    int32_t* cnt;              // [T_cap][ns_per_token] arrivals, zeroed by the prep kernel
    const int32_t* kvalid;     // [T_cap] kept routes of each token
    const int32_t* perm_src;   // grouped row -> route
    const int32_t* dst;        // route -> grouped row (-1 if dropped)
    const float* sorted_probs; // [T_cap][k] in canonical order
    float* O;                  // fp32 FC2 rows [rows][H]
    float* out;                // [T_cap][H]
    int H;
    int k;
    int ns_per_token;          // ceil(H / 256)
};

// All threads of the workgroup call this after storing the O values of rows
// [row0, row0 + rows) and columns [256 ns, 256 ns + 256).  list: LDS scratch of
// at least rows + 1 ints.
// Store of one FC2 value (write-back; published by the release fence below).
__device__ __forceinline__ void store_fc2(float* p, float v) { *p = v; }

__device__ __forceinline__ void fused_finalize(const FinArgs& f, int row0, int rows, int ns, int* list)
{
    __builtin_amdgcn_s_waitcnt(0);         // this wave's FC2 stores have completed
    __syncthreads();                       // ... and every other wave's
    if (threadIdx.x < 64) {
        if (threadIdx.x == 0) list[0] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        for (int r = threadIdx.x; r < rows; r += 64) {
            const int route = f.perm_src[row0 + r];
            const int t = route / f.k;
            const int old = __hip_atomic_fetch_add(&f.cnt[(int64_t)t * f.ns_per_token + ns], 1,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == f.kvalid[t] - 1) list[1 + atomicAdd(&list[0], 1)] = t;
        }
    }
    __syncthreads();
    const int nl = list[0];
    if (nl == 0) return;
    const int c0 = ns * 256;
    for (int q = threadIdx.x; q < nl * 256; q += blockDim.x) {
        const int i = q >> 8, c = c0 + (q & 255);
        if (c >= f.H) continue;
        const int t = list[1 + i];
        float acc = 0.0f;
        for (int j = 0; j < f.k; ++j) {
            const int d = f.dst[(int64_t)t * f.k + j];
            if (d < 0) continue;
            const float o = __hip_atomic_load(&f.O[(int64_t)d * f.H + c], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            acc = __builtin_fmaf(f.sorted_probs[(int64_t)t * f.k + j], o, acc);
        }
        f.out[(int64_t)t * f.H + c] = acc;
    }
}

}  // namespace moe
