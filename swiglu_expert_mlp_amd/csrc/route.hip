// K0: router top-k with canonical (ascending expert id) output.
//
// Megatron-Core API docs, core.transformer.moe.training_matches_inference,
// `_route`: the router returns [tokens, topk] probabilities and expert ids.
// Megatron-LM PR #7830, "1. Mega backend for generation": the ids are put in
// a canonical order (ascending) before the combine.
//
// One wavefront per token.  Selection is on the logits (softmax is monotone,
// so this selects the same experts as selecting on probabilities, without
// ties that fp32 rounding of the probabilities could create); ties go to the
// lower expert id.  The renormalized probability of a selected expert is
// softmax over all E followed by division by the selected mass, which equals
// exp(l_j - m) / sum_{selected} exp(l_i - m) with m the largest logit; the
// kernel evaluates that form in fp32.
#include "common.h"

namespace moe {

// Wave-wide argmax of (value, id): larger value wins, equal values go to the
// smaller id.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& id)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(v, off, kWave);
        int oid = __shfl_xor(id, off, kWave);
        if (ov > v || (ov == v && oid < id)) { v = ov; id = oid; }
    }
}

template <int PER_LANE>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    int64_t T_cap, const int32_t* __restrict__ live_ptr,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ probs,
                                                    WsHeader* __restrict__ hdr)
{
    const int lane = threadIdx.x & 63;
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    if (blockIdx.x == 0 && threadIdx.x == 0 && hdr != nullptr)
        hdr->route_err = (live < 0 ? kErrLiveNeg : 0u) | (live > T_cap ? kErrLiveHigh : 0u);

    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t t = wave0; t < T; t += nwaves) {
        const float* row = logits + t * E;
        float l[PER_LANE];
        bool taken[PER_LANE];
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            int e = lane + kWave * i;
            l[i] = e < E ? row[e] : -INFINITY;
            taken[i] = e >= E;
        }
        int sel[kMaxTopk];
        float selv[kMaxTopk];
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int bid = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                int e = lane + kWave * i;
                if (!taken[i] && (l[i] > bv || (l[i] == bv && e < bid))) { bv = l[i]; bid = e; }
            }
            wave_argmax(bv, bid);
            sel[j] = bid;
            selv[j] = bv;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i)
                if (lane + kWave * i == bid) taken[i] = true;
        }
        // sel[0] holds the largest logit.  Canonical order: ascending id.
        const float m = selv[0];
        for (int a = 1; a < k; ++a)
            for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
                int ti = sel[b]; sel[b] = sel[b - 1]; sel[b - 1] = ti;
                float tv = selv[b]; selv[b] = selv[b - 1]; selv[b - 1] = tv;
            }
        float z[kMaxTopk];
        float S = 0.0f;
        for (int j = 0; j < k; ++j) { z[j] = expf(selv[j] - m); S += z[j]; }
        if (lane < k) {
            float zj = 0.0f;
            int idj = 0;
            for (int j = 0; j < k; ++j) if (j == lane) { zj = z[j]; idj = sel[j]; }
            ids[t * k + lane] = idj;
            probs[t * k + lane] = zj / S;
        }
    }
}

hipError_t launch_route(const float* logits, int64_t T_cap, const int32_t* live, int E, int k,
                        int32_t* ids, float* probs, WsHeader* hdr, int num_cu, hipStream_t s)
{
    int64_t waves_needed = T_cap;
    int64_t blocks = (waves_needed + 3) / 4;
    int64_t cap = (int64_t)num_cu * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    dim3 grid((unsigned)blocks), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T_cap, live, E, k, ids, probs, hdr);
    else if (E <= 128)
        hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T_cap, live, E, k, ids, probs, hdr);
    else if (E <= 256)
        hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T_cap, live, E, k, ids, probs, hdr);
    else if (E <= 512)
        hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T_cap, live, E, k, ids, probs, hdr);
    else
        hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T_cap, live, E, k, ids, probs, hdr);
    return hipGetLastError();
}

}  // namespace moe
