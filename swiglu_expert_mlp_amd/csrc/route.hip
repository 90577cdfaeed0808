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

// Order-preserving integer key of a logit: a larger logit has a larger key;
// -0 and +0 share one key (they compare equal); NaN gets key 0, below every
// number (-inf is 0x007fffff), as does the padding past E.
__device__ __forceinline__ uint32_t route_key(float v)
{
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;
    const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return v != v ? 0u : key;
}

// lanes below this one with their bit set in mask
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Selection: the top k of (logit, id) in the order larger logit first, equal
// logits by the smaller id.  The k-th largest key T is found bit by bit (the
// largest T with at least k keys >= T: 32 compare-and-count steps, the counts
// from the wave's comparison masks); keys above T are taken, and of the keys
// equal to T the smallest ids fill the remaining places.  Ids run in the
// order (i, lane), e = lane + 64 i, so a prefix count over the masks gives both
// the tie rank and the output position (ascending id).
template <int PER_LANE>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    int64_t T_cap, const int32_t* __restrict__ live_ptr,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ probs,
                                                    WsHeader* __restrict__ hdr)
{
    __shared__ int32_t sel_id[4][kMaxTopk];
    __shared__ float sel_z[4][kMaxTopk];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x / kWave;
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    if (blockIdx.x == 0 && threadIdx.x == 0 && hdr != nullptr)
        hdr->err = (live < 0 ? kErrLiveNeg : 0u) | (live > T_cap ? kErrLiveHigh : 0u);

    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + wv;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t t = wave0; t < T; t += nwaves) {
        const float* row = logits + t * E;
        float l[PER_LANE];
        uint32_t key[PER_LANE];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int e = lane + kWave * i;
            l[i] = e < E ? row[e] : -INFINITY;
            key[i] = e < E ? route_key(l[i]) : 0u;
            if (e < E) mx = fmaxf(mx, l[i]);
        }
        uint32_t thr = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i)
                cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] >= cand));
            if (cnt >= k) thr = cand;
        }
        int above = 0;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] > thr));
        const int need = k - above;
        bool sel[PER_LANE];
        int before = 0;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const uint64_t eq = __builtin_amdgcn_ballot_w64(key[i] == thr);
            sel[i] = key[i] > thr || (key[i] == thr && before + lanes_below(eq) < need);
            before += __builtin_popcountll(eq);
        }
        // the largest logit (no selected logit is NaN unless fewer than k are numbers)
        mx = row16_max(mx);
        float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 0));
#pragma unroll
        for (int r = 16; r < 64; r += 16)
            m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), r)));
        // each selected route to its place in ascending-id order
        before = 0;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const uint64_t sm = __builtin_amdgcn_ballot_w64(sel[i]);
            if (sel[i]) {
                const int pos = before + lanes_below(sm);
                sel_id[wv][pos] = lane + kWave * i;
                sel_z[wv][pos] = expf(l[i] - m);
            }
            before += __builtin_popcountll(sm);
        }
        const int c_id = lane < k ? sel_id[wv][lane] : 0;
        const float c_z = lane < k ? sel_z[wv][lane] : 0.0f;
        // the selected mass, summed in ascending-id order
        float S = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxTopk; ++i)
            if (i < k)
                S += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c_z), i));
        if (lane < k) {
            ids[t * k + lane] = c_id;
            probs[t * k + lane] = c_z / S;
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
