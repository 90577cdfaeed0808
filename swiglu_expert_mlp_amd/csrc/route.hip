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

// (value, id) order of the selection: larger value first, equal values go to
// the smaller id.
__device__ __forceinline__ bool ahead(float ov, int oid, float v, int id)
{
    return ov > v || (ov == v && oid < id);
}

template <int CTRL>
__device__ __forceinline__ void dpp_amax_step(float& v, int& id)
{
    const float ov = __builtin_bit_cast(float,
        __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
    const int oid = __builtin_amdgcn_mov_dpp(id, CTRL, 0xF, 0xF, false);
    if (ahead(ov, oid, v, id)) { v = ov; id = oid; }
}

// Wave-wide argmax of (value, id).  Within each 16-lane row: DPP exchanges
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror),
// after which every lane of a row holds the row's winner; the four row
// winners are then combined from lanes 0, 16, 32, 48.  The result is
// wave-uniform.
__device__ __forceinline__ void wave_argmax(float& v, int& id)
{
    dpp_amax_step<0xB1>(v, id);
    dpp_amax_step<0x4E>(v, id);
    dpp_amax_step<0x141>(v, id);
    dpp_amax_step<0x140>(v, id);
    float bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    int bid = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float ov = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), r));
        const int oid = __builtin_amdgcn_readlane(id, r);
        if (ahead(ov, oid, bv, bid)) { bv = ov; bid = oid; }
    }
    v = bv;
    id = bid;
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
        hdr->err = (live < 0 ? kErrLiveNeg : 0u) | (live > T_cap ? kErrLiveHigh : 0u);

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
        // k rounds of argmax over the experts not yet taken; lane j keeps the
        // j-th winner (descending logit)
        int my_id = 0x7fffffff;
        float my_v = -INFINITY, m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j) {
            if (j >= k) continue;
            float bv = -INFINITY;
            int bid = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                int e = lane + kWave * i;
                if (!taken[i] && ahead(l[i], e, bv, bid)) { bv = l[i]; bid = e; }
            }
            wave_argmax(bv, bid);
            if (j == 0) m = bv;                       // the largest logit
            if (lane == j) { my_id = bid; my_v = bv; }
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i)
                if (lane + kWave * i == bid) taken[i] = true;
        }
        // canonical order: the rank of lane j's id among the k selected ids;
        // lane j's pair moves to lane rank_j (ids are distinct)
        int rank = 0;
#pragma unroll
        for (int i = 0; i < kMaxTopk; ++i)
            if (i < k && __builtin_amdgcn_readlane(my_id, i) < my_id) ++rank;
        const float z = lane < k ? expf(my_v - m) : 0.0f;
        const int dest = (lane < k ? rank : lane) * 4;
        const int c_id = __builtin_amdgcn_ds_permute(dest, my_id);
        const float c_z = __builtin_bit_cast(float, __builtin_amdgcn_ds_permute(dest, __builtin_bit_cast(int, z)));
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
