// K1: canonical sort of each token's routes, expert histogram, prefix sum,
// tile table and a stable row scatter.
//
// Megatron-LM PR #7830, "1. Mega backend for generation": a token's routes
// are summed in canonical (ascending expert id) order.  cudnn-frontend
// PR #448, MoeEp class docstring: routed rows are grouped by expert in
// ascending order and kept in token-major route order inside an expert.
// Megatron-LM PR #8367, "Problem": the token count is a device-side value,
// so every kernel here reads it from device memory.
//
// Three launches, each with a grid that never depends on the live count:
//   prep_count   one workgroup per 256-token chunk (chunks past the live
//                count exit at once): canonical sort, per-chunk expert counts
//                and each route's stable rank inside its chunk (wave ballots,
//                so the ranks are deterministic, not atomic-order dependent);
//   prep_scan    one workgroup: chunk prefix per expert, exclusive scan over
//                experts, M-tile table, error word;
//   prep_scatter one thread per route: position = expert offset + chunk base
//                + rank; perm_src[position] = route, dst[route] = position.
#include "common.h"

namespace moe {

__device__ __forceinline__ int32_t clamp_live(int32_t live, int64_t T_cap)
{
    return live < 0 ? 0 : (live > T_cap ? (int32_t)T_cap : live);
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024).
// Returns the exclusive prefix; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* total, int* lds /* >= 32 ints */)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
    }
    if (lane == 63) lds[wid] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) { int c = lds[w]; lds[w] = run; run += c; }
        lds[31] = run;
    }
    __syncthreads();
    int excl = lds[wid] + inc - v;
    *total = lds[31];
    __syncthreads();
    return excl;
}

template <int K>
__global__ void __launch_bounds__(256) prep_count_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ probs, int64_t T_cap,
    const int32_t* __restrict__ live_ptr, int E, int32_t* __restrict__ sorted_ids,
    float* __restrict__ sorted_probs, int32_t* __restrict__ local_rank,
    int32_t* __restrict__ chunk_counts, uint32_t* __restrict__ chunk_err)
{
    __shared__ int wcnt[4][kMaxExperts];
    const int T = clamp_live(*live_ptr, T_cap);
    const int c = blockIdx.x;
    const int t0 = c * kChunkTok;
    if (t0 >= T) return;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = t0 + threadIdx.x;
    const bool valid = t < T;

    // canonical sort of this token's (id, prob) pairs: insertion sort keeps
    // equal ids (a contract violation) in their listed order
    int id[K];
    float p[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        id[j] = valid ? ids[(int64_t)t * K + j] : -1;
        p[j] = valid ? probs[(int64_t)t * K + j] : 0.0f;
    }
#pragma unroll
    for (int a = 1; a < K; ++a)
#pragma unroll
        for (int b = a; b > 0; --b)
            if (id[b - 1] > id[b]) {
                int ti = id[b]; id[b] = id[b - 1]; id[b - 1] = ti;
                float tp = p[b]; p[b] = p[b - 1]; p[b - 1] = tp;
            }
    uint32_t err = 0;
    if (valid) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            sorted_ids[(int64_t)t * K + j] = id[j];
            sorted_probs[(int64_t)t * K + j] = p[j];
            if (id[j] < 0 || id[j] >= E) err |= kErrBadId;
            if (j > 0 && id[j] == id[j - 1]) err |= kErrDupId;
        }
    }
    // in-wave stable ranks: route (t, j) precedes (t', j') iff t < t' or
    // (t == t' and j < j'); rank = earlier routes of this wave with the same id
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rank[K];
#pragma unroll
    for (int j = 0; j < K; ++j) rank[j] = -1;
    for (int e = 0; e < E; ++e) {
        uint64_t m[K];
        int tot = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            m[j] = __ballot(valid && id[j] == e);
            tot += __popcll(m[j]);
        }
        if (tot == 0) {
            if (lane == 0) wcnt[wid][e] = 0;
            continue;
        }
        int before = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) before += __popcll(m[j] & lt);
        int same_tok = 0;
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (valid && id[j] == e) { rank[j] = before + same_tok; ++same_tok; }
        if (lane == 0) wcnt[wid][e] = tot;
    }
    __syncthreads();
    // chunk counts and the wave's base inside the chunk
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (rank[j] >= 0) {
            int e = id[j];
            int base = 0;
            for (int w = 0; w < wid; ++w) base += wcnt[w][e];
            rank[j] += base;
        }
        if (valid) local_rank[(int64_t)t * K + j] = rank[j];
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        chunk_counts[(int64_t)c * E + e] = wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
    // OR of the error bits of the chunk
    uint64_t any_bad = __ballot(err & kErrBadId), any_dup = __ballot(err & kErrDupId);
    __shared__ uint32_t werr[4];
    if (lane == 0) werr[wid] = (any_bad ? kErrBadId : 0u) | (any_dup ? kErrDupId : 0u);
    __syncthreads();
    if (threadIdx.x == 0) chunk_err[c] = werr[0] | werr[1] | werr[2] | werr[3];
}

// One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) prep_scan_kernel(
    int64_t T_cap, const int32_t* __restrict__ live_ptr, int E, int k,
    int32_t* __restrict__ chunk_base, const uint32_t* __restrict__ chunk_err,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int2* __restrict__ tiles,
    WsHeader* __restrict__ hdr)
{
    __shared__ int lds[32];
    const int32_t live = *live_ptr;
    const int T = clamp_live(live, T_cap);
    const int nch = (T + kChunkTok - 1) / kChunkTok;
    const int e = threadIdx.x;
    // per-expert prefix over chunks (chunk order = token order)
    int run = 0;
    if (e < E) {
        for (int c = 0; c < nch; ++c) {
            int v = chunk_base[(int64_t)c * E + e];
            chunk_base[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    int cnt = e < E ? run : 0;
    int total;
    int off = block_exclusive_scan(cnt, &total, lds);
    if (e < E) {
        counts[e] = cnt;
        offsets[e] = off;
        for (int c = 0; c < nch; ++c) chunk_base[(int64_t)c * E + e] += off;
    }
    if (e == 0) offsets[E] = total;
    // M-tile table: expert e owns ceil(count / kBM) tiles
    int nt = (cnt + kBM - 1) / kBM;
    int ntotal;
    int tfirst = block_exclusive_scan(nt, &ntotal, lds);
    for (int i = 0; i < nt; ++i) tiles[tfirst + i] = make_int2(e, off + i * kBM);
    // error word: OR over the live chunks plus the live-count checks
    uint32_t err = 0;
    for (int c = e; c < nch; c += blockDim.x) err |= chunk_err[c];
    uint64_t b1 = __ballot(err & kErrBadId), b2 = __ballot(err & kErrDupId);
    __shared__ uint32_t werr[16];
    if ((threadIdx.x & 63) == 0) werr[threadIdx.x >> 6] = (b1 ? kErrBadId : 0u) | (b2 ? kErrDupId : 0u);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t all = (live < 0 ? kErrLiveNeg : 0u) | (live > T_cap ? kErrLiveHigh : 0u);
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) all |= werr[w];
        hdr->fwd_err = all;
        hdr->T = T;
        hdr->n_tiles = ntotal;
        hdr->n_rows = total;
    }
}

__global__ void __launch_bounds__(256) prep_scatter_kernel(
    int64_t T_cap, const int32_t* __restrict__ live_ptr, int E, int k,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ dst)
{
    const int T = clamp_live(*live_ptr, T_cap);
    const int64_t R = (int64_t)T * k;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R;
         r += (int64_t)gridDim.x * blockDim.x) {
        int e = sorted_ids[r];
        int rk = local_rank[r];
        if (rk < 0 || e < 0 || e >= E) { dst[r] = -1; continue; }
        int c = (int)((r / k) / kChunkTok);
        int pos = chunk_base[(int64_t)c * E + e] + rk;
        perm_src[pos] = (int32_t)r;
        dst[r] = pos;
    }
}

hipError_t launch_prep(const int32_t* ids, const float* probs, int64_t T_cap, const int32_t* live,
                       int E, int k, int num_cu, char* ws, const WsLayout& L, hipStream_t s)
{
    int32_t* sorted_ids = (int32_t*)(ws + L.sorted_ids);
    float* sorted_probs = (float*)(ws + L.sorted_probs);
    int32_t* local_rank = (int32_t*)(ws + L.local_rank);
    int32_t* chunk_base = (int32_t*)(ws + L.chunk_base);
    uint32_t* chunk_err = (uint32_t*)(ws + L.chunk_err);
    dim3 g1((unsigned)L.nchunks), b1(256);
#define PREP_CASE(KK)                                                                        \
    case KK:                                                                                 \
        hipLaunchKernelGGL(prep_count_kernel<KK>, g1, b1, 0, s, ids, probs, T_cap, live, E,  \
                           sorted_ids, sorted_probs, local_rank, chunk_base, chunk_err);     \
        break;
    switch (k) {
        PREP_CASE(1) PREP_CASE(2) PREP_CASE(3) PREP_CASE(4) PREP_CASE(5) PREP_CASE(6)
        PREP_CASE(7) PREP_CASE(8) PREP_CASE(9) PREP_CASE(10) PREP_CASE(11) PREP_CASE(12)
        PREP_CASE(13) PREP_CASE(14) PREP_CASE(15) PREP_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef PREP_CASE
    hipLaunchKernelGGL(prep_scan_kernel, dim3(1), dim3(1024), 0, s, T_cap, live, E, k, chunk_base,
                       chunk_err, (int32_t*)(ws + L.counts), (int32_t*)(ws + L.offsets),
                       (int2*)(ws + L.tiles), (WsHeader*)(ws + L.hdr));
    int64_t R = T_cap * k;
    int64_t blocks = (R + 255) / 256;
    if (blocks > (int64_t)num_cu * 4) blocks = (int64_t)num_cu * 4;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(prep_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s, T_cap, live, E,
                       k, sorted_ids, local_rank, chunk_base, (int32_t*)(ws + L.perm_src),
                       (int32_t*)(ws + L.dst));
    return hipGetLastError();
}

}  // namespace moe
