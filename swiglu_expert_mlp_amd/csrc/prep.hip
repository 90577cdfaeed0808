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
// Launches, with grids that never depend on the live count:
//   prep_kernel    one workgroup per 256-token chunk (chunks past the live
//                  count exit at once): canonical sort, then per expert a
//                  256-bit map of the chunk's tokens that route to it (LDS
//                  atomic OR, order-independent); a route's stable rank inside
//                  the chunk is the number of set bits below its token, and
//                  the chunk's count the bits set in all.
//   prep_finish    one workgroup: the prefix over chunks (per expert, staged
//                  through LDS in coalesced slabs) and over experts, the M-tile
//                  tables and the header (error word, live count, tile counts).
//   prep_scatter   one thread per route: position = expert offset + the
//                  chunk's base inside the expert + rank; perm_src[position] =
//                  route, dst[route] = position.
// A launch whose capacity fits one chunk (T_cap <= 256 tokens, the decode
// sizes) runs as a single workgroup that keeps the counts in LDS, finishes
// and scatters its own routes; the host then launches neither prep_finish
// nor prep_scatter.  No launch reads a value that an earlier forward left in
// the workspace, so a new workspace needs no initialisation.
// A route whose id is outside [0, E), or repeats an id already listed for the
// token (contract violations), is dropped: it has no row and dst = -1.
#include "common.h"

namespace moe {

__device__ __forceinline__ int32_t clamp_live(int32_t live, int64_t T_cap)
{
    return live < 0 ? 0 : (live > T_cap ? (int32_t)T_cap : live);
}

// Block-wide exclusive scans of three ints per thread at once (blockDim.x <=
// 1024): the shuffles of the three run side by side.  v[i] becomes its
// exclusive prefix, total[i] the sum.
__device__ void block_exclusive_scan3(int (&v)[3], int (&total)[3], int* lds /* >= 96 ints */)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    int inc[3] = {v[0], v[1], v[2]};
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) o[i] = __shfl_up(inc[i], off, kWave);
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (lane >= off) inc[i] += o[i];
    }
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < 3; ++i) lds[32 * i + wid] = inc[i];
    __syncthreads();
    if (threadIdx.x < 3) {
        int run = 0;
        for (int w = 0; w < nw; ++w) { int c = lds[32 * threadIdx.x + w]; lds[32 * threadIdx.x + w] = run; run += c; }
        lds[32 * threadIdx.x + 31] = run;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        v[i] = lds[32 * i + wid] + inc[i] - v[i];
        total[i] = lds[32 * i + 31];
    }
    __syncthreads();
}

constexpr int kSlab = kMaxExperts * (kChunkTok / 32);   // ints of the LDS token bitmaps

struct PrepArgs {
    const int32_t* ids;
    const float* probs;
    int64_t T_cap;
    const int32_t* live;
    int E;
    int32_t* sorted_ids;
    float* sorted_probs;
    int32_t* local_rank;
    int32_t* chunk_base;     // [nchunks][E]: chunk counts, then global bases
    uint32_t* chunk_err;
    int32_t* counts;
    int32_t* offsets;
    int2* tiles;
    int2* tiles_big;
    int32_t* ready;          // single-launch FFN readiness counters (zeroed here)
    // single-launch finalize (null when the forward runs a separate finalize):
    // per live token and 512-column block, the token's kept-route count
    int32_t* fin_cnt;
    int fin_nt;              // 512-column blocks per token: ceil(H / 512)
    int fin_H;
    int fin_mode;            // combine: 0 fp32, 1 bf16, 2 rows
    void* fin_out;           // the forward's output (tokens with no kept route)
    WsHeader* hdr;
    int32_t* perm_src;
    int32_t* dst;
};

// Prefix over chunks and experts, tile table, header (one workgroup).
// With local_cnt (single-chunk launch) the per-expert counts come from LDS,
// the expert offsets go to local_off (LDS) instead of the chunk bases, and
// local_err is the chunk's error bits.
__device__ void prep_finish(const PrepArgs& a, int T, int nch, int32_t live, int* lds,
                            int* slab /* kSlab ints of LDS */, const int* local_cnt = nullptr,
                            int* local_off = nullptr, uint32_t local_err = 0)
{
    const int E = a.E;
    constexpr int PER = kMaxExperts / 256;          // experts per thread
    int cnt[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) cnt[q] = 0;
    if (local_cnt) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = threadIdx.x * PER + q;
            if (e < E) cnt[q] = local_cnt[e];
        }
    } else {
        // chunk counts [nch][E] -> each chunk's base inside its expert (exclusive
        // prefix over chunks), a slab of whole chunk rows at a time through LDS
        const int cs = kSlab / E > 0 ? kSlab / E : 1;
        for (int c0 = 0; c0 < nch; c0 += cs) {
            const int nc = nch - c0 < cs ? nch - c0 : cs;
            int32_t* g = a.chunk_base + (int64_t)c0 * E;
            // 32 loads per thread in flight before any is stored, a whole slab
            // in one round trip (a load-store loop waited for each load in
            // turn: 32 round trips, ~9 us of a 21 us launch at 16K tokens and
            // 128 experts); an index past the slab's end is
            // clamped to its last entry, which it then reads and writes again
            // (no branch, so no load is held back behind one)
            const int n = nc * E;
            for (int i0 = threadIdx.x; i0 < n; i0 += 32 * blockDim.x) {
                int v[32];
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    v[j] = __builtin_nontemporal_load(&g[min(i0 + j * (int)blockDim.x, n - 1)]);
#pragma unroll
                for (int j = 0; j < 32; ++j) slab[min(i0 + j * (int)blockDim.x, n - 1)] = v[j];
            }
            __syncthreads();
            // here expert e is thread e % 256's (consecutive threads, consecutive
            // words: no bank conflicts, and at most 128 experts one expert per
            // thread); eight chunks' counts read before any is replaced (one LDS
            // round trip per eight chunks instead of one per chunk)
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int e = q * 256 + threadIdx.x;
                if (e < E) {
                    int c = 0;
                    for (; c + 8 <= nc; c += 8) {
                        int v[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) v[j] = slab[(c + j) * E + e];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            slab[(c + j) * E + e] = cnt[q];
                            cnt[q] += v[j];
                        }
                    }
                    for (; c < nc; ++c) {
                        const int v = slab[c * E + e];
                        slab[c * E + e] = cnt[q];
                        cnt[q] += v;
                    }
                }
            }
            __syncthreads();
            for (int i = threadIdx.x; i < nc * E; i += blockDim.x) g[i] = slab[i];
            __syncthreads();
        }
        // the totals back to the layout below (experts PER t .. PER t + PER - 1
        // are thread t's), through the slab
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = q * 256 + threadIdx.x;
            if (e < E) slab[e] = cnt[q];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = threadIdx.x * PER + q;
            cnt[q] = e < E ? slab[e] : 0;
        }
    }
    int mine = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) mine += cnt[q];
    // M tiles: an expert with at most kBigMin rows goes to the 64-row tiles,
    // a larger one to the 256-row tiles
    int ntile_mine = 0, nbig_mine = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (cnt[q] > kBigMin) nbig_mine += (cnt[q] + kBigBMRows - 1) / kBigBMRows;
        else ntile_mine += (cnt[q] + kBM - 1) / kBM;
    }
    bool multi_mine = false;                       // an expert of more than one 64-row tile
#pragma unroll
    for (int q = 0; q < PER; ++q) multi_mine |= cnt[q] > kBM;
    const int multi = __syncthreads_or(multi_mine);
    int sc[3] = {mine, ntile_mine, nbig_mine}, tot[3];
    block_exclusive_scan3(sc, tot, lds);
    int off = sc[0], tfirst = sc[1], bfirst = sc[2];
    const int total = tot[0], ntotal = tot[1], nbig = tot[2];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = threadIdx.x * PER + q;
        if (e < E) {
            a.counts[e] = cnt[q];
            a.offsets[e] = off;
            if (local_off) local_off[e] = off;
            if (cnt[q] > kBigMin) {
                const int nt = (cnt[q] + kBigBMRows - 1) / kBigBMRows;
                for (int i = 0; i < nt; ++i) a.tiles_big[bfirst + i] = make_int2(e, off + i * kBigBMRows);
                bfirst += nt;
            } else {
                const int nt = (cnt[q] + kBM - 1) / kBM;
                for (int i = 0; i < nt; ++i) a.tiles[tfirst + i] = make_int2(e, off + i * kBM);
                tfirst += nt;
            }
        }
        off += cnt[q];
    }
    if (threadIdx.x == 0) a.offsets[E] = total;
    // the readiness counters of every 64-row M tile (a 256-row tile counts as
    // four) start at zero for the forward that follows
    for (int i = threadIdx.x; i < ntotal + 4 * nbig; i += blockDim.x) a.ready[i] = 0;
    uint32_t err = 0;
    if (local_cnt) err = threadIdx.x == 0 ? local_err : 0u;
    else
        for (int c = threadIdx.x; c < nch; c += blockDim.x)
            err |= __builtin_nontemporal_load(&a.chunk_err[c]);
    uint64_t b1 = __ballot(err & kErrBadId), b2 = __ballot(err & kErrDupId);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = (b1 ? kErrBadId : 0) | (b2 ? kErrDupId : 0);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t all = (live < 0 ? kErrLiveNeg : 0u) | (live > a.T_cap ? kErrLiveHigh : 0u);
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) all |= (uint32_t)lds[w];
        a.hdr->err = all;
        a.hdr->T = T;
        a.hdr->n_tiles = ntotal;
        a.hdr->n_tiles_big = nbig;
        a.hdr->multi_tile = multi ? 1 : 0;
        a.hdr->n_rows = total;
    }
}

template <int K>
__global__ void __launch_bounds__(256) prep_kernel(PrepArgs a)
{
    __shared__ uint32_t bm[kMaxExperts * (kChunkTok / 32)];
    __shared__ int lds[96];
    __shared__ int loc[2 * kMaxExperts];         // single-chunk launch: counts, offsets
    const int c = blockIdx.x;
    const int t = c * kChunkTok + threadIdx.x;
    // this token's (id, prob) pairs, read for every row inside the capacity so
    // that these loads go out beside the live count's instead of after it
    int id[K];
    float p[K];
    const bool in_cap = t < a.T_cap;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        id[j] = in_cap ? a.ids[(int64_t)t * K + j] : -1;
        // no probabilities (row mode): every route has probability 1
        p[j] = in_cap ? (a.probs ? a.probs[(int64_t)t * K + j] : 1.0f) : 0.0f;
    }
    const int32_t live = *a.live;
    const int T = clamp_live(live, a.T_cap);
    const int nch = (T + kChunkTok - 1) / kChunkTok;
    const int E = a.E;
    const bool single = gridDim.x == 1;          // T_cap <= one chunk
    if (c >= nch && !single) return;
    for (int i = threadIdx.x; i < E * (kChunkTok / 32); i += blockDim.x) bm[i] = 0;
    const bool valid = t < T;

    // canonical sort of this token's pairs (stable insertion sort)
#pragma unroll
    for (int j = 0; j < K; ++j) {
        id[j] = valid ? id[j] : -1;
        p[j] = valid ? p[j] : 0.0f;
    }
#pragma unroll
    for (int x = 1; x < K; ++x)
#pragma unroll
        for (int y = x; y > 0; --y)
            if (id[y - 1] > id[y]) {
                int ti = id[y]; id[y] = id[y - 1]; id[y - 1] = ti;
                float tp = p[y]; p[y] = p[y - 1]; p[y - 1] = tp;
            }
    uint32_t err = 0;
    bool keep[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const bool in = id[j] >= 0 && id[j] < E;
        const bool dup = j > 0 && id[j] == id[j - 1];
        keep[j] = valid && in && !dup;
        if (valid && !in) err |= kErrBadId;
        if (valid && dup) err |= kErrDupId;
        if (valid) {
            a.sorted_ids[(int64_t)t * K + j] = id[j];
            a.sorted_probs[(int64_t)t * K + j] = p[j];
        }
    }
    if (a.fin_cnt && valid) {
        // the single-launch finalize counts every 512-column block of this
        // token down from its kept routes; with none kept, no FC2 tile ever
        // reaches the token, so its output (+0 in every combine, as the
        // separate finalize writes it) is written here
        int nk = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) nk += keep[j] ? 1 : 0;
        for (int b = 0; b < a.fin_nt; ++b) a.fin_cnt[(int64_t)t * a.fin_nt + b] = nk;
        if (nk == 0) {
            if (a.fin_mode == 1) {
                uint16_t* o = (uint16_t*)a.fin_out + (int64_t)t * a.fin_H;
                for (int i = 0; i < a.fin_H; ++i) o[i] = 0;
            } else {
                const int64_t n = a.fin_mode == 2 ? (int64_t)K * a.fin_H : (int64_t)a.fin_H;
                float* o = (float*)a.fin_out + (int64_t)t * n;
                for (int64_t i = 0; i < n; ++i) o[i] = 0.0f;
            }
        }
    }
    __syncthreads();
    const int word = threadIdx.x >> 5, bit = threadIdx.x & 31;
#pragma unroll
    for (int j = 0; j < K; ++j)
        if (keep[j]) atomicOr(&bm[id[j] * 8 + word], 1u << bit);
    __syncthreads();
    // stable rank = tokens of this chunk below t that route to the same expert:
    // the expert's 8 bitmap words in two 16-byte reads, the words below this
    // token's counted whole, its own word below its bit (no dependent reads)
    int rank[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        rank[j] = -1;
        if (keep[j]) {
            const uint4 m0 = *(const uint4*)&bm[id[j] * 8];
            const uint4 m1 = *(const uint4*)&bm[id[j] * 8 + 4];
            const uint32_t m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            int r = 0;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint32_t mask = w < word ? ~0u : (w == word ? (1u << bit) - 1u : 0u);
                r += __popc(m[w] & mask);
            }
            rank[j] = r;
        }
        if (valid && !single) a.local_rank[(int64_t)t * K + j] = rank[j];
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const uint4 m0 = *(const uint4*)&bm[e * 8];
        const uint4 m1 = *(const uint4*)&bm[e * 8 + 4];
        const int n = __popc(m0.x) + __popc(m0.y) + __popc(m0.z) + __popc(m0.w) +
                      __popc(m1.x) + __popc(m1.y) + __popc(m1.z) + __popc(m1.w);
        if (single) loc[e] = n;
        else a.chunk_base[(int64_t)c * E + e] = n;
    }
    uint64_t any_bad = __ballot(err & kErrBadId), any_dup = __ballot(err & kErrDupId);
    if ((threadIdx.x & 63) == 0)
        lds[threadIdx.x >> 6] = (any_bad ? kErrBadId : 0) | (any_dup ? kErrDupId : 0);
    __syncthreads();
    uint32_t ce = 0;
    for (int w = 0; w < 4; ++w) ce |= (uint32_t)lds[w];
    if (single) {
        // the only chunk: finish from LDS, then each thread places its own routes
        __syncthreads();
        prep_finish(a, T, nch, live, lds, (int*)bm, loc, loc + kMaxExperts, ce);
        __syncthreads();
        if (valid) {
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int64_t r = (int64_t)t * K + j;
                if (keep[j]) {
                    const int pos = loc[kMaxExperts + id[j]] + rank[j];
                    a.perm_src[pos] = (int32_t)r;
                    a.dst[r] = pos;
                } else {
                    a.dst[r] = -1;
                }
            }
        }
        return;
    }
    if (threadIdx.x == 0) a.chunk_err[c] = ce;
}

// The prefix over every chunk's counts, run as its own single-workgroup launch
// once every prep_kernel workgroup has written its chunk (stream order).
__global__ void __launch_bounds__(256) prep_finish_kernel(PrepArgs a)
{
    __shared__ int slab[kSlab];
    __shared__ int lds[96];
    const int32_t live = *a.live;
    const int T = clamp_live(live, a.T_cap);
    const int nch = (T + kChunkTok - 1) / kChunkTok;
    prep_finish(a, T, nch, live, lds, slab);
}

__global__ void __launch_bounds__(256) prep_scatter_kernel(
    int64_t T_cap, const int32_t* __restrict__ live_ptr, int E, int k,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ dst)
{
    const int T = clamp_live(*live_ptr, T_cap);
    const int64_t R = (int64_t)T * k;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R;
         r += (int64_t)gridDim.x * blockDim.x) {
        int rk = local_rank[r];
        if (rk < 0) { dst[r] = -1; continue; }
        int e = sorted_ids[r];
        int c = (int)((r / k) / kChunkTok);
        int pos = offsets[e] + chunk_base[(int64_t)c * E + e] + rk;
        perm_src[pos] = (int32_t)r;
        dst[r] = pos;
    }
}

hipError_t launch_prep(const int32_t* ids, const float* probs, int64_t T_cap, const int32_t* live,
                       int E, int k, int num_cu, char* ws, const WsLayout& L, hipStream_t s,
                       int fin_H, int fin_mode, void* fin_out)
{
    PrepArgs a;
    a.fin_cnt = fin_out ? (int32_t*)(ws + L.fin_cnt) : nullptr;
    a.fin_nt = (fin_H + kFinCols - 1) / kFinCols;
    a.fin_H = fin_H;
    a.fin_mode = fin_mode;
    a.fin_out = fin_out;
    a.ids = ids;
    a.probs = probs;
    a.T_cap = T_cap;
    a.live = live;
    a.E = E;
    a.sorted_ids = (int32_t*)(ws + L.sorted_ids);
    a.sorted_probs = (float*)(ws + L.sorted_probs);
    a.local_rank = (int32_t*)(ws + L.local_rank);
    a.chunk_base = (int32_t*)(ws + L.chunk_base);
    a.chunk_err = (uint32_t*)(ws + L.chunk_err);
    a.counts = (int32_t*)(ws + L.counts);
    a.offsets = (int32_t*)(ws + L.offsets);
    a.tiles = (int2*)(ws + L.tiles);
    a.tiles_big = (int2*)(ws + L.tiles_big);
    a.ready = (int32_t*)(ws + L.ready);
    a.hdr = (WsHeader*)(ws + L.hdr);
    a.perm_src = (int32_t*)(ws + L.perm_src);
    a.dst = (int32_t*)(ws + L.dst);
    dim3 g1((unsigned)L.nchunks), b1(256);
#define PREP_CASE(KK)                                                        \
    case KK:                                                                 \
        hipLaunchKernelGGL(prep_kernel<KK>, g1, b1, 0, s, a);                \
        break;
    switch (k) {
        PREP_CASE(1) PREP_CASE(2) PREP_CASE(3) PREP_CASE(4) PREP_CASE(5) PREP_CASE(6)
        PREP_CASE(7) PREP_CASE(8) PREP_CASE(9) PREP_CASE(10) PREP_CASE(11) PREP_CASE(12)
        PREP_CASE(13) PREP_CASE(14) PREP_CASE(15) PREP_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef PREP_CASE
    if (L.nchunks == 1) return hipGetLastError();   // single workgroup scattered its routes
    hipLaunchKernelGGL(prep_finish_kernel, dim3(1), dim3(256), 0, s, a);
    int64_t R = T_cap * k;
    int64_t blocks = (R + 255) / 256;
    if (blocks > (int64_t)num_cu * 4) blocks = (int64_t)num_cu * 4;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(prep_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s, T_cap, live, E,
                       k, a.sorted_ids, a.local_rank, a.chunk_base, a.offsets,
                       (int32_t*)(ws + L.perm_src), (int32_t*)(ws + L.dst));
    return hipGetLastError();
}

}  // namespace moe
