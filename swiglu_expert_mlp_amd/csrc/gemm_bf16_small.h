// K3 / K4, bf16 tiles of experts with at most 128 rows (64-row M tiles):
// grouped expert GEMMs on CDNA4 MFMA, bf16 operands, fp32 accumulate.
//
// Megatron-LM PR #7830, "1. Mega backend for generation": gate and up are
// stacked in one FC1 weight, interleaved in blocks of 32 rows, K-major.
// Megatron-LM PR #7798, "Background": the activation and the FC2-input
// conversion are fused into the FC1 epilogue; probabilities are applied after
// FC2 (the FC2 rows here are unweighted).
//
// Arithmetic contract (what makes every token's output independent of the
// launch): each output element is  acc = 0; for k0 = 0, 16, 32, ... :
// acc = MFMA_32x32x16_bf16(A[row, k0:k0+16], B[col, k0:k0+16], acc), with the
// same instruction and the same K order whatever the tile, the row's position
// inside its tile, or the number of rows of the launch.  Nothing splits K.
// The 256-row tiles (gemm_bf16_big.h) follow the same contract.
//
// These tiles stream the expert weights (each weight byte serves at most 64
// rows).  A workgroup of 8 waves takes a tile of up to 64 rows x 512 columns,
// wave w owning 64 columns (FC1: one gate/up interleave block = 32 SwiGLU
// outputs, the gate half and the up half one 32-column MFMA block each, so
// the gate and up of an output sit in the same lane).  Each 32-wide K step moves the tile's 32 weight blocks (1 KB each,
// stored in MFMA lane order; the 32 blocks of one step of a 512-column group
// are one contiguous 32 KB run of the kernel-weight buffer) and one 16-row x
// 64-byte activation block per row group (a quad of lanes per row, chunks
// permuted as in the 256-row tiles) into one stage of a 4-stage LDS ring by
// direct global->LDS loads, three stages in flight, and a barrier per step
// keeps the 8 waves together.  Measured at decode sizes: with one private
// register ring per wave instead, the two waves sharing a SIMD were served
// unevenly (one half of a workgroup finished its weight stream ~20 us after
// the other) and the launch lasted until the slowest; and the contiguous
// 32 KB step moves HBM->LDS at ~6.1 TB/s where 32 blocks 64 KB apart (one
// column's K steps contiguous instead) reach ~4.8 TB/s.
#pragma once

#include "gemm_bf16_big.h"

namespace moe {

constexpr int kSmallCols = 512;                 // columns per tile (8 waves x 64)
constexpr int kSmallRing = 4;
constexpr int kSmallStage = (4 + 32) * 1024;    // 4 activation + 32 weight blocks
constexpr int kSmallLds = kSmallRing * kSmallStage;

// s_waitcnt vmcnt(n) for a run-time n in 0..15 (a per-wave count of loads per
// step times the steps still allowed in flight)
__device__ __forceinline__ void wait_vmcnt_upto15(int n)
{
    switch (n) {
        case 0: BIG_WAIT_VMCNT(0); break;
        case 1: BIG_WAIT_VMCNT(1); break;
        case 2: BIG_WAIT_VMCNT(2); break;
        case 3: BIG_WAIT_VMCNT(3); break;
        case 4: BIG_WAIT_VMCNT(4); break;
        case 5: BIG_WAIT_VMCNT(5); break;
        case 6: BIG_WAIT_VMCNT(6); break;
        case 7: BIG_WAIT_VMCNT(7); break;
        case 8: BIG_WAIT_VMCNT(8); break;
        case 9: BIG_WAIT_VMCNT(9); break;
        case 10: BIG_WAIT_VMCNT(10); break;
        default: BIG_WAIT_VMCNT(0); break;
    }
}

__device__ __forceinline__ int small_col_tiles(const GemmArgs& g) { return (g.N + kSmallCols - 1) / kSmallCols; }


// FC1 tile done (single-launch FFN): every wave's stores complete, then one
// thread releases them at device scope (the L2's dirty lines written back)
// and counts the tile in its M tile's readiness counter.
__device__ __forceinline__ void small_release(const GemmArgs& g, int mt)
{
    BIG_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(g.ready + mt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The single-launch FFN (FC1 and FC2 tiles in one persistent launch, every
// workgroup running all its FC1 tiles before any FC2 tile): FUSE = 1, an FC1
// tile releases its SwiGLU rows (device scope) and counts itself in its M
// tile's readiness counter; FUSE = 2, an FC2 tile issues its first weight
// loads, waits until `need` FC1 column tiles of its M tile are counted (a
// bounded wait: past about 0.2 s it flags kErrFusedWait and goes on), and
// reads the rows with coherent loads.  The wait always ends, since every
// FC1 tile is taken by a workgroup that is already running (one per CU).
constexpr int kFuseWaitTicks = 20000000;        // wall-clock ticks (100 MHz): 0.2 s
constexpr int kCoherentLoad = 16;               // cache policy sc1 (device-coherent)

// Single-launch finalize (FUSE = 3: an FC2 tile of the fused launch): once
// the tile's fp32 rows are stored, they are released at device scope (every
// wave's stores complete, the L2's dirty lines written back) and each row's
// token counts its 512-column block down; the workgroup that takes a count
// to zero holds the last of that token's rows in the block and combines the
// block at once, reading the other routes' rows (written by workgroups on any
// XCD) with device-coherent loads.  No wait: a workgroup that is not the last
// goes on to its next tile.  A tile holds one expert's rows, and a token
// routes to an expert at most once, so a token appears at most once per tile.
// The combine is the separate finalize's arithmetic (fp32 fused multiply-adds
// of probability and row from +0 in canonical order, skipping dropped
// routes; its bf16 rounding; or row mode).  The lanes that counted a token
// to zero stage its k row indices and probabilities in LDS (one round trip
// for all of them), then the 8 waves share the jobs: a job is one token's
// whole 512-column block (8 columns per lane) when k <= 8, or a 256-column
// half (4 per lane) above, so that a job's k row loads (issued back to back,
// one round trip) fit 64 registers.
static_assert(kFinCols == kSmallCols && kFinCols == 64 * 8, "finalize blocks");
struct SmallFinLds {
    int n;                                       // tokens this workgroup combines
    int tok[kBM];
    int dst[kBM][kMaxTopk];                      // their routes' grouped rows (-1: dropped)
    float prob[kBM][kMaxTopk];                   // and probabilities (1 when none are applied)
};

// device-coherent 8-byte load: a relaxed device-scope atomic load (sc1)
__device__ __forceinline__ float2 fin_load2(const float* p)
{
    const uint64_t v = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// The combine jobs of one wave: NR routes at most, CPL columns per lane.
template <int NR, int CPL>
__device__ __forceinline__ void small_fin_jobs(const GemmArgs& g, const SmallFinLds* fl, int ct)
{
    constexpr int kJobs = kFinCols / (64 * CPL);  // jobs per token block
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int H = g.N, k = g.topk;
    const float* O = (const float*)g.out;
    const int njobs = fl->n * kJobs;
    for (int q = wid; q < njobs; q += 8) {
        const int i = q / kJobs;
        const int c = ct * kFinCols + (q % kJobs) * 64 * CPL + CPL * lane;
        // H is a multiple of 32, so a lane's columns are all inside or all past it
        const bool in = c < H;
        const int t = __builtin_amdgcn_readfirstlane(fl->tok[i]);
        int d[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) d[j] = j < k ? __builtin_amdgcn_readfirstlane(fl->dst[i][j]) : -1;
        float2 o[NR][CPL / 2];
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int h = 0; h < CPL / 2; ++h) {
                o[j][h] = make_float2(0.0f, 0.0f);
                if (d[j] >= 0 && in) o[j][h] = fin_load2(O + (int64_t)d[j] * H + c + 2 * h);
            }
        // the stores are per-lane predicated (no early exit)
        if (g.fin_mode == 2) {
            // row mode: every route alone, one fma from +0 (a dropped route stays +0)
#pragma unroll
            for (int j = 0; j < NR; ++j)
                if (j < k && in) {
                    float* dstp = (float*)g.fin_out + ((int64_t)t * k + j) * H + c;
#pragma unroll
                    for (int h = 0; h < CPL / 4; ++h) {
                        float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        if (d[j] >= 0)
                            r = make_float4(__builtin_fmaf(1.0f, o[j][2 * h].x, 0.0f),
                                            __builtin_fmaf(1.0f, o[j][2 * h].y, 0.0f),
                                            __builtin_fmaf(1.0f, o[j][2 * h + 1].x, 0.0f),
                                            __builtin_fmaf(1.0f, o[j][2 * h + 1].y, 0.0f));
                        *(float4*)(dstp + 4 * h) = r;
                    }
                }
        } else {
            float acc[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int j = 0; j < NR; ++j)
                if (d[j] >= 0) {
                    const float p = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fl->prob[i][j])));
#pragma unroll
                    for (int h = 0; h < CPL / 2; ++h) {
                        acc[2 * h] = __builtin_fmaf(p, o[j][h].x, acc[2 * h]);
                        acc[2 * h + 1] = __builtin_fmaf(p, o[j][h].y, acc[2 * h + 1]);
                    }
                }
            if (in) {
                if (g.fin_mode == 0) {
                    float* dstp = (float*)g.fin_out + (int64_t)t * H + c;
#pragma unroll
                    for (int h = 0; h < CPL / 4; ++h)
                        *(float4*)(dstp + 4 * h) = make_float4(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
                } else {
                    uint16_t* dstp = (uint16_t*)g.fin_out + (int64_t)t * H + c;
#pragma unroll
                    for (int h = 0; h < CPL / 4; ++h)
                        *(uint2*)(dstp + 4 * h) = make_uint2(
                            (uint32_t)f32_to_bf16_bits(acc[4 * h]) | ((uint32_t)f32_to_bf16_bits(acc[4 * h + 1]) << 16),
                            (uint32_t)f32_to_bf16_bits(acc[4 * h + 2]) | ((uint32_t)f32_to_bf16_bits(acc[4 * h + 3]) << 16));
                }
            }
        }
    }
}

__device__ __forceinline__ void small_finalize(const GemmArgs& g, SmallFinLds* fl, int ct, int row0,
                                               int rows)
{
    const int lane = threadIdx.x & 63;
    const int NT = small_col_tiles(g);           // g.N = H: output column blocks per token
    const int k = g.topk;
    BIG_WAIT_VMCNT(0);                           // this wave's row stores are complete
    __builtin_amdgcn_s_barrier();                // and every wave's
    if (threadIdx.x < 64) {
        int t = 0;
        bool last = false;
        if (lane < rows) {
            t = g.fin_route[row0 + lane] / g.topk;
            last = __hip_atomic_fetch_add(g.fin_cnt + (int64_t)t * NT + ct, -1, __ATOMIC_RELEASE,
                                          __HIP_MEMORY_SCOPE_AGENT) == 1;
        }
        const uint64_t m = __ballot(last);
        if (last) {
            const int i = __popcll(m & ((1ull << lane) - 1ull));
            fl->tok[i] = t;
            int d[kMaxTopk];
            float p[kMaxTopk];
#pragma unroll
            for (int j = 0; j < kMaxTopk; ++j)
                if (j < k) {
                    d[j] = g.fin_dst[(int64_t)t * k + j];
                    p[j] = g.fin_prob ? g.fin_prob[(int64_t)t * k + j] : 1.0f;
                }
#pragma unroll
            for (int j = 0; j < kMaxTopk; ++j)
                if (j < k) {
                    fl->dst[i][j] = d[j];
                    fl->prob[i][j] = p[j];
                }
        }
        if (lane == 0) fl->n = __popcll(m);
    }
    __syncthreads();
    if (k <= 8) small_fin_jobs<8, 8>(g, fl, ct);
    else small_fin_jobs<16, 4>(g, fl, ct);
}

// n_small: the number of 64-row M tiles; n_big: the number of 256-row M
// tiles this launch also runs, as four 64-row tiles each (0 when a launch of
// the 256-row design takes them); (e0, row00): the table entry of this
// workgroup's first tile (xcd_first_tile()), read by the caller before the counts
// were known.
// WPOL: the cache policy of the weight stream (kNonTemporal when every
// expert's rows fit one 64-row tile, else the default; the caller reads which
// from the header).
template <bool FC1, bool PROB, int FUSE, int WPOL>
__device__ __forceinline__ void small_tiles(const GemmArgs& g, char* smem, int n_small, int n_big,
                                            int e0, int row00, int need = 0, SmallFinLds* fin_lds = nullptr)
{
    const int NTs = small_col_tiles(g);
    const int total = (n_small + 4 * n_big) * NTs;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int K = g.K;
    const int nsteps = K / 32;
    const int nt16 = g.N / 16;
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    // 32 x 16 fragment lanes of sub-step q (8-wide K chunks 2 q, 2 q + 1): A row
    // l % 32 of a 32-row block, chunk 2 q + l / 32; B column l % 32, lane
    // 16 (2 q + l / 32) + l % 16 of its 16-column block
    int a_off[2], b_off[2];
    {
        const int r = lane & 31, r16 = r & 15, hi = lane >> 5;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = 2 * q + hi;
            a_off[q] = (r >> 4) * 1024 + 16 * (4 * r16 + (c ^ big_swz(r16)));
            b_off[q] = (r >> 4) * 1024 + 16 * (16 * c + r16);
        }
    }
    const int c32 = lane & 31, hi = lane >> 5;

    const int first = xcd_first_tile();
    for (int tile = first; tile < total; tile += gridDim.x) {
        const int mt = tile / NTs, ct = tile - mt * NTs;
        int e = e0, row0 = row00;
        if (mt >= n_small) {
            // a 256-row tile run as four 64-row tiles
            const int* te = (const int*)(g.tiles_big + ((mt - n_small) >> 2));
            e = ld_const(te);
            row0 = ld_const(te + 1) + kBM * ((mt - n_small) & 3);
        } else if (tile != first) {
            const int* te = (const int*)(g.tiles + mt);
            e = ld_const(te);
            row0 = ld_const(te + 1);
        }
        const int cb = ct * 8 + wid;                 // this wave's 64-column block
        const bool has_cols = cb < n_cb;
        const uint16_t* bblk[4];
        int bstep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c16 = min(cb * 4 + j, nt16 - 1);
            bblk[j] = g.W + ((int64_t)e * nt16 * nsteps + wblock_index(c16, 0, nt16, nsteps)) * 512 + 8 * lane;
            bstep[j] = (int)wblock_step(c16, nt16) * 512;
        }
        auto issue_b = [&](int s) {
            char* st = smem + (s % kSmallRing) * kSmallStage;
            if (has_cols) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_global_load_lds(bblk[j] + (int64_t)bstep[j] * s,
                                                     (lds_void_t*)(st + (4 + 4 * wid + j) * 1024), 16, 0,
                                                     WPOL);
            }
        };
        // a 64-row part of a 256-row tile may lie past its expert's rows
        int rows = 0;
        if (mt >= n_small) {
            rows = min(kBM, ld_const(g.offsets + e + 1) - row0);
            if (rows <= 0) continue;                 // uniform across the workgroup
        }
        // every wave finished the previous tile's LDS reads before the ring is
        // refilled; step 0's weights go out before the row count and the
        // gathered rows (a further round trip) are known
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        issue_b(0);
        if (mt < n_small) rows = min(kBM, ld_const(g.offsets + e + 1) - row0);
        const int ng = (rows + 15) >> 4;             // 16-row activation blocks
        const int nb = (rows + 31) >> 5;             // 32-row MFMA blocks
        const bool has_a = wid < ng;                 // this wave loads activation block wid
        const int nl = (has_a ? 1 : 0) + (has_cols ? 4 : 0);

        const uint16_t* arow = g.A;
        if (has_a) {
            const int r = min(16 * wid + (lane >> 2), rows - 1);
            int64_t src = row0 + r;
            if constexpr (FC1) src = g.perm_src[src] / g.topk;
            arow = g.A + src * K + 8 * ((lane & 3) ^ big_swz(lane >> 2));
        }
        if constexpr (FUSE >= 2) {
            // the waves that load rows wait for the FC1 tiles of this M tile
            if (has_a) {
                const int32_t* rp = g.ready + mt;
                int v = __hip_atomic_load(rp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v < need) {
                    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                    while (v < need) {
                        __builtin_amdgcn_s_sleep(2);
                        v = __hip_atomic_load(rp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)kFuseWaitTicks) {
                            if (lane == 0) atomicOr(g.err, kErrFusedWait);
                            break;
                        }
                    }
                }
            }
        }
        auto issue_a = [&](int s) {
            if (has_a) {
                char* dst = smem + (s % kSmallRing) * kSmallStage + wid * 1024;
                if constexpr (FUSE >= 2)
                    __builtin_amdgcn_global_load_lds(arow + 32 * s, (lds_void_t*)dst, 16, 0, kCoherentLoad);
                else
                    big_load_block(arow + 32 * s, dst);
            }
        };
        auto issue = [&](int s) { issue_a(s); issue_b(s); };

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // a step's loads stay contiguous in issue order (step 0: weights, then rows)
        issue_a(0);
#pragma unroll
        for (int s = 1; s < kSmallRing - 1; ++s)
            if (s < nsteps) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // step s landed when at most the later in-flight steps remain
            wait_vmcnt_upto15(min(kSmallRing - 2, nsteps - 1 - s) * nl);
            __builtin_amdgcn_s_barrier();
            if (s + kSmallRing - 1 < nsteps) issue(s + kSmallRing - 1);
            if (has_cols) {
                const char* st = smem + (s % kSmallRing) * kSmallStage;
                // B blocks 4 wid + 2 j and + 1 hold the wave's 32-column block j
                bf16x8 a[2][2], b[2][2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        b[q][j] = big_frag(st + (4 + 4 * wid + 2 * j) * 1024 + b_off[q]);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (i < nb) a[q][i] = big_frag(st + 2 * i * 1024 + a_off[q]);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (i < nb)
#pragma unroll
                            for (int j = 0; j < 2; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q][i], b[q][j], acc[i][j], 0, 0, 0);
            }
        }

        // epilogue: lane holds column l % 32 of each 32-column block and rows
        // 8 (v / 4) + 4 (l / 32) + v % 4 of each 32-row block
        if (!has_cols) {
            if constexpr (FUSE == 1) small_release(g, mt);
            if constexpr (FUSE == 3) small_finalize(g, fin_lds, ct, row0, rows);
            continue;
        }
        if constexpr (FC1) {
            // column block 0 is the gate half, 1 the up half of interleave block cb
            const int F = g.N / 2;
            uint16_t* hb = (uint16_t*)g.out;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
                    if (i < nb && r < rows) {
                        const float pr = PROB ? fc1_row_prob(g.row_prob, g.perm_src, row0 + r) : 1.0f;
                        hb[(int64_t)(row0 + r) * F + cb * 32 + c32] =
                            f32_to_bf16_bits(swiglu_f32(acc[i][0][v], acc[i][1][v]) * pr);
                    }
                }
        } else {
            float* ob = (float*)g.out;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = cb * 64 + 32 * j + c32;
                if (cb * 64 + 32 * j < g.N) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int r = 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
                            if (i < nb && r < rows) ob[(int64_t)(row0 + r) * g.N + col] = acc[i][j][v];
                        }
                }
            }
        }
        if constexpr (FUSE == 1) small_release(g, mt);
        if constexpr (FUSE == 3) small_finalize(g, fin_lds, ct, row0, rows);
    }
}

}  // namespace moe
