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
// launch): each output element is  acc = 0; for k0 = 0, 32, 64, ... :
// acc = MFMA_16x16x32_bf16(A[row, k0:k0+32], B[col, k0:k0+32], acc), with the
// same instruction and the same K order whatever the tile, the row's position
// inside its tile, or the number of rows of the launch.  Nothing splits K.
// The 256-row tiles (gemm_bf16_lds.h) follow the same contract.
//
// These tiles stream the expert weights (each weight byte serves at most 64
// rows).  A workgroup of 8 waves takes a tile of up to 64 rows x 512 columns,
// wave w owning 64 columns (FC1: one gate/up interleave block = 32 SwiGLU
// outputs).  Each 32-wide K step moves the tile's 32 weight blocks (1 KB each,
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

#include "gemm_bf16_lds.h"

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
        case 0: WAIT_VMCNT(0); break;
        case 1: WAIT_VMCNT(1); break;
        case 2: WAIT_VMCNT(2); break;
        case 3: WAIT_VMCNT(3); break;
        case 4: WAIT_VMCNT(4); break;
        case 5: WAIT_VMCNT(5); break;
        case 6: WAIT_VMCNT(6); break;
        case 7: WAIT_VMCNT(7); break;
        case 8: WAIT_VMCNT(8); break;
        case 9: WAIT_VMCNT(9); break;
        case 10: WAIT_VMCNT(10); break;
        default: WAIT_VMCNT(0); break;
    }
}

__device__ __forceinline__ int small_col_tiles(const GemmArgs& g) { return (g.N + kSmallCols - 1) / kSmallCols; }

// n_mt: the number of 64-row M tiles; (e0, row00): the table entry of this
// workgroup's first tile (blockIdx.x), read by the caller before n_mt was known.
template <bool FC1>
__device__ __forceinline__ void small_tiles(const GemmArgs& g, char* smem, int n_mt, int e0, int row00)
{
    const int NTs = small_col_tiles(g);
    const int total = n_mt * NTs;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int K = g.K;
    const int nsteps = K / 32;
    const int nt16 = g.N / 16;
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    const int a_off = 16 * (4 * (lane & 15) + ((lane >> 4) ^ a_swz(lane & 15)));
    const int r16 = lane & 15, kg = lane >> 4;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / NTs, ct = tile - mt * NTs;
        int e = e0, row0 = row00;
        if (tile != (int)blockIdx.x) {
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
                    load_block_to_lds(bblk[j] + (int64_t)bstep[j] * s, st + (4 + 4 * wid + j) * 1024);
            }
        };
        // every wave finished the previous tile's LDS reads before the ring is
        // refilled; step 0's weights go out before the row count and the
        // gathered rows (a further round trip) are known
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        issue_b(0);
        const int rows = min(kBM, ld_const(g.offsets + e + 1) - row0);
        const int ng = (rows + 15) >> 4;
        const bool has_a = wid < ng;                 // this wave loads activation block wid
        const int nl = (has_a ? 1 : 0) + (has_cols ? 4 : 0);

        const uint16_t* arow = g.A;
        if (has_a) {
            const int r = min(16 * wid + (lane >> 2), rows - 1);
            int64_t src = row0 + r;
            if constexpr (FC1) src = g.perm_src[src] / g.topk;
            arow = g.A + src * K + 8 * ((lane & 3) ^ a_swz(lane >> 2));
        }
        auto issue_a = [&](int s) {
            if (has_a) load_block_to_lds(arow + 32 * s, smem + (s % kSmallRing) * kSmallStage + wid * 1024);
        };
        auto issue = [&](int s) { issue_a(s); issue_b(s); };

        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
                bf16x8 a[4], b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = __builtin_bit_cast(bf16x8, *(const uint4*)(st + (4 + 4 * wid + j) * 1024 + 16 * lane));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i < ng) a[i] = __builtin_bit_cast(bf16x8, *(const uint4*)(st + i * 1024 + a_off));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i < ng)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }

        // epilogue: lane holds rows 4 kg + v of each 16-row group, column r16 of each block
        if (!has_cols) continue;
        if constexpr (FC1) {
            const int F = g.N / 2;
            uint16_t* hb = (uint16_t*)g.out;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * i + 4 * kg + v;
                    if (i < ng && r < rows) {
                        const int64_t row = row0 + r;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const float gt = acc[i][h][v];
                            const float up = acc[i][h + 2][v];
                            const float hv = gt / (1.0f + __expf(-gt)) * up;
                            hb[row * F + cb * 32 + 16 * h + r16] = f32_to_bf16_bits(hv);
                        }
                    }
                }
        } else {
            float* ob = (float*)g.out;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * i + 4 * kg + v;
                    if (i < ng && r < rows) {
                        const int64_t row = row0 + r;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int col = cb * 64 + 16 * j + r16;
                            if (col < g.N) ob[row * g.N + col] = acc[i][j][v];
                        }
                    }
                }
        }
    }
}

}  // namespace moe
