// K3 / K4, streaming design (experts with at most 128 rows): grouped expert
// GEMMs on CDNA4 MFMA, bf16 operands, fp32 accumulate.
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
//
// Work decomposition: a persistent grid of fixed size walks the device-built
// tile table (expert, first row) x N tiles.  A workgroup is 4 waves; each
// wave owns 64 output columns (FC1: one interleave block = 32 gate + 32 up
// columns, i.e. 32 SwiGLU outputs) and all rows of the M tile (up to 64, in
// 16-row MFMA groups; groups past the expert's row count are skipped).
// Operands are streamed from global memory straight into registers in the
// MFMA lane layout: lane l holds row (l % 16) and the 8 K values starting at
// 8 * (l / 16) of each 32-wide K step, for both operands.  Rows past the
// expert's count read a clamped, valid row; their results are discarded.
#pragma once

#include "gemm_args.h"

namespace moe {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <bool FC1, int NG>
__device__ __forceinline__ void tile_body(const GemmArgs& g, int e, int row0, int rows, int cb)
{
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K;
    const uint16_t* ap[NG];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg) {
        int r = 16 * rg + r16;
        if (r >= rows) r = rows - 1;
        int row = row0 + r;
        if constexpr (FC1) {
            int t = g.perm_src[row] / g.topk;
            ap[rg] = g.A + (int64_t)t * K + 8 * kg;
        } else {
            ap[rg] = g.A + (int64_t)row * K + 8 * kg;
        }
    }
    // B fragments: the weight is stored as 1 KB blocks of 16 rows x 32 K in
    // lane order, [expert][row / 16][k / 32]; a lane reads its 16 bytes at
    // block + 16 * lane, so one load instruction of a wave is 1 KB contiguous.
    const int nt16 = g.N / 16;
    const uint16_t* bp[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        int c16 = cb * 4 + ct;
        if (c16 >= nt16) c16 = nt16 - 1;
        bp[ct] = g.W + ((int64_t)e * nt16 + c16) * (int64_t)(K / 32) * 512 + 8 * lane;
    }
    f32x4 acc[NG][4];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rg][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Ring of D K-steps in flight: step s lives in slot s % D.  The MFMA order
    // is still k0 = 0, 32, 64, ... for every element; only the load schedule
    // runs ahead.  D shrinks as the row groups grow, so that every variant
    // fits two 4-wave workers per CU in 256 registers per lane.
    constexpr int D = NG <= 2 ? 4 : (NG == 3 ? 3 : 2);
    const int nsteps = K / 32;
    uint4 ar[D][NG], br[D][4];
    // weights are read once per tile: non-temporal loads keep them from
    // evicting the activation rows that the other N tiles of the M tile reuse
    // (measured: decode FC1 98.5 -> 93.2 us, FC2 64.6 -> 61.5 us)
    auto load = [&](int d, int s) {
#pragma unroll
        for (int rg = 0; rg < NG; ++rg) ar[d][rg] = *(const uint4*)(ap[rg] + 32 * s);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) br[d][ct] = load_stream16(bp[ct] + 512 * s);
    };
    auto mfma = [&](int d) {
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[rg][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(ar[d][rg]), as_bf16x8(br[d][ct]), acc[rg][ct], 0, 0, 0);
    };
    int s0 = 0;
    if (nsteps >= D) {
#pragma unroll
        for (int d = 0; d < D; ++d) load(d, d);
        // steady state: every slot is consumed and refilled D steps ahead
        for (; s0 + 2 * D <= nsteps; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                mfma(d);
                load(d, s0 + D + d);
            }
        }
        // drain the ring, refilling only with steps that exist
#pragma unroll
        for (int d = 0; d < D; ++d) {
            mfma(d);
            if (s0 + D + d < nsteps) load(d, s0 + D + d);
        }
        s0 += D;
    }
    // remaining steps (fewer than D), one at a time
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (s0 + d < nsteps) {
            if (nsteps < D) load(d, s0 + d);
            mfma(d);
        }
    }

    // epilogue: lane holds rows 4 * kg + i (i < 4) of each group, column r16 of each tile
    if constexpr (FC1) {
        const int F = g.N / 2;
        uint16_t* hb = (uint16_t*)g.out;
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = 16 * rg + 4 * kg + i;
                if (r < rows) {
                    int64_t row = row0 + r;
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        float gt = acc[rg][ct][i];
                        float up = acc[rg][ct + 2][i];
                        float h = gt / (1.0f + __expf(-gt)) * up;
                        hb[row * F + cb * 32 + 16 * ct + r16] = f32_to_bf16_bits(h);
                    }
                }
            }
    } else {
        float* ob = (float*)g.out;
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = 16 * rg + 4 * kg + i;
                if (r < rows) {
                    int64_t row = row0 + r;
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        int col = cb * 64 + 16 * ct + r16;
                        if (col < g.N) ob[row * g.N + col] = acc[rg][ct][i];
                    }
                }
            }
    }
}

// The streaming tile loop of one 4-wave worker (wid = its wave 0..3):
// workers take the 64-row M tiles x N tiles in a strided order.
template <bool FC1>
__device__ __forceinline__ void stream_tiles(const GemmArgs& g, int worker, int nworkers, int wid)
{
    const int n_mt = g.hdr->n_tiles;
    const int total = n_mt * g.n_tiles_n;
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    for (int tile = worker; tile < total; tile += nworkers) {
        const int mt = tile / g.n_tiles_n;
        const int nt = tile - mt * g.n_tiles_n;
        const int2 te = g.tiles[mt];
        const int e = te.x, row0 = te.y;
        int rows = g.offsets[e + 1] - row0;
        if (rows > kBM) rows = kBM;
        const int cb = nt * 4 + wid;
        if (cb >= n_cb || rows <= 0) continue;
        const int ng = (rows + 15) >> 4;
        switch (ng) {
            case 1: tile_body<FC1, 1>(g, e, row0, rows, cb); break;
            case 2: tile_body<FC1, 2>(g, e, row0, rows, cb); break;
            case 3: tile_body<FC1, 3>(g, e, row0, rows, cb); break;
            default: tile_body<FC1, 4>(g, e, row0, rows, cb); break;
        }
    }
}

}  // namespace moe
