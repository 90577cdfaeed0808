// K3 / K4: grouped expert GEMMs on CDNA4 MFMA, bf16 operands, fp32 accumulate.
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
    const uint16_t* bp[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        int col = cb * 64 + 16 * ct + r16;
        if (col >= g.N) col = g.N - 1;
        bp[ct] = g.W + ((int64_t)e * g.N + col) * K + 8 * kg;
    }
    f32x4 acc[NG][4];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rg][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 an[NG], bn[4];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg) an[rg] = *(const uint4*)(ap[rg]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) bn[ct] = *(const uint4*)(bp[ct]);
    for (int k0 = 0; k0 < K; k0 += 32) {
        uint4 ac[NG], bc[4];
#pragma unroll
        for (int rg = 0; rg < NG; ++rg) ac[rg] = an[rg];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bc[ct] = bn[ct];
        if (k0 + 32 < K) {
#pragma unroll
            for (int rg = 0; rg < NG; ++rg) an[rg] = *(const uint4*)(ap[rg] + k0 + 32);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) bn[ct] = *(const uint4*)(bp[ct] + k0 + 32);
        }
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[rg][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(ac[rg]), as_bf16x8(bc[ct]), acc[rg][ct], 0, 0, 0);
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

template <bool FC1>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(GemmArgs g)
{
    const int n_mt = g.hdr->n_tiles;
    const int total = n_mt * g.n_tiles_n;
    const int wid = threadIdx.x >> 6;
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
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

hipError_t launch_gemm_bf16(bool fc1, const GemmArgs& g, int num_cu, hipStream_t s)
{
    dim3 grid((unsigned)(num_cu * 3)), block(256);
    if (fc1)
        hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, block, 0, s, g);
    else
        hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, block, 0, s, g);
    return hipGetLastError();
}

}  // namespace moe
