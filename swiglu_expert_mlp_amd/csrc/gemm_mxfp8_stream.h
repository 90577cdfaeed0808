// K3 / K4 for MXFP8, streaming design (experts with at most 128 rows):
// grouped expert GEMMs on the CDNA4 block-scaled MFMA
// (E4M3 x E4M3 with one E8M0 scale per 32 elements of K, fp32 accumulate).
//
// Megatron-LM PR #7798, "Background": the activation and the FC2-input
// quantization are fused into the FC1 epilogue.  cudnn-frontend PR #448:
// MXFP8 = E4M3 data with an E8M0 scale per 32-element block.  The SwiGLU
// output is re-quantized per 32-element block of F in the FC1 epilogue
// (scale = power-of-two ceiling of the block's max magnitude / 448).
//
// Arithmetic contract: acc = 0; for k0 = 0, 128, 256, ... :
// acc = MFMA_SCALE_16x16x128_E4M3(A[row, k0:k0+128], B[col, k0:k0+128], acc)
// with the scales of the four 32-blocks, in that order for every row, tile
// and launch.  A K tail shorter than 128 is padded with zero codes.
//
// Lane layout of one 128-wide K step (both operands; the weights are stored
// pre-arranged in it, the activations are gathered from row-major rows): lane l holds row (l % 16);
// its first 16 bytes are K = 16 * (l / 16) + [0, 16) and its last 16 bytes are
// K = 64 + 16 * (l / 16) + [0, 16).  The scale byte of lane l applies to the
// 32-block (l / 16) of the step, i.e. 32-block q is made of the first halves
// (q < 2) or second halves (q >= 2) of lane groups 2 (q % 2) and 2 (q % 2) + 1.
// Work decomposition: a persistent grid over (M tile, N tile), a worker of 4
// waves x 64 columns per tile, up to 64 rows per M tile.
//
// W4: MXFP4 weights (E2M1 codes with one E8M0 scale per 32 elements of K)
// against the same MXFP8 activations: the B operand of a 128-wide K step is
// then 16 bytes per lane, lane l holding K = 32 (l / 16) + [0, 32) of column
// l % 16 (two codes per byte, the lower K in the low nibble; measured on the
// MI355X), so a block of 16 columns is 1 KB; the scale of lane l covers the
// same 32-block (l / 16).  Same contract, with the E2M1 B format.
#pragma once

#include "gemm_args.h"

namespace moe {

template <bool FC1, int NG, bool W4, bool PROB>
__device__ __forceinline__ void mx_tile_body(const MxGemmArgs& g, int e, int row0, int rows,
                                             int cb)
{
    constexpr int kBlk = W4 ? 1024 : 2048;    // bytes of a 16-column x 128-K weight block
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K, KB = K / 32;
    const uint8_t* ap[NG];
    const uint8_t* as[NG];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg) {
        int r = 16 * rg + r16;
        if (r >= rows) r = rows - 1;
        int64_t arow = row0 + r;
        if constexpr (FC1) arow = g.perm_src[arow] / g.topk;
        ap[rg] = g.A + arow * K + 16 * kg;
        as[rg] = g.As + arow * KB + kg;
    }
    // B fragments: 2 KB (MXFP4: 1 KB) blocks of 16 rows x 128 K,
    // [expert][row / 16][k / 128], in lane order (MXFP8: two 1 KB halves, 16
    // codes per lane each); scales in 256-byte groups of 4 K-steps, one dword
    // per lane (byte = step % 4).
    // MXFP4: blocks in 512-column groups (wblock_index): K step s of column
    // block c16 at wblock_index(c16, 0) + s * wblock_step(c16), the scale
    // group of steps 4q .. 4q + 3 likewise with q for s
    const int nt16 = g.N / 16, KS = (K + 127) / 128, KQ = (KS + 3) / 4;
    const uint8_t* bp[4];
    const uint32_t* bs[4];
    int bstep[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        int c16 = cb * 4 + ct;
        if (c16 >= nt16) c16 = nt16 - 1;
        const int64_t blk = (int64_t)e * nt16 + c16;
        if constexpr (W4) {
            bstep[ct] = (int)wblock_step(c16, nt16);
            bp[ct] = g.W + ((int64_t)e * nt16 * KS + wblock_index(c16, 0, nt16, KS)) * 1024 + 16 * lane;
            bs[ct] = (const uint32_t*)(g.Ws + ((int64_t)e * nt16 * KQ + wblock_index(c16, 0, nt16, KQ)) * 256) + lane;
        } else {
            bstep[ct] = 1;
            bp[ct] = g.W + blk * KS * kBlk + 16 * lane;
            bs[ct] = (const uint32_t*)(g.Ws + blk * KQ * 256) + lane;
        }
    }
    f32x4 acc[NG][4];
#pragma unroll
    for (int rg = 0; rg < NG; ++rg)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rg][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += 128) {
        // K is a multiple of 32: each 16-byte half and each 32-block is either
        // inside K or entirely past it (then zero codes, scale 2^0)
        const bool lo_in = k0 + 16 * kg < K, hi_in = k0 + 64 + 16 * kg < K;
        const bool s_in = k0 + 32 * kg < K;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        i32x8 a[NG], b[4];
        int sa[NG], sb[4];
#pragma unroll
        for (int rg = 0; rg < NG; ++rg) {
            uint4 lo = lo_in ? *(const uint4*)(ap[rg] + k0) : z;
            uint4 hi = hi_in ? *(const uint4*)(ap[rg] + k0 + 64) : z;
            a[rg] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sa[rg] = s_in ? (int)as[rg][k0 / 32] : 127;
        }
        const int step = k0 / 128;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            // padded blocks hold zero codes and scale 2^0, so no K check here;
            // weights are read once per tile (non-temporal, see the bf16 kernel)
            if constexpr (W4) {
                // the upper half of an E2M1 operand is not read by the MFMA
                const uint4 lo = load_stream16(bp[ct] + step * bstep[ct] * 1024);
                b[ct] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
            } else {
                const uint4 lo = load_stream16(bp[ct] + step * 2048);
                const uint4 hi = load_stream16(bp[ct] + step * 2048 + 1024);
                b[ct] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                              (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            sb[ct] = (int)((bs[ct][(step >> 2) * bstep[ct] * 64] >> (8 * (step & 3))) & 0xffu);
        }
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                // A format 0 (E4M3); B format 0 (E4M3) or 4 (E2M1)
                acc[rg][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a[rg], b[ct], acc[rg][ct], 0, W4 ? 4 : 0, 0, sa[rg], 0, sb[ct]);
    }

    if constexpr (FC1) {
        // SwiGLU, then the per-32 requantization of this interleave block's 32
        // outputs of each row: 16 lanes (same kg) x 2 tiles hold one row's block.
        const int F = g.N / 2, FB = F / 32;
        uint8_t* hq = (uint8_t*)g.out;
#pragma unroll
        for (int rg = 0; rg < NG; ++rg)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float h0, h1;
                int r = 16 * rg + 4 * kg + i;
                {
                    // the 16 lanes of one requantization block hold one row: one probability
                    const float pr = (PROB && r < rows) ? fc1_row_prob(g.row_prob, g.perm_src, row0 + r) : 1.0f;
                    float gt = acc[rg][0][i], up = acc[rg][2][i];
                    h0 = swiglu_f32(gt, up) * pr;
                    gt = acc[rg][1][i]; up = acc[rg][3][i];
                    h1 = swiglu_f32(gt, up) * pr;
                }
                const float amax = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
                int e8 = e8m0_exponent(amax);
                float inv = e8 == 127 ? __uint_as_float(1u << 22)
                                      : __uint_as_float((uint32_t)(127 - e8) << 23);
                if (r < rows) {
                    int64_t row = row0 + r;
                    const uint32_t c2 = cvt_e4m3x2(h0 * inv, h1 * inv);
                    hq[row * F + cb * 32 + r16] = (uint8_t)c2;
                    hq[row * F + cb * 32 + 16 + r16] = (uint8_t)(c2 >> 8);
                    if (r16 == 0) g.out_scale[row * FB + cb] = (uint8_t)(e8 + 127);
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

// The streaming tile loop of one 4-wave worker (wid = its wave 0..3): the
// 64-row tiles of the streaming table, and the large experts' 256-row tiles as
// four 64-row tiles each when the LDS-staged loop does not apply (K not a
// multiple of 128).
template <bool FC1, bool W4, bool PROB>
__device__ __forceinline__ void mx_stream_tiles(const MxGemmArgs& g, int worker, int nworkers, int wid)
{
    const int n_small = g.hdr->n_tiles;
    const int n_mt = n_small + (g.stream_big ? 4 * g.hdr->n_tiles_big : 0);
    const int total = n_mt * g.n_tiles_n;
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    for (int tile = worker; tile < total; tile += nworkers) {
        const int mt = tile / g.n_tiles_n;
        const int nt = tile - mt * g.n_tiles_n;
        int2 te;
        if (mt < n_small) {
            te = g.tiles[mt];
        } else {
            const int b = mt - n_small;
            te = g.tiles_big[b >> 2];
            te.y += kBM * (b & 3);
        }
        const int e = te.x, row0 = te.y;
        int rows = g.offsets[e + 1] - row0;
        if (rows > kBM) rows = kBM;
        const int cb = nt * 4 + wid;
        if (cb >= n_cb || rows <= 0) continue;
        const int ng = (rows + 15) >> 4;
        switch (ng) {
            case 1: mx_tile_body<FC1, 1, W4, PROB>(g, e, row0, rows, cb); break;
            case 2: mx_tile_body<FC1, 2, W4, PROB>(g, e, row0, rows, cb); break;
            case 3: mx_tile_body<FC1, 3, W4, PROB>(g, e, row0, rows, cb); break;
            default: mx_tile_body<FC1, 4, W4, PROB>(g, e, row0, rows, cb); break;
        }
    }
}

}  // namespace moe
