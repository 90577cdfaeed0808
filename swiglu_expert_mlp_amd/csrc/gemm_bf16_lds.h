// K3 / K4, LDS-staged design (experts with more than 128 rows): grouped GEMM on CDNA4 MFMA,
// bf16 operands, fp32 accumulate.
//
// Same arithmetic contract as the 64-row tiles of gemm_bf16_small.h (and
// therefore bitwise the same results for a row): every output element is acc = 0; for k0 = 0, 32, ... :
// acc = MFMA_16x16x32_bf16(A[row, k0:k0+32], B[col, k0:k0+32], acc).  Only
// the decomposition differs: a workgroup computes a 256 x 256 tile, each of
// its 8 waves a 128 x 64 part (8 x 4 MFMA blocks, accumulators in registers;
// for FC1 the 64 columns are one gate/up interleave block), with both
// operands staged through LDS in 32-wide K stages,
// a ring of 4 stages with 3 in flight.  Stages are filled with direct global->LDS loads
// (global_load_lds_dwordx4): one wave instruction moves one 16 x 32 operand
// block (1 KB) into LDS.  The weight blocks are stored in MFMA lane order in
// the kernel-weight buffer (1 KB each; one K step of a tile's 16 column blocks
// is a contiguous 16 KB run) and land as stored.
// Activation blocks are gathered 16 rows x 64 bytes at a time with a quad of
// lanes per row, each quad one 64-byte segment (lane-to-row by lane % 16
// spreads every quad over four rows and moves a third less per second through
// the L1), and land with a row's four 16-byte chunks permuted so that the
// fragment reads stay free of bank conflicts.
//
// Tiles: the device-built table of 256-row M tiles (experts with more than
// 128 rows) x 256-column N tiles.  The persistent grid
// is one workgroup per CU; tiles are split into 8 contiguous ranges, one per
// XCD (workgroups are dispatched round-robin over the XCDs), so the tiles of
// one expert, which share activation and weight slices, run on one XCD and
// share its L2.  Within an expert the tiles go column tile by column tile, so
// that all of its row tiles read a weight slice at the same time (measured:
// 22% less FC1 traffic than row-tile order at 16K tokens).
#pragma once

#include <type_traits>

#include "gemm_args.h"

namespace moe {

constexpr int kBigBM = 256;
constexpr int kBigBN = 256;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void load_block_to_lds(const void* gsrc, void* lds_dst)
{
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const char* base, int lane)
{
    return __builtin_bit_cast(bf16x8, *(const uint4*)(base + 16 * lane));
}

// chunk permutation of an activation block row (measured free of LDS bank
// conflicts for the fragment reads)
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 3; }

constexpr int kRing = 4;          // LDS stages (one 32-wide K step each)
constexpr int kStageBytes = 32 * 1024;

// s_waitcnt with only a vector-memory bound (expcnt and lgkmcnt left at max).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// The LDS-staged tile loop of one 8-wave workgroup (one workgroup per CU).
// smem: the kernel's LDS, at least kRing * kStageBytes bytes, 1 KB aligned;
// n_mt: the number of 256-row M tiles.
template <bool FC1>
__device__ __forceinline__ void lds_tiles(const GemmArgs& g, char* smem_base, int n_mt)
{
    // [stage][A 16 blocks | B 16 blocks] of 1 KB (16 rows or columns x 32 K)
    char (*smem)[kStageBytes] = (char (*)[kStageBytes])smem_base;
    const int NT = (g.N + kBigBN - 1) / kBigBN;
    const int total = n_mt * NT;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 8 waves, wave-uniform
    const int wm = wid >> 2, wn = wid & 3;                        // 2 x 4 waves
    const int K = g.K;
    const int nsteps = K / 32;                                    // 32-wide K steps
    const int nt16 = g.N / 16;
    // fragment lane (row l % 16, chunk l / 16) of an activation block
    const int a_off = 16 * (4 * (lane & 15) + ((lane >> 4) ^ a_swz(lane & 15)));

    // contiguous range of tiles for this XCD, strided over its workgroups
    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int chunk = (total + 7) / 8;
    const int t_begin = xcd * chunk;
    const int t_end = min(total, t_begin + chunk);
    for (int tile = t_begin + (blockIdx.x >> 3); tile < t_end; tile += per_xcd) {
        // the tiles of one expert (its m_e row tiles x NT column tiles) keep their
        // index range but are walked column tile by column tile: the expert's
        // row tiles for one column tile run together and share its weight slice
        const int2 te0 = g.tiles_big[tile / NT];
        const int e = te0.x;
        const int base = g.offsets[e], cnt = g.offsets[e + 1] - base;
        const int m_e = (cnt + kBigBM - 1) / kBigBM;
        const int b_e = tile / NT - (te0.y - base) / kBigBM;     // the expert's first row tile
        const int u = tile - b_e * NT;
        const int nt = u / m_e, mi = u - nt * m_e;
        const int row0 = base + mi * kBigBM;
        int rows = cnt - mi * kBigBM;
        if (rows > kBigBM) rows = kBigBM;
        const int n0 = nt * kBigBN;

        // loads: wave w moves the A blocks of row groups 2w, 2w+1 and the B
        // blocks of column groups 2w, 2w+1 of each K step (4 instructions)
        // activation blocks: a quad of lanes fetches one row's 64 bytes (lane i's
        // 16 bytes land at LDS slot i), chunk c of block row r at slot 4 r + (c ^ sw(r))
        const uint16_t* arow[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = lane >> 2;
            int r = 16 * (2 * wid + i) + rr;
            if (r >= rows) r = rows - 1;
            const int row = row0 + r;
            int64_t src_row = row;
            if constexpr (FC1) src_row = g.perm_src[row] / g.topk;
            arow[i] = g.A + src_row * K + 8 * ((lane & 3) ^ a_swz(rr));
        }
        const uint16_t* bblk[2];
        int bstep[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c16 = n0 / 16 + 2 * wid + i;
            if (c16 >= nt16) c16 = nt16 - 1;
            bblk[i] = g.W + ((int64_t)e * nt16 * nsteps + wblock_index(c16, 0, nt16, nsteps)) * 512 + 8 * lane;
            bstep[i] = (int)wblock_step(c16, nt16) * 512;
        }
        auto issue = [&](int s) {
            char* st = smem[s % kRing];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                load_block_to_lds(arow[i] + 32 * s, st + (2 * wid + i) * 1024);
                load_block_to_lds(bblk[i] + (int64_t)bstep[i] * s, st + 16 * 1024 + (2 * wid + i) * 1024);
            }
        };

        f32x4 acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // every wave finished the previous tile's LDS reads before the ring is
        // refilled; a bare barrier (no vmcnt drain) lets the previous tile's
        // output stores overlap the first loads of this tile
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int s = 0; s < kRing - 1; ++s)
            if (s < nsteps) issue(s);
        // the K loop for a wave whose half of the tile holds NG valid 16-row
        // groups: groups wholly past the tile's rows (the last tile of an
        // expert) read no fragments and issue no MFMAs, which frees the SIMD's
        // matrix pipe for the other wave on it; no valid row changes
        auto kloop = [&](auto NGC) {
            constexpr int NG = decltype(NGC)::value;
            for (int s = 0; s < nsteps; ++s) {
                // step s landed when at most the later in-flight steps remain
                const int later = min(kRing - 2, nsteps - 1 - s);
                if (later >= 2) WAIT_VMCNT(8);
                else if (later == 1) WAIT_VMCNT(4);
                else WAIT_VMCNT(0);
                // a bare barrier: each wave has waited for its own loads of step s,
                // and __syncthreads() would also wait for the steps still in flight
                __builtin_amdgcn_s_barrier();
                // refill the slot every wave finished reading in the previous step
                if (s + kRing - 1 < nsteps) issue(s + kRing - 1);
                if constexpr (NG > 0) {
                    const char* As = smem[s % kRing];
                    const char* Bs = As + 16 * 1024;
                    bf16x8 a[NG], b[4];
#pragma unroll
                    for (int i = 0; i < NG; ++i)
                        a[i] = __builtin_bit_cast(bf16x8, *(const uint4*)(As + (8 * wm + i) * 1024 + a_off));
#pragma unroll
                    for (int j = 0; j < 4; ++j) b[j] = lds_frag(Bs + (4 * wn + j) * 1024, lane);
#pragma unroll
                    for (int i = 0; i < NG; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                    // issue all fragment reads before the MFMAs: left alone, the
                    // scheduler reads two A fragments at a time and waits for them
                    // between groups of eight MFMAs (four LDS round trips per step)
                    __builtin_amdgcn_sched_group_barrier(0x100, NG + 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NG, 0);
                }
            }
        };
        const int ngw = min(8, max(0, (rows - 128 * wm + 15) >> 4));
        switch (ngw) {
            case 8: kloop(std::integral_constant<int, 8>{}); break;
            case 7: kloop(std::integral_constant<int, 7>{}); break;
            case 6: kloop(std::integral_constant<int, 6>{}); break;
            case 5: kloop(std::integral_constant<int, 5>{}); break;
            case 4: kloop(std::integral_constant<int, 4>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            default: kloop(std::integral_constant<int, 0>{}); break;
        }

        // epilogue: lane holds rows 4 (lane / 16) + v of each 16-row group, column lane % 16
        const int r16 = lane & 15, kg = lane >> 4;
        const int c0 = n0 + 64 * wn;                 // this wave's 64 columns
        if constexpr (FC1) {
            // one interleave block: tiles 0, 1 gate and 2, 3 up of the same 32 outputs
            const int F = g.N / 2;
            const int cb = c0 / 64;
            uint16_t* hb = (uint16_t*)g.out;
            if (c0 < g.N) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = 128 * wm + 16 * i + 4 * kg + v;
                        if (r < rows) {
                            const int64_t row = row0 + r;
#pragma unroll
                            for (int ct = 0; ct < 2; ++ct) {
                                const float gt = acc[i][ct][v];
                                const float up = acc[i][ct + 2][v];
                                const float h = gt / (1.0f + __expf(-gt)) * up;
                                hb[row * F + cb * 32 + 16 * ct + r16] = f32_to_bf16_bits(h);
                            }
                        }
                    }
            }
        } else {
            float* ob = (float*)g.out;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 128 * wm + 16 * i + 4 * kg + v;
                    if (r < rows) {
                        const int64_t row = row0 + r;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int col = c0 + 16 * j + r16;
                            if (col < g.N) ob[row * g.N + col] = acc[i][j][v];
                        }
                    }
                }
        }
    }
}

}  // namespace moe
