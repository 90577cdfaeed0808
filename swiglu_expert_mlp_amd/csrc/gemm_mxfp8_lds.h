// K3 / K4 for MXFP8, LDS-staged design (experts with more than 128 rows): grouped GEMM on the
// CDNA4 block-scaled MFMA (E4M3 x E4M3, one E8M0 scale per 32 elements of K,
// fp32 accumulate).  Used when K is a multiple of 128 (otherwise the streaming
// kernel takes these tiles too; the choice depends on the shape only).
//
// Same arithmetic contract as gemm_mxfp8.hip (and therefore bitwise the same
// results for a row): acc = 0; for k0 = 0, 128, 256, ... :
// acc = MFMA_SCALE_16x16x128_E4M3(A[row, k0:k0+128], B[col, k0:k0+128], acc)
// with the scales of the step's four 32-blocks.
//
// Decomposition: a workgroup computes a 256 x 256 tile of the device-built
// table of 256-row M tiles; each of its 8 waves a 128 x 64 part (8 x 4 MFMA
// blocks).  Everything a K step reads is staged through LDS by direct
// global->LDS loads, double buffered, one wait and one barrier per step (the
// next step's loads run while the current one computes):
//  * activation codes: an instruction moves 8 rows x 128 bytes (a step of a
//    row is one cache line).  In LDS rows are 128 bytes apart and the row's
//    eight 16-byte chunks are permuted, chunk c of tile row r at position
//    c ^ (r mod 8), which keeps the fragment reads (16 rows, one chunk each)
//    free of bank conflicts; the permutation is applied on the global side.
//  * weight codes: the kernel-weight buffer holds 2 KB blocks (16 columns x
//    128 K, two 1 KB halves in MFMA lane order), moved into LDS as they are.
//    W4 (MXFP4 weights, E2M1 B format): 1 KB blocks, half of the B region.
//  * activation scales: the step's 4 scale bytes of each of the 256 rows, one
//    dword per lane (rows are 4-byte aligned because K is a multiple of 128),
//    placed so that the 8 row groups of a fragment lane are 8 consecutive
//    dwords (tile row 128 m + 16 i + r at dword (16 m + r) * 8 + i).
//  * weight scales: the 256-byte group (4 steps of one 16-column block) of
//    the kernel-weight buffer that holds the step, for each column block.
//
// Tiles are split into 8 contiguous ranges, one per XCD (workgroups are
// dispatched round-robin over the XCDs), so the tiles of one expert share an
// L2; within an expert they go column tile by column tile, so that all of its
// row tiles read a weight slice at the same time.
#pragma once

#include <type_traits>

#include "gemm_args.h"

namespace moe {

constexpr int kMxBigBM = 256;
constexpr int kMxBigBN = 256;
// one stage: A codes 32 KB | B codes 32 KB | A scales 1 KB | B scales 4 KB
constexpr int kMxStage = 69 * 1024;
constexpr int kMxAsOff = 64 * 1024, kMxBsOff = 65 * 1024;

typedef __attribute__((address_space(3))) void mx_lds_void;

__device__ __forceinline__ void mx_load_block_to_lds(const void* gsrc, void* lds_dst)
{
    __builtin_amdgcn_global_load_lds(gsrc, (mx_lds_void*)lds_dst, 16, 0, 0);
}

// weight blocks: FC2's with the non-temporal cache policy (measured at 16K
// tokens: FC2 466 -> 447 us; FC1, whose row tiles reuse them through the L2,
// 728 -> 766 us with it, so FC1 keeps the default)
template <bool FC1>
__device__ __forceinline__ void mx_load_wblock_to_lds(const void* gsrc, void* lds_dst)
{
    __builtin_amdgcn_global_load_lds(gsrc, (mx_lds_void*)lds_dst, 16, 0, FC1 ? 0 : kNonTemporal);
}

__device__ __forceinline__ void mx_load_dword_to_lds(const void* gsrc, void* lds_dst)
{
    __builtin_amdgcn_global_load_lds(gsrc, (mx_lds_void*)lds_dst, 4, 0, 0);
}

__device__ __forceinline__ i32x8 mx_frag(uint4 lo, uint4 hi)
{
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

#define MX_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt(0x0F70)

// The LDS-staged tile loop of one 8-wave workgroup (one workgroup per CU).
// Requires K % 128 == 0.
template <bool FC1, bool W4, bool PROB>
__device__ __forceinline__ void mx_lds_tiles(const MxGemmArgs& g)
{
    // the two stages are separate LDS objects, always addressed with
    // compile-time selection (the step loop is unrolled by 2): the compiler
    // can then tell a fragment read from a direct load into the other stage
    // and does not drain the loads in flight
    __shared__ __attribute__((aligned(1024))) char st0[kMxStage];
    __shared__ __attribute__((aligned(1024))) char st1[kMxStage];
    const int n_mt = g.hdr->n_tiles_big;
    const int NT = (g.N + kMxBigBN - 1) / kMxBigBN;
    const int total = n_mt * NT;
    const int lane = threadIdx.x & 63;
    // wave-uniform: scalar registers for everything derived from the wave index
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 8 waves
    const int wm = wid >> 2, wn = wid & 3;                               // 2 x 4 waves
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K, KB = K / 32;
    const int KS = K / 128, KQ = (KS + 3) / 4;
    const int nt16 = g.N / 16;

    // fragment offsets inside a 16-row activation group (2 KB): first and
    // second 16-byte K chunk of the lane's row
    const int a_lo = r16 * 128 + ((kg ^ (r16 & 7)) << 4);
    const int a_hi = r16 * 128 + (((kg + 4) ^ (r16 & 7)) << 4);

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
        const int m_e = (cnt + kMxBigBM - 1) / kMxBigBM;
        const int b_e = tile / NT - (te0.y - base) / kMxBigBM;     // the expert's first row tile
        const int u = tile - b_e * NT;
        const int nt = u / m_e, mi = u - nt * m_e;
        const int row0 = base + mi * kMxBigBM;
        int rows = cnt - mi * kMxBigBM;
        if (rows > kMxBigBM) rows = kMxBigBM;
        const int n0 = nt * kMxBigBN;

        // activation code loads: blocks 4 wid + i (8 rows each); lane -> row
        // 8 j + lane / 8, LDS position lane % 8 <- chunk (lane % 8) ^ (row % 8)
        const uint8_t* aptr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 8 * (4 * wid + i) + (lane >> 3);
            const int r = rr < rows ? rr : rows - 1;
            int64_t src = row0 + r;
            if constexpr (FC1) src = g.perm_src[row0 + r] / g.topk;
            aptr[i] = g.A + src * K + 16 * ((lane & 7) ^ (rr & 7));
        }
        // activation scale loads (waves 0-3): dword q = 64 wid + lane holds tile
        // row 128 (q / 128) + 16 (q % 8) + (q / 8) % 16, 4 bytes per step
        const uint8_t* sptr;
        {
            const int q = 64 * (wid & 3) + lane;
            const int rr = 128 * (q >> 7) + 16 * (q & 7) + ((q >> 3) & 15);
            const int r = rr < rows ? rr : rows - 1;
            int64_t src = row0 + r;
            if constexpr (FC1) src = g.perm_src[row0 + r] / g.topk;
            sptr = g.As + src * KB;
        }
        // weight code and scale loads: column blocks 2 wid + i
        // weight blocks of K step s: MXFP8 [expert][c16][s] (2 KB); MXFP4 in
        // 512-column groups (wblock_index, 1 KB codes / 256-byte scale groups)
        int64_t bblk[2], b4[2], q4[2], w4s[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c16 = n0 / 16 + 2 * wid + i;
            if (c16 >= nt16) c16 = nt16 - 1;
            bblk[i] = (int64_t)e * nt16 + c16;
            b4[i] = (int64_t)e * nt16 * KS + wblock_index(c16, 0, nt16, KS);
            q4[i] = (int64_t)e * nt16 * KQ + wblock_index(c16, 0, nt16, KQ);
            w4s[i] = wblock_step(c16, nt16);
        }
        // loads of step s into stage Q
        auto issue = [&](auto QC, int s) {
            constexpr int Q = decltype(QC)::value;
            char* st = (Q & 1) ? st1 : st0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mx_load_block_to_lds(aptr[i] + 128 * s, st + (4 * wid + i) * 1024);
            if constexpr (W4) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    mx_load_wblock_to_lds<FC1>(g.W + (b4[i] + s * w4s[i]) * 1024 + 16 * lane,
                                         st + 32768 + (2 * wid + i) * 1024);
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        mx_load_wblock_to_lds<FC1>(g.W + (bblk[i] * KS + s) * 2048 + h * 1024 + 16 * lane,
                                             st + 32768 + ((2 * wid + i) * 2 + h) * 1024);
            }
            if (wid < 4) mx_load_dword_to_lds(sptr + 4 * s, st + kMxAsOff + 256 * wid);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                mx_load_dword_to_lds(g.Ws + (W4 ? q4[i] + (s >> 2) * w4s[i] : bblk[i] * KQ + (s >> 2)) * 256 +
                                         4 * lane,
                                     st + kMxBsOff + (2 * wid + i) * 256);
        };

        f32x4 acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // one K step in stage P: wait for its loads (issued one step ago) in
        // every wave, refill the other stage (read by every wave in the
        // previous step), compute
        auto step = [&](auto PC, int s) {
            constexpr int P = decltype(PC)::value;
            MX_WAIT_VMCNT0();
            __builtin_amdgcn_s_barrier();
            const char* As = P ? st1 : st0;
            const char* Bs = As + 32768 + 16 * lane;
            const char* Sa = As + kMxAsOff + (16 * wm + r16) * 32;
            const uint8_t* Sb = (const uint8_t*)As + kMxBsOff + 4 * lane + (s & 3);
            // the weight fragments and all scales are read before the next
            // stage's loads are issued
            i32x8 b[4];
            int sb[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                if constexpr (W4)   // the upper half of an E2M1 operand is not read
                    b[ct] = mx_frag(*(const uint4*)(Bs + (4 * wn + ct) * 1024), make_uint4(0, 0, 0, 0));
                else
                    b[ct] = mx_frag(*(const uint4*)(Bs + (4 * wn + ct) * 2048),
                                    *(const uint4*)(Bs + (4 * wn + ct) * 2048 + 1024));
                sb[ct] = Sb[(4 * wn + ct) * 256];
            }
            const uint4 sa_lo = *(const uint4*)Sa, sa_hi = *(const uint4*)(Sa + 16);
            if (s + 1 < KS) issue(std::integral_constant<int, P ^ 1>{}, s + 1);
            const uint32_t sad[8] = {sa_lo.x, sa_lo.y, sa_lo.z, sa_lo.w,
                                     sa_hi.x, sa_hi.y, sa_hi.z, sa_hi.w};
            // FC1: activation fragments in four groups of two, each group's reads
            // issued while the previous group's MFMAs run; the explicit
            // lgkmcnt(0) before a group's reads is what tells the compiler that
            // the previous group has landed (after the direct loads above it
            // would otherwise wait for every LDS read before each MFMA)
            i32x8 af[2][2];
            auto read_group = [&](int gr, i32x8 (&dst)[2]) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const char* ag = As + (8 * wm + 2 * gr + q) * 2048;
                    dst[q] = mx_frag(*(const uint4*)(ag + a_lo), *(const uint4*)(ag + a_hi));
                }
            };
            auto mfma_group = [&](int gr, const i32x8 (&src)[2]) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int i = 2 * gr + q;
                    const int sa = (int)((sad[i] >> (8 * kg)) & 0xffu);
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        // A format 0 (E4M3); B format 0 (E4M3) or 4 (E2M1)
                        acc[i][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            src[q], b[ct], acc[i][ct], 0, W4 ? 4 : 0, 0, sa, 0, sb[ct]);
                }
            };
            if constexpr (FC1) {
                read_group(0, af[0]);
#pragma unroll
                for (int gr = 0; gr < 4; ++gr) {
                    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): group gr is in
                    if (gr + 1 < 4) read_group(gr + 1, af[(gr + 1) & 1]);
                    mfma_group(gr, af[gr & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // FC2 is bound by its loads and output stores; the grouped reads
                // only added register spills there
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const char* ag = As + (8 * wm + i) * 2048;
                    const i32x8 a = mx_frag(*(const uint4*)(ag + a_lo), *(const uint4*)(ag + a_hi));
                    const int sa = (int)((sad[i] >> (8 * kg)) & 0xffu);
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[i][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a, b[ct], acc[i][ct], 0, W4 ? 4 : 0, 0, sa, 0, sb[ct]);
                }
            }
        };

        // every wave finished the previous tile's LDS reads before the stages refill
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        issue(std::integral_constant<int, 0>{}, 0);
        for (int s2 = 0; s2 < KS; s2 += 2) {
            step(std::integral_constant<int, 0>{}, s2);
            if (s2 + 1 < KS) step(std::integral_constant<int, 1>{}, s2 + 1);
        }

        // epilogue: lane holds rows 4 (lane / 16) + v of each 16-row group, column lane % 16
        const int c0 = n0 + 64 * wn;                 // this wave's 64 columns
        if constexpr (FC1) {
            // SwiGLU of one interleave block (tiles 0, 1 gate and 2, 3 up of the
            // same 32 outputs), then the per-32 requantization of each row's 32
            // outputs, held by the 16 lanes of one lane group
            const int F = g.N / 2, FB = F / 32;
            const int cb = c0 / 64;
            uint8_t* hq = (uint8_t*)g.out;
            if (c0 < g.N) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = 128 * wm + 16 * i + 4 * kg + v;
                        // the 16 lanes of one requantization block hold one row: one probability
                        const float pr = (PROB && r < rows) ? fc1_row_prob(g.row_prob, g.perm_src, row0 + r) : 1.0f;
                        float gt = acc[i][0][v], up = acc[i][2][v];
                        const float h0 = gt / (1.0f + __expf(-gt)) * up * pr;
                        gt = acc[i][1][v]; up = acc[i][3][v];
                        const float h1 = gt / (1.0f + __expf(-gt)) * up * pr;
                        float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                        for (int off = 1; off < 16; off <<= 1)
                            amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
                        const int e8 = e8m0_exponent(amax);
                        const float inv = e8 == 127 ? __uint_as_float(1u << 22)
                                                    : __uint_as_float((uint32_t)(127 - e8) << 23);
                        if (r < rows) {
                            const int64_t row = row0 + r;
                            const uint32_t c2 = cvt_e4m3x2(h0 * inv, h1 * inv);
                            hq[row * F + cb * 32 + r16] = (uint8_t)c2;
                            hq[row * F + cb * 32 + 16 + r16] = (uint8_t)(c2 >> 8);
                            if (r16 == 0) g.out_scale[row * FB + cb] = (uint8_t)(e8 + 127);
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
