// K3 / K4, bf16, 256-row tiles (experts with more than 128 rows): grouped
// expert GEMMs on CDNA4 MFMA, bf16 operands, fp32 accumulate.
//
// Arithmetic contract shared with the 64-row tiles (gemm_bf16_small.h), which
// makes a row's output independent of the tile that computes it: every output
// element is  acc = 0; for k0 = 0, 16, 32, ... :
// acc = MFMA_32x32x16_bf16(A[row, k0:k0+16], B[col, k0:k0+16], acc).
//
// Decomposition: one workgroup of 8 waves per CU (two per SIMD, so that one
// wave's barrier and memory waits overlap the other's matrix work), a 256 x
// 256 output tile per workgroup, each wave a 128 x 64 part (4 x 2 MFMA blocks
// of 32 x 32; FC1: the 64 columns are one gate/up interleave block).  Operands
// reach LDS by direct global->LDS loads (one wave instruction moves 1 KB)
// through two stages of 64 K each (one computed while the other fills), one
// barrier per stage.  A 64-wide K stage makes every activation load a whole
// 128-byte line (8 lanes per gathered row): the L1 keeps a bounded number of
// line requests in flight, and half-line requests had cut the rate at which a
// CU pulled operands from the L2 by a fifth.
//  * activation stage: 256 rows x 128 bytes, row r's 16-byte chunk c at slot
//    c ^ (r mod 8), which keeps the 8-lane phases of a fragment read on
//    distinct banks;
//  * weight stage: the two 32-wide K steps of the tile's 16 column blocks
//    (1 KB each, 16 columns x 32 K in the lane order of the stored kernel
//    weights; one K step of a 512-column group is contiguous in the buffer).
// Inside a stage a wave computes four 16-wide sub-steps, reading the next
// sub-step's fragments while the current sub-step's 8 MFMAs run.
//
// Epilogue: the wave's results go through LDS (the stage the next tile has not
// yet been given) and leave as 16-byte stores of whole row segments: FC1
// SwiGLU rows as bf16, FC2 rows as fp32.  Stores through buffer descriptors
// that cover exactly the tile's valid rows drop the rows past them.
//
// Tiles: the device-built table of 256-row M tiles x 256-column N tiles, split
// into 8 contiguous ranges, one per XCD (workgroups are dispatched round-robin
// over the XCDs), so the tiles of one expert, which share activation and
// weight slices, run on one XCD and share its L2; within an expert they go
// column tile by column tile, so that all of its row tiles read a weight
// slice at the same time.
#pragma once

#include <type_traits>

#include "gemm_args.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only a vector-memory bound (expcnt and lgkmcnt left at max).
#define BIG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

__device__ __forceinline__ void big_load_block(const void* gsrc, void* lds_dst)
{
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ bf16x8 big_frag(const char* p)
{
    return __builtin_bit_cast(bf16x8, *(const uint4*)p);
}

// chunk permutation of a 64-byte activation row in the 64-row tiles
__device__ __forceinline__ int big_swz(int r) { return (r >> 1) & 3; }

constexpr int kBigTM = 256, kBigTN = 256;
constexpr int kBigKS = 64;                      // K per stage
constexpr int kBigStage = 64 * 1024;            // activations 32 KB | weights 2 x 16 KB
constexpr int kBigWOff = 32 * 1024;             // weight part of a stage
constexpr int kBigALoads = 4, kBigWLoads = 4;   // direct loads per wave per stage
constexpr int kBigLoads = kBigALoads + kBigWLoads;
constexpr int kBigEpi = 8 * 1024;               // a wave's epilogue region (in a stage)

// third dword of a raw buffer descriptor on CDNA (32-bit data format, no
// swizzle, no stride): byte-addressed accesses with a range check on the
// per-lane offset
constexpr int kBigRsrcWord3 = 0x00020000;

// Operand sources of one tile for one wave.  Direct loads go through buffer
// descriptors (wave-uniform); the per-lane offsets are fixed for the tile and
// the K position is a scalar offset, so no address register changes inside
// the K loop.
struct BigSrc {
    __amdgpu_buffer_rsrc_t ar;  // activation rows (FC1: x; FC2: this tile's SwiGLU rows)
    __amdgpu_buffer_rsrc_t wr;  // this expert's weight section
    int aoff[kBigALoads];       // per activation load: the lane's row and chunk at stage 0
    int woff[2];                // the wave's two weight blocks at K step 0 (bytes)
    int wstep;                  // bytes from one 32-wide K step of a weight block to the next
    int nst;                    // stages (K / 64)
    int wid;
};

// the 8 direct loads of stage s into st: activation blocks 4 wid + i (rows
// 32 wid + 8 i + lane / 8), weight blocks 2 wid + i of both K steps
__device__ __forceinline__ void big_issue(const BigSrc& t, char* st, int s)
{
#pragma unroll
    for (int i = 0; i < kBigALoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t.ar, (lds_void_t*)(st + (4 * t.wid + i) * 1024), 16,
                                                 t.aoff[i], 128 * s, 0, 0);
    // the instruction's immediate offset would move the LDS destination too, so
    // the block's place in the weight buffer goes into the scalar offset
    const int lane16 = 16 * (threadIdx.x & 63);
    static_assert(kBigWLoads == 4, "two weight blocks of both K steps");
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                t.wr, (lds_void_t*)(st + kBigWOff + h * 16384 + (2 * t.wid + i) * 1024), 16, lane16,
                t.woff[i] + t.wstep * (2 * s + h), 0, 0);
}

struct BigFrag {
    bf16x8 a[4], b[2];
};

// Lane offsets of the fragments of sub-step q (K 16 q .. 16 q + 15 of a
// stage): A row l % 32 of a 32-row block, 16-byte chunk 2 q + l / 32 (at its
// permuted slot); B column l % 32 of a pair of 16-column blocks, lane
// 16 (2 (q % 2) + l / 32) + l % 16 of its block in K step q / 2.
struct BigLanes {
    int a[4];                   // per q, inside a 32-row block
    int b[2];                   // per q % 2, inside a pair of 16-column blocks
};

// (B first: the MFMAs run row block by row block, so each A fragment is needed
// one MFMA pair after the one before)
template <int Q>
__device__ __forceinline__ void big_read(const char* st, const BigLanes& ln, int wm, int wn, BigFrag& f)
{
#pragma unroll
    for (int j = 0; j < 2; ++j)
        f.b[j] = big_frag(st + kBigWOff + (Q >> 1) * 16384 + (4 * wn + 2 * j) * 1024 + ln.b[Q & 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = big_frag(st + (128 * wm + 32 * i) * 128 + ln.a[Q]);
}

__device__ __forceinline__ void big_mma(f32x16 (&acc)[4][2], const BigFrag& f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// One sub-step: the MFMAs of the fragments in cur, with the 6 fragment reads
// of the next sub-step (sub-step Q of the stage at st, into nxt) placed
// between them, one read after each of the first 6 MFMAs; nothing moves across
// the phase's ends (the compiler otherwise bunched the reads, waited for each
// right away, and sank the stage's direct loads down to the next wait).
template <int Q>
__device__ __forceinline__ void big_phase(f32x16 (&acc)[4][2], const BigFrag& cur, const char* st,
                                          const BigLanes& ln, int wm, int wn, BigFrag& nxt)
{
    big_read<Q>(st, ln, wm, wn, nxt);
    big_mma(acc, cur);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop of a tile.  On entry stage 0 (in s0) and, with two or more
// stages, stage 1 (in s1; the last kBigLoads loads of this wave) are in
// flight.  MMA = false: a wave whose 128 rows all lie past the tile's rows
// only keeps the loads and barriers in step with the others.  Every stage
// boundary inside the loop is unconditional, so that the compiler sees each
// stage's loads waited for before its reads and adds no waits of its own.
template <bool MMA>
__device__ __forceinline__ void big_kloop(const BigSrc& t, char* s0, char* s1, const BigLanes& ln, int wm,
                                          int wn, f32x16 (&acc)[4][2])
{
    const int nst = t.nst;
    BigFrag x, y;
    if (nst > 1) BIG_WAIT_VMCNT(kBigLoads);
    else BIG_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if constexpr (MMA) big_read<0>(s0, ln, wm, wn, x);

    // sub-steps 0 .. 2 of the stage in cur (sub-step 0's fragments in x),
    // reading sub-steps 1 .. 3 (the last into y)
    auto body = [&](const char* cur) {
        if constexpr (MMA) {
            big_phase<1>(acc, x, cur, ln, wm, wn, y);
            big_phase<2>(acc, y, cur, ln, wm, wn, x);
            big_phase<3>(acc, x, cur, ln, wm, wn, y);
        }
    };
    // a stage boundary: this wave's loads of the next stage landed and its
    // reads of the current one are done; after the barrier both hold for every
    // wave, and the current stage's buffer may be refilled
    auto boundary = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        BIG_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // sub-step 3 of the stage before (in y) with sub-step 0 of the stage in nxt read
    auto into = [&](const char* nxt) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MMA) big_phase<0>(acc, y, nxt, ln, wm, wn, x);
    };
    int s = 0;
    for (; s + 2 < nst; s += 2) {
        body(s0);
        boundary();
        big_issue(t, s0, s + 2);
        into(s1);
        body(s1);
        boundary();
        // issued on every path (a load issued on one path only made the
        // compiler wait on all loads in flight before later fragment reads):
        // with an odd number of stages the last pass loads the last stage
        // once more, into s1, which no later fragment read uses (the caller
        // waits for it before s1 serves the epilogue)
        big_issue(t, s1, min(s + 3, nst - 1));
        into(s0);
    }
    // the last one or two stages (already issued)
    body(s0);
    if (s + 1 < nst) {
        boundary();
        into(s1);
        body(s1);
    }
    if constexpr (MMA) big_mma(acc, y);              // the last sub-step
}

// The 256-row tile loop of one 8-wave workgroup (one workgroup per CU).
// n_mt: the number of 256-row M tiles.  Requires K % 64 == 0 (the launch
// sends other shapes to the 64-row kernel).
template <bool FC1, bool PROB>
__device__ __forceinline__ void big_tiles(const GemmArgs& g, int n_mt)
{
    __shared__ __attribute__((aligned(1024))) char lds0[kBigStage];
    __shared__ __attribute__((aligned(1024))) char lds1[kBigStage];
    __shared__ float lds_p[PROB ? kBigTM : 1];

    const int NT = (g.N + kBigTN - 1) / kBigTN;
    const int total = n_mt * NT;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 8 waves, wave-uniform
    const int wm = wid >> 2, wn = wid & 3;                        // 2 x 4 waves of 128 x 64
    const int K = g.K;
    const int ks32 = K / 32;
    const int nt16 = g.N / 16;

    BigSrc t;
    t.nst = K / kBigKS;
    t.wid = wid;
    BigLanes ln;
    {
        const int r = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int q = 0; q < 4; ++q) ln.a[q] = r * 128 + 16 * ((2 * q + hi) ^ (r & 7));
#pragma unroll
        for (int h = 0; h < 2; ++h) ln.b[h] = ((r >> 4) & 1) * 1024 + 16 * (16 * (2 * h + hi) + (r & 15));
    }
    if constexpr (FC1)
        t.ar = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, 0x7fffffff, kBigRsrcWord3);

    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int chunk = (total + 7) / 8;
    const int t_begin = xcd * chunk;
    const int t_end = min(total, t_begin + chunk);

    // A tile's place: its expert, first grouped row, row count and first column.
    struct TilePos { int e, row0, rows, n0; };
    auto locate = [&](int tile) {
        // the tiles of one expert (its m_e row tiles x NT column tiles) keep their
        // index range but are walked column tile by column tile
        const int2 te0 = g.tiles_big[tile / NT];
        const int e = te0.x;
        const int base = g.offsets[e], cnt = g.offsets[e + 1] - base;
        const int m_e = (cnt + kBigTM - 1) / kBigTM;
        const int b_e = tile / NT - (te0.y - base) / kBigTM;     // the expert's first row tile
        const int u = tile - b_e * NT;
        const int nt = u / m_e, mi = u - nt * m_e;
        return TilePos{e, base + mi * kBigTM, min(kBigTM, cnt - mi * kBigTM), nt * kBigTN};
    };
    // activation loads: lane -> row 32 wid + 8 i + lane / 8 (the last valid
    // row past the tile's rows), 16-byte chunk (lane % 8) ^ (row % 8) at LDS
    // slot lane % 8; weight loads: the wave's 16-column blocks 2 wid, 2 wid + 1
    // of the tile (a block past the last column re-reads the last column
    // block, whose columns are never stored; the blocks of a tile lie in one
    // 512-column group, so they share the step distance)
    auto sources = [&](const TilePos& p) {
        if constexpr (!FC1)
            t.ar = __builtin_amdgcn_make_buffer_rsrc((void*)(g.A + (int64_t)p.row0 * K), (short)0,
                                                     0x7fffffff, kBigRsrcWord3);
#pragma unroll
        for (int i = 0; i < kBigALoads; ++i) {
            const int rr = 32 * wid + 8 * i + (lane >> 3);
            int64_t src_row = min(rr, p.rows - 1);
            if constexpr (FC1) src_row = g.perm_src[p.row0 + src_row] / g.topk;
            t.aoff[i] = (int)(src_row * K * 2) + 16 * ((lane & 7) ^ (rr & 7));
        }
        t.wr = __builtin_amdgcn_make_buffer_rsrc((void*)(g.W + (int64_t)p.e * nt16 * ks32 * 512),
                                                 (short)0, nt16 * ks32 * 1024, kBigRsrcWord3);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            t.woff[i] = (int)wblock_index(min(p.n0 / 16 + 2 * wid + i, nt16 - 1), 0, nt16, ks32) * 1024;
        t.wstep = (int)wblock_step(min(p.n0 / 16, nt16 - 1), nt16) * 1024;
    };

    int tile = t_begin + (blockIdx.x >> 3);
    if (tile >= t_end) return;
    TilePos pos = locate(tile);
    sources(pos);
    big_issue(t, lds0, 0);
    if (t.nst > 1) big_issue(t, lds1, 1);
    char* const ep = lds1 + wid * kBigEpi;          // this wave's epilogue region
    while (true) {
        const int row0 = pos.row0, rows = pos.rows, n0 = pos.n0;
        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        const bool active = rows > 128 * wm;        // wave-uniform
        if (active) big_kloop<true>(t, lds0, lds1, ln, wm, wn, acc);
        else big_kloop<false>(t, lds0, lds1, ln, wm, wn, acc);

        // every wave finished reading the stages (and, with an odd number of
        // stages, the K loop's repeated last stage landed in lds1); the next
        // tile's stage 0 goes out before this tile's epilogue, stage 1 after it
        // (the epilogue passes through lds1)
        const int next = tile + per_xcd;
        const bool more = next < t_end;
        if (t.nst & 1) BIG_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        TilePos npos{};
        if (more) {
            npos = locate(next);
            sources(npos);
            big_issue(t, lds0, 0);
        }
        // FC1 with the probabilities applied inside FC1: the tile's row
        // probabilities, staged once for all waves
        if constexpr (FC1 && PROB) {
            if (threadIdx.x < kBigTM) {
                const int r = threadIdx.x;
                lds_p[r] = r < rows ? g.row_prob[g.perm_src[row0 + r]] : 1.0f;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
        }

        // epilogue: lane holds column l % 32 of each 32-column block and rows
        // 8 (v / 4) + 4 (l / 32) + v % 4 of each 32-row block
        if (active) {
            const int hi = lane >> 5, c32 = lane & 31;
            if constexpr (FC1) {
                // interleave block ib: column block 0 the gate half, 1 the up half
                const int F = g.N / 2;
                const int ib = n0 / 64 + wn;
                if (ib * 64 < g.N) {
                    // the wave's 128 x 32 SwiGLU outputs as bf16 rows of 64 bytes in
                    // ep, rows 4 m .. 4 m + 3 with odd m in swapped row pairs (the two
                    // rows a write instruction covers fall in different bank halves)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int rr = 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
                            float h = swiglu_f32(acc[i][0][v], acc[i][1][v]);
                            if constexpr (PROB) h *= lds_p[128 * wm + rr];
                            *(uint16_t*)(ep + ((rr * 64 + 2 * c32) ^ (((rr >> 2) & 1) << 6))) =
                                f32_to_bf16_bits(h);
                        }
                    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                        (void*)((uint16_t*)g.out + (int64_t)row0 * F), (short)0, rows * F * 2, kBigRsrcWord3);
                    const int c = lane & 3;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int rr = (lane >> 2) + 16 * k;
                        const u32x4_t val =
                            *(const u32x4_t*)(ep + ((rr * 64 + 16 * c) ^ (((rr >> 2) & 1) << 6)));
                        __builtin_amdgcn_raw_buffer_store_b128(
                            val, orr, ((128 * wm + rr) * F + ib * 32 + 8 * c) * 2, 0, 0);
                    }
                }
            } else {
                const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)((float*)g.out + (int64_t)row0 * g.N), (short)0, rows * g.N * 4, kBigRsrcWord3);
                const int c = lane & 15;
                const int col = n0 + 64 * wn + 4 * c;   // this lane's 4 stored columns
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // one 32-row block at a time: 32 x 64 fp32 in ep, rows of 256
                    // bytes, halves swapped in rows 4 m .. 4 m + 3 with odd m
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int rr = 8 * (v >> 2) + 4 * hi + (v & 3);
                            *(float*)(ep + ((rr * 256 + 4 * (32 * j + c32)) ^ (((rr >> 2) & 1) << 7))) =
                                acc[i][j][v];
                        }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int rr = (lane >> 4) + 4 * k;
                        const u32x4_t val =
                            *(const u32x4_t*)(ep + ((rr * 256 + 16 * c) ^ (((rr >> 2) & 1) << 7)));
                        if (col < g.N)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                val, orr, ((128 * wm + 32 * i + rr) * g.N + col) * 4, 0, 0);
                    }
                }
            }
        }
        // every wave is done with lds1 before the next tile's stage 1 fills it
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        if (!more) break;
        if (t.nst > 1) big_issue(t, lds1, 1);
        tile = next;
        pos = npos;
    }
}

}  // namespace moe
