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
constexpr int kBigEpi = 4 * 1024;               // a wave's epilogue region (LDS of its own)
constexpr int kBigPOff = 2 * 1024;              // FC1: the wave's row probabilities in it
// 16-byte stores per wave per tile (FC1: 128 rows x 32 bf16; FC2: 128 rows x
// 64 fp32); every wave issues exactly this many, and the next K loop counts them
template <bool FC1>
constexpr int big_stores() { return FC1 ? 8 : 32; }

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
// 32 wid + 8 i + lane / 8), weight blocks 2 wid + i of both K steps.  WPOL:
// the weights' cache policy (FC2: non-temporal, measured 686 -> 664 us at
// 16K tokens; FC1: default, which its row tiles' L2 reuse needs, 989 -> 1049
// us with non-temporal)
template <int WPOL>
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
                t.woff[i] + t.wstep * (2 * s + h), 0, WPOL);
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

// The K loop of a tile (two or more stages).  On entry this wave's loads of
// stage 0 (into s0) and stage 1 (into s1) are in flight, followed by AFTER
// further vector-memory operations (the previous tile's stores, which may
// drain while this tile runs).  Every load issue is unconditional (a load
// issued on one path only made the compiler wait on all loads in flight before
// later fragment reads): where no stage is left to load, the last stage is
// loaded once more into s0, which no later fragment read of the tile uses.
template <int AFTER, int WPOL>
__device__ __forceinline__ void big_kloop(const BigSrc& t, char* s0, char* s1, const BigLanes& ln, int wm,
                                          int wn, f32x16 (&acc)[4][2])
{
    static_assert(AFTER + kBigLoads <= 63, "vmcnt bound");
    const int nst = t.nst;                           // >= 2
    BigFrag x, y;
    // both stages landed (waiting for stage 0 alone made the compiler add a
    // wait for everything in flight before the first fragment reads)
    BIG_WAIT_VMCNT(AFTER);
    __builtin_amdgcn_s_barrier();
    big_read<0>(s0, ln, wm, wn, x);

    // sub-steps 0 .. 2 of the stage in cur (sub-step 0's fragments in x),
    // reading sub-steps 1 .. 3 (the last into y)
    auto body = [&](const char* cur) {
        big_phase<1>(acc, x, cur, ln, wm, wn, y);
        big_phase<2>(acc, y, cur, ln, wm, wn, x);
        big_phase<3>(acc, x, cur, ln, wm, wn, y);
    };
    // a stage boundary: this wave's loads of the next stage landed (N: the
    // vector-memory operations issued after them) and its reads of the current
    // one are done; after the barrier both hold for every wave, and the current
    // stage's buffer may be refilled
    auto boundary = [&](auto NC) {
        constexpr int N = decltype(NC)::value;
        __builtin_amdgcn_sched_barrier(0);
        BIG_WAIT_VMCNT(N);
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // sub-step 3 of the stage before (in y) with sub-step 0 of the stage in nxt read
    auto into = [&](const char* nxt) {
        __builtin_amdgcn_sched_barrier(0);
        big_phase<0>(acc, y, nxt, ln, wm, wn, x);
    };
    using Now = std::integral_constant<int, 0>;
    // stage 0 (stage 1 has landed too)
    body(s0);
    boundary(std::integral_constant<int, AFTER>{});
    big_issue<WPOL>(t, s0, min(2, nst - 1));
    into(s1);
    int s = 1;
    // stage s in s1, stage s + 1 (if any) in flight into s0
    for (; s + 2 < nst; s += 2) {
        body(s1);
        boundary(Now{});
        big_issue<WPOL>(t, s1, s + 2);
        into(s0);
        body(s0);
        boundary(Now{});
        big_issue<WPOL>(t, s0, min(s + 3, nst - 1));
        into(s1);
    }
    body(s1);
    if (s + 1 < nst) {
        boundary(Now{});
        into(s0);
        body(s0);
    }
    big_mma(acc, y);                                 // the last sub-step
}

// The 256-row tile loop of one 8-wave workgroup (one workgroup per CU).
// n_mt: the number of 256-row M tiles.  Requires K % 64 == 0 and K >= 128
// (the launch sends other shapes to the 64-row kernel).
template <bool FC1, bool PROB>
__device__ __forceinline__ void big_tiles(const GemmArgs& g, int n_mt)
{
    __shared__ __attribute__((aligned(1024))) char lds0[kBigStage];
    __shared__ __attribute__((aligned(1024))) char lds1[kBigStage];
    __shared__ __attribute__((aligned(1024))) char lds_x[8 * kBigEpi];   // the waves' epilogue regions

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
    constexpr int kWPol = FC1 ? 0 : kNonTemporal;
    big_issue<kWPol>(t, lds0, 0);
    big_issue<kWPol>(t, lds1, 1);
    // the K loop counts the previous tile's stores among the operations after
    // its first stages; before the first tile the same number of stores go to
    // an empty descriptor (the range check drops them all; distinct offsets, so
    // that none is merged away)
    constexpr int kStores = big_stores<FC1>();
    {
        const __amdgpu_buffer_rsrc_t none =
            __builtin_amdgcn_make_buffer_rsrc(g.out, (short)0, 0, kBigRsrcWord3);
#pragma unroll
        for (int k = 0; k < kStores; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, none, 16 * lane + 1024 * k, 0, 0);
    }
    char* const ep = lds_x + wid * kBigEpi;         // this wave's epilogue region
    while (true) {
        const int row0 = pos.row0, rows = pos.rows, n0 = pos.n0;
        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // every wave runs the same K loop, also one whose 128 rows all lie past
        // the tile's rows (its results are dropped by the store descriptor): a
        // second, load-only loop for such waves made the compiler wait for all
        // loads and stores in flight at every tile's first fragment reads
        big_kloop<kStores, kWPol>(t, lds0, lds1, ln, wm, wn, acc);

        // every wave finished reading the stages: the next tile's two stages go
        // out before this tile's epilogue (which has LDS of its own), so they
        // land while it runs, and its stores drain while the next tile runs.
        // The loads go out on every path (after the last tile they load its
        // first stages again, waited for before the exit): a load issued on one
        // path only made the compiler wait on all loads in flight before the
        // next K loop's first fragment reads.
        const int next = tile + per_xcd;
        const bool more = next < t_end;
        __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        // FC1 with the probabilities applied inside FC1: the wave's 128 row
        // probabilities, fetched before the loads below so that waiting for
        // them does not wait for those
        float pr0 = 1.0f, pr1 = 1.0f;
        if constexpr (FC1 && PROB) {
            const int r0 = 128 * wm + lane, r1 = r0 + 64;
            if (r0 < rows) pr0 = g.row_prob[g.perm_src[row0 + r0]];
            if (r1 < rows) pr1 = g.row_prob[g.perm_src[row0 + r1]];
        }
        TilePos npos = pos;
        if (more) {
            npos = locate(next);
            sources(npos);
        }
        big_issue<kWPol>(t, lds0, 0);
        big_issue<kWPol>(t, lds1, 1);

        // epilogue: lane holds column l % 32 of each 32-column block and rows
        // 8 (v / 4) + 4 (l / 32) + v % 4 of each 32-row block.  The lane index
        // goes through an opaque copy so that the compiler derives the epilogue's
        // many per-lane offsets here instead of hoisting them out of the tile
        // loop (they would stay live across the K loop and spill).  Every wave
        // issues exactly kStores stores: rows past the tile's rows (all of an
        // idle wave's) fall outside the store descriptor, and columns past N get
        // an offset outside it.
        int elane = lane;
        asm volatile("" : "+v"(elane));
        const int hi = elane >> 5, c32 = elane & 31;
        if constexpr (FC1) {
            // interleave block ib: column block 0 the gate half, 1 the up half;
            // one 32-row block at a time as bf16 rows of 64 bytes in ep, rows
            // 4 m .. 4 m + 3 with odd m in swapped row pairs (the two rows a write
            // instruction covers fall in different bank halves)
            const int F = g.N / 2;
            const int ib = n0 / 64 + wn;
            const bool cols = ib * 64 < g.N;
            const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((uint16_t*)g.out + (int64_t)row0 * F), (short)0, rows * F * 2, kBigRsrcWord3);
            const float* pw = (const float*)(ep + kBigPOff);
            if constexpr (PROB) {
                ((float*)(ep + kBigPOff))[elane] = pr0;
                ((float*)(ep + kBigPOff))[elane + 64] = pr1;
            }
            const int c = elane & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rr = 8 * (v >> 2) + 4 * hi + (v & 3);
                    float h = swiglu_f32(acc[i][0][v], acc[i][1][v]);
                    if constexpr (PROB) h *= pw[32 * i + rr];
                    // (the offset through an opaque copy: a 16-bit LDS store whose
                    // constant part the compiler folds into the instruction made
                    // it wait for the next tile's direct loads first)
                    int ea = (rr * 64 + 2 * c32) ^ (((rr >> 2) & 1) << 6);
                    asm volatile("" : "+v"(ea));
                    *(uint16_t*)(ep + ea) = f32_to_bf16_bits(h);
                }
                static_assert(big_stores<true>() == 4 * 2, "4 row blocks x 2 stores");
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int rr = (elane >> 2) + 16 * k;
                    const u32x4_t val = *(const u32x4_t*)(ep + ((rr * 64 + 16 * c) ^ (((rr >> 2) & 1) << 6)));
                    const int off = cols ? ((128 * wm + 32 * i + rr) * F + ib * 32 + 8 * c) * 2 : 0x7ffffff0;
                    __builtin_amdgcn_raw_buffer_store_b128(val, orr, off, 0, 0);
                }
            }
        } else {
            const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((float*)g.out + (int64_t)row0 * g.N), (short)0, rows * g.N * 4, kBigRsrcWord3);
            const int c = elane & 15;
            const int col = n0 + 64 * wn + 4 * c;       // this lane's 4 stored columns
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    // 16 rows (v in 8 hv .. 8 hv + 7) x 64 fp32 in ep, rows of 256
                    // bytes, halves swapped in rows 4 m .. 4 m + 3 with odd m
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 8 * hv; v < 8 * hv + 8; ++v) {
                            const int lr = 8 * ((v >> 2) & 1) + 4 * hi + (v & 3);
                            *(float*)(ep + ((lr * 256 + 4 * (32 * j + c32)) ^ (((lr >> 2) & 1) << 7))) =
                                acc[i][j][v];
                        }
                    static_assert(big_stores<false>() == 4 * 2 * 4, "4 row blocks x 2 halves x 4 stores");
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int lr = (elane >> 4) + 4 * k;
                        const u32x4_t val =
                            *(const u32x4_t*)(ep + ((lr * 256 + 16 * c) ^ (((lr >> 2) & 1) << 7)));
                        const int off = col < g.N ? ((128 * wm + 32 * i + 16 * hv + lr) * g.N + col) * 4
                                                  : 0x7ffffff0;
                        __builtin_amdgcn_raw_buffer_store_b128(val, orr, off, 0, 0);
                    }
                }
        }
        if (!more) {
            BIG_WAIT_VMCNT(0);          // the repeated loads land before the LDS is released
            break;
        }
        tile = next;
        pos = npos;
    }
}

}  // namespace moe
