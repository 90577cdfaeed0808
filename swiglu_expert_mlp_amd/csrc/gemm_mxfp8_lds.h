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
//  * activation scales: in chunks of 8 K steps (a row's 32 scale bytes, one
//    16-byte load per lane, row r at r * 32), double buffered beside the
//    stages; a chunk is loaded while the one before it is in use.  (A 4-byte
//    load of every row at every step had each step request 256 cache lines
//    for 1 KB of scales: 55 us of a 630 us FC1 at 16K tokens.)
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
// one stage: A codes 32 KB | B codes 32 KB | B scales 4 KB
constexpr int kMxStage = 68 * 1024;
constexpr int kMxBsOff = 64 * 1024;
// activation scales: two 8 KB chunk buffers (256 rows x 32 bytes) and a 1 KB
// landing area for the scale loads of the steps that start no chunk
constexpr int kMxScChunk = 8 * 1024;
constexpr int kMxScBytes = 2 * kMxScChunk + 1024;

typedef __attribute__((address_space(3))) void mx_lds_void;

__device__ __forceinline__ i32x8 mx_frag(uint4 lo, uint4 hi)
{
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// s_waitcnt with only a vector-memory bound (expcnt and lgkmcnt left at max)
#define MX_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

typedef unsigned mx_u32x4 __attribute__((ext_vector_type(4)));

// third dword of a raw buffer descriptor (32-bit format, no swizzle or
// stride): byte-addressed stores with a range check on the offset, which
// drops the rows past a tile's valid rows
constexpr int kMxRsrcWord3 = 0x00020000;

// Epilogue (after the K loop; the second stage's LDS holds no operands then).
// FC1: the tile's 256 rows x 128 code bytes, row r's four 32-byte segments
// (one per wave column, one interleave block each) at slot wn ^ ((r / 4) mod 4),
// which spreads the rows one write instruction covers over the banks; inside
// a segment the code pair (column q, column 16 + q) at bytes 2 q, 2 q + 1.
// The waves' row probabilities (PROB) after the codes.
constexpr int kMxEpiProb = 32 * 1024;
// FC2: 8 KB per wave (32 rows x 64 fp32 at a time).
constexpr int kMxEpiWave = 8 * 1024;
static_assert(kMxEpiProb + 8 * 512 <= kMxStage && 8 * kMxEpiWave <= kMxStage, "epilogue fits a stage");
// stores per wave per tile (every wave issues exactly these; the next tile's
// first wait lets them drain while its first stage is already in)
template <bool FC1>
constexpr int mx_stores() { return FC1 ? 4 + 2 : 32; }

// The lane index computed afresh (mbcnt, in a volatile asm statement, which
// the compiler neither hoists nor merges): values derived from it are not
// hoisted out of the tile loop, where they would outlive the K loop and spill
// (a spill reload waits for every load in flight).
__device__ __forceinline__ int mx_lane_fresh()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

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
    __shared__ __attribute__((aligned(1024))) char scl[kMxScBytes];
    const int n_mt = g.hdr->n_tiles_big;
    const int NT = (g.N + kMxBigBN - 1) / kMxBigBN;
    const int total = n_mt * NT;
    const int lane = threadIdx.x & 63;
    // wave-uniform: scalar registers for everything derived from the wave index
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 8 waves
    const int wm = wid >> 2, wn = wid & 3;                               // 2 x 4 waves
    const int K = g.K, KB = K / 32;
    const int KS = K / 128, KQ = (KS + 3) / 4;
    const int nt16 = g.N / 16;


    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int chunk = (total + 7) / 8;
    const int t_begin = xcd * chunk;
    const int t_end = min(total, t_begin + chunk);
    int tile = t_begin + (blockIdx.x >> 3);
    if (tile >= t_end) return;

    // A tile's place: its expert, first grouped row, row count and first column.
    struct MxPos { int e, row0, rows, n0; };
    auto locate = [&](int t) {
        // the tiles of one expert (its m_e row tiles x NT column tiles) keep their
        // index range but are walked column tile by column tile: the expert's
        // row tiles for one column tile run together and share its weight slice
        const int2 te0 = g.tiles_big[t / NT];
        const int e = te0.x;
        const int base = g.offsets[e], cnt = g.offsets[e + 1] - base;
        const int m_e = (cnt + kMxBigBM - 1) / kMxBigBM;
        const int b_e = t / NT - (te0.y - base) / kMxBigBM;     // the expert's first row tile
        const int u = t - b_e * NT;
        const int nt = u / m_e, mi = u - nt * m_e;
        return MxPos{e, base + mi * kMxBigBM, min(kMxBigBM, cnt - mi * kMxBigBM), nt * kMxBigBN};
    };

    // Operand sources of one tile.  Direct loads go through buffer descriptors
    // (wave-uniform); the per-lane offsets are fixed for the tile and the K
    // step is a scalar offset, so no address register changes inside the K
    // loop (the instruction's immediate offset would move the LDS destination
    // too, so it stays 0).
    __amdgpu_buffer_rsrc_t ar, asr, wr, wsr;
    int aoff[4], soff;           // per lane: activation rows (codes; scales of row (64 wid + lane) / 2)
    int woff[2], wstep[2];       // the wave's two weight column blocks: K step 0, bytes per K step
    int qoff[2], qstep[2];       // their scale groups: step 0, bytes per 4 steps
    const __amdgpu_buffer_rsrc_t anone = __builtin_amdgcn_make_buffer_rsrc(g.out, (short)0, 0, kMxRsrcWord3);
    auto sources = [&](const MxPos& p) {
        const int lane = mx_lane_fresh();
        // activation code loads: blocks 4 wid + i (8 rows each); lane -> row
        // 8 j + lane / 8, LDS position lane % 8 <- chunk (lane % 8) ^ (row % 8);
        // activation scale loads: thread 64 wid + lane loads half lane % 2 of
        // tile row (64 wid + lane) / 2's chunk (16 of its 32 bytes).  FC1
        // gathers the rows: all five row lookups go out before any is used (one
        // round trip, not five).
        const int64_t abase = FC1 ? 0 : (int64_t)p.row0;
        ar = __builtin_amdgcn_make_buffer_rsrc((void*)(g.A + abase * K), (short)0, 0x7fffffff, kMxRsrcWord3);
        // the scale range ends exactly at the scale tensor's end: the last
        // chunk of a row whose K is not a multiple of 8 steps reads on into the
        // next row (never used), and past the last row the range check drops it
        const int64_t sc_left = g.a_bytes / 32 - abase * KB;
        asr = __builtin_amdgcn_make_buffer_rsrc((void*)(g.As + abase * KB), (short)0,
                                                (int)(sc_left < 0x7fffffff ? sc_left : 0x7fffffff), kMxRsrcWord3);
        int src[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            int rr;
            if (i < 4) {
                rr = 8 * (4 * wid + i) + (lane >> 3);
            } else {
                rr = (64 * wid + lane) >> 1;
            }
            src[i] = rr < p.rows ? rr : p.rows - 1;
            if constexpr (FC1) src[i] = g.perm_src[p.row0 + src[i]];
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            if constexpr (FC1) src[i] /= g.topk;
            if (i < 4) {
                const int rr = 8 * (4 * wid + i) + (lane >> 3);
                aoff[i] = src[i] * K + 16 * ((lane & 7) ^ (rr & 7));
            } else {
                soff = src[i] * KB + 16 * (lane & 1);
            }
        }
        // weight code and scale loads: column blocks 2 wid + i of the expert's
        // section; codes MXFP8 [c16][s] (2 KB blocks), MXFP4 in 512-column
        // groups (wblock_index, 1 KB blocks); scales in 256-byte groups of 4 steps
        wr = __builtin_amdgcn_make_buffer_rsrc((void*)(g.W + (int64_t)p.e * nt16 * KS * (W4 ? 1024 : 2048)),
                                               (short)0, 0x7fffffff, kMxRsrcWord3);
        wsr = __builtin_amdgcn_make_buffer_rsrc((void*)(g.Ws + (int64_t)p.e * nt16 * KQ * 256), (short)0,
                                                0x7fffffff, kMxRsrcWord3);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c16 = p.n0 / 16 + 2 * wid + i;
            if (c16 >= nt16) c16 = nt16 - 1;
            if constexpr (W4) {
                woff[i] = (int)wblock_index(c16, 0, nt16, KS) * 1024;
                wstep[i] = (int)wblock_step(c16, nt16) * 1024;
                qoff[i] = (int)wblock_index(c16, 0, nt16, KQ) * 256;
                qstep[i] = (int)wblock_step(c16, nt16) * 256;
            } else {
                woff[i] = c16 * KS * 2048;
                wstep[i] = 2048;
                qoff[i] = c16 * KQ * 256;
                qstep[i] = 256;
            }
        }
    };
    // loads of step s into stage Q (fl: the lane index)
    auto issue = [&](auto QC, int s, int fl) {
        constexpr int Q = decltype(QC)::value;
        const int lane16 = 16 * fl, lane4 = 4 * fl;
        char* st = (Q & 1) ? st1 : st0;
        // the weights' cache policy: FC2's non-temporal (measured at 16K tokens:
        // FC2 466 -> 447 us); FC1, whose row tiles reuse a weight slice through
        // the L2, keeps the default (728 -> 766 us with non-temporal loads)
        constexpr int wpol = FC1 ? 0 : kNonTemporal;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (mx_lds_void*)(st + (4 * wid + i) * 1024), 16, aoff[i],
                                                     128 * s, 0, 0);
        if constexpr (W4) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (mx_lds_void*)(st + 32768 + (2 * wid + i) * 1024), 16,
                                                         lane16, woff[i] + s * wstep[i], 0, wpol);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        wr, (mx_lds_void*)(st + 32768 + ((2 * wid + i) * 2 + h) * 1024), 16, lane16,
                        woff[i] + s * 2048 + h * 1024, 0, wpol);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wsr, (mx_lds_void*)(st + kMxBsOff + (2 * wid + i) * 256), 4,
                                                     lane4, qoff[i] + (s >> 2) * qstep[i], 0, 0);
    };
    // the activation-scale load of K step s: chunk c = s / 8 + 1 (into buffer
    // c mod 2) when s starts chunk s / 8 and chunk c exists; otherwise the
    // same load through an empty descriptor (the range check drops it) into
    // the landing area.  No branch: a branch around it made the compiler
    // wait for the previous tile's stores before the first step's fragment
    // reads, and this form measured no slower.  The destination stays inside
    // one LDS object, its offset through an opaque copy (as a choice between
    // two pointers the compiler can no longer tell it apart from the stages
    // and waits for every direct load before any later LDS access).  The
    // tile's first chunk goes out with its first stage.
    const int nch = (KS + 7) >> 3;
    auto issue_scales = [&](bool first, int s) {
        const int c = first ? 0 : (s >> 3) + 1;
        const bool real = first || ((s & 7) == 0 && c < nch);
        int dst = real ? (c & 1) * kMxScChunk + 1024 * wid : 2 * kMxScChunk;
        asm volatile("" : "+s"(dst));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(real ? asr : anone, (mx_lds_void*)(scl + dst), 16, soff, 32 * c,
                                                 0, 0);
    };

    f32x4 acc[8][4];
    int kst = KS;       // the step count, re-derived per tile (see the tile loop)

    // one K step in stage P: wait for its loads (issued one step ago; before a
    // tile's first step, the AFTER stores of the previous tile's epilogue came
    // after them) in every wave, refill the other stage (read by every wave in
    // the previous step), compute
    auto step = [&](auto PC, auto AC, int s) {
        constexpr int P = decltype(PC)::value;
        constexpr int AFTER = decltype(AC)::value;
        MX_WAIT_VMCNT(AFTER);
        __builtin_amdgcn_s_barrier();
        // per-lane offsets from a fresh lane index (kept across the steps they
        // would take registers the K loop needs)
        const int fl = mx_lane_fresh();
        const int r16 = fl & 15, kg = fl >> 4;
        // fragment offsets inside a 16-row activation group (2 KB): first and
        // second 16-byte K chunk of the lane's row
        const int a_lo = r16 * 128 + ((kg ^ (r16 & 7)) << 4);
        const int a_hi = r16 * 128 + (((kg + 4) ^ (r16 & 7)) << 4);
        const char* As = P ? st1 : st0;
        const char* Bs = As + 32768 + 16 * fl;
        const char* Sa = scl + ((s >> 3) & 1) * kMxScChunk + (128 * wm + r16) * 32 + (s & 7) * 4;
        const uint8_t* Sb = (const uint8_t*)As + kMxBsOff + 4 * fl + (s & 3);
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
        uint32_t sad[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sad[i] = *(const uint32_t*)(Sa + 512 * i);   // tile row + 16 i
        if (s + 1 < kst) issue(std::integral_constant<int, P ^ 1>{}, s + 1, fl);
        issue_scales(false, s);
        // activation fragments in four groups of two, each group's reads
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
        read_group(0, af[0]);
#pragma unroll
        for (int gr = 0; gr < 4; ++gr) {
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): group gr is in
            if (gr + 1 < 4) read_group(gr + 1, af[(gr + 1) & 1]);
            mfma_group(gr, af[gr & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    MxPos pos = locate(tile);
    sources(pos);
    issue(std::integral_constant<int, 0>{}, 0, lane);
    issue_scales(true, 0);
    // the first tile's first wait counts the previous epilogue's stores too:
    // before the first tile the same number of stores go to an empty
    // descriptor (the range check drops them; distinct offsets, so that none
    // is merged away)
    constexpr int kStores = mx_stores<FC1>();
    static_assert(kStores + 16 <= 63, "vmcnt bound");
    {
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(g.out, (short)0, 0, kMxRsrcWord3);
#pragma unroll
        for (int k = 0; k < kStores; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(mx_u32x4{0u, 0u, 0u, 0u}, none, 16 * lane + 1024 * k, 0, 0);
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    while (true) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // an opaque copy: the compiler otherwise hoists the steps' loop-invariant
        // conditions out of the tile loop, where they outlive everything and spill
        kst = KS;
        asm volatile("" : "+s"(kst));
        step(I0{}, std::integral_constant<int, kStores>{}, 0);
        for (int s2 = 1; s2 < kst; s2 += 2) {
            step(I1{}, I0{}, s2);
            if (s2 + 1 < kst) step(I0{}, I0{}, s2 + 1);
        }

        // every wave finished its fragment reads of both stages: the next
        // tile's first stage goes out before this tile's epilogue, which works
        // in the second stage's LDS, so it lands while the epilogue runs, and
        // the epilogue's stores drain while the next tile's first step runs.
        // The load goes out on every path (after the last tile it loads that
        // tile's first stage again, waited for before the exit): a load issued
        // on one path only makes the compiler wait on every load in flight.
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        const int next = tile + per_xcd;
        const bool more = next < t_end;
        const int row0 = pos.row0, rows = pos.rows, n0 = pos.n0;
        // FC1 with the probabilities applied inside FC1: the wave's 128 row
        // probabilities, fetched before the loads below so that waiting for
        // them does not wait for those
        float pr0 = 1.0f, pr1 = 1.0f;
        if constexpr (FC1 && PROB) {
            const int r0 = 128 * wm + lane, r1 = r0 + 64;
            if (r0 < rows) pr0 = fc1_row_prob(g.row_prob, g.perm_src, row0 + r0);
            if (r1 < rows) pr1 = fc1_row_prob(g.row_prob, g.perm_src, row0 + r1);
        }
        if (more) {
            pos = locate(next);
            sources(pos);
        }
        issue(I0{}, 0, mx_lane_fresh());
        issue_scales(true, 0);
        __builtin_amdgcn_sched_barrier(0);

        // epilogue: lane holds rows 16 i + 4 (lane / 16) + v of the wave's 128
        // rows, column 16 j + lane % 16 of its 64 columns (per-lane offsets from
        // a fresh lane index, derived here).
        const int elane = mx_lane_fresh();
        const int er16 = elane & 15, ekg = elane >> 4;
        const int c0 = n0 + 64 * wn;                 // this wave's 64 columns
        if constexpr (FC1) {
            // SwiGLU of one interleave block (tiles 0, 1 gate and 2, 3 up of the
            // same 32 outputs), then the per-32 requantization of each row's 32
            // outputs, held by the 16 lanes of one lane group
            const int F = g.N / 2, FB = F / 32;
            const int cb0 = n0 / 64;                 // the tile's first interleave block
            float* const xpr = (float*)(st1 + kMxEpiProb) + 128 * wid;
            if constexpr (PROB) {
                xpr[elane] = pr0;
                xpr[elane + 64] = pr1;
            }
            // scale bytes: after the loop, lane (q, kg) keeps the scale of row
            // 16 (4 h + q / 4) + 4 kg + q % 4 in sc[h]
            uint32_t sc[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 16 * i + 4 * ekg + v;
                    const float pr = PROB ? xpr[lr] : 1.0f;
                    float gt = acc[i][0][v], up = acc[i][2][v];
                    const float h0 = swiglu_f32(gt, up) * pr;
                    gt = acc[i][1][v]; up = acc[i][3][v];
                    const float h1 = swiglu_f32(gt, up) * pr;
                    const float amax = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
                    const int e8 = e8m0_exponent(amax);
                    const float inv = e8 == 127 ? __uint_as_float(1u << 22)
                                                : __uint_as_float((uint32_t)(127 - e8) << 23);
                    int ea = (128 * wm + lr) * 128 + 32 * (wn ^ ekg) + 2 * er16;
                    asm volatile("" : "+v"(ea));
                    *(uint16_t*)(st1 + ea) = (uint16_t)cvt_e4m3x2(h0 * inv, h1 * inv);
                    if (er16 == 4 * (i & 3) + v) sc[i >> 2] = (uint32_t)(e8 + 127);
                    __builtin_amdgcn_sched_barrier(0);
                }
            // scale bytes [row][F / 32]: one per row and interleave block
            {
                const __amdgpu_buffer_rsrc_t srr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(g.out_scale + (int64_t)row0 * FB), (short)0, rows * FB, kMxRsrcWord3);
                const bool cols = c0 < g.N;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 128 * wm + 16 * (4 * h + (er16 >> 2)) + 4 * ekg + (er16 & 3);
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc[h], srr,
                                                         cols ? r * FB + cb0 + wn : 0x7ffffff0, 0, 0);
                }
            }
            // codes: every wave's segments are in; a thread takes two (row,
            // segment) items and stores each as two 16-byte pieces (the
            // segment's even bytes are columns 0 .. 15, its odd bytes 16 .. 31)
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((uint8_t*)g.out + (int64_t)row0 * F), (short)0, rows * F, kMxRsrcWord3);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int item = 64 * wid + elane + 512 * k;
                const int r = item >> 2, w = item & 3;
                const char* seg = st1 + r * 128 + 32 * (w ^ ((r >> 2) & 3));
                const uint4 d0 = *(const uint4*)seg, d1 = *(const uint4*)(seg + 16);
                const mx_u32x4 lo{__builtin_amdgcn_perm(d0.y, d0.x, 0x06040200u),
                                  __builtin_amdgcn_perm(d0.w, d0.z, 0x06040200u),
                                  __builtin_amdgcn_perm(d1.y, d1.x, 0x06040200u),
                                  __builtin_amdgcn_perm(d1.w, d1.z, 0x06040200u)};
                const mx_u32x4 hi{__builtin_amdgcn_perm(d0.y, d0.x, 0x07050301u),
                                  __builtin_amdgcn_perm(d0.w, d0.z, 0x07050301u),
                                  __builtin_amdgcn_perm(d1.y, d1.x, 0x07050301u),
                                  __builtin_amdgcn_perm(d1.w, d1.z, 0x07050301u)};
                const int off = (cb0 + w) * 64 < g.N ? r * F + (cb0 + w) * 32 : 0x7ffffff0;
                __builtin_amdgcn_raw_buffer_store_b128(lo, orr, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(hi, orr, off + 16, 0, 0);
            }
        } else {
            // 32 rows x 64 fp32 at a time in the wave's region, rows of 256
            // bytes, 64-byte column groups at group ^ ((row / 4) mod 4)
            char* const ep = st1 + wid * kMxEpiWave;
            const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((float*)g.out + (int64_t)row0 * g.N), (short)0, rows * g.N * 4, kMxRsrcWord3);
            const int c = er16;
            const int col = c0 + 4 * c;              // this lane's 4 stored columns
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int lr = 16 * ii + 4 * ekg + v;
                            *(float*)(ep + lr * 256 + ((64 * j + 4 * er16) ^ (64 * ekg))) = acc[2 * p + ii][j][v];
                        }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int lr = ekg + 4 * k;
                    const mx_u32x4 val = *(const mx_u32x4*)(ep + lr * 256 + ((16 * c) ^ (64 * ((lr >> 2) & 3))));
                    const int off = col < g.N ? ((128 * wm + 32 * p + lr) * g.N + col) * 4 : 0x7ffffff0;
                    __builtin_amdgcn_raw_buffer_store_b128(val, orr, off, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (!more) {
            MX_WAIT_VMCNT(0);          // the repeated loads land before the LDS is released
            break;
        }
        tile = next;
    }
}

}  // namespace moe
