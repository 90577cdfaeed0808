// K3 / K4 for MXFP4 weights, 64-row tiles (experts with at most 128 rows, and
// at decode-sized batches the larger experts as 64-row tiles too; K a
// multiple of 128, operands below 2 GiB): E2M1 weights with one E8M0 scale per
// 32 along K against E4M3 activations with the same scaling, on the CDNA4
// block-scaled MFMA (16x16x128, B in the E2M1 format), fp32 accumulate.
//
// Same arithmetic contract as the streaming tiles (gemm_mxfp8_stream.h): acc =
// 0; for k0 = 0, 128, ... : acc = MFMA_SCALE(A[row, k0:k0+128], B[col,
// k0:k0+128], acc) with the step's four scales, so a row's bits do not depend
// on which design ran it.
//
// A workgroup of 8 waves takes up to 64 rows x 512 columns, wave w owning 64
// columns (FC1: one gate/up interleave block).  Everything a K step reads
// arrives in LDS by direct loads:
//  - the weights of a wave's columns (4 KB of codes, their 1 KB of scale
//    groups) and the tile's activation scales go to a 3-slot ring of that
//    wave's own, refilled by the wave as soon as it has read a slot, so the
//    weights run three steps ahead of the multiply;
//  - the tile's activation codes (64 rows x 128 bytes, 8 rows loaded by each
//    wave) go to a 3-slot ring shared by the workgroup, two steps ahead, with
//    one barrier per step (a step's codes have landed in every wave, and the
//    slot refilled next has been read by every wave).
// With nothing but direct loads in flight, each wave waits for its own loads
// with one vmcnt count.  Every step issues the same loads (past the last step
// they re-read it into a slot nobody reads again), so the count is uniform.
// (A wave that also had plain register loads in flight could not rely on such
// counts: measured on the MI355X, outputs then came out wrong from run to run.)
// The weights are packed in 512-column groups (wblock_index), so the 32 code
// blocks of a tile's K step are one contiguous 32 KB and their scale groups
// one contiguous 8 KB.
#pragma once

#include "gemm_args.h"

namespace moe {

constexpr int kMx4Cols = 512;                    // columns per tile (8 waves x 64)
constexpr int kMx4Slot = 4096 + 1024 + 256;      // one wave's weight slot: codes, scale groups, activation scales
constexpr int kMx4SlotAll = 8 * kMx4Slot;         // one weight slot of all 8 waves
constexpr int kMx4ASlot = 64 * 128;              // one activation-code slot: 64 rows x 128 bytes
// Direct loads per wave and step, by what issues them (the waits below are
// derived from these counts; each issuing loop is bounded by its constant)
constexpr int kMx4CodeLoads = 4;                 // issue_w: 4 weight-code blocks of 1 KB
constexpr int kMx4ScaleLoads = 4;                // issue_w: 4 weight-scale groups
constexpr int kMx4ActScaleLoads = 1;             // issue_w: the activation scales
constexpr int kMx4WLoads = kMx4CodeLoads + kMx4ScaleLoads + kMx4ActScaleLoads;
constexpr int kMx4ALoads = 1;                    // issue_a: the activation codes
constexpr int kMx4Loads = kMx4WLoads + kMx4ALoads;
// Issue order: W(0) A(0) W(1) A(1) W(2), then step t issues A(t + 2) W(t + 3).
// At step s's wait, after the last load of A(s) come W(s+1) A(s+1) W(s+2) and
// after the last load of W(s) one more (A(s)); the smaller count is the bound.
constexpr int kMx4StepWait = 2 * kMx4WLoads + kMx4ALoads;
static_assert(kMx4StepWait == 2 * kMx4Loads - 1 && kMx4StepWait <= 63, "vmcnt bound");

typedef __attribute__((address_space(3))) void mx4_lds_void;

// third dword of a raw buffer descriptor on CDNA (32-bit data format, no
// swizzle, no stride): byte-addressed loads with a range check
constexpr int kMx4RsrcWord3 = 0x00020000;

#define MX4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Ring slots: three weight-slot objects (w*: this wave's part) and three
// activation-slot objects (q*), each addressed with a static slot number so
// the compiler can tell a read of one slot from a direct load into another.
struct Mx4Ring {
    char *w0, *w1, *w2, *q0, *q1, *q2;
};

template <bool FC1, int NG, bool PROB>
__device__ __forceinline__ void mx4_tile(const MxGemmArgs& g, const Mx4Ring& rg, int wid, int e, int row0,
                                         int rows, int cb, bool has_cols)
{
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K, KB = K / 32, KS = K / 128, KQ = KS / 4 + ((KS % 4) ? 1 : 0);
    const int nt16 = g.N / 16;

    // Direct loads through buffer descriptors (wave-uniform, scalar registers)
    // with a per-lane offset register fixed for the tile and the step in a
    // scalar offset: no per-lane address register is rewritten while a load
    // that reads it is in flight.
    //  activation codes: lane -> tile row 8 wid + lane / 8, LDS chunk lane % 8
    //  holds the row's 16-byte chunk (lane % 8) ^ (row % 8)
    int aoff;
    {
        const int rr = 8 * wid + (lane >> 3);
        int64_t src = row0 + min(rr, rows - 1);
        if constexpr (FC1) src = g.perm_src[src] / g.topk;
        aoff = (int)(src * K) + 16 * ((lane & 7) ^ (rr & 7));
    }
    //  activation scales: lane L -> the step's 4 scale bytes of tile row L
    int soff;
    {
        int64_t src = row0 + min(lane, rows - 1);
        if constexpr (FC1) src = g.perm_src[src] / g.topk;
        soff = (int)(src * KB);
    }
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, 0x7fffffff, kMx4RsrcWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void*)g.As, (short)0, 0x7fffffff, kMx4RsrcWord3);
    //  weights: the expert's section, block (c16, t) at wblock_index(c16, t); a
    //  wave without columns re-reads the last column block (loads stay
    //  uniform, the multiply is skipped)
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.W + (int64_t)e * nt16 * KS * 1024), (short)0, nt16 * KS * 1024, kMx4RsrcWord3);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.Ws + (int64_t)e * nt16 * KQ * 256), (short)0, nt16 * KQ * 256, kMx4RsrcWord3);
    int b0[4], bw[4], q0[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c16 = min(cb * 4 + j, nt16 - 1);
        b0[j] = (int)wblock_index(c16, 0, nt16, KS);
        q0[j] = (int)wblock_index(c16, 0, nt16, KQ);
        bw[j] = (int)wblock_step(c16, nt16);
    }
    const int boff = 16 * lane, qoff = 4 * lane;

    // activation codes of step s into shared slot q: 1 load
    auto issue_a = [&](int s, char* q) {
        const int t = min(s, KS - 1);
        static_assert(kMx4ALoads == 1, "issue_a issues one load");
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (mx4_lds_void*)(q + wid * 1024), 16, aoff, 128 * t, 0, 0);
        __builtin_amdgcn_sched_barrier(0);      // the vmcnt count below assumes source order
    };
    // weights of step s (+ activation scales) into this wave's slot w: kMx4WLoads loads
    auto issue_w = [&](int s, char* w) {
        const int t = min(s, KS - 1);
        static_assert(kMx4CodeLoads == 4 && kMx4ScaleLoads == 4 && kMx4ActScaleLoads == 1,
                      "a wave loads its 4 column blocks' codes and scale groups");
#pragma unroll
        for (int j = 0; j < kMx4CodeLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (mx4_lds_void*)(w + j * 1024), 16, boff,
                                                     (b0[j] + t * bw[j]) * 1024, 0, kNonTemporal);
#pragma unroll
        for (int j = 0; j < kMx4ScaleLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (mx4_lds_void*)(w + 4096 + j * 256), 4, qoff,
                                                     (q0[j] + (t >> 2) * bw[j]) * 256, 0, kNonTemporal);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (mx4_lds_void*)(w + 5120), 4, soff, 4 * t, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4 acc[NG][4];
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment offsets inside a 16-row group (2 KB): the lane row's 16-byte K chunks kg and kg + 4
    const int a_lo = r16 * 128 + ((kg ^ (r16 & 7)) << 4);
    const int a_hi = r16 * 128 + (((kg + 4) ^ (r16 & 7)) << 4);

    // Step s waits until its weights and codes landed (kMx4StepWait).  Only
    // direct loads may be in flight here: vmcnt also counts plain vector loads
    // and stores, and one more of them anywhere between two steps' loads would
    // let the count pass before step s's data is in LDS.
    auto step = [&](int s, const char* w, const char* q, char* qn) {
        MX4_WAIT_VMCNT(kMx4StepWait);
        __builtin_amdgcn_s_barrier();
        i32x8 a[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const uint4 lo = *(const uint4*)(q + i * 2048 + a_lo);
            const uint4 hi = *(const uint4*)(q + i * 2048 + a_hi);
            a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        uint4 bl[4];
        int sb[4], sa[NG];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bl[j] = *(const uint4*)(w + j * 1024 + 16 * lane);
            sb[j] = ((const uint8_t*)w)[4096 + j * 256 + 4 * lane + (s & 3)];
        }
#pragma unroll
        for (int i = 0; i < NG; ++i) sa[i] = ((const uint8_t*)w)[5120 + 4 * (16 * i + r16) + kg];
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): both slots read
        issue_a(s + 2, qn);                     // into the slot every wave read at step s - 1
        issue_w(s + 3, (char*)w);               // into this wave's slot just read
        if (has_cols) {
#pragma unroll
            for (int i = 0; i < NG; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // the upper half of an E2M1 operand is not read by the MFMA
                    const i32x8 b = {(int)bl[j].x, (int)bl[j].y, (int)bl[j].z, (int)bl[j].w, 0, 0, 0, 0};
                    // A format 0 (E4M3), B format 4 (E2M1)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a[i], b, acc[i][j], 0, 4, 0, sa[i], 0, sb[j]);
                }
        }
    };

    // every wave has read the previous tile's slots before they refill
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_w(0, rg.w0);
    issue_a(0, rg.q0);
    issue_w(1, rg.w1);
    issue_a(1, rg.q1);
    issue_w(2, rg.w2);
    // unrolled by three: static slots of both rings (step s reads w[s % 3],
    // q[s % 3] and refills q[(s + 2) % 3])
    int s = 0;
    for (; s + 3 <= KS; s += 3) {
        step(s, rg.w0, rg.q0, rg.q2);
        step(s + 1, rg.w1, rg.q1, rg.q0);
        step(s + 2, rg.w2, rg.q2, rg.q1);
    }
    if (s < KS) step(s, rg.w0, rg.q0, rg.q2);
    if (s + 1 < KS) step(s + 1, rg.w1, rg.q1, rg.q0);
    // the loads past the last step land before the slots are reused
    MX4_WAIT_VMCNT(0);
    if (!has_cols) return;

    // epilogue: lane holds rows 4 kg + v of each 16-row group, column r16 of each block
    if constexpr (FC1) {
        // SwiGLU, then the per-32 requantization of this interleave block's
        // 32 outputs of each row (16 lanes x 2 blocks hold one row's block)
        const int F = g.N / 2, FB = F / 32;
        uint8_t* hq = (uint8_t*)g.out;
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * kg + v;
                // the 16 lanes of one requantization block hold one row: one probability
                const float pr = (PROB && r < rows) ? fc1_row_prob(g.row_prob, g.perm_src, row0 + r) : 1.0f;
                float gt = acc[i][0][v], up = acc[i][2][v];
                const float h0 = swiglu_f32(gt, up) * pr;
                gt = acc[i][1][v]; up = acc[i][3][v];
                const float h1 = swiglu_f32(gt, up) * pr;
                const float amax = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
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
    } else {
        float* ob = (float*)g.out;
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * kg + v;
                if (r < rows) {
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

// The 64-row tile loop of one 8-wave workgroup; K % 128 == 0.  Every wave
// takes part in every tile (the barriers), a wave past N without columns.
// With lds_small == 2 the 256-row table follows, four 64-row tiles per entry.
template <bool FC1, bool PROB>
__device__ __forceinline__ void mx4_small_tiles(const MxGemmArgs& g, const Mx4Ring& ring)
{
    const int n_small = ld_const(&g.hdr->n_tiles);
    const int n_mt = n_small + (g.lds_small == 2 ? 4 * ld_const(&g.hdr->n_tiles_big) : 0);
    const int NTs = (g.N + kMx4Cols - 1) / kMx4Cols;
    const int total = n_mt * NTs;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int n_cb = g.N / 64 + ((g.N % 64) ? 1 : 0);
    Mx4Ring rg = ring;
    rg.w0 += wid * kMx4Slot;
    rg.w1 += wid * kMx4Slot;
    rg.w2 += wid * kMx4Slot;
    for (int tile = xcd_first_tile(); tile < total; tile += gridDim.x) {
        const int mt = tile / NTs, ct = tile - mt * NTs;
        const int* te = mt < n_small ? (const int*)(g.tiles + mt) : (const int*)(g.tiles_big + ((mt - n_small) >> 2));
        const int e = ld_const(te), row0 = ld_const(te + 1) + (mt < n_small ? 0 : kBM * ((mt - n_small) & 3));
        const int rows = min(kBM, ld_const(g.offsets + e + 1) - row0);
        if (rows <= 0) continue;                     // uniform across the workgroup
        const int cb = ct * 8 + wid;
        const bool has_cols = cb < n_cb;
        switch ((rows + 15) >> 4) {
            case 1: mx4_tile<FC1, 1, PROB>(g, rg, wid, e, row0, rows, cb, has_cols); break;
            case 2: mx4_tile<FC1, 2, PROB>(g, rg, wid, e, row0, rows, cb, has_cols); break;
            case 3: mx4_tile<FC1, 3, PROB>(g, rg, wid, e, row0, rows, cb, has_cols); break;
            default: mx4_tile<FC1, 4, PROB>(g, rg, wid, e, row0, rows, cb, has_cols); break;
        }
    }
}

}  // namespace moe
