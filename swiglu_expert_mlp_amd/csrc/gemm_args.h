// Launch arguments of the grouped expert GEMMs (shared by host and device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Cache policy of the weight streams of the 64-row tiles when every expert's
// rows fit one 64-row M tile (each weight byte then read once per launch):
// non-temporal.  Measured at decode sizes (64 experts, hidden 2048, FFN 1024):
// FC1 90.5 -> 82.8 us, FC2 53.5 -> 49.6 us.  With experts of several 64-row
// tiles, which share a weight slice through the L2, the default policy (the
// single-launch FFN at 16K tokens: 3.73 ms/step with it, 5.08 with
// non-temporal loads).
constexpr int kNonTemporal = 2;

// 16-byte load with the non-temporal (streaming) cache policy.
__device__ __forceinline__ uint4 load_stream16(const void* p)
{
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v v = __builtin_nontemporal_load((const u32x4v*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Load of a table that an earlier launch wrote and this launch only reads, at a
// wave-uniform address: through the constant address space it becomes a scalar
// load, kept apart from the vector-memory count of the tile's loads and stores.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p)
{
    return *(const __attribute__((address_space(4))) T*)p;
}

// A persistent 64-row tile loop's first tile; the loop then steps by the grid.
// Each round of the grid is split into 8 contiguous runs, one per XCD
// (workgroups are dispatched round-robin over the XCDs; the grid is a multiple
// of 8), so that the column tiles of one M tile run on one XCD and share its
// L2: at decode sizes an expert's whole FC1 (and FC2) runs on one XCD, and in
// the single-launch FFN an FC2 tile waits only for FC1 tiles of its own XCD.
// Measured (bf16, one MI355X): decode 148.4 -> 146.1 us per forward, a
// 65,536-token capacity with 512 live 670 -> 655 us.
__device__ __forceinline__ int xcd_first_tile()
{
    return (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3));
}

// FC1 with the routes' probabilities applied inside FC1 (row_prob: the
// canonical probabilities, indexed by route t * k + j): the probability of a
// grouped row.  The kernels take this path as a compile-time variant (PROB):
// a run-time branch around the load made the compiler wait on every load in
// flight in the default epilogues.
__device__ __forceinline__ float fc1_row_prob(const float* row_prob, const int32_t* perm_src,
                                              int64_t row)
{
    return row_prob[perm_src[row]];
}

// bf16 operands.
struct GemmArgs {
    const uint16_t* A;         // FC1: x [T_cap][H]; FC2: hbuf [rows][F]
    const uint16_t* W;         // FC1: packed W1 [E][2F][H]; FC2: W2 [E][H][F]
    const int32_t* perm_src;   // FC1: grouped row -> route (t * k + j)
    const int2* tiles;         // (expert, first row) per 64-row M tile
    const int2* tiles_big;     // (expert, first row) per 256-row M tile (LDS-staged kernel)
    const int32_t* offsets;    // [E + 1]
    const WsHeader* hdr;       // n_tiles, n_tiles_big
    void* out;                 // FC1: hbuf bf16 [rows][F]; FC2: obuf fp32 [rows][H]
    int N;                     // FC1: 2F; FC2: H
    int K;                     // FC1: H;  FC2: F
    int topk;
    int n_tiles_n;             // N tiles per M tile (4 waves x 64 columns each)
    int max_tiles;             // capacity of `tiles` (entries)
    int small_takes_big;       // 1: one launch, the 64-row kernel also runs the 256-row
                               // tiles (as four 64-row tiles each): token capacity <= 1024,
                               // or a shape the 256-row kernel does not take
    const float* row_prob;     // FC1: probabilities applied to the SwiGLU rows, or null
    // single-launch FFN (FC1 and FC2 in one persistent launch): per 64-row M
    // tile, the count of FC1 column tiles whose SwiGLU rows are released
    int32_t* ready;
    uint32_t* err;             // the header's error word (a readiness wait past its limit)
    // single-launch finalize (the FC2 half of the fused launch): per live token
    // and 512-column block of the output, the number of the token's FC2 rows
    // not yet written (prep sets it to the token's kept routes)
    int32_t* fin_cnt;
    const int32_t* fin_route;  // grouped row -> route (t * k + j)
    const int32_t* fin_dst;    // route -> grouped row, -1 for a dropped route
    const float* fin_prob;     // canonical probabilities, or null (every p is 1)
    void* fin_out;             // the forward's output
    int fin_mode;              // 0: fp32 chain, 1: bf16 of it, 2: rows
};

// MXFP8 operands: E4M3 codes with one E8M0 scale byte per 32 elements of K.
struct MxGemmArgs {
    const uint8_t* A;          // FC1: xq [T_cap][H]; FC2: hbuf codes [rows][F]
    const uint8_t* As;         // FC1: xs [T_cap][H/32]; FC2: hbuf scales [rows][F/32]
    const uint8_t* W;          // FC1: packed W1 codes [E][2F][H]; FC2: W2 codes [E][H][F]
    const uint8_t* Ws;         // scales [E][N][K/32]
    const int32_t* perm_src;
    const int2* tiles;
    const int2* tiles_big;
    const int32_t* offsets;
    const WsHeader* hdr;
    void* out;                 // FC1: hbuf codes [rows][F]; FC2: obuf fp32 [rows][H]
    uint8_t* out_scale;        // FC1: hbuf scales [rows][F/32]
    int N;
    int K;
    int topk;
    int n_tiles_n;
    int stream_big;            // 1: the streaming kernel also takes the 256-row tiles
                               // (as four 64-row tiles each); 0: the LDS-staged kernel does
    int lds_small;             // MXFP4: 0: the streaming loop takes the 64-row tiles; 1: the
                               // LDS-staged 64-row kernel does; 2: that kernel also takes the
                               // 256-row tiles (four 64-row tiles each, no 256-row launch)
    int small_batch;           // 1: decode-sized batch (the caller's token capacity <= 1024)
    int64_t a_bytes;           // bytes of A (rows x K)
    const float* row_prob;     // FC1: probabilities applied to the SwiGLU rows, or null
};

}  // namespace moe
