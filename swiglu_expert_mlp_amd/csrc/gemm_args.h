// Launch arguments of the grouped expert GEMMs (shared by host and device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

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
};

}  // namespace moe
