// Shared device-side definitions of the MI355X (gfx950) routed-MoE library.
//
// Vector types for the CDNA4 MFMA operands, number-format conversions done
// in registers, and the workspace layout that every kernel and the host code
// agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 1024;
constexpr int kChunkTok = 256;       // tokens per prep workgroup
// bf16 kernel-weight blocks (1 KB: 16 columns x 32 K in MFMA lane order) of one
// expert's N x K section, in 512-column groups: [n16 / 32][K step][n16 % 32], so
// one K step of a group is contiguous (the last group may be narrower).
__host__ __device__ inline int64_t wblock_index(int64_t n16, int64_t s, int64_t nt16, int64_t ks)
{
    const int64_t g = n16 >> 5;
    const int64_t w = nt16 - 32 * g < 32 ? nt16 - 32 * g : 32;
    return g * 32 * ks + s * w + (n16 & 31);
}
// distance in blocks from one K step of column block n16 to the next
__host__ __device__ inline int64_t wblock_step(int64_t n16, int64_t nt16)
{
    const int64_t g = n16 >> 5;
    return nt16 - 32 * g < 32 ? nt16 - 32 * g : 32;
}

constexpr int kBM = 64;              // rows per M tile of the small-expert GEMM tiles
constexpr int kBigBMRows = 256;      // rows per M tile of the LDS-staged GEMMs
constexpr int kBigMin = 128;         // experts with more rows than this use the LDS-staged GEMMs
constexpr int kFinCols = 512;        // output columns per count of the single-launch finalize
                                     // (the 64-row tiles' column width)

// Error bits reported by moe_check (same values as the header's MOE_DEVERR_*).
constexpr uint32_t kErrBadId = 1u;
constexpr uint32_t kErrDupId = 2u;
constexpr uint32_t kErrLiveHigh = 4u;
constexpr uint32_t kErrLiveNeg = 8u;
constexpr uint32_t kErrFusedWait = 16u;

// ---------------------------------------------------------------- formats

// SwiGLU of one gate/up pair in fp32, silu(g) * u = g / (1 + exp(-g)) * u, the
// division as a multiply by the hardware reciprocal (v_rcp_f32, within 1 ulp).
// Every GEMM epilogue (bf16 and MX) calls this one function, so the tile
// designs agree bit for bit.  Large negative g: exp(-g) = inf, rcp(inf) = 0, so the result
// is a signed zero; large positive g: rcp(1) = 1, so the result is g * u.
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Maximum over the 16 lanes of a DPP row (lanes 16 m .. 16 m + 15), the lanes
// that hold one row of a 16 x 16 MFMA block: v_max_f32 with the row rotated
// by 1, 2, 4, 8 on its first operand.  Each s_nop gives the two wait states a
// DPP read of a VGPR needs after a VALU write to it.  Equal to an fmaxf
// reduction for every value the epilogues produce (no signaling NaN).
__device__ __forceinline__ float row16_max(float x)
{
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "+v"(x));
    return x;
}

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v)
{
    __bf16 b = static_cast<__bf16>(v);
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b)
{
    return __uint_as_float(b << 16);
}

// Exponent e of the E8M0 block scale: the smallest e in [-127, 127] with
// amax <= 448 * 2^e.  With amax = 1.m * 2^E (normal), 448 = 1.75 * 2^8, so
// e = E - 8 when 1.m <= 1.75 (mantissa field <= 0x600000), else E - 7.
// Zero and subnormal amax fall below 448 * 2^-127 and give -127.
// (The zero / subnormal case needs no branch: exponent field 0 gives e <= -134,
// which the clamp takes to -127.)
__device__ __forceinline__ int e8m0_exponent(float amax)
{
    uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
    int ef = (int)(u >> 23);
    int e = ef - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E8M0 exponent of an MXFP4 block: the smallest e with amax <= 6 * 2^e (the
// power-of-two ceiling of amax / 6), clamped to [-127, 127]; amax == 0 (or an
// fp32 subnormal, whose block then scales to below 2^-126 * 2^127 = 2) gives
// -127.  From the fp32 bits: amax = 2^E (1 + m) needs e = E - 2 when
// 1 + m <= 1.5 and E - 1 otherwise.
__device__ __forceinline__ int e8m0_exponent_fp4(float amax)
{
    uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
    int ef = (int)(u >> 23);   // 0 gives e <= -128, clamped to -127 below
    int e = ef - 127 - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// fp32 -> E2M1 code (OCP MX FP4: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) for
// |v| <= 6, round to nearest with ties to the even code; the sign is kept.
// The intervals between neighbouring magnitudes, with each midpoint going to
// the neighbour whose mantissa bit is 0.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v)
{
    const float a = fabsf(v);
    const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f  ? 4u : a < 3.5f  ? 5u : a <= 5.0f  ? 6u : 7u;
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// fp32 -> E4M3FN codes with the hardware converter (v_cvt_pk_fp8_f32): round
// to nearest even, the OCP E4M3FN encoding.  Callers pass finite values with
// |v| <= 448, which the MX block scale guarantees; on that range the converter
// is exact rounding (checked exhaustively against a bit-level software
// rounding of every such fp32 value).  x2: code of a in byte 0, b in byte 1.
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// four codes, a in byte 0 .. d in byte 3
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---------------------------------------------------------------- workspace

// Byte layout of the caller's workspace.  Offsets are 256-byte aligned.
struct WsLayout {
    size_t hdr;            // WsHeader
    size_t counts;         // int32 [E]
    size_t offsets;        // int32 [E + 1]
    size_t chunk_base;     // int32 [nchunks][E]: chunk counts, then global bases
    size_t chunk_err;      // uint32 [nchunks]
    size_t local_rank;     // int32 [T_cap * k]
    size_t sorted_ids;     // int32 [T_cap * k]
    size_t sorted_probs;   // float [T_cap * k]
    size_t perm_src;       // int32 [T_cap * k]
    size_t dst;            // int32 [T_cap * k]
    size_t tiles;          // int2 [max_tiles]: (expert, first row), 64-row GEMM tiles
    size_t tiles_big;      // int2 [max_tiles_big]: (expert, first row), LDS-staged GEMM tiles
    size_t ready;          // int32 [max_tiles + 4 max_tiles_big]: single-launch FFN readiness counters
    size_t fin_cnt;        // int32 [T_cap][ceil(H / 512)]: single-launch finalize, routes still to come
    size_t hbuf;           // bf16 [T_cap * k][F] or E4M3 [T_cap * k][F]
    size_t hscale;         // E8M0 [T_cap * k][F / 32] (mxfp8)
    size_t obuf;           // float [T_cap * k][H]
    size_t xq;             // E4M3 [T_cap][H] (mxfp8)
    size_t xs;             // E8M0 [T_cap][H / 32] (mxfp8)
    size_t total;
    int64_t nchunks;
    int64_t max_tiles;
    int64_t max_tiles_big;
};

// Every field is written by the launch that produces it before any later
// launch reads it, so the header needs no initialisation.
struct WsHeader {
    uint32_t err;          // contract-violation bits of the last route or forward
    int32_t multi_tile;    // 1: some expert needs more than one 64-row M tile
    int32_t T;             // live tokens of the last forward (clamped)
    int32_t n_tiles;       // M tiles in the tile table
    int32_t n_rows;        // routed rows with a valid expert
    int32_t n_tiles_big;   // M tiles in the LDS-staged table
    int32_t pad[58];
};

static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

}  // namespace moe
