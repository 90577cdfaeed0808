// K6: kernel-weight buffer pack (and MXFP8 quantization), K2: MXFP8
// quantization of the activations.
//
// Megatron-LM PR #7830, "1. Mega backend for generation": the kernel weight
// layout interleaves gate and up in blocks of 32 rows and is K-major; the
// caller owns the buffer, so a refit rewrites it in place.  cudnn-frontend
// PR #448: MXFP8 carries one E8M0 scale per 32 elements; the scale here is
// the power-of-two ceiling of the block's max magnitude / 448, so every code
// fits E4M3 without saturation.
//
// Packed FC1 row 64 b + i of an expert is gate row 32 b + i (i < 32) or up
// row F + 32 b + (i - 32) (i >= 32); FC2 rows keep their order.  MXFP8 blocks
// run along K (H for FC1 rows, F for FC2 rows), so the interleave moves whole
// rows and never splits a block.
//
// The rows are then tiled into MFMA operand blocks so that one wave's operand
// load is one contiguous 1 KB read (layout formulas in include/moe.h):
//   bf16:  16 rows x 32 K per 1 KB block, lane order (lane = 16 * (k%32 / 8)
//          + n%16, 8 elements per lane); an expert's blocks in 512-row groups
//          [n/512][k/32][(n/16)%32] (the last group as wide as what is left),
//          so one K step of a group is one contiguous run of blocks.
//   MXFP8: 16 rows x 128 K per 2 KB block = two 1 KB halves (K%128 < 64 and
//          >= 64), lane = 16 * (k%64 / 16) + n%16, 16 codes per lane; blocks
//          [expert][n/16][k/128]; E8M0 scales 4 K-steps per lane dword:
//          256 B groups [expert][n/16][k/512], byte (k/128)%4 of lane
//          16 * ((k/32)%4) + n%16.
//   MXFP4: 16 rows x 128 K per 1 KB block, lane = 16 * (k%128 / 32) + n%16,
//          32 E2M1 codes per lane as 16 bytes (the lower K in the low nibble);
//          blocks in 512-row groups [n/512][k/128][(n/16)%32] like bf16;
//          scale groups [n/512][k/512][(n/16)%32], otherwise as MXFP8.  The
//          scale is the power-of-two ceiling of the block's max magnitude / 6.
#include "common.h"

namespace moe {

__device__ __forceinline__ int64_t fc1_src_row(int64_t packed, int64_t F)
{
    int64_t b = packed >> 6, i = packed & 63;
    return i < 32 ? 32 * b + i : F + 32 * b + (i - 32);
}

// bf16 tiled layout: one thread writes one lane's 16 bytes (8 elements) of a
// block.  N rows of K elements per expert; fc1 selects the interleaved order.
__global__ void __launch_bounds__(256) pack_bf16_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int E, int N,
                                                        int K, int F, int fc1)
{
    const int64_t ks = K / 32, nt = N / 16;
    const int64_t n_pieces = (int64_t)E * nt * ks * 64;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pieces;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i & 63);
        int64_t blk = i >> 6;                       // (e * nt + n16) * ks + s
        const int64_t s = blk % ks;
        blk /= ks;
        const int64_t n16 = blk % nt, e = blk / nt;
        const int64_t n = n16 * 16 + (lane & 15);
        const int64_t k = s * 32 + (lane >> 4) * 8;
        const int64_t srow = fc1 ? fc1_src_row(n, F) : n;
        const int64_t o = (e * nt * ks + wblock_index(n16, s, nt, ks)) * 64 + lane;
        ((uint4*)dst)[o] = *(const uint4*)(src + ((e * N + srow) * K + k));
    }
}

// Quantize one 32-element block of bf16 values: 32 E4M3 codes and the E8M0
// scale byte.
__device__ __forceinline__ void quant_block32(const uint16_t* __restrict__ src,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scale)
{
    const uint4* s4 = (const uint4*)src;
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = s4[q];
    const uint32_t* w = (const uint32_t*)v;
    float f[32];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        f[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
        f[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(f[q]));
    int e8 = e8m0_exponent(amax);
    // 2^-e8 exactly; 2^-127 is an fp32 subnormal
    float inv = e8 == 127 ? __uint_as_float(1u << 22) : __uint_as_float((uint32_t)(127 - e8) << 23);
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        out[q] = cvt_e4m3x4(f[4 * q] * inv, f[4 * q + 1] * inv, f[4 * q + 2] * inv, f[4 * q + 3] * inv);
    }
    uint4* d4 = (uint4*)codes;
    d4[0] = make_uint4(out[0], out[1], out[2], out[3]);
    d4[1] = make_uint4(out[4], out[5], out[6], out[7]);
    *scale = (uint8_t)(e8 + 127);
}

// MXFP8 weights, tiled layout.  One thread quantizes one 32-element block
// (row n, block q of K) and writes its 32 codes as two 16-byte pieces (the
// block's halves go to lanes kg = 2 (q%2) and 2 (q%2) + 1 of one half of the
// K-step) and its scale byte.  Padding past K (codes 0, scale 2^0) is written
// by the threads of the blocks q >= K/32 up to the padded size.
__global__ void __launch_bounds__(256) pack_mx_kernel(const uint16_t* __restrict__ src,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, int E, int N,
                                                      int K, int F, int fc1)
{
    const int64_t KS = (K + 127) / 128, KQ = (KS + 3) / 4, nt = N / 16;
    const int64_t nbk = KQ * 16;                  // padded 32-blocks per row
    const int64_t n_items = (int64_t)E * N * nbk;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_items;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t q = i % nbk;
        const int64_t row = i / nbk;               // e * N + n
        const int64_t e = row / N, n = row - e * N;
        const int64_t n16 = n >> 4, r16 = n & 15;
        const int64_t step = q >> 2, kg = q & 3;
        uint8_t* sc = scales + ((e * nt + n16) * KQ + (step >> 2)) * 256 +
                      ((kg * 16 + r16) * 4) + (step & 3);
        if (q >= K / 32) {
            *sc = 127;
            if (step < KS) {
                // the two 16-byte pieces of this (padded) block
                const int64_t half = (kg >> 1), lg = (kg & 1) * 2;
                uint8_t* base = codes + (((e * nt + n16) * KS + step) * 2 + half) * 1024;
                *(uint4*)(base + ((lg + 0) * 16 + r16) * 16) = make_uint4(0, 0, 0, 0);
                *(uint4*)(base + ((lg + 1) * 16 + r16) * 16) = make_uint4(0, 0, 0, 0);
            }
            continue;
        }
        const int64_t srow = fc1 ? fc1_src_row(n, F) : n;
        alignas(16) uint8_t c32[32];
        quant_block32(src + (e * N + srow) * K + q * 32, c32, sc);
        const int64_t half = kg >> 1, lg = (kg & 1) * 2;   // K%128 = 32 kg + [0, 32)
        uint8_t* base = codes + (((e * nt + n16) * KS + step) * 2 + half) * 1024;
        *(uint4*)(base + ((lg + 0) * 16 + r16) * 16) = *(const uint4*)(c32);
        *(uint4*)(base + ((lg + 1) * 16 + r16) * 16) = *(const uint4*)(c32 + 16);
    }
}

// MXFP4 weights, tiled layout.  One thread quantizes one 32-element block
// (row n, block q of K) and writes its 32 codes as the 16 bytes of lane
// 16 (q % 4) + n % 16 of the row's 1 KB block of K step q / 4; blocks past
// K/32 (the padding of the last step) get zero codes and scale 127.  The code
// blocks and the 256-byte scale groups of an expert are in 512-column groups
// (wblock_index), so one K step of a group is one contiguous run.
__global__ void __launch_bounds__(256) pack_mx4_kernel(const uint16_t* __restrict__ src,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int E, int N,
                                                       int K, int F, int fc1)
{
    const int64_t KS = (K + 127) / 128, KQ = (KS + 3) / 4, nt = N / 16;
    const int64_t nbk = KQ * 16;                  // padded 32-blocks per row
    const int64_t n_items = (int64_t)E * N * nbk;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_items;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t q = i % nbk;
        const int64_t row = i / nbk;               // e * N + n
        const int64_t e = row / N, n = row - e * N;
        const int64_t n16 = n >> 4, r16 = n & 15;
        const int64_t step = q >> 2, kg = q & 3;
        uint8_t* sc = scales + (e * nt * KQ + wblock_index(n16, step >> 2, nt, KQ)) * 256 +
                      ((kg * 16 + r16) * 4) + (step & 3);
        uint4* dst = (uint4*)(codes + (e * nt * KS + wblock_index(n16, step, nt, KS)) * 1024 +
                              (kg * 16 + r16) * 16);
        if (q >= K / 32) {
            *sc = 127;
            if (step < KS) *dst = make_uint4(0, 0, 0, 0);
            continue;
        }
        const int64_t srow = fc1 ? fc1_src_row(n, F) : n;
        const uint4* s4 = (const uint4*)(src + (e * N + srow) * K + q * 32);
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = s4[j];
        const uint32_t* w = (const uint32_t*)v;
        float f[32];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            f[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
            f[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
        const int e4 = e8m0_exponent_fp4(amax);
        // 2^-e4 exactly; 2^-127 is an fp32 subnormal
        const float inv = e4 == 127 ? __uint_as_float(1u << 22) : __uint_as_float((uint32_t)(127 - e4) << 23);
        uint32_t out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) word |= f32_to_e2m1(f[8 * j + t] * inv) << (4 * t);
            out[j] = word;
        }
        *dst = make_uint4(out[0], out[1], out[2], out[3]);
        *sc = (uint8_t)(e4 + 127);
    }
}

// K2: x rows < live quantized per 32-block of H.  A lane converts 8 elements
// (one 16-byte load, one 8-byte store); the 4 lanes of a quad hold one
// 32-block and exchange their partial amax with two DPP steps (quad_perm
// [1,0,3,2] and [2,3,0,1]), so every lane derives the same E8M0 exponent.
__global__ void __launch_bounds__(256) quant_x_mx_kernel(const uint16_t* __restrict__ x,
                                                         int64_t T_cap, const int32_t* __restrict__ live_ptr,
                                                         int H, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales)
{
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    const int nb = H / 32;
    const int64_t n = T * (H / 8);                      // 8-element groups, quads never straddle rows
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x; i0 < n; i0 += stride) {
        // whole waves stay in the loop together (the DPP steps need the quad's lanes)
        const int64_t i = i0 + threadIdx.x;
        const bool in = i < n;
        uint4 v = in ? ((const uint4*)x)[i] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
            f[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
        }
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
        amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                               __builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false)));
        amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                               __builtin_bit_cast(int, amax), 0x4E, 0xF, 0xF, false)));
        const int e8 = e8m0_exponent(amax);
        // 2^-e8 exactly; 2^-127 is an fp32 subnormal
        const float inv = e8 == 127 ? __uint_as_float(1u << 22) : __uint_as_float((uint32_t)(127 - e8) << 23);
        uint32_t out[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            out[q] = cvt_e4m3x4(f[4 * q] * inv, f[4 * q + 1] * inv, f[4 * q + 2] * inv, f[4 * q + 3] * inv);
        }
        if (in) {
            ((uint2*)codes)[i] = make_uint2(out[0], out[1]);
            if ((i & 3) == 0) {
                const int64_t t = (i / 4) / nb, b = (i / 4) - t * nb;
                scales[t * nb + b] = (uint8_t)(e8 + 127);
            }
        }
    }
}

hipError_t launch_quant_x(const uint16_t* x, int64_t T_cap, const int32_t* live, int H,
                          uint8_t* codes, uint8_t* scales, int num_cu, hipStream_t s)
{
    hipLaunchKernelGGL(quant_x_mx_kernel, dim3(num_cu * 8), dim3(256), 0, s, x, T_cap, live, H,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                            int F, int num_cu, hipStream_t s)
{
    uint16_t* p1 = (uint16_t*)kbuf;
    uint16_t* p2 = p1 + (int64_t)E * 2 * F * H;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(num_cu * 8), dim3(256), 0, s, w1, p1, E, 2 * F, H, F, 1);
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(num_cu * 8), dim3(256), 0, s, w2, p2, E, H, F, F, 0);
    return hipGetLastError();
}

static size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// Section sizes of the MXFP8 buffer (codes and scales of FC1, then FC2).
void mx_section_bytes(int E, int H, int F, size_t* c1, size_t* c2, size_t* s1, size_t* s2)
{
    auto codes = [&](int64_t N, int64_t K) { return (size_t)E * (N / 16) * ((K + 127) / 128) * 2048; };
    auto scl = [&](int64_t N, int64_t K) {
        int64_t KS = (K + 127) / 128;
        return (size_t)E * (N / 16) * ((KS + 3) / 4) * 256;
    };
    *c1 = up256(codes(2 * F, H));
    *c2 = up256(codes(H, F));
    *s1 = up256(scl(2 * F, H));
    *s2 = up256(scl(H, F));
}

// Section sizes of the MXFP4 buffer (codes and scales of FC1, then FC2).
void mx4_section_bytes(int E, int H, int F, size_t* c1, size_t* c2, size_t* s1, size_t* s2)
{
    auto codes = [&](int64_t N, int64_t K) { return (size_t)E * (N / 16) * ((K + 127) / 128) * 1024; };
    auto scl = [&](int64_t N, int64_t K) {
        int64_t KS = (K + 127) / 128;
        return (size_t)E * (N / 16) * ((KS + 3) / 4) * 256;
    };
    *c1 = up256(codes(2 * F, H));
    *c2 = up256(codes(H, F));
    *s1 = up256(scl(2 * F, H));
    *s2 = up256(scl(H, F));
}

hipError_t launch_pack_mxfp4(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                             int F, int num_cu, hipStream_t s)
{
    size_t c1, c2, s1, s2;
    mx4_section_bytes(E, H, F, &c1, &c2, &s1, &s2);
    uint8_t* pc1 = kbuf;
    uint8_t* pc2 = pc1 + c1;
    uint8_t* ps1 = pc2 + c2;
    uint8_t* ps2 = ps1 + s1;
    hipLaunchKernelGGL(pack_mx4_kernel, dim3(num_cu * 8), dim3(256), 0, s, w1, pc1, ps1, E, 2 * F, H, F, 1);
    hipLaunchKernelGGL(pack_mx4_kernel, dim3(num_cu * 8), dim3(256), 0, s, w2, pc2, ps2, E, H, F, F, 0);
    return hipGetLastError();
}

hipError_t launch_pack_mxfp8(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                             int F, int num_cu, hipStream_t s)
{
    size_t c1, c2, s1, s2;
    mx_section_bytes(E, H, F, &c1, &c2, &s1, &s2);
    uint8_t* pc1 = kbuf;
    uint8_t* pc2 = pc1 + c1;
    uint8_t* ps1 = pc2 + c2;
    uint8_t* ps2 = ps1 + s1;
    hipLaunchKernelGGL(pack_mx_kernel, dim3(num_cu * 8), dim3(256), 0, s, w1, pc1, ps1, E, 2 * F, H, F, 1);
    hipLaunchKernelGGL(pack_mx_kernel, dim3(num_cu * 8), dim3(256), 0, s, w2, pc2, ps2, E, H, F, F, 0);
    return hipGetLastError();
}

}  // namespace moe
