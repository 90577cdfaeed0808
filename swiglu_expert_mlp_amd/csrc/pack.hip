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
#include "common.h"

namespace moe {

__device__ __forceinline__ int64_t fc1_src_row(int64_t packed, int64_t F)
{
    int64_t b = packed >> 6, i = packed & 63;
    return i < 32 ? 32 * b + i : F + 32 * b + (i - 32);
}

// bf16: copy 16-byte pieces of rows into their packed position.
__global__ void __launch_bounds__(256) pack_fc1_bf16_kernel(const uint16_t* __restrict__ w1,
                                                            uint16_t* __restrict__ p1, int E,
                                                            int H, int F)
{
    const int64_t per_row = H / 8;
    const int64_t n = (int64_t)E * 2 * F * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t prow = i / per_row, piece = i - prow * per_row;
        int64_t e = prow / (2 * F), pr = prow - e * 2 * F;
        int64_t src = (e * 2 * F + fc1_src_row(pr, F)) * per_row + piece;
        ((uint4*)p1)[i] = ((const uint4*)w1)[src];
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
        uint32_t c0 = f32_to_e4m3(f[4 * q] * inv), c1 = f32_to_e4m3(f[4 * q + 1] * inv);
        uint32_t c2 = f32_to_e4m3(f[4 * q + 2] * inv), c3 = f32_to_e4m3(f[4 * q + 3] * inv);
        out[q] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    uint4* d4 = (uint4*)codes;
    d4[0] = make_uint4(out[0], out[1], out[2], out[3]);
    d4[1] = make_uint4(out[4], out[5], out[6], out[7]);
    *scale = (uint8_t)(e8 + 127);
}

// Weight rows: one thread per 32-element block; FC1 rows are taken in the
// packed (interleaved) order.
template <bool FC1_ORDER>
__global__ void __launch_bounds__(256) quant_rows_mx_kernel(const uint16_t* __restrict__ src,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t rows, int cols, int F)
{
    const int nb = cols / 32;
    const int64_t n = rows * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = i / nb;
        int b = (int)(i - r * nb);
        int64_t sr = r;
        if constexpr (FC1_ORDER) {
            int64_t e = r / (2 * F), pr = r - e * 2 * F;
            sr = e * 2 * F + fc1_src_row(pr, F);
        }
        quant_block32(src + sr * cols + b * 32, codes + r * cols + b * 32, scales + r * nb + b);
    }
}

// K2: x rows < live quantized per 32-block of H.
__global__ void __launch_bounds__(256) quant_x_mx_kernel(const uint16_t* __restrict__ x,
                                                         int64_t T_cap, const int32_t* __restrict__ live_ptr,
                                                         int H, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales)
{
    const int32_t live = *live_ptr;
    const int64_t T = live < 0 ? 0 : (live > T_cap ? T_cap : live);
    const int nb = H / 32;
    const int64_t n = T * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t t = i / nb;
        int b = (int)(i - t * nb);
        quant_block32(x + t * H + b * 32, codes + t * H + b * 32, scales + t * nb + b);
    }
}

hipError_t launch_quant_x(const uint16_t* x, int64_t T_cap, const int32_t* live, int H,
                          uint8_t* codes, uint8_t* scales, int num_cu, hipStream_t s)
{
    hipLaunchKernelGGL(quant_x_mx_kernel, dim3(num_cu * 4), dim3(256), 0, s, x, T_cap, live, H,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                            int F, int num_cu, hipStream_t s)
{
    uint16_t* p1 = (uint16_t*)kbuf;
    uint16_t* p2 = p1 + (int64_t)E * 2 * F * H;
    hipLaunchKernelGGL(pack_fc1_bf16_kernel, dim3(num_cu * 8), dim3(256), 0, s, w1, p1, E, H, F);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return hipMemcpyAsync(p2, w2, sizeof(uint16_t) * (size_t)E * H * F, hipMemcpyDeviceToDevice, s);
}

static size_t up256(size_t v) { return (v + 255) / 256 * 256; }

hipError_t launch_pack_mxfp8(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                             int F, int num_cu, hipStream_t s)
{
    size_t n1 = (size_t)E * 2 * F * H, n2 = (size_t)E * H * F;
    uint8_t* c1 = kbuf;
    uint8_t* c2 = c1 + up256(n1);
    uint8_t* s1 = c2 + up256(n2);
    uint8_t* s2 = s1 + up256(n1 / 32);
    hipLaunchKernelGGL(quant_rows_mx_kernel<true>, dim3(num_cu * 8), dim3(256), 0, s, w1, c1, s1,
                       (int64_t)E * 2 * F, H, F);
    hipLaunchKernelGGL(quant_rows_mx_kernel<false>, dim3(num_cu * 8), dim3(256), 0, s, w2, c2, s2,
                       (int64_t)E * H, F, F);
    return hipGetLastError();
}

}  // namespace moe
