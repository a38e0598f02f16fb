// Epilogue of every convolution kernel: one fp32 accumulator -> one element
// of y (OutSpec, launch.hpp):
//
//   v = scale[co] * (acc + bias[co])        (either factor optional)
//
// the bias of the convolution call of "Unifying Convolutions and GEMM"
// (Sec. 5) and the learned per-channel scale of "Fast and Memory-Efficient
// Wavelet Convolutions via I/O-Aware Reformulation" (scale folding: by
// linearity s * (X * W + b) = X * (s W) + s b, so the scale costs no pass of
// its own), applied here to the fp32 accumulator so that the folded weights
// are never rounded to the input dtype; then rounded once, to nearest even,
// to the storage type of y and stored at its NCHW or NHWC offset.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "lds_dma.hpp"

namespace im2win {

__device__ __forceinline__ float out_value(const OutSpec &o, int co, float acc)
{
    float v = acc;
    if (o.bias) v += o.bias[co];
    if (o.scale) v *= o.scale[co];
    return v;
}

// bfloat16 bits of an fp32 value, rounded to nearest even (the low 16 bits
// decide, ties to the even result); a NaN stays a quiet NaN
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// binary16 bits of an fp32 value (the conversion instruction rounds to
// nearest even in the default mode)
__device__ __forceinline__ uint32_t f16_bits(float f)
{
    return uint32_t(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

__device__ __forceinline__ uint32_t half_bits(const OutSpec &o, float v)
{
    return o.type == 1 ? f16_bits(v) : bf16_bits(v);
}

// element offset of output (n, co, p), p = ho * Wo + wo
__device__ __forceinline__ int64_t out_offset(const OutSpec &o, int64_t n, int co, int64_t p)
{
    return o.nhwc ? (n * o.plane + p) * o.Cout + co : (n * o.Cout + co) * o.plane + p;
}

// v (already through out_value) at element offset off
__device__ __forceinline__ void out_put(const OutSpec &o, int64_t off, float v)
{
    if (o.type == 0)
        static_cast<float *>(o.y)[off] = v;
    else
        static_cast<uint16_t *>(o.y)[off] = uint16_t(half_bits(o, v));
}

// one accumulator of output (n, co, p)
__device__ __forceinline__ void out_store(const OutSpec &o, int64_t n, int co, int64_t p, float acc)
{
    out_put(o, out_offset(o, n, co, p), out_value(o, co, acc));
}

// 4 accumulators of channel co at consecutive elements off .. off+3 of y (NCHW
// positions p .. p+3 of one plane), off a multiple of 4: one 16-byte (fp32)
// or 8-byte (fp16/bf16) store
__device__ __forceinline__ void out_store4(const OutSpec &o, int64_t off, int co, const floatx4_t &acc)
{
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = out_value(o, co, acc[k]);
    if (o.type == 0) {
        *reinterpret_cast<floatx4_t *>(static_cast<float *>(o.y) + off) = floatx4_t{v[0], v[1], v[2], v[3]};
    } else {
        const uint2 h{half_bits(o, v[0]) | (half_bits(o, v[1]) << 16), half_bits(o, v[2]) | (half_bits(o, v[3]) << 16)};
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o.y) + off) = h;
    }
}

// 4 accumulators of channels co0 .. co0+3 (co0 a multiple of 4) at output
// position p of image img: the layout of the window-GEMM kernels' lanes
// (D[co][column]). NHWC y with Cout % 4 == 0: one vector store of the 4
// channels; otherwise one store per channel below Cout.
__device__ __forceinline__ void out_store_cols4(const OutSpec &o, int64_t img, int co0, int64_t p,
                                                const floatx4_t &acc)
{
    if (o.nhwc && (o.Cout & 3) == 0) {
        if (co0 >= o.Cout) return;
        const int64_t off = (img * o.plane + p) * o.Cout + co0;
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = out_value(o, co0 + k, acc[k]);
        if (o.type == 0) {
            *reinterpret_cast<floatx4_t *>(static_cast<float *>(o.y) + off) = floatx4_t{v[0], v[1], v[2], v[3]};
        } else {
            const uint2 h{half_bits(o, v[0]) | (half_bits(o, v[1]) << 16),
                          half_bits(o, v[2]) | (half_bits(o, v[3]) << 16)};
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o.y) + off) = h;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (co0 + k < o.Cout) out_store(o, img, co0 + k, p, acc[k]);
}

}  // namespace im2win
