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
#include <type_traits>

#include "../launch.hpp"
#include "lds_dma.hpp"

namespace im2win {

// The per-channel factors of the epilogue, read once per output channel: a
// missing scale is 1 and a missing bias 0, so that v = (acc + b) * s holds in
// every case (exact for the plain case: x + 0 and x * 1 round to x)
struct ChanEpi {
    float s, b;
};

__device__ __forceinline__ ChanEpi chan_epi(const OutSpec &o, int co)
{
    return ChanEpi{o.scale ? o.scale[co] : 1.f, o.bias ? o.bias[co] : 0.f};
}

__device__ __forceinline__ float epi_apply(const ChanEpi &e, float acc) { return (acc + e.b) * e.s; }

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

// storage type of y as a compile-time tag (0 fp32, 1 fp16, 2 bf16)
template <int T>
using YType = std::integral_constant<int, T>;

// run f(YType<t>) for the output type of o: one branch per call, so that the
// loops inside f hold no test of the type
template <typename F>
__device__ __forceinline__ void with_ytype(const OutSpec &o, F &&f)
{
    if (o.type == 1)
        f(YType<1>{});
    else if (o.type == 2)
        f(YType<2>{});
    else
        f(YType<0>{});
}

template <int T>
__device__ __forceinline__ uint32_t half_of(float v)
{
    return T == 1 ? f16_bits(v) : bf16_bits(v);
}

// one value (already through the epilogue) at element offset off
template <int T>
__device__ __forceinline__ void put1(void *y, int64_t off, float v)
{
    if constexpr (T == 0)
        static_cast<float *>(y)[off] = v;
    else
        static_cast<uint16_t *>(y)[off] = uint16_t(half_of<T>(v));
}

// four values at consecutive elements off .. off+3, off a multiple of 4: one
// 16-byte (fp32) or 8-byte (fp16/bf16) store
template <int T>
__device__ __forceinline__ void put4(void *y, int64_t off, float v0, float v1, float v2, float v3)
{
    if constexpr (T == 0) {
        *reinterpret_cast<floatx4_t *>(static_cast<float *>(y) + off) = floatx4_t{v0, v1, v2, v3};
    } else {
        const uint2 h{half_of<T>(v0) | (half_of<T>(v1) << 16), half_of<T>(v2) | (half_of<T>(v3) << 16)};
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + off) = h;
    }
}

// element offset of output (n, co, p), p = ho * Wo + wo
__device__ __forceinline__ int64_t out_offset(const OutSpec &o, int64_t n, int co, int64_t p)
{
    return o.nhwc ? (n * o.plane + p) * o.Cout + co : (n * o.Cout + co) * o.plane + p;
}

// one accumulator of output (n, co, p), for the paths that store element by
// element (T the output type of o)
template <int T>
__device__ __forceinline__ void out_store(const OutSpec &o, int64_t n, int co, int64_t p, float acc)
{
    put1<T>(o.y, out_offset(o, n, co, p), epi_apply(chan_epi(o, co), acc));
}

// 4 accumulators of channels co0 .. co0+3 (co0 a multiple of 4) at output
// position p of image img: the layout of the window-GEMM kernels' lanes
// (D[co][column]). NHWC y with Cout % 4 == 0: one vector store of the 4
// channels; otherwise one store per channel below Cout.
template <int T>
__device__ __forceinline__ void out_store_cols4(const OutSpec &o, int64_t img, int co0, int64_t p,
                                                const floatx4_t &acc)
{
    if (o.nhwc && (o.Cout & 3) == 0) {
        if (co0 >= o.Cout) return;
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = epi_apply(chan_epi(o, co0 + k), acc[k]);
        put4<T>(o.y, (img * o.plane + p) * o.Cout + co0, v[0], v[1], v[2], v[3]);
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (co0 + k < o.Cout) out_store<T>(o, img, co0 + k, p, acc[k]);
}

}  // namespace im2win
