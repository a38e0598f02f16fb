// Filter staging: reorder w[Cout][Cin][KH][KW] into the K order in which the
// window-GEMM walks a window. The im2win paper keeps the filter in a layout
// whose taps follow the window's element order ("Enabling Memory-efficient
// Im2win Convolution ...", Sec. III-C, end); here that order is:
//   fp32 path (row-interleaved windows):
//       out[cb][ci][kh][kw][j] = w[cb*16 + j][ci][kh][kw]      (j < 16)
//     16 output channels innermost, so one scalar load brings the 16 filter
//     values a wave multiplies against one window element;
//   fp16/bf16 path (channels-last windows):
//       out[co][(kw*KH + kh)*Cin_pad + ci] = w[co][ci][kh][kw]
//     matching the contiguous window run (kw outer, kh, channels inner).
// Cells with no filter value (padded channels, rows, K tail) are zero.
// Pure copies of raw bits (element bodies in stage_body.hpp; the forward
// call usually runs them inside the first pack launch instead).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "stage_body.hpp"

namespace im2win {
namespace {

template <typename E>
__global__ __launch_bounds__(256) void stage_row_kernel(const E *__restrict__ w, E *__restrict__ out,
                                                        int Cout, int K, int rows)
{
    stage_row_elems(w, out, Cout, K, rows, blockIdx.x * blockDim.x + threadIdx.x,
                    gridDim.x * blockDim.x);
}

template <typename E>
__global__ __launch_bounds__(256) void stage_cl_kernel(const E *__restrict__ w, E *__restrict__ out,
                                                       int Cout, int Cin, int KH, int KW,
                                                       int Cin_pad, int row_len)
{
    stage_cl_elems(w, out, Cout, Cin, KH, KW, Cin_pad, row_len,
                   blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

__global__ __launch_bounds__(256) void stage_cl_vec8_kernel(const uint16_t *__restrict__ w,
                                                            uint16_t *__restrict__ out, int Cout, int Cin,
                                                            int KH, int KW, int Cin_pad, int row_len)
{
    stage_cl_vec8(w, out, Cout, Cin, KH, KW, Cin_pad, row_len, blockIdx.x * blockDim.x + threadIdx.x,
                  gridDim.x * blockDim.x);
}

// NHWC filters (w [Cout][KH][KW][Cin]) into the channels-last K order:
// out[co][(kw*KH + kh)*Cin_pad + ci] = w[co][kh][kw][ci]; every element of
// the rows x row_len staged filter is written (zero past Cout, Cin and K).
__global__ __launch_bounds__(256) void stage_cl_ohwi_kernel(const uint16_t *__restrict__ w,
                                                            uint16_t *__restrict__ out, int Cout, int Cin,
                                                            int KH, int KW, int Cin_pad, int rows, int row_len)
{
    const int krun = KW * KH * Cin_pad;
    const unsigned total = unsigned(rows) * unsigned(row_len);
    for (unsigned e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
        const int co = int(e / unsigned(row_len));
        const int k = int(e) - co * row_len;
        uint16_t v = 0;
        if (co < Cout && k < krun) {
            const int pos = k / Cin_pad;
            const int ci = k - pos * Cin_pad;
            const int kw = pos / KH;
            const int kh = pos - kw * KH;
            if (ci < Cin) v = w[((co * KH + kh) * KW + kw) * Cin + ci];
        }
        out[e] = v;
    }
}

unsigned grid_for(int64_t total)
{
    int64_t b = (total + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return unsigned(b);
}

}  // namespace

hipError_t launch_stage_row(const StageArgs &a, hipStream_t s)
{
    const int K = a.Cin * a.KH * a.KW;
    const dim3 grid(grid_for(int64_t(a.rows) * K));
    if (a.esize == 4)
        hipLaunchKernelGGL(stage_row_kernel<uint32_t>, grid, dim3(256), 0, s,
                           static_cast<const uint32_t *>(a.w), static_cast<uint32_t *>(a.out),
                           a.Cout, K, a.rows);
    else
        hipLaunchKernelGGL(stage_row_kernel<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.w), static_cast<uint16_t *>(a.out),
                           a.Cout, K, a.rows);
    return hipGetLastError();
}

hipError_t launch_stage_cl(const StageArgs &a, hipStream_t s)
{
    if (a.ohwi) {
        if (a.esize != 2) return hipErrorInvalidValue;
        hipLaunchKernelGGL(stage_cl_ohwi_kernel, dim3(grid_for(int64_t(a.rows) * a.row_len)), dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.w), static_cast<uint16_t *>(a.out), a.Cout, a.Cin,
                           a.KH, a.KW, a.Cin_pad, a.rows, a.row_len);
        return hipGetLastError();
    }
    if (a.esize == 2 && a.Cin_pad % 8 == 0 && a.row_len % 8 == 0) {
        // one 16-byte output vector per thread
        hipLaunchKernelGGL(stage_cl_vec8_kernel, dim3(grid_for(int64_t(a.Cout) * (a.row_len / 8))), dim3(256),
                           0, s, static_cast<const uint16_t *>(a.w), static_cast<uint16_t *>(a.out),
                           a.Cout, a.Cin, a.KH, a.KW, a.Cin_pad, a.row_len);
        return hipGetLastError();
    }
    const dim3 grid(grid_for(int64_t(a.rows) * a.row_len));
    if (a.esize == 4)
        hipLaunchKernelGGL(stage_cl_kernel<uint32_t>, grid, dim3(256), 0, s,
                           static_cast<const uint32_t *>(a.w), static_cast<uint32_t *>(a.out),
                           a.Cout, a.Cin, a.KH, a.KW, a.Cin_pad, a.row_len);
    else
        hipLaunchKernelGGL(stage_cl_kernel<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.w), static_cast<uint16_t *>(a.out),
                           a.Cout, a.Cin, a.KH, a.KW, a.Cin_pad, a.row_len);
    return hipGetLastError();
}

}  // namespace im2win
