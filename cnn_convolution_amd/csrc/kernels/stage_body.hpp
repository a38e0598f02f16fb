// Filter staging, element by element: the bodies shared by the stand-alone
// staging kernels and by the pack launch that carries the staging along
// (extra workgroups ahead of the pack's own). Orders:
//   fp32 path (row-interleaved windows):
//       out[cb][ci][kh][kw][j] = w[cb*16 + j][ci][kh][kw]      (j < 16)
//   fp16/bf16 path (channels-last windows):
//       out[co][(kw*KH + kh)*Cin_pad + ci] = w[co][ci][kh][kw]
// Cells with no filter value (padded channels, rows, K tail) are zero.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace im2win {

// the staging job a pack launch may carry (blocks == 0: none)
struct StageFold {
    const void *w;
    void *out;
    int Cout, Cin, KH, KW, Cin_pad, rows, row_len;
    int blocks;              // workgroups given to the staging, ahead of the pack's
};

// Indices are 32-bit: every buffer holds fewer than 2^31 elements (checked
// by the library before anything is launched); the loop counters are
// unsigned so that e + step (< 2^31 + 2^24) cannot wrap.
template <typename E>
__device__ __forceinline__ void stage_row_elems(const E *__restrict__ w, E *__restrict__ out, int Cout,
                                                int K, int rows, unsigned first, unsigned step)
{
    // out index = (cb*K + k)*16 + j ; co = cb*16 + j ; w index = co*K + k
    const unsigned total = unsigned(rows) * unsigned(K);
    for (unsigned e = first; e < total; e += step) {
        const int j = int(e & 15u);
        const int t = int(e >> 4);
        const int cb = t / K;
        const int k = t - cb * K;
        const int co = cb * 16 + j;
        out[e] = co < Cout ? w[co * K + k] : E(0);
    }
}

template <typename E>
__device__ __forceinline__ void stage_cl_elems(const E *__restrict__ w, E *__restrict__ out, int Cout,
                                               int Cin, int KH, int KW, int Cin_pad, int row_len,
                                               unsigned first, unsigned step)
{
    const int krun = KW * KH * Cin_pad;
    const unsigned total = unsigned(Cout) * unsigned(row_len);
    for (unsigned e = first; e < total; e += step) {
        const int co = int(e / unsigned(row_len));
        const int k = int(e) - co * row_len;
        E v = E(0);
        if (k < krun) {
            const int pos = k / Cin_pad;
            const int ci = k - pos * Cin_pad;
            const int kw = pos / KH;
            const int kh = pos - kw * KH;
            if (ci < Cin) v = w[((co * Cin + ci) * KH + kh) * KW + kw];
        }
        out[e] = v;
    }
}

// Channels-last order, 16 bytes at a time: one 8-channel group of one
// filter position per step, gathered from w with the channel stride KH*KW
// and stored as one 16-byte vector. For 16-bit elements with Cin_pad and
// row_len multiples of 8 (out rows 16-byte aligned); the caller checks.
__device__ __forceinline__ void stage_cl_vec8(const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
                                              int Cout, int Cin, int KH, int KW, int Cin_pad, int row_len,
                                              unsigned first, unsigned step)
{
    const int krun = KW * KH * Cin_pad;
    const int gpr = row_len >> 3;                 // 8-element groups per row
    const unsigned total = unsigned(Cout) * unsigned(gpr);
    const int taps = KH * KW;
    for (unsigned gi = first; gi < total; gi += step) {
        const int co = int(gi / unsigned(gpr));
        const int k = (int(gi) - co * gpr) * 8;
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        if (k < krun) {
            const int pos = k / Cin_pad;
            const int ci0 = k - pos * Cin_pad;
            const int kw = pos / KH;
            const int kh = pos - kw * KH;
            const uint16_t *src = w + (co * Cin + ci0) * taps + kh * KW + kw;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h = ci0 + e < Cin ? uint32_t(src[e * taps]) : 0u;
                v[e >> 1] |= h << (16 * (e & 1));
            }
        }
        *reinterpret_cast<uint4 *>(out + size_t(co) * row_len + k) = uint4{v[0], v[1], v[2], v[3]};
    }
}

}  // namespace im2win
