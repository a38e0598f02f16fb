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

}  // namespace im2win
