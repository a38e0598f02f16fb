// fp32 window-GEMM on the vector ALUs (the full-precision im2win kernel of
// "Enabling Memory-efficient Im2win Convolution ...", Sec. III-F, on CDNA4).
//
//   y[n][co][ho][wo] = sum_ci sum_kh sum_kw T[r][ci][(wo*s + kw)*KH + kh] * w[co][ci][kh][kw]
//
// with T the row-interleaved window tensor of one chunk of window rows
// r = n*Ho + ho (Eq. (2)) and the window index of the im2win convolution,
// Eq. (3), read as (wo*s + kw)*KH + kh.
//
// Work split. A lane owns NT consecutive output columns of one window row and
// 16 output channels; a wave owns 16 channels, so the filter values it needs
// at each tap are wave-uniform and come in through scalar loads (SGPR
// operands of v_fmac_f32) with no LDS traffic. For each input channel the
// lane's NT windows overlap: their union is ONE contiguous run of
// ((NT-1)*s + KW)*KH elements of T, loaded with 16-byte vector loads and
// reused from registers for all NT*KH*KW taps (the overlapping-window reuse
// of Sec. III-C). The run of the next channel is loaded while the current one
// is consumed (register double buffering). Waves of a workgroup cover
// different channel blocks of the same columns, so their loads of the run hit
// the same L1 lines.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

constexpr int MT = 16;   // output channels per wave (per lane)

template <int NT>
__device__ __forceinline__ void store_cols(float *__restrict__ dst, const float (&a)[NT], int nvalid,
                                           bool vec_ok)
{
    if constexpr (NT == 4) {
        if (vec_ok && nvalid == 4) {
            *reinterpret_cast<float4 *>(dst) = make_float4(a[0], a[1], a[2], a[3]);
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
        if (j < nvalid) dst[j] = a[j];
}

// Shapes known at compile time: KH, KW, S, NT.
template <int KH, int KW, int S, int NT>
__global__ __launch_bounds__(256) void gemm_valu_kernel(
    const float *__restrict__ win, const float *__restrict__ wst, float *__restrict__ y, int rows,
    int row0, int Cin, int pos_pad, int row_elems, int Ho, int Wo, int Cout, int slots,
    int waves_m, int tiles_m)
{
    constexpr int L = ((NT - 1) * S + KW) * KH;   // run length per channel
    constexpr int LV = (L + 3) / 4;               // 16-byte vectors per run
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int waves_n = 4 / waves_m;
    const int wm = wave % waves_m, wn = wave / waves_m;
    const int cb = tm * waves_m + wm;             // 16-channel block of this wave
    if (cb * MT >= Cout) return;
    const int g = (tn * waves_n + wn) * 64 + lane;
    const int rl = g / slots;
    const int slot = g - rl * slots;
    const bool lane_ok = rl < rows;
    const int wo0 = slot * NT;
    const int nvalid = lane_ok ? min(NT, Wo - wo0) : 0;
    const int lvalid = nvalid > 0 ? ((nvalid - 1) * S + KW) * KH : 0;
    const float *run = win + int64_t(lane_ok ? rl : 0) * row_elems + wo0 * S * KH;
    const float *wcb = wst + int64_t(cb) * Cin * (KH * KW * MT);

    float acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[m][j] = 0.f;

    float v[LV * 4], vn[LV * 4];
#pragma unroll
    for (int i = 0; i < LV; ++i) {
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (4 * i < lvalid) q = *reinterpret_cast<const float4 *>(run + 4 * i);
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    for (int ci = 0; ci < Cin; ++ci) {
        if (ci + 1 < Cin) {
            const float *nrun = run + int64_t(ci + 1) * pos_pad;
#pragma unroll
            for (int i = 0; i < LV; ++i) {
                float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
                if (4 * i < lvalid) q = *reinterpret_cast<const float4 *>(nrun + 4 * i);
                vn[4 * i] = q.x; vn[4 * i + 1] = q.y; vn[4 * i + 2] = q.z; vn[4 * i + 3] = q.w;
            }
        }
        const float *wc = wcb + ci * (KH * KW * MT);
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const float *a = wc + (kh * KW + kw) * MT;   // wave-uniform: scalar loads
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const float x = v[(j * S + kw) * KH + kh];
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[m][j] = __builtin_fmaf(a[m], x, acc[m][j]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < LV * 4; ++i) v[i] = vn[i];
    }
    if (nvalid <= 0) return;
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const bool vec_ok = (Wo % 4) == 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int co = cb * MT + m;
        if (co < Cout)
            store_cols<NT>(y + ((int64_t(n) * Cout + co) * Ho + ho) * Wo + wo0, acc[m], nvalid,
                           vec_ok);
    }
}

// Any shape: taps loaded one element at a time (used for shapes without a
// compiled specialisation; same work split, NT = 4).
__global__ __launch_bounds__(256) void gemm_valu_generic_kernel(
    const float *__restrict__ win, const float *__restrict__ wst, float *__restrict__ y, int rows,
    int row0, int Cin, int pos_pad, int row_elems, int KH, int KW, int S, int Ho, int Wo, int Cout,
    int slots, int waves_m, int tiles_m)
{
    constexpr int NT = 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int waves_n = 4 / waves_m;
    const int wm = wave % waves_m, wn = wave / waves_m;
    const int cb = tm * waves_m + wm;
    if (cb * MT >= Cout) return;
    const int g = (tn * waves_n + wn) * 64 + lane;
    const int rl = g / slots;
    const int slot = g - rl * slots;
    const bool lane_ok = rl < rows;
    const int wo0 = slot * NT;
    const int nvalid = lane_ok ? min(NT, Wo - wo0) : 0;
    const float *run = win + int64_t(lane_ok ? rl : 0) * row_elems + wo0 * S * KH;
    const int taps = KH * KW;
    const float *wcb = wst + int64_t(cb) * Cin * taps * MT;

    float acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[m][j] = 0.f;

    for (int ci = 0; ci < Cin; ++ci) {
        const float *rc = run + int64_t(ci) * pos_pad;
        for (int kh = 0; kh < KH; ++kh) {
            for (int kw = 0; kw < KW; ++kw) {
                const float *a = wcb + (int64_t(ci) * taps + kh * KW + kw) * MT;
                float x[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) x[j] = j < nvalid ? rc[(j * S + kw) * KH + kh] : 0.f;
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[m][j] = __builtin_fmaf(a[m], x[j], acc[m][j]);
            }
        }
    }
    if (nvalid <= 0) return;
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const bool vec_ok = (Wo % 4) == 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int co = cb * MT + m;
        if (co < Cout)
            store_cols<NT>(y + ((int64_t(n) * Cout + co) * Ho + ho) * Wo + wo0, acc[m], nvalid,
                           vec_ok);
    }
}

template <int KH, int KW, int S, int NT>
hipError_t launch_spec(const ValuGemmArgs &a, hipStream_t s)
{
    const int slots = (a.Wo + NT - 1) / NT;
    const int cblocks = a.Cout_stage / MT;
    const int waves_m = cblocks >= 4 ? 4 : (cblocks >= 2 ? 2 : 1);
    const int waves_n = 4 / waves_m;
    const int tiles_m = (cblocks + waves_m - 1) / waves_m;
    const int64_t groups = int64_t(a.rows) * slots;
    const int64_t tiles_n = (groups + 64 * waves_n - 1) / (64 * waves_n);
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    hipLaunchKernelGGL((gemm_valu_kernel<KH, KW, S, NT>), grid, dim3(256), 0, s, a.win, a.wst, a.y,
                       a.rows, a.row0, a.Cin, a.pos_pad, a.row_elems, a.Ho, a.Wo, a.Cout, slots,
                       waves_m, tiles_m);
    return hipGetLastError();
}

hipError_t launch_generic(const ValuGemmArgs &a, hipStream_t s)
{
    constexpr int NT = 4;
    const int slots = (a.Wo + NT - 1) / NT;
    const int cblocks = a.Cout_stage / MT;
    const int waves_m = cblocks >= 4 ? 4 : (cblocks >= 2 ? 2 : 1);
    const int waves_n = 4 / waves_m;
    const int tiles_m = (cblocks + waves_m - 1) / waves_m;
    const int64_t groups = int64_t(a.rows) * slots;
    const int64_t tiles_n = (groups + 64 * waves_n - 1) / (64 * waves_n);
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    hipLaunchKernelGGL(gemm_valu_generic_kernel, grid, dim3(256), 0, s, a.win, a.wst, a.y, a.rows,
                       a.row0, a.Cin, a.pos_pad, a.row_elems, a.KH, a.KW, a.stride, a.Ho, a.Wo,
                       a.Cout, slots, waves_m, tiles_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_valu_f32(const ValuGemmArgs &a, hipStream_t s)
{
    // compiled specialisations (NT*S*KH is a multiple of 4: 16-byte aligned runs)
    if (a.KH == 3 && a.KW == 3 && a.stride == 1) return launch_spec<3, 3, 1, 4>(a, s);
    if (a.KH == 3 && a.KW == 3 && a.stride == 2) return launch_spec<3, 3, 2, 4>(a, s);
    if (a.KH == 7 && a.KW == 7 && a.stride == 2) return launch_spec<7, 7, 2, 2>(a, s);
    if (a.KH == 5 && a.KW == 5 && a.stride == 1) return launch_spec<5, 5, 1, 4>(a, s);
    if (a.KH == 1 && a.KW == 1 && a.stride == 1) return launch_spec<1, 1, 1, 4>(a, s);
    return launch_generic(a, s);
}

}  // namespace im2win
