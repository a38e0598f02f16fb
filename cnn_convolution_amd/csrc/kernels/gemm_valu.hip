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
#include "epilogue.hpp"
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

// Wave -> (channel split, channel block, column group). The 4 waves of a
// workgroup form ks x waves_m x waves_n; waves that differ only in the split
// index own the same outputs and sum their partials through LDS at the end.
struct ValuMap {
    int ksi, cb, g;
    bool active;
};

__device__ __forceinline__ ValuMap valu_map(int wave, int lane, int ks, int waves_m, int tiles_m,
                                            int Cout)
{
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int waves_n = 4 / (ks * waves_m);
    const int ksi = wave % ks;
    const int rest = wave / ks;
    const int wm = rest % waves_m, wn = rest / waves_m;
    ValuMap m;
    m.ksi = ksi;
    m.cb = tm * waves_m + wm;                  // 16-channel block of this wave
    m.g = (tn * waves_n + wn) * 64 + lane;     // column group of this lane
    m.active = m.cb * MT < Cout;
    return m;
}

// Sum the ks channel-split partials of acc into the split-0 wave (fixed order).
template <int NT>
__device__ __forceinline__ void valu_reduce(float (&acc)[MT][NT], float *red, int wave, int lane,
                                            int ks)
{
    const int ksi = wave % ks;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (ksi != 0) {
#pragma unroll
            for (int m = 0; m < MT / 2; ++m)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    red[((wave * (MT / 2) + m) * NT + j) * 64 + lane] = acc[h * (MT / 2) + m][j];
        }
        __syncthreads();
        if (ksi == 0) {
            for (int k = 1; k < ks; ++k) {
#pragma unroll
                for (int m = 0; m < MT / 2; ++m)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[h * (MT / 2) + m][j] +=
                            red[(((wave + k) * (MT / 2) + m) * NT + j) * 64 + lane];
            }
        }
        __syncthreads();
    }
}

template <int NT>
__device__ __forceinline__ void valu_store(const float (&acc)[MT][NT], const OutSpec &o, int cb,
                                           int rl, int row0, int wo0, int nvalid, int Ho, int Wo,
                                           int Cout)
{
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const bool vec_ok = (Wo % 4) == 0;
    const int64_t p = int64_t(ho) * Wo + wo0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int co = cb * MT + m;
        if (co >= Cout) continue;
        if (o.plain) {
            store_cols<NT>(static_cast<float *>(o.y) + (int64_t(n) * Cout + co) * o.plane + p, acc[m], nvalid,
                           vec_ok);
        } else {
            with_ytype(o, [&](auto tc) {
                constexpr int T = decltype(tc)::value;
                const ChanEpi e = chan_epi(o, co);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nvalid) put1<T>(o.y, out_offset(o, n, co, p + j), epi_apply(e, acc[m][j]));
            });
        }
    }
}

// Shapes known at compile time: KH, KW, S, NT.
template <int KH, int KW, int S, int NT>
__global__ __launch_bounds__(256) void gemm_valu_kernel(
    const float *__restrict__ win, const float *__restrict__ wst, const OutSpec o, int rows,
    int row0, int Cin, int pos_pad, int row_elems, int Ho, int Wo, int Cout, int slots,
    int waves_m, int tiles_m, int ks)
{
    constexpr int L = ((NT - 1) * S + KW) * KH;   // run length per channel
    constexpr int LV = (L + 3) / 4;               // 16-byte vectors per run
    __shared__ float red[4 * (MT / 2) * NT * 64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const ValuMap mp = valu_map(wave, lane, ks, waves_m, tiles_m, Cout);
    const int rl = mp.g / slots;
    const int slot = mp.g - rl * slots;
    const bool lane_ok = mp.active && rl < rows;
    const int wo0 = slot * NT;
    const int nvalid = lane_ok ? min(NT, Wo - wo0) : 0;
    const int lvalid = nvalid > 0 ? ((nvalid - 1) * S + KW) * KH : 0;
    const float *run = win + int64_t(lane_ok ? rl : 0) * row_elems + wo0 * S * KH;
    const float *wcb = wst + int64_t(mp.active ? mp.cb : 0) * Cin * (KH * KW * MT);

    float acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[m][j] = 0.f;

    if (mp.active) {
        float v[LV * 4], vn[LV * 4];
        // Loads are unconditional: a vector past this lane's valid run reads
        // the run start instead (a load under a branch would make the compiler
        // wait for it at the join). Values past the valid run only ever meet
        // the columns j >= nvalid, which are never stored, so no masking.
        auto load_run = [&](const float *src, float (&dst)[LV * 4]) {
#pragma unroll
            for (int i = 0; i < LV; ++i) {
                const float4 q = *reinterpret_cast<const float4 *>(src + (4 * i < lvalid ? 4 * i : 0));
                dst[4 * i] = q.x;
                dst[4 * i + 1] = q.y;
                dst[4 * i + 2] = q.z;
                dst[4 * i + 3] = q.w;
            }
        };
        load_run(run + int64_t(mp.ksi < Cin ? mp.ksi : 0) * pos_pad, v);
        for (int ci = mp.ksi; ci < Cin; ci += ks) {
            // next channel of this split (the last iteration reloads its own run)
            load_run(run + int64_t(ci + ks < Cin ? ci + ks : ci) * pos_pad, vn);
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
    }
    if (ks > 1) valu_reduce<NT>(acc, red, wave, lane, ks);
    if (mp.ksi != 0 || nvalid <= 0) return;
    valu_store<NT>(acc, o, mp.cb, rl, row0, wo0, nvalid, Ho, Wo, Cout);
}

// Any shape: taps loaded one element at a time (used for shapes without a
// compiled specialisation; same work split, NT = 4).
__global__ __launch_bounds__(256) void gemm_valu_generic_kernel(
    const float *__restrict__ win, const float *__restrict__ wst, const OutSpec o, int rows,
    int row0, int Cin, int pos_pad, int row_elems, int KH, int KW, int S, int Ho, int Wo, int Cout,
    int slots, int waves_m, int tiles_m, int ks)
{
    constexpr int NT = 4;
    __shared__ float red[4 * (MT / 2) * NT * 64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const ValuMap mp = valu_map(wave, lane, ks, waves_m, tiles_m, Cout);
    const int rl = mp.g / slots;
    const int slot = mp.g - rl * slots;
    const bool lane_ok = mp.active && rl < rows;
    const int wo0 = slot * NT;
    const int nvalid = lane_ok ? min(NT, Wo - wo0) : 0;
    const float *run = win + int64_t(lane_ok ? rl : 0) * row_elems + wo0 * S * KH;
    const int taps = KH * KW;
    const float *wcb = wst + int64_t(mp.active ? mp.cb : 0) * Cin * taps * MT;

    float acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[m][j] = 0.f;

    if (mp.active) {
        for (int ci = mp.ksi; ci < Cin; ci += ks) {
            const float *rc = run + int64_t(ci) * pos_pad;
            for (int kh = 0; kh < KH; ++kh) {
                for (int kw = 0; kw < KW; ++kw) {
                    const float *a = wcb + (int64_t(ci) * taps + kh * KW + kw) * MT;
                    float x[NT];
#pragma unroll
                    for (int j = 0; j < NT; ++j) x[j] = rc[j < nvalid ? (j * S + kw) * KH + kh : 0];
#pragma unroll
                    for (int j = 0; j < NT; ++j)
#pragma unroll
                        for (int m = 0; m < MT; ++m) acc[m][j] = __builtin_fmaf(a[m], x[j], acc[m][j]);
                }
            }
        }
    }
    if (ks > 1) valu_reduce<NT>(acc, red, wave, lane, ks);
    if (mp.ksi != 0 || nvalid <= 0) return;
    valu_store<NT>(acc, o, mp.cb, rl, row0, wo0, nvalid, Ho, Wo, Cout);
}

struct ValuGrid {
    int slots, waves_m, tiles_m, ks;
    unsigned blocks;
};

ValuGrid valu_grid(const ValuGemmArgs &a, int NT)
{
    ValuGrid g{};
    g.ks = (a.ksplit == 2 || a.ksplit == 4) ? a.ksplit : 1;
    g.slots = (a.Wo + NT - 1) / NT;
    const int cblocks = a.Cout_stage / MT;
    const int per = 4 / g.ks;                  // waves per split index
    g.waves_m = cblocks >= per ? per : (cblocks >= 2 && per >= 2 ? 2 : 1);
    const int waves_n = per / g.waves_m;
    g.tiles_m = (cblocks + g.waves_m - 1) / g.waves_m;
    const int64_t groups = int64_t(a.rows) * g.slots;
    const int64_t tiles_n = (groups + 64 * waves_n - 1) / (64 * waves_n);
    g.blocks = static_cast<unsigned>(g.tiles_m * tiles_n);
    return g;
}

template <int KH, int KW, int S, int NT>
hipError_t launch_spec(const ValuGemmArgs &a, hipStream_t s)
{
    const ValuGrid g = valu_grid(a, NT);
    hipLaunchKernelGGL((gemm_valu_kernel<KH, KW, S, NT>), dim3(g.blocks), dim3(256), 0, s, a.win,
                       a.wst, a.out, a.rows, a.row0, a.Cin, a.pos_pad, a.row_elems, a.Ho, a.Wo, a.Cout,
                       g.slots, g.waves_m, g.tiles_m, g.ks);
    return hipGetLastError();
}

hipError_t launch_generic(const ValuGemmArgs &a, hipStream_t s)
{
    const ValuGrid g = valu_grid(a, 4);
    hipLaunchKernelGGL(gemm_valu_generic_kernel, dim3(g.blocks), dim3(256), 0, s, a.win, a.wst, a.out,
                       a.rows, a.row0, a.Cin, a.pos_pad, a.row_elems, a.KH, a.KW, a.stride, a.Ho,
                       a.Wo, a.Cout, g.slots, g.waves_m, g.tiles_m, g.ks);
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
    if (a.KH == 11 && a.KW == 11 && a.stride == 4) return launch_spec<11, 11, 4, 1>(a, s);
    return launch_generic(a, s);
}

}  // namespace im2win
