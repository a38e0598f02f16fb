// Implicit im2win convolution for layers with few input channels (Cin <= 8:
// the RGB stem and its kind), fp16 / bf16 and fp32, on the matrix cores.
//
// With a handful of channels the window rows of Eq. (2) of "Enabling
// Memory-efficient Im2win Convolution with Multi-precision Support on GPU
// CUDA and Tensor Cores" (Sec. III-B) are short in channels and long in
// positions, so they are built in LDS in the channels-last order of the
// window tensor: window row ho holds, for every column w < W_win =
// (Wo - 1) * s + KW and filter row kh, the CP (4 or 8, zero-padded) channels
// of input position (ho * s - pad + kh, w - pad). The window of output
// column wo is then ONE contiguous run of K = KW * KH * CP elements starting
// at wo * s * KH * CP, contracted against the filter held in LDS in the same
// K order (kw, kh, ci) (Sec. III-C Eq. (3), Sec. III-D) — the contraction of the
// window form with the window rows in LDS instead of HBM.
//
// A workgroup of eight waves owns a block of 64 output channels and walks a
// contiguous range of row blocks (R output rows of one image, R * Wo <= 512).
// It puts its filter block into LDS once: 64 rows of Kp elements in the
// window's K order, Kp = K rounded up to the MFMA K step, zero at padded
// channels and past K, each LDS row 16 bytes longer than Kp so that the 16
// rows a fragment read touches fall in different bank groups. Launches of at
// most one workgroup per CU gather it straight from w as stored
// (w[co][ci][kh][kw]: no staging launch, no workspace); larger launches read
// it from the filter staged in that order in the workspace ([Cout][Kp], as
// the channels-last staging writes it), since each of their workgroups would
// otherwise pay for the scattered 2- or 4-byte gathers again.
// Per row block it builds the R window rows (zero outside the image; the
// gathers of the next row block are in flight while this one is contracted
// and stored), and after a barrier each wave contracts its 16-output blocks
// of the flattened R x Wo outputs. The elements past K
// in a run are the next columns' window elements (or zeroed slack at the end
// of a row) and meet zero filter taps. The product is formed transposed,
// D[output][co], and stored as 16-byte vectors, or through an LDS transpose
// where output rows are not a multiple of 4 long (out_blocks.hpp).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../launch.hpp"
#include "lds_dma.hpp"
#include "out_blocks.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

constexpr int kNarrowThreads = 512;

struct NarrowKArgs {
    const void *x;
    const void *w;
    OutSpec out;            // y and its epilogue
    int Cin, H, W, Cout, KH, KW, stride, pad, Ho, Wo;
    int K, Kp;              // window run KW*KH*CP and its padded length
    int Wwin;               // (Wo - 1) * stride + KW
    int L, Lp;              // window row elements W_win*KH*CP, and per row in LDS (with slack)
    int R, row_groups, co_blocks;
    int groups;             // workgroups per 64-channel block (gridDim.x / co_blocks)
    int rowvec;             // CP 4, W % 4 == 0, x aligned: the ROWS kernels (window rows from whole input rows)
};

// dword p (0..3) of a 16-byte vector
__device__ __forceinline__ uint32_t dword_at(const uint4 &v, int p)
{
    return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
}

// One 16-byte vector of the filter block, gathered from w as stored: vector
// v is row r = v / (Kp / VE) (output channel cb*64 + r; rows past Cout read
// row Cout-1 and are never stored) and K elements k0 .. k0+VE-1, k0 = (v mod
// (Kp / VE)) * VE. Element k is channel ci = k mod CP of window position
// k / CP = kw * KH + kh, i.e. w[co][ci][kh][kw], or zero for ci >= Cin or
// k >= K. A vector covers VE / CP whole positions (VE >= CP) or part of one
// (fp32 with CP = 8), so one division by KH per vector.
template <int CP, typename T>
__device__ __forceinline__ uint4 gather_filter_vec(const NarrowKArgs &a, const T *w, int cb, int v)
{
    constexpr int VE = 16 / sizeof(T);
    const int fv_row = a.Kp / VE;
    const int r = v / fv_row;
    const int k0 = (v - r * fv_row) * VE;
    const int co = min(cb * 64 + r, a.Cout - 1);
    const T *wr = w + int64_t(co) * a.Cin * a.KH * a.KW;
    const int pos0 = k0 / CP;
    int kw = pos0 / a.KH;
    int kh = pos0 - kw * a.KH;
    T o[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        int ci;
        if constexpr (VE >= CP) {
            if (e > 0 && e % CP == 0 && ++kh == a.KH) {   // next window position
                kh = 0;
                ++kw;
            }
            ci = e % CP;
        } else {
            ci = k0 % CP + e;
        }
        const bool in = ci < a.Cin && k0 + e < a.K;
        const T val = wr[in ? (ci * a.KH + kh) * a.KW + kw : 0];   // every load in bounds
        o[e] = in ? val : T(0);
    }
    uint4 q;
    __builtin_memcpy(&q, o, 16);
    return q;
}

// Vector v of the filter block: gathered from w as stored (GATHER), or read
// from the staged rows [Cout][Kp] in the workspace.
template <int CP, bool GATHER, typename T>
__device__ __forceinline__ uint4 filter_vec(const NarrowKArgs &a, const T *w, int cb, int v)
{
    if constexpr (GATHER) {
        return gather_filter_vec<CP>(a, w, cb, v);
    } else {
        constexpr int VE = 16 / sizeof(T);
        const int fv_row = a.Kp / VE;
        const int r = v / fv_row;
        const int row = min(cb * 64 + r, a.Cout - 1);
        return *reinterpret_cast<const uint4 *>(w + int64_t(row) * a.Kp + (v - r * fv_row) * VE);
    }
}

// The filter block into LDS rows of FS elements, FB vectors per thread in
// flight at a time.
template <int CP, bool GATHER, int FB, typename T>
__device__ __forceinline__ void load_filter(const NarrowKArgs &a, const T *w, T *fl, int FS, int cb, int tid)
{
    constexpr int V = 16 / sizeof(T);
    const int fv_row = a.Kp / V;
    const int fvec = 64 * fv_row;
    for (int f0 = 0; f0 < fvec; f0 += FB * kNarrowThreads) {
        uint4 fv[FB];
#pragma unroll
        for (int j = 0; j < FB; ++j)
            fv[j] = filter_vec<CP, GATHER>(a, w, cb, min(f0 + tid + j * kNarrowThreads, fvec - 1));
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int v = f0 + tid + j * kNarrowThreads;
            if (v < fvec) {
                const int r = v / fv_row;
                *reinterpret_cast<uint4 *>(fl + r * FS + (v - r * fv_row) * V) = fv[j];
            }
        }
    }
}

// The rw window rows of output rows ho0 .. ho0+rw-1: units (row i, filter row
// kh, window column wc), consecutive lanes on consecutive input columns so
// that each load instruction reads one contiguous stretch of an input row; a
// unit writes the CP channels of position (wc, kh) as one vector. A thread
// holds UB units per round: fetch_window issues a round's loads into
// registers, put_window writes them (and, on the last round, zeroes the slack
// after each row), so that the next row block's loads can be in flight while
// the current one is contracted.
template <int CP, int UB, typename T>
struct WinRegs {
    T v[UB][CP];
    bool in[UB];
};

// Unit u = (i * KH + kh) * Wwin + wc as its digits, and a step of
// kNarrowThreads units as digits (di, dkh, dwc) of the same radices, so that
// a thread walks its units with adds and compares instead of two divisions
// each (STEP; measured on the fp16 stem, one row block per workgroup: 50.1
// -> 41.8 us). The persistent form, whose registers are already spilling
// with the next block's gathers held, keeps the divisions (stepping there
// measured 142 -> 154 us on the fp32 stem).
struct UnitPos {
    int i, kh, wc;
};

__device__ __forceinline__ UnitPos unit_pos(const NarrowKArgs &a, int u)
{
    const int upr = a.KH * a.Wwin;
    UnitPos p;
    p.i = u / upr;
    const int q = u - p.i * upr;
    p.kh = q / a.Wwin;
    p.wc = q - p.kh * a.Wwin;
    return p;
}

__device__ __forceinline__ void unit_next(const NarrowKArgs &a, UnitPos &p, const UnitPos &d)
{
    p.wc += d.wc;
    p.kh += d.kh;
    p.i += d.i;
    if (p.wc >= a.Wwin) {
        p.wc -= a.Wwin;
        ++p.kh;
    }
    if (p.kh >= a.KH) {
        p.kh -= a.KH;
        ++p.i;
    }
}

template <bool STEP, int CP, int UB, typename T>
__device__ __forceinline__ void fetch_window(const NarrowKArgs &a, const T *ximg, int ho0, int rw, int u0,
                                             int tid, WinRegs<CP, UB, T> &r)
{
    const int units = rw * a.KH * a.Wwin;
    const int HW = a.H * a.W;
    const UnitPos d = unit_pos(a, kNarrowThreads);
    UnitPos p = unit_pos(a, u0 + tid);
#pragma unroll
    for (int j = 0; j < UB; ++j) {
        if constexpr (STEP) {
            if (j > 0) unit_next(a, p, d);
        } else {
            p = unit_pos(a, min(u0 + tid + j * kNarrowThreads, units - 1));
        }
        const int ih = (ho0 + p.i) * a.stride - a.pad + p.kh;
        const int iw = p.wc - a.pad;
        // (without STEP the unit is clamped to the last one; put_window skips
        // units past the end in both forms)
        r.in[j] = (!STEP || u0 + tid + j * kNarrowThreads < units) && unsigned(ih) < unsigned(a.H) &&
                  unsigned(iw) < unsigned(a.W);
        const int src = r.in[j] ? ih * a.W + iw : 0;
#pragma unroll
        for (int c = 0; c < CP; ++c) r.v[j][c] = ximg[min(c, a.Cin - 1) * HW + src];
    }
}

template <bool STEP, int CP, int UB, typename T>
__device__ __forceinline__ void put_window(const NarrowKArgs &a, T *win, int rw, int u0, int tid,
                                           const WinRegs<CP, UB, T> &r)
{
    constexpr int V = 16 / sizeof(T);
    const int units = rw * a.KH * a.Wwin;
    const UnitPos d = unit_pos(a, kNarrowThreads);
    UnitPos p = unit_pos(a, u0 + tid);
#pragma unroll
    for (int j = 0; j < UB; ++j) {
        const int u = u0 + tid + j * kNarrowThreads;
        if (u >= units) break;
        if constexpr (STEP) {
            if (j > 0) unit_next(a, p, d);
        } else {
            p = unit_pos(a, u);
        }
        const int i = p.i, kh = p.kh, wc = p.wc;
        T o[CP];
#pragma unroll
        for (int c = 0; c < CP; ++c) o[c] = (r.in[j] && c < a.Cin) ? r.v[j][c] : T(0);
        T *dst = win + i * a.Lp + (wc * a.KH + kh) * CP;
        if constexpr (CP * sizeof(T) == 8) {
            uint2 q2;
            __builtin_memcpy(&q2, o, 8);
            *reinterpret_cast<uint2 *>(dst) = q2;
        } else {
#pragma unroll
            for (int c = 0; c < CP; c += V) {
                uint4 q4;
                __builtin_memcpy(&q4, o + c, 16);
                *reinterpret_cast<uint4 *>(dst + c) = q4;
            }
        }
    }
    if (u0 + UB * kNarrowThreads >= units) {
        const int slack = a.Lp - a.L;
        for (int v = tid; v < rw * slack; v += kNarrowThreads) {
            const int i = v / slack;
            win[i * a.Lp + a.L + (v - i * slack)] = T(0);
        }
    }
}

// One row block per workgroup: the filter block's vectors (FB per thread) and
// the window units (UB per thread) of a round all in flight together, then
// written; normally a single round.
template <int CP, bool GATHER, int FB, int UB, typename T>
__device__ __forceinline__ void load_block(const NarrowKArgs &a, const T *ximg, const T *w, T *fl, T *win,
                                           int FS, int cb, int ho0, int rw, int tid)
{
    constexpr int V = 16 / sizeof(T);
    const int fv_row = a.Kp / V;
    const int fvec = 64 * fv_row;
    const int units = rw * a.KH * a.Wwin;
    for (int f0 = 0, u0 = 0; f0 < fvec || u0 < units; f0 += FB * kNarrowThreads, u0 += UB * kNarrowThreads) {
        uint4 fv[FB];
#pragma unroll
        for (int j = 0; j < FB; ++j)
            fv[j] = filter_vec<CP, GATHER>(a, w, cb, min(f0 + tid + j * kNarrowThreads, fvec - 1));
        WinRegs<CP, UB, T> wr;
        if (u0 < units) fetch_window<true>(a, ximg, ho0, rw, u0, tid, wr);
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int v = f0 + tid + j * kNarrowThreads;
            if (v < fvec) {
                const int r = v / fv_row;
                *reinterpret_cast<uint4 *>(fl + r * FS + (v - r * fv_row) * V) = fv[j];
            }
        }
        if (u0 < units) put_window<true>(a, win, rw, u0, tid, wr);
    }
}

// Window rows from whole input rows (CP = 4, W % 4 == 0, x aligned to 4
// elements): unit (input row r of the block, 4-column group g) reads the 4
// columns 4g .. 4g+3 of each channel (one 8-byte load in half precision,
// 16-byte in fp32; consecutive lanes on consecutive groups), turns them in
// registers into 4 positions of 4 channels, and writes each position into
// every window row (i, kh) that interleaves this input row (kh = r - i *
// stride), so that an input element is read once per row block rather than
// once per window row holding it (7x7 stride 2, 4 output rows: 13 input rows
// against 28 window row segments), with a quarter of the load instructions
// and of the registers a prefetched round holds. The window's padding columns
// (wc < pad, wc >= pad + W) are zeroed apart.
constexpr int kRowVecUnits = 2;                      // units per thread per round

template <typename T>
struct RowRegs {
    using Q = std::conditional_t<sizeof(T) == 2, uint2, uint4>;   // 4 columns of one channel
    Q v[kRowVecUnits][4];
};

template <typename T>
__device__ __forceinline__ int row_units(const NarrowKArgs &a, int rw)
{
    return ((rw - 1) * a.stride + a.KH) * (a.W >> 2);
}

template <typename T>
__device__ __forceinline__ void fetch_rows(const NarrowKArgs &a, const T *ximg, int ho0, int rw, int u0, int tid,
                                           RowRegs<T> &q)
{
    using Q = typename RowRegs<T>::Q;
    const int G4 = a.W >> 2;
    const int units = row_units<T>(a, rw);
    const int HW = a.H * a.W;
#pragma unroll
    for (int j = 0; j < kRowVecUnits; ++j) {
        const int u = min(u0 + tid + j * kNarrowThreads, units - 1);
        const int r = u / G4;
        const int g = u - r * G4;
        const int ih = ho0 * a.stride - a.pad + r;
        const int src = (unsigned(ih) < unsigned(a.H) ? ih * a.W : 0) + 4 * g;   // every load in bounds
#pragma unroll
        for (int c = 0; c < 4; ++c) q.v[j][c] = *reinterpret_cast<const Q *>(ximg + min(c, a.Cin - 1) * HW + src);
    }
}

template <typename T>
__device__ __forceinline__ void put_rows(const NarrowKArgs &a, T *win, int ho0, int rw, int u0, int tid,
                                         const RowRegs<T> &q)
{
    using Q = typename RowRegs<T>::Q;
    const int G4 = a.W >> 2;
    const int units = row_units<T>(a, rw);
#pragma unroll
    for (int j = 0; j < kRowVecUnits; ++j) {
        const int u = u0 + tid + j * kNarrowThreads;
        if (u >= units) break;
        const int r = u / G4;
        const int g = u - r * G4;
        const int ih = ho0 * a.stride - a.pad + r;
        const bool in = unsigned(ih) < unsigned(a.H);
        Q v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (in && c < a.Cin) ? q.v[j][c] : Q{};
        // position p (column 4g + p): element p of each channel's 4 columns
        Q pos[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if constexpr (sizeof(T) == 2) {
                const uint32_t sel = (p & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t d0 = p < 2 ? v[0].x : v[0].y, d1 = p < 2 ? v[1].x : v[1].y;
                const uint32_t d2 = p < 2 ? v[2].x : v[2].y, d3 = p < 2 ? v[3].x : v[3].y;
                pos[p] = Q{__builtin_amdgcn_perm(d1, d0, sel), __builtin_amdgcn_perm(d3, d2, sel)};
            } else {
                pos[p] = Q{dword_at(v[0], p), dword_at(v[1], p), dword_at(v[2], p), dword_at(v[3], p)};
            }
        }
        // window rows i with 0 <= r - i * stride < KH
        const int num = r - a.KH + 1;
        const int i_lo = num > 0 ? (num + a.stride - 1) / a.stride : 0;
        const int i_hi = min(rw - 1, r / a.stride);
        for (int i = i_lo; i <= i_hi; ++i) {
            const int kh = r - i * a.stride;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int wc = 4 * g + p + a.pad;
                if (wc < a.Wwin) *reinterpret_cast<Q *>(win + i * a.Lp + (wc * a.KH + kh) * 4) = pos[p];
            }
        }
    }
}

// zero the padding columns of the rw window rows, and the slack after each
template <typename T>
__device__ __forceinline__ void zero_row_pads(const NarrowKArgs &a, T *win, int rw, int tid)
{
    using Q = typename RowRegs<T>::Q;
    const int right = max(0, a.Wwin - a.pad - a.W);
    const int npad = a.pad + right;
    const int n = rw * a.KH * npad;
    for (int v = tid; v < n; v += kNarrowThreads) {
        const int ik = v / npad;
        const int col = v - ik * npad;
        const int i = ik / a.KH;
        const int kh = ik - i * a.KH;
        const int wc = col < a.pad ? col : a.pad + a.W + (col - a.pad);
        *reinterpret_cast<Q *>(win + i * a.Lp + (wc * a.KH + kh) * 4) = Q{};
    }
    const int slack = a.Lp - a.L;
    for (int v = tid; v < rw * slack; v += kNarrowThreads) {
        const int i = v / slack;
        win[i * a.Lp + a.L + (v - i * slack)] = T(0);
    }
}

// every row-unit round of a row block after the first, fetched and written
template <typename T>
__device__ __forceinline__ void rows_rest(const NarrowKArgs &a, const T *ximg, T *win, int ho0, int rw, int tid)
{
    for (int u0 = kRowVecUnits * kNarrowThreads; u0 < row_units<T>(a, rw); u0 += kRowVecUnits * kNarrowThreads) {
        RowRegs<T> more;
        fetch_rows(a, ximg, ho0, rw, u0, tid, more);
        put_rows(a, win, ho0, rw, u0, tid, more);
    }
}

// One row block per workgroup from whole input rows: the filter block's
// vectors and a round of row units in flight together, then written.
template <bool GATHER, int FB, typename T>
__device__ __forceinline__ void load_block_rows(const NarrowKArgs &a, const T *ximg, const T *w, T *fl, T *win,
                                                int FS, int cb, int ho0, int rw, int tid)
{
    constexpr int V = 16 / sizeof(T);
    const int fv_row = a.Kp / V;
    const int fvec = 64 * fv_row;
    const int units = row_units<T>(a, rw);
    constexpr int UR = kRowVecUnits * kNarrowThreads;
    for (int f0 = 0, u0 = 0; f0 < fvec || u0 < units; f0 += FB * kNarrowThreads, u0 += UR) {
        uint4 fv[FB];
#pragma unroll
        for (int j = 0; j < FB; ++j)
            fv[j] = filter_vec<4, GATHER>(a, w, cb, min(f0 + tid + j * kNarrowThreads, fvec - 1));
        RowRegs<T> q;
        if (u0 < units) fetch_rows(a, ximg, ho0, rw, u0, tid, q);
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int v = f0 + tid + j * kNarrowThreads;
            if (v < fvec) {
                const int r = v / fv_row;
                *reinterpret_cast<uint4 *>(fl + r * FS + (v - r * fv_row) * V) = fv[j];
            }
        }
        if (u0 < units) put_rows(a, win, ho0, rw, u0, tid, q);
    }
    zero_row_pads(a, win, rw, tid);
}

// this workgroup's row blocks [t_begin, t_end): image and first output row
__device__ __forceinline__ void task_rows(const NarrowKArgs &a, int t, int &n, int &ho0, int &rw)
{
    n = t / a.row_groups;
    ho0 = (t - n * a.row_groups) * a.R;
    rw = min(a.R, a.Ho - ho0);
}

// ---- fp16 / bf16 -------------------------------------------------------------
// ROWS (CP = 4 only): window rows from whole input rows (load_block_rows)
template <int CP, bool BF16, bool PIPE, bool GATHER, bool ROWS>
__global__ __launch_bounds__(kNarrowThreads) void conv_implicit_narrow_kernel(const NarrowKArgs a, int ntasks)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int FS = a.Kp + 8;                         // filter row stride in LDS (elements)
    uint16_t *const fl = lds;                        // [64][FS]
    uint16_t *const win = lds + 64 * FS;             // [R][Lp], then the store scratch

    const int cb = blockIdx.x % a.co_blocks;
    const int g = blockIdx.x / a.co_blocks;
    const int t_begin = int(int64_t(ntasks) * g / a.groups);
    const int t_end = int(int64_t(ntasks) * (g + 1) / a.groups);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const uint16_t *const wsrc = static_cast<const uint16_t *>(a.w);  // w, or the staged rows
    constexpr int UB = CP == 4 ? 16 : 8;
    constexpr int UBR = UB * kNarrowThreads;         // window units per round
    const uint16_t *const x = static_cast<const uint16_t *>(a.x);
    const int64_t img = int64_t(a.Cin) * a.H * a.W;
    // contraction and stores of one row block, after its window rows are in LDS
    auto run_block = [&](int n, int ho0, int rw) __attribute__((always_inline)) {
        const int outs = rw * a.Wo;
        int b0, nb;
        wave_blocks(wave, outs, b0, nb);
        // this lane's window run (A row) of each block and filter row (B column)
        int abase[4];
        const int step = a.stride * a.KH * CP;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int m = min((b0 + s) * 16 + (lane & 15), outs - 1);
            const int i = m / a.Wo;
            abase[s] = i * a.Lp + (m - i * a.Wo) * step + 8 * (lane >> 4);
        }
        const int bbase = (lane & 15) * FS + 8 * (lane >> 4);
        floatx4_t acc[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const int nk = a.Kp >> 5;
        auto contract = [&](auto nbc) {
            constexpr int NBW = decltype(nbc)::value;
#pragma unroll 2
            for (int kk = 0; kk < nk; ++kk) {
                uint4 af[NBW], bf[4];
#pragma unroll
                for (int s = 0; s < NBW; ++s) af[s] = *reinterpret_cast<const uint4 *>(win + abase[s] + kk * 32);
#pragma unroll
                for (int c = 0; c < 4; ++c) bf[c] = *reinterpret_cast<const uint4 *>(fl + bbase + c * 16 * FS + kk * 32);
#pragma unroll
                for (int s = 0; s < NBW; ++s)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(af[s], bf[c], acc[s][c]);
            }
        };
        if (nb >= 4) contract(std::integral_constant<int, 4>{});
        else if (nb == 3) contract(std::integral_constant<int, 3>{});
        else if (nb == 2) contract(std::integral_constant<int, 2>{});
        else if (nb == 1) contract(std::integral_constant<int, 1>{});
        if ((a.Wo & 3) == 0 && a.out.type == 0) {
            if (nb > 0) store_blocks<4, true>(acc, nb, b0, lane, a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
        } else {
            __syncthreads();                         // the window rows are dead: their LDS is store scratch
            if (nb > 0)
                store_blocks_lds(acc, nb, b0, lane, reinterpret_cast<float *>(win) + wave * kStoreScratchFloats,
                                 a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
        }
    };
    if constexpr (!PIPE) {
        // one row block: filter and window loads in one round trip
        int n, ho0, rw;
        task_rows(a, t_begin, n, ho0, rw);
        if constexpr (ROWS)
            load_block_rows<GATHER, 4>(a, x + n * img, wsrc, fl, win, FS, cb, ho0, rw, tid);
        else
            load_block<CP, GATHER, 4, UB>(a, x + n * img, wsrc, fl, win, FS, cb, ho0, rw, tid);
        __syncthreads();
        run_block(n, ho0, rw);
    } else {
        // persistent: the filter once; the first round of each row block's
        // gathers in flight during the previous block's contraction (the
        // first block's together with the filter loads)
        WinRegs<CP, UB, uint16_t> nxt;
        {
            int n, ho0, rw;
            task_rows(a, t_begin, n, ho0, rw);
            fetch_window<false>(a, x + n * img, ho0, rw, 0, tid, nxt);
        }
        load_filter<CP, GATHER, 4>(a, wsrc, fl, FS, cb, tid);
        for (int t = t_begin; t < t_end; ++t) {
            int n, ho0, rw;
            task_rows(a, t, n, ho0, rw);
            if (t != t_begin) __syncthreads();       // the previous block's window rows (scratch) are dead
            put_window<false>(a, win, rw, 0, tid, nxt);
            for (int u0 = UBR; u0 < rw * a.KH * a.Wwin; u0 += UBR) {
                WinRegs<CP, UB, uint16_t> more;
                fetch_window<false>(a, x + n * img, ho0, rw, u0, tid, more);
                put_window<false>(a, win, rw, u0, tid, more);
            }
            if (t + 1 < t_end) {
                int n1, h1, r1;
                task_rows(a, t + 1, n1, h1, r1);
                fetch_window<false>(a, x + n1 * img, h1, r1, 0, tid, nxt);
            }
            __syncthreads();
            run_block(n, ho0, rw);
        }
    }
}

// ---- fp32: v_mfma_f32_16x16x4_f32; K in slices of 16 elements, lane group
// g = lane / 16 holding elements 4g .. 4g + 3 of a slice as one vector and
// feeding element j to K step j (window runs and filter alike) -------------
template <int CP, bool PIPE, bool GATHER, bool ROWS>
__global__ __launch_bounds__(kNarrowThreads) void conv_implicit_narrow_f32_kernel(const NarrowKArgs a, int ntasks)
{
    extern __shared__ __attribute__((aligned(16))) float ldsf[];
    const int FS = a.Kp + 4;
    float *const fl = ldsf;                          // [64][FS]
    float *const win = ldsf + 64 * FS;               // [R][Lp], then the store scratch

    const int cb = blockIdx.x % a.co_blocks;
    const int g = blockIdx.x / a.co_blocks;
    const int t_begin = int(int64_t(ntasks) * g / a.groups);
    const int t_end = int(int64_t(ntasks) * (g + 1) / a.groups);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const float *const wsrc = static_cast<const float *>(a.w);        // w, or the staged rows
    constexpr int UB = CP == 4 ? 16 : 8;
    constexpr int UBR = UB * kNarrowThreads;         // window units per round
    const float *const x = static_cast<const float *>(a.x);
    const int64_t img = int64_t(a.Cin) * a.H * a.W;
    // contraction and stores of one row block, after its window rows are in LDS
    auto run_block = [&](int n, int ho0, int rw) __attribute__((always_inline)) {
        const int outs = rw * a.Wo;
        int b0, nb;
        wave_blocks(wave, outs, b0, nb);
        int abase[4];
        const int step = a.stride * a.KH * CP;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int m = min((b0 + s) * 16 + (lane & 15), outs - 1);
            const int i = m / a.Wo;
            abase[s] = i * a.Lp + (m - i * a.Wo) * step + 4 * (lane >> 4);
        }
        const int bbase = (lane & 15) * FS + 4 * (lane >> 4);
        floatx4_t acc[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const int nsl = nb > 0 ? a.Kp >> 4 : 0;
        for (int sl = 0; sl < nsl; ++sl) {
            floatx4_t af[4], bf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (s < nb) af[s] = *reinterpret_cast<const floatx4_t *>(win + abase[s] + sl * 16);
#pragma unroll
            for (int c = 0; c < 4; ++c) bf[c] = *reinterpret_cast<const floatx4_t *>(fl + bbase + c * 16 * FS + sl * 16);
            // with CP = 4 a K step j takes channel j of every position (each
            // lane group's 4 elements are one position): the steps of the
            // zero-padded channels j >= Cin would only add 0 * 0, so they are
            // not issued (the 3-channel stem: a quarter of the products)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (CP == 4 && j >= a.Cin) break;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s >= nb) break;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[s][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[s][j], bf[c][j], acc[s][c], 0, 0, 0);
                }
            }
        }
        if ((a.Wo & 3) == 0 && a.out.type == 0) {
            if (nb > 0) store_blocks<4, true>(acc, nb, b0, lane, a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
        } else {
            __syncthreads();
            if (nb > 0)
                store_blocks_lds(acc, nb, b0, lane, win + wave * kStoreScratchFloats, a.out, n, a.Cout, cb, a.Ho,
                                 a.Wo, ho0, outs);
        }
    };
    if constexpr (!PIPE) {
        // one row block: filter and window loads in one round trip
        int n, ho0, rw;
        task_rows(a, t_begin, n, ho0, rw);
        if constexpr (ROWS)
            load_block_rows<GATHER, 4>(a, x + n * img, wsrc, fl, win, FS, cb, ho0, rw, tid);
        else
            load_block<CP, GATHER, 4, UB>(a, x + n * img, wsrc, fl, win, FS, cb, ho0, rw, tid);
        __syncthreads();
        run_block(n, ho0, rw);
    } else if constexpr (ROWS) {
        // persistent, window rows from whole input rows: the first round of
        // each row block's row units in flight during the previous block's
        // contraction
        RowRegs<float> nxt;
        {
            int n, ho0, rw;
            task_rows(a, t_begin, n, ho0, rw);
            fetch_rows(a, x + n * img, ho0, rw, 0, tid, nxt);
        }
        load_filter<CP, GATHER, 4>(a, wsrc, fl, FS, cb, tid);
        for (int t = t_begin; t < t_end; ++t) {
            int n, ho0, rw;
            task_rows(a, t, n, ho0, rw);
            if (t != t_begin) __syncthreads();       // the previous block's window rows (scratch) are dead
            put_rows(a, win, ho0, rw, 0, tid, nxt);
            rows_rest(a, x + n * img, win, ho0, rw, tid);
            zero_row_pads(a, win, rw, tid);
            if (t + 1 < t_end) {
                int n1, h1, r1;
                task_rows(a, t + 1, n1, h1, r1);
                fetch_rows(a, x + n1 * img, h1, r1, 0, tid, nxt);
            }
            __syncthreads();
            run_block(n, ho0, rw);
        }
    } else {
        // persistent: the filter once; the first round of each row block's
        // gathers in flight during the previous block's contraction (the
        // first block's together with the filter loads)
        WinRegs<CP, UB, float> nxt;
        {
            int n, ho0, rw;
            task_rows(a, t_begin, n, ho0, rw);
            fetch_window<false>(a, x + n * img, ho0, rw, 0, tid, nxt);
        }
        load_filter<CP, GATHER, 4>(a, wsrc, fl, FS, cb, tid);
        for (int t = t_begin; t < t_end; ++t) {
            int n, ho0, rw;
            task_rows(a, t, n, ho0, rw);
            if (t != t_begin) __syncthreads();       // the previous block's window rows (scratch) are dead
            put_window<false>(a, win, rw, 0, tid, nxt);
            for (int u0 = UBR; u0 < rw * a.KH * a.Wwin; u0 += UBR) {
                WinRegs<CP, UB, float> more;
                fetch_window<false>(a, x + n * img, ho0, rw, u0, tid, more);
                put_window<false>(a, win, rw, u0, tid, more);
            }
            if (t + 1 < t_end) {
                int n1, h1, r1;
                task_rows(a, t + 1, n1, h1, r1);
                fetch_window<false>(a, x + n1 * img, h1, r1, 0, tid, nxt);
            }
            __syncthreads();
            run_block(n, ho0, rw);
        }
    }
}

}  // namespace

hipError_t launch_conv_implicit_narrow(const ImplicitArgs &h, hipStream_t s)
{
    const int cp = h.narrow_cp;
    const int kstep = h.f32 ? 16 : 32;
    NarrowKArgs a{};
    a.x = h.x;
    a.w = h.wst;                                     // w as stored, or the staged rows
    a.out = h.out;
    a.Cin = h.Cin;
    a.H = h.H;
    a.W = h.W;
    a.Cout = h.Cout;
    a.KH = h.KH;
    a.KW = h.KW;
    a.stride = h.stride;
    a.pad = h.pad;
    a.Ho = h.Ho;
    a.Wo = h.Wo;
    a.K = h.KW * h.KH * cp;
    a.Kp = (a.K + kstep - 1) / kstep * kstep;
    a.Wwin = (h.Wo - 1) * h.stride + h.KW;
    a.L = a.Wwin * h.KH * cp;
    const int vec = h.f32 ? 4 : 8;
    a.Lp = (a.L + a.Kp - a.K + vec - 1) / vec * vec;
    a.R = h.R;
    a.row_groups = (h.Ho + h.R - 1) / h.R;
    a.co_blocks = (h.Cout + 63) / 64;
    // window rows from whole input rows: 4 channels per position, rows of 4k
    // elements, x aligned to 4 elements
    a.rowvec = cp == 4 && h.W % 4 == 0 && (reinterpret_cast<uintptr_t>(h.x) & (h.f32 ? 15 : 7)) == 0;
    // the kernel's assumptions: CP channels hold Cin, every window start is a
    // whole 16-byte vector, the outputs of a block fit 32 MFMA blocks, and
    // element offsets of the image fit 32 bits
    const int es = h.f32 ? 4 : 2;
    if ((cp != 4 && cp != 8) || h.Cin < 1 || h.Cin > cp || (h.stride * h.KH * cp * es) % 16 != 0 ||
        h.kstage != a.Kp || h.R < 1 || int64_t(h.R) * h.Wo > 512 || h.Wo < 1 || h.Ho < 1 ||
        int64_t(h.Cin) * h.H * h.W >= (int64_t(1) << 31) ||
        int64_t(h.Cout) * h.Cin * h.KH * h.KW >= (int64_t(1) << 31) ||
        implicit_narrow_lds_bytes(es, a.Kp, a.Lp, h.R) > kImplicitMaxLdsBytes)
        return hipErrorInvalidValue;
    // workgroups: co_blocks x groups, each group walking a contiguous range of
    // the N * row_groups row blocks with its filter block gathered once
    a.groups = h.groups;
    int ntasks = h.N * a.row_groups;
    const int64_t blocks = int64_t(a.co_blocks) * a.groups;
    if (a.groups < 1 || a.groups > ntasks || blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = size_t(implicit_narrow_lds_bytes(es, a.Kp, a.Lp, h.R));
    // one row block per workgroup, or persistent workgroups that prefetch the
    // next row block's gathers (more registers: one workgroup per CU)
    const bool pipe = a.groups < ntasks;
    // the filter gathered from w (the plan then keeps no staged filter), or
    // read from the staged rows
    const bool gather = narrow_gathers_filter(blocks);
    const void *kern;
#define IM2WIN_NARROW_PICK(P, G)                                                                                   \
    if (h.f32)                                                                                                     \
        kern = cp == 8   ? reinterpret_cast<const void *>(conv_implicit_narrow_f32_kernel<8, P, G, false>)         \
               : a.rowvec ? reinterpret_cast<const void *>(conv_implicit_narrow_f32_kernel<4, P, G, true>)         \
                          : reinterpret_cast<const void *>(conv_implicit_narrow_f32_kernel<4, P, G, false>);       \
    else if (h.bf16)                                                                                               \
        kern = cp == 8   ? reinterpret_cast<const void *>(conv_implicit_narrow_kernel<8, true, P, G, false>)       \
               : a.rowvec ? reinterpret_cast<const void *>(conv_implicit_narrow_kernel<4, true, P, G, true>)       \
                          : reinterpret_cast<const void *>(conv_implicit_narrow_kernel<4, true, P, G, false>);     \
    else                                                                                                           \
        kern = cp == 8   ? reinterpret_cast<const void *>(conv_implicit_narrow_kernel<8, false, P, G, false>)      \
               : a.rowvec ? reinterpret_cast<const void *>(conv_implicit_narrow_kernel<4, false, P, G, true>)      \
                          : reinterpret_cast<const void *>(conv_implicit_narrow_kernel<4, false, P, G, false>);
    // persistent launches have at most 256 workgroups: always the gathered filter
    if (pipe && !gather) return hipErrorInvalidValue;
    if (pipe) {
        IM2WIN_NARROW_PICK(true, true)
    } else if (gather) {
        IM2WIN_NARROW_PICK(false, true)
    } else {
        IM2WIN_NARROW_PICK(false, false)
    }
#undef IM2WIN_NARROW_PICK
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    void *args[] = {&a, &ntasks};
    const hipError_t e = hipLaunchKernel(kern, dim3(unsigned(blocks)), dim3(kNarrowThreads), args, lds, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace im2win
