// im2win pack: the window tensor of "Enabling Memory-efficient Im2win
// Convolution with Multi-precision Support on GPU CUDA and Tensor Cores",
// Sec. III-B, Eq. (2), with zero padding. Window row r = n*Ho + ho holds, for
// every padded column w < W_win and filter row kh, the value
//     xp[n][ci][ho*stride + kh][w]  (= x[n][ci][ho*stride+kh-pad][w-pad], or 0)
// at position pos = w*KH + kh. Two storage orders:
//   row-interleaved  T[r][ci][pos]   (pos_pad positions per channel)
//   channels-last    T[r][pos][ci]   (Cin_pad channels per position)
// Both kernels are pure copies on the raw bits (no arithmetic on values), so
// the result is bit-identical to the definition. Both are HBM-bound.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "../launch.hpp"
#include "stage_body.hpp"

namespace im2win {
namespace {

// ---------------------------------------------------------------- row-interleaved
// One wave per task = (window row r, group of up to CPW channels). A lane
// writes consecutive positions q of each channel's run (coalesced stores) and
// reads the input element (kh, w) = (q mod KH, q div KH) of the KH input rows,
// which a wave touches as KH short contiguous segments (L1-resident). Four
// positions per lane and all channels of the group are loaded before any is
// stored, so 4*CPW independent loads are in flight. KH is a template
// parameter for the common filter heights (q div KH becomes a multiply).
constexpr int CPW = 8;    // channels per wave task
constexpr int QU = 4;     // positions per lane per step

template <typename E, int KHT>
__global__ __launch_bounds__(256) void pack_row_kernel(
    const E *__restrict__ x, E *__restrict__ out, int Cin, int H, int W, int KH_rt, int stride,
    int pad, int Ho, int Wwin, int pos_pad, int row_elems, int row0, int rows, int cgroups,
    StageFold fs)
{
    if (int(blockIdx.x) < fs.blocks) {            // filter staging carried by this launch
        stage_row_elems(static_cast<const E *>(fs.w), static_cast<E *>(fs.out), fs.Cout,
                        fs.Cin * fs.KH * fs.KW, fs.rows, blockIdx.x * 256u + threadIdx.x,
                        unsigned(fs.blocks) * 256u);
        return;
    }
    const int KH = KHT > 0 ? KHT : KH_rt;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int task = (int(blockIdx.x) - fs.blocks) * 4 + wave;
    if (task >= rows * cgroups) return;            // no barriers in this kernel
    const int rl = task / cgroups;
    const int c0 = (task - rl * cgroups) * CPW;
    const int nc = min(CPW, Cin - c0);
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const int used = Wwin * KH;
    const int ih0 = ho * stride - pad;
    const E *xc = x + (int64_t(n) * Cin + c0) * H * W;
    E *o = out + int64_t(rl) * row_elems + int64_t(c0) * pos_pad;
    const int64_t cstride = int64_t(H) * W;
    for (int qb = 0; qb < pos_pad; qb += 64 * QU) {
        int src[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int q = qb + u * 64 + lane;
            src[u] = -1;
            if (q < used) {
                const int w = q / KH;
                const int kh = q - w * KH;
                const int ih = ih0 + kh;
                const int iw = w - pad;
                if (ih >= 0 && ih < H && iw >= 0 && iw < W) src[u] = ih * W + iw;
            }
        }
        // unconditional loads from valid addresses, masked after (no branch)
        E v[CPW][QU];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const E t = xc[(c < nc ? c : 0) * cstride + (src[u] >= 0 ? src[u] : 0)];
                v[c][u] = (src[u] >= 0) ? t : E(0);
            }
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            if (c >= nc) break;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const int q = qb + u * 64 + lane;
                if (q < pos_pad) o[int64_t(c) * pos_pad + q] = v[c][u];
            }
        }
    }
}

// ---------------------------------------------------------------- channels-last
// Workgroup = (window row r, block of CB channels), looping over blocks of PW
// padded columns and passes of up to KHB filter rows.
// Phase 1 stages T[ci][kh][w] in LDS: lanes along w (coalesced reads), each
// wave takes 4 channels x KHB filter rows at a time so that up to 16
// independent loads are in flight. Phase 2 reads CG x 8 blocks (CG channels x
// 8 columns) as 16-byte LDS rows, transposes them in registers and writes
// CG-channel vectors, so global writes run along ci, the innermost dimension
// of the window tensor (8 lanes cover one 128-byte run of 64 channels).
// Channel rows of the LDS tile are skewed by 16 bytes so that the phase-2 reads
// of 8 channels hit 8 different bank groups.
constexpr int PW = 64;             // padded columns per pass (one per lane)
constexpr int CB = 64;             // channels per workgroup
constexpr int KHB = 4;             // filter rows per pass
constexpr int LDS_PITCH = PW + 8;  // elements per (ci, kh) LDS row (16-byte multiple)
constexpr int CSTRIDE = KHB * LDS_PITCH + 8;   // elements per channel (skew: 592 bytes)
constexpr int CU1 = 4;             // channels per wave per phase-1 step

// 16-bit lanes of a 32-bit word
__device__ __forceinline__ uint32_t lo16(uint32_t v) { return v & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t v) { return v >> 16; }

template <int CG>
__global__ __launch_bounds__(256) void pack_cl_kernel(
    const uint16_t *__restrict__ x, uint16_t *__restrict__ out, int Cin, int H, int W, int KH,
    int stride, int pad, int Ho, int Wwin, int Cin_pad, int row_elems, int row0, int cblocks)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[CB * CSTRIDE];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int cbk = blockIdx.x % cblocks;
    const int rl = blockIdx.x / cblocks;
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const int c0 = cbk * CB;
    const int cb = min(CB, Cin_pad - c0);        // channels in this block (multiple of CG)
    const int ih0 = ho * stride - pad;
    const int64_t cstride = int64_t(H) * W;
    const uint16_t *xb = x + (int64_t(n) * Cin + c0) * cstride;
    uint16_t *orow = out + int64_t(rl) * row_elems;
    const int cgroups = cb / CG;

    for (int w0 = 0; w0 < Wwin; w0 += PW) {
        const int iw = w0 + lane - pad;
        const bool col_ok = iw >= 0 && iw < W && w0 + lane < Wwin;
        for (int kh0 = 0; kh0 < KH; kh0 += KHB) {
            const int khn = min(KHB, KH - kh0);
            // phase 1: tile[ci*CSTRIDE + kh*LDS_PITCH + lane]
            for (int cs = wave * CU1; cs < cb; cs += 4 * CU1) {
                uint16_t v[CU1][KHB];
#pragma unroll
                for (int u = 0; u < CU1; ++u)
#pragma unroll
                    for (int kh = 0; kh < KHB; ++kh) {
                        const int c = cs + u;
                        const int ih = ih0 + kh0 + kh;
                        const bool ok = kh < khn && c0 + c < Cin && ih >= 0 && ih < H && col_ok;
                        // unconditional load from a valid address, masked after (no branch)
                        const uint16_t t = xb[ok ? int64_t(c) * cstride + ih * W + iw : 0];
                        v[u][kh] = ok ? t : uint16_t(0);
                    }
#pragma unroll
                for (int u = 0; u < CU1; ++u)
#pragma unroll
                    for (int kh = 0; kh < KHB; ++kh)
                        if (kh < khn && cs + u < cb)
                            tile[(cs + u) * CSTRIDE + kh * LDS_PITCH + lane] = v[u][kh];
            }
            __syncthreads();
            // phase 2: (kh, column group of 8, channel group of CG)
            const int items = khn * (PW / 8) * cgroups;
            for (int i = threadIdx.x; i < items; i += 256) {
                const int cg = i % cgroups;
                const int t = i / cgroups;
                const int wg = t % (PW / 8);
                const int kh = t / (PW / 8);
                const int wbase = w0 + wg * 8;
                if (wbase >= Wwin) continue;
                uint32_t rowv[CG][4];
#pragma unroll
                for (int e = 0; e < CG; ++e) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(
                        &tile[(cg * CG + e) * CSTRIDE + kh * LDS_PITCH + wg * 8]);
                    rowv[e][0] = q.x; rowv[e][1] = q.y; rowv[e][2] = q.z; rowv[e][3] = q.w;
                }
                uint16_t *dst = orow + (int64_t(wbase) * KH + kh0 + kh) * Cin_pad + c0 + cg * CG;
                const int64_t wstep = int64_t(KH) * Cin_pad;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (wbase + j >= Wwin) break;
                    uint32_t o[CG / 2];
#pragma unroll
                    for (int q = 0; q < CG / 2; ++q) {
                        const uint32_t a = rowv[2 * q][j >> 1];
                        const uint32_t c = rowv[2 * q + 1][j >> 1];
                        o[q] = (j & 1) ? (hi16(a) | (c & 0xffff0000u)) : (lo16(a) | (c << 16));
                    }
                    if constexpr (CG == 8) {
                        *reinterpret_cast<uint4 *>(dst + j * wstep) = make_uint4(o[0], o[1], o[2], o[3]);
                    } else {
                        *reinterpret_cast<uint2 *>(dst + j * wstep) = make_uint2(o[0], o[1]);
                    }
                }
            }
            __syncthreads();
        }
    }
    // zero the row tail past W_win*KH*Cin_pad (alignment padding), once per row
    if (cbk == 0) {
        const int used = Wwin * KH * Cin_pad;
        for (int q = used + threadIdx.x; q < row_elems; q += 256) orow[q] = 0;
    }
}

// ---------------------------------------------------------------- channels-last, row-staged
// Workgroup = (window row r, block of cblk channels). Every channel of the
// block needs the same KH input rows ih in [ho*stride - pad, ... + KH),
// clipped to [0, H); in NCHW those rows are ONE contiguous run of len
// elements per channel. Phase 1 copies each run into LDS as whole aligned
// 16-byte chunks (a chunk may start up to 7 elements before the run, the
// offset is kept per channel), issuing U chunk loads per wave before the
// first wait. Phase 2 walks the output vectors of the row in storage order,
// one per thread: CG channels at one position (w, kh) are gathered from the
// LDS runs (zero outside the input or past Cin) and stored as one 16-byte
// (CG = 8) or 8-byte (CG = 4) vector, so consecutive lanes write consecutive
// bytes of the window row. One barrier per workgroup.
constexpr int LU = 8;   // chunk loads in flight per lane in phase 1

template <int CG>
__global__ __launch_bounds__(256) void pack_cl_staged_kernel(
    const uint16_t *__restrict__ x, uint16_t *__restrict__ out, int Cin, int H, int W, int KH,
    int stride, int pad, int Ho, int Wwin, int Cin_pad, int row_elems, int row0, int cblocks,
    int cblk, int cp, int nck, int x_elems, int x_chunks, StageFold fs)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t run[];   // [cblk][cp]
    if (int(blockIdx.x) < fs.blocks) {            // filter staging carried by this launch
        if (fs.Cin_pad % 8 == 0 && fs.row_len % 8 == 0)
            stage_cl_vec8(static_cast<const uint16_t *>(fs.w), static_cast<uint16_t *>(fs.out), fs.Cout,
                          fs.Cin, fs.KH, fs.KW, fs.Cin_pad, fs.row_len,
                          blockIdx.x * 256u + threadIdx.x, unsigned(fs.blocks) * 256u);
        else
            stage_cl_elems(static_cast<const uint16_t *>(fs.w), static_cast<uint16_t *>(fs.out), fs.Cout,
                           fs.Cin, fs.KH, fs.KW, fs.Cin_pad, fs.row_len,
                           blockIdx.x * 256u + threadIdx.x, unsigned(fs.blocks) * 256u);
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const int bid = int(blockIdx.x) - fs.blocks;
    const int cbk = bid % cblocks;
    const int rl = bid / cblocks;
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const int c0 = cbk * cblk;
    const int cb = min(cblk, Cin_pad - c0);      // channels stored (multiple of CG)
    const int cin_b = min(cb, Cin - c0);          // of which real (the rest are zero padding)
    const int ih0 = ho * stride - pad;
    const int ihA = max(ih0, 0);
    const int ihB = min(ih0 + KH, H);
    const int len = ihB > ihA ? (ihB - ihA) * W : 0;   // run length per channel
    const int HW = H * W;
    const int g0 = (n * Cin + c0) * HW + ihA * W;        // run start of channel c0 (elements)
    const uint4 *x16 = reinterpret_cast<const uint4 *>(x);

    // ---- phase 1: runs -> LDS, chunk k of channel c at run[c*cp + 8k]
    const int lpc = nck < 64 ? nck : 64;          // lanes per channel
    const int cpi = 64 / lpc;                     // channels per wave instruction
    const int csub = lane / lpc;
    const int k0 = lane - csub * lpc;
    const int ksteps = (nck + lpc - 1) / lpc;
    const int cgrp = (cin_b + 4 * cpi - 1) / (4 * cpi);
    const int slots = len > 0 ? cgrp * ksteps : 0;
    const int spill = cblk * cp + lane * 8;       // per-lane 16-byte slot after the runs
    for (int s0 = 0; s0 < slots; s0 += LU) {
        uint4 v[LU];
        int dst[LU];
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            const int sl = s0 + u;
            const int q = sl / ksteps;            // wave-uniform
            const int ks = sl - q * ksteps;
            const int c = (q * 4 + wave) * cpi + csub;
            const int k = ks * lpc + k0;
            const int g = g0 + c * HW;
            const int a = (g >> 3) + k;           // chunk index in x
            const bool ok = sl < slots && csub < cpi && c < cin_b &&
                            a <= ((g + len - 1) >> 3) && a < x_chunks;
            v[u] = x16[ok ? a : 0];               // unconditional, from a valid address
            dst[u] = ok ? c * cp + k * 8 : spill;  // lanes with nothing to copy write their own
        }                                         // slot past the runs (no branch)
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            uint32_t *d32 = reinterpret_cast<uint32_t *>(run + dst[u]);
            d32[0] = v[u].x; d32[1] = v[u].y; d32[2] = v[u].z; d32[3] = v[u].w;
        }
    }
    // the chunk holding the last elements of x when x_elems is not a multiple
    // of 8: a 16-byte load would cross the end of x, copy it element-wise
    if ((x_elems & 7) != 0 && len > 0) {
        for (int c = tid; c < cin_b; c += 256) {
            const int g = g0 + c * HW;
            const int last = g + len - 1;
            const int a = last >> 3;
            if (a >= x_chunks) {
                const int k = a - (g >> 3);
                for (int j = max(g, a * 8); j <= last; ++j) run[c * cp + k * 8 + (j - a * 8)] = x[j];
            }
        }
    }
    // channels past Cin (zero padding of the last group): zero runs, so that
    // phase 2 reads them like any other channel
    for (int i = cin_b * cp + tid; i < cb * cp; i += 256) run[i] = 0;
    __syncthreads();

    // ---- phase 2: output vectors (cg, kh, w) of this block, cg fastest
    const int cgroups = cb / CG;
    const int total = Wwin * KH * cgroups;
    int cg = tid % cgroups;
    int t = tid / cgroups;
    int kh = t % KH;
    int w = t / KH;
    const int dcg = 256 % cgroups;
    const int dt = 256 / cgroups;
    const int dkh = dt % KH;
    const int dw = dt / KH;
    // element e of a vector (channel cg*CG + e) sits at run offset
    // (cg*CG + e)*cp + shift + inner, where the run of channel c starts
    // shift = (g0 + c*HW) mod 8 elements into its first chunk; cg*CG*HW is a
    // multiple of 8 (CG = 8, or CG = 4 with one group), so e*cp + shift is the
    // same for every vector: wave-uniform offsets
    int eo[CG];
#pragma unroll
    for (int e = 0; e < CG; ++e) eo[e] = e * cp + ((g0 + e * HW) & 7);
    uint16_t *orow = out + int64_t(rl) * row_elems + c0;
    const int khn = max(ihB - ihA, 0);                     // staged rows (0: all padding)
    auto advance = [&](int &cg_, int &kh_, int &w_) {      // by 256 vectors
        cg_ += dcg;
        int carry = cg_ >= cgroups;
        cg_ -= carry ? cgroups : 0;
        kh_ += dkh + carry;
        carry = kh_ >= KH;
        kh_ -= carry ? KH : 0;
        w_ += dw + carry;
    };
    auto gather = [&](int cg_, int kh_, int w_, uint32_t (&o)[CG / 2]) {
        const int ihr = ih0 + kh_ - ihA;                   // row inside the staged runs
        const int iw = w_ - pad;
        const bool ok = unsigned(ihr) < unsigned(khn) && unsigned(iw) < unsigned(W);
        const int base = ok ? cg_ * CG * cp + ihr * W + iw : 0;
        uint32_t e32[CG];
#pragma unroll
        for (int e = 0; e < CG; ++e) e32[e] = run[base + eo[e]];
        const uint32_t m = ok ? 0xffffffffu : 0u;
#pragma unroll
        for (int q = 0; q < CG / 2; ++q) o[q] = (e32[2 * q] | (e32[2 * q + 1] << 16)) & m;
    };
    auto put = [&](int cg_, int kh_, int w_, const uint32_t (&o)[CG / 2]) {
        uint16_t *dst = orow + (w_ * KH + kh_) * Cin_pad + cg_ * CG;
        if constexpr (CG == 8)
            *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        else
            *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
    };
    // two vectors per trip: both gathers are issued before either store waits
    for (int vi = tid; vi < total; vi += 512) {
        int cg1 = cg, kh1 = kh, w1 = w;
        advance(cg1, kh1, w1);
        uint32_t o0[CG / 2], o1[CG / 2];
        gather(cg, kh, w, o0);
        gather(cg1, kh1, w1, o1);
        put(cg, kh, w, o0);
        if (vi + 256 < total) put(cg1, kh1, w1, o1);
        cg = cg1; kh = kh1; w = w1;
        advance(cg, kh, w);
    }
    // zero the row tail past W_win*KH*Cin_pad (alignment padding), once per row
    if (cbk == 0) {
        const int used = Wwin * KH * Cin_pad;
        uint16_t *orow0 = out + int64_t(rl) * row_elems;
        for (int q = used + tid; q < row_elems; q += 256) orow0[q] = 0;
    }
}

// Channels-last window rows from NHWC x: element (pos = w*KH + kh, ci) of
// window row r = n*Ho + ho is x[n][ho*stride + kh - pad][w - pad][ci], zero
// outside the image and for the padding channels ci >= Cin; every element of
// the row's row_elems, the spare tail included, is written. One 16-byte
// output vector per thread, consecutive threads on consecutive vectors of a
// row: with Cin % 8 == 0 it is 8 channels of one input position, one 16-byte
// load (the channels of a position are contiguous in NHWC); else 2-byte
// gathers.
__global__ __launch_bounds__(256) void pack_cl_nhwc_kernel(const uint16_t *__restrict__ x,
                                                           uint16_t *__restrict__ out, int Cin, int H, int W,
                                                           int KH, int stride, int pad, int Ho, int Wwin,
                                                           int Cin_pad, int row_elems, int row0, int rows)
{
    const int vpr = row_elems >> 3;
    const int npos = Wwin * KH;
    const int64_t total = int64_t(rows) * vpr;
    for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < total; t += int64_t(gridDim.x) * 256) {
        const int rl = int(t / vpr);
        const int e0 = int(t - int64_t(rl) * vpr) * 8;
        const int r = row0 + rl;
        const int n = r / Ho;
        const int ho = r - n * Ho;
        uint4 o{0u, 0u, 0u, 0u};
        if (Cin % 8 == 0) {                             // Cin_pad == Cin
            const int pos = e0 / Cin;
            if (pos < npos) {
                const int c0 = e0 - pos * Cin;
                const int wc = pos / KH;
                const int kh = pos - wc * KH;
                const int ih = ho * stride + kh - pad;
                const int iw = wc - pad;
                if (unsigned(ih) < unsigned(H) && unsigned(iw) < unsigned(W))
                    o = *reinterpret_cast<const uint4 *>(x + ((int64_t(n) * H + ih) * W + iw) * Cin + c0);
            }
        } else {
            uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = e0 + e;
                const int pos = k / Cin_pad;
                const int ci = k - pos * Cin_pad;
                if (pos < npos && ci < Cin) {
                    const int wc = pos / KH;
                    const int kh = pos - wc * KH;
                    const int ih = ho * stride + kh - pad;
                    const int iw = wc - pad;
                    if (unsigned(ih) < unsigned(H) && unsigned(iw) < unsigned(W))
                        v[e >> 1] |= uint32_t(x[((int64_t(n) * H + ih) * W + iw) * Cin + ci]) << (16 * (e & 1));
                }
            }
            o = uint4{v[0], v[1], v[2], v[3]};
        }
        *reinterpret_cast<uint4 *>(out + int64_t(rl) * row_elems + e0) = o;
    }
}

}  // namespace

// staging workgroups a pack launch carries: about 4 filter elements per
// thread
static StageFold make_fold(const StageArgs *f, int64_t elems)
{
    StageFold fs{};
    if (!f) return fs;
    fs.w = f->w;
    fs.out = f->out;
    fs.Cout = f->Cout;
    fs.Cin = f->Cin;
    fs.KH = f->KH;
    fs.KW = f->KW;
    fs.Cin_pad = f->Cin_pad;
    fs.rows = f->rows;
    fs.row_len = f->row_len;
    const int64_t b = (elems + 1023) / 1024;
    fs.blocks = int(b < 2048 ? (b > 0 ? b : 1) : 2048);
    return fs;
}

template <typename E>
hipError_t launch_pack_row_t(const PackArgs &a, hipStream_t s, const StageFold &fs)
{
    const int cgroups = (a.Cin + CPW - 1) / CPW;
    const int64_t tasks = int64_t(a.rows) * cgroups;
    const dim3 grid(static_cast<unsigned>((tasks + 3) / 4 + fs.blocks));
    const E *x = static_cast<const E *>(a.x);
    E *out = static_cast<E *>(a.out);
#define IM2WIN_PACK_ROW(K)                                                                       \
    hipLaunchKernelGGL((pack_row_kernel<E, K>), grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W,   \
                       a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.pos_pad, a.row_elems, a.row0,       \
                       a.rows, cgroups, fs)
    switch (a.KH) {
    case 1: IM2WIN_PACK_ROW(1); break;
    case 3: IM2WIN_PACK_ROW(3); break;
    case 5: IM2WIN_PACK_ROW(5); break;
    case 7: IM2WIN_PACK_ROW(7); break;
    default: IM2WIN_PACK_ROW(0); break;
    }
#undef IM2WIN_PACK_ROW
    return hipGetLastError();
}

hipError_t launch_pack_row(const PackArgs &a, hipStream_t s, const StageArgs *fold, bool *folded)
{
    const StageFold fs = make_fold(fold, fold ? int64_t(fold->rows) * fold->Cin * fold->KH * fold->KW : 0);
    if (folded) *folded = fold != nullptr;
    return a.esize == 4 ? launch_pack_row_t<uint32_t>(a, s, fs) : launch_pack_row_t<uint16_t>(a, s, fs);
}

// LDS budget of the row-staged channels-last pack (per workgroup)
constexpr int kStagedLdsBytes = 63 * 1024;   // plus 1 KB of spill slots: within 64 KB

hipError_t launch_pack_cl(const PackArgs &a, hipStream_t s, const StageArgs *fold, bool *folded)
{
    if (a.nhwc) {
        if (folded) *folded = false;
        if (a.esize != 2 || a.row_elems % 8 != 0 || a.Cin_pad % 4 != 0) return hipErrorInvalidValue;
        const int64_t vecs = int64_t(a.rows) * (a.row_elems / 8);
        const int64_t blocks = std::min<int64_t>((vecs + 255) / 256, 1 << 18);
        hipLaunchKernelGGL(pack_cl_nhwc_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.x), static_cast<uint16_t *>(a.out), a.Cin, a.H,
                           a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad, a.row_elems, a.row0, a.rows);
        return hipGetLastError();
    }
    if (folded) *folded = false;
    if (a.esize != 2) return hipErrorInvalidValue;
    const auto *x = static_cast<const uint16_t *>(a.x);
    auto *out = static_cast<uint16_t *>(a.out);
    const int cg = a.Cin_pad % 8 == 0 ? 8 : (a.Cin_pad == 4 ? 4 : 0);
    if (cg == 0) return hipErrorInvalidValue;
    // row-staged form: one LDS run of KH input rows per channel
    const int nck = (a.KH * a.W + 14) / 8;          // 16-byte chunks per run, worst alignment
    int cp = 8 * nck + 2;                            // LDS pitch: odd number of 4-byte words
    if ((cp / 2) % 2 == 0) cp += 2;
    int cblk = (kStagedLdsBytes / (2 * cp)) / cg * cg;
    const int x_elems = a.N * a.Cin * a.H * a.W;
    // A block must hold the channels of at least one whole 128-byte line per
    // position (64 channels, or all of them): narrower blocks leave every
    // line of the row to be written piecewise by several workgroups, which
    // the tiled form avoids. IM2WIN_PACK_FORM=staged|tiled overrides (sweeps).
    bool staged = cblk >= (a.Cin_pad < 64 ? a.Cin_pad : 64);
    if (const char *e = std::getenv("IM2WIN_PACK_FORM")) {
        if (std::strcmp(e, "staged") == 0) staged = true;
        if (std::strcmp(e, "tiled") == 0) staged = false;
    }
    if (staged && cblk >= cg && x_elems >= 8) {
        cblk = cblk < a.Cin_pad ? cblk : a.Cin_pad;
        // keep at least ~2 workgroups per CU: split channels when rows are few
        while (int64_t(a.rows) * ((a.Cin_pad + cblk - 1) / cblk) < 512 && cblk >= 128)
            cblk = (cblk / 2) / cg * cg;
        const int cblocks = (a.Cin_pad + cblk - 1) / cblk;
        const size_t lds = (size_t(cblk) * cp + 64 * 8) * 2;   // runs + per-lane spill slots
        const StageFold fs = make_fold(fold, fold ? int64_t(fold->rows) * fold->row_len : 0);
        if (folded) *folded = fold != nullptr;
        const dim3 grid2(static_cast<unsigned>(int64_t(a.rows) * cblocks + fs.blocks));
        if (cg == 8)
            hipLaunchKernelGGL(pack_cl_staged_kernel<8>, grid2, dim3(256), lds, s, x, out, a.Cin,
                               a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad,
                               a.row_elems, a.row0, cblocks, cblk, cp, nck, x_elems, x_elems >> 3, fs);
        else
            hipLaunchKernelGGL(pack_cl_staged_kernel<4>, grid2, dim3(256), lds, s, x, out, a.Cin,
                               a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad,
                               a.row_elems, a.row0, cblocks, cblk, cp, nck, x_elems, x_elems >> 3, fs);
        return hipGetLastError();
    }
    // very wide rows: tiled form (64 columns x 4 filter rows x 64 channels per pass)
    const int cblocks = (a.Cin_pad + CB - 1) / CB;
    const dim3 grid(static_cast<unsigned>(int64_t(a.rows) * cblocks));
    if (cg == 8)
        hipLaunchKernelGGL(pack_cl_kernel<8>, grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W, a.KH,
                           a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad, a.row_elems, a.row0, cblocks);
    else
        hipLaunchKernelGGL(pack_cl_kernel<4>, grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W, a.KH,
                           a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad, a.row_elems, a.row0, cblocks);
    return hipGetLastError();
}

}  // namespace im2win
