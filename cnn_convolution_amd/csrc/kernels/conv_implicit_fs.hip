// fp16 / bf16 implicit im2win convolution, filter-stationary form, for a
// short K (KW*KH*Cin <= 576): each workgroup keeps one 64-row block of the
// staged filter in registers for its whole life and walks a contiguous range
// of output tiles, so the filter is read once per workgroup instead of once
// per tile and the K loop of a tile has no barrier and no filter traffic.
//
// Output tile and window rows as in conv_implicit.hip: R window rows
// (n, ho0 ..) x WB output columns of one image, NB = 64*FN GEMM columns (the
// rest padding); the tile's window rows ("Enabling Memory-efficient Im2win
// Convolution ...", Sec. III-B Eq. (2)) are held as one channels-innermost
// patch of IR = (R-1)*s + KH input rows x IW = (WB-1)*s + KW columns per
// 64-channel block, one 128-byte LDS row per (block, position), granule g of
// row r in slot g ^ (r & 7). The contraction is Sec. III-C Eq. (3) in the window's
// K order (kw, kh, ci).
//
// The four waves lie 2 x 2 over the tile: each holds its 32 filter rows for
// the whole K as MFMA A fragments (K/32 x 2 fragments of 16 bytes per lane)
// and multiplies them with 16*FN of the tile's columns. Per tile: the loads of the next tile's patch are issued
// first (2-byte gathers through a buffer resource, 8 channels of one
// position per 16-byte vector), the current tile is multiplied from the LDS
// patch, its outputs are stored, the prefetched patch is written to the
// other LDS buffer, and one barrier ends the tile.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../launch.hpp"
#include "lds_dma.hpp"

namespace im2win {
namespace {

constexpr int KI = kStageK;
constexpr int kFsPrefetch = 6;   // gathered patch vectors per thread held for the next tile
constexpr int kFsUnits = 2;      // row-chunk units per thread held for the next tile (aligned rows)

struct FsKArgs {
    const uint16_t *x;
    const uint16_t *wst;
    float *y;
    int Cin, H, W, Cout, KH, KW, stride, pad, Ho, Wo;
    int kstage;
    int R, WB, IR, IW;
    int tiles_ho, tiles_wo, tiles_m;
    int col_tiles;          // N * tiles_ho * tiles_wo
    int groups;             // workgroups per 64-row filter block (gridDim.x / tiles_m)
};

template <int NKF, int FN, bool BF16, bool VEC>
__global__ __launch_bounds__(256, 1) void conv_implicit_fs_kernel(const FsKArgs a)
{
    constexpr int NB = 32 * FN;             // two waves along N, 16*FN columns each
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave & 1;                // 32-row half of the filter block
    const int wn = wave >> 1;               // half of the tile's columns
    const int tm = blockIdx.x % a.tiles_m;
    const int grp = blockIdx.x / a.tiles_m;
    const int m0 = tm * 64;
    // contiguous range of column tiles for this workgroup; neighbouring
    // workgroups of one XCD (blockIdx stride 8) take neighbouring ranges
    const int G = a.groups;
    const int xcd = grp & 7, gi = grp >> 3;
    const int per8 = G >> 3, rem8 = G & 7;
    const int lg = xcd * per8 + min(xcd, rem8) + gi;          // logical group, XCD-contiguous
    const int per = a.col_tiles / G, rem = a.col_tiles % G;
    const int c_begin = lg * per + min(lg, rem);
    const int c_end = c_begin + per + (lg < rem ? 1 : 0);

    const int HW = a.H * a.W;
    const int P = a.IR * a.IW;
    const int nblk = a.Cin / KI;
    const int V = nblk * P * 8;
    uint16_t *const pbuf0 = lds;
    uint16_t *const pbuf1 = lds + nblk * P * KI;

    // filter fragments: row m0 + 32*wm + 16i + (lane & 15) (clamped), K
    // values 32*ks + 8*(lane >> 4) .. +7
    uint4 af[2][NKF];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = min(m0 + 32 * wm + 16 * i + (lane & 15), a.Cout - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(a.wst + int64_t(row) * a.kstage + 8 * (lane >> 4));
#pragma unroll
        for (int ks = 0; ks < NKF; ++ks) af[i][ks] = src[ks * 4];
    }
    // all filter loads complete here, on every path: no wait for them can be
    // carried into the tile loop (where it would also wait for the prefetch)
    wait_vm<0>();
    // patch row offset of every 32-K step (wave-uniform): its channel block
    // and its tap (kw, kh)
    int dq[NKF];
#pragma unroll
    for (int ks = 0; ks < NKF; ++ks) {
        const int k0 = ks * 32;
        const int t = k0 / a.Cin;                 // tap index kw*KH + kh
        const int kw = t / a.KH;
        const int kh = t - kw * a.KH;
        const int blk = (k0 - t * a.Cin) / KI;
        dq[ks] = blk * P + kh * a.IW + kw;
    }

    auto tile_origin = [&](int c, int &n, int &ho0, int &wo0) {
        const int two = c % a.tiles_wo;
        const int t2 = c / a.tiles_wo;
        const int tho = t2 % a.tiles_ho;
        n = t2 / a.tiles_ho;
        ho0 = tho * a.R;
        wo0 = two * a.WB;
    };

    // Patch of tile c, in two steps: load_patch only issues the loads;
    // store_patch (after the current tile's multiply) packs and writes them,
    // so their latency overlaps the MFMAs.
    //
    // VEC (rows of x 16-byte aligned: W a multiple of 8): a unit is 8
    // channels x 8 consecutive input columns (one aligned 16-byte chunk of
    // each channel's row), loaded as 8 16-byte vectors and transposed in
    // registers into 8 patch vectors; columns outside x are written as zeros
    // by a second small pass. Otherwise: one patch vector (8 channels of one
    // position) per 8 two-byte gathers, vector v = (blk*8 + g)*P + q.
    constexpr int NU = VEC ? kFsUnits : kFsPrefetch;
    constexpr int NE = VEC ? 1 : 8;
    uint4 rv[VEC ? kFsUnits : 1][8];
    unsigned short raw[VEC ? 1 : kFsPrefetch][8];
    bool pin[NU];
    int pdst[NU];
    int piw0 = 0, pjlo = 0;
    (void)NE;
    auto load_patch = [&](int c) {
        int n, ho0, wo0;
        tile_origin(c, n, ho0, wo0);
        const int ih0 = ho0 * a.stride - a.pad;
        const int iw0 = wo0 * a.stride - a.pad;
        const uint16_t *ximg = a.x + int64_t(n) * a.Cin * HW;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(ximg), short(0), int(unsigned(a.Cin) * unsigned(HW) * 2u),
            0x00020000);
        if constexpr (VEC) {
            const int lo = max(iw0, 0), hi = min(iw0 + a.IW, a.W);
            const int jlo = lo >> 3;
            const int nch = hi > lo ? ((hi - 1) >> 3) - jlo + 1 : 0;
            const int U = nblk * 8 * a.IR * nch;
            piw0 = iw0;
            pjlo = jlo;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int v = u * 256 + int(threadIdx.x);
                const int rn = a.IR * max(nch, 1);
                const int bg = v / rn;                // blk*8 + g
                const int rem = v - bg * rn;
                const int r = rem / max(nch, 1);
                const int jj = rem - r * max(nch, 1);
                const int ih = ih0 + r;
                pin[u] = v < U && unsigned(ih) < unsigned(a.H);
                pdst[u] = v < U ? (bg << 16) | (r << 8) | jj : -1;   // unpacked in store_patch
                const unsigned off = pin[u] ? unsigned(bg * 8 * HW + ih * a.W + (jlo + jj) * 8) * 2u : 0u;
                if (pin[u]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        rv[u][e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 xr, int(off), int(unsigned(e * HW) * 2u), 0));
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int v = u * 256 + int(threadIdx.x);
                const int bg = v / P;                 // blk*8 + g
                const int q = v - bg * P;
                const int ihl = q / a.IW;
                const int ih = ih0 + ihl;
                const int iw = iw0 + (q - ihl * a.IW);
                pin[u] = v < V && unsigned(ih) < unsigned(a.H) && unsigned(iw) < unsigned(a.W);
                const int row = (bg >> 3) * P + q;
                pdst[u] = v < V ? row * KI + (((bg & 7) ^ (row & 7)) << 3) : -1;
                const unsigned off = pin[u] ? unsigned(bg * 8 * HW + ih * a.W + iw) * 2u : 0u;
                if (pin[u]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        raw[u][e] = __builtin_amdgcn_raw_buffer_load_b16(xr, int(off), int(unsigned(e * HW) * 2u), 0);
                }
            }
        }
    };
    auto store_patch = [&](uint16_t *buf) {
        if constexpr (VEC) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (pdst[u] < 0) continue;
                const int bg = pdst[u] >> 16, r = (pdst[u] >> 8) & 255, jj = pdst[u] & 255;
                const int blk = bg >> 3, g = bg & 7;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int iwl = (pjlo + jj) * 8 + t - piw0;
                    if (iwl < 0 || iwl >= a.IW) continue;
                    // position t of channels 2k, 2k+1: the low (t even) or high
                    // (t odd) halves of dword t/2 of their rows
                    const unsigned sel = (t & 1) ? 0x07060302u : 0x05040100u;
                    const int d = t >> 1;
                    auto pick = [&](int e) {
                        const uint4 &q4 = rv[u][e];
                        return d == 0 ? q4.x : d == 1 ? q4.y : d == 2 ? q4.z : q4.w;
                    };
                    uint4 o;
                    o.x = pin[u] ? __builtin_amdgcn_perm(pick(1), pick(0), sel) : 0u;
                    o.y = pin[u] ? __builtin_amdgcn_perm(pick(3), pick(2), sel) : 0u;
                    o.z = pin[u] ? __builtin_amdgcn_perm(pick(5), pick(4), sel) : 0u;
                    o.w = pin[u] ? __builtin_amdgcn_perm(pick(7), pick(6), sel) : 0u;
                    const int row = blk * P + r * a.IW + iwl;
                    *reinterpret_cast<uint4 *>(buf + row * KI + ((g ^ (row & 7)) << 3)) = o;
                }
            }
            // columns outside x: zeros (left: iw < 0, right: iw >= W)
            const int padl = max(-piw0, 0), padr = max(piw0 + a.IW - a.W, 0);
            const int npad = padl + padr;
            const int Z = nblk * 8 * a.IR * npad;
            for (int z = int(threadIdx.x); z < Z; z += 256) {
                const int bg = z / (a.IR * npad);
                const int rem = z - bg * (a.IR * npad);
                const int r = rem / npad;
                const int k = rem - r * npad;
                const int iwl = k < padl ? k : a.IW - padr + (k - padl);
                const int row = (bg >> 3) * P + r * a.IW + iwl;
                *reinterpret_cast<uint4 *>(buf + row * KI + (((bg & 7) ^ (row & 7)) << 3)) = uint4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (pdst[u] < 0) continue;
                uint4 o;
                // (a byte permute needs no zero-extension of the 16-bit loads)
                o.x = pin[u] ? __builtin_amdgcn_perm(raw[u][1], raw[u][0], 0x05040100u) : 0u;
                o.y = pin[u] ? __builtin_amdgcn_perm(raw[u][3], raw[u][2], 0x05040100u) : 0u;
                o.z = pin[u] ? __builtin_amdgcn_perm(raw[u][5], raw[u][4], 0x05040100u) : 0u;
                o.w = pin[u] ? __builtin_amdgcn_perm(raw[u][7], raw[u][6], 0x05040100u) : 0u;
                *reinterpret_cast<uint4 *>(buf + pdst[u]) = o;
            }
        }
    };

    if (c_begin < c_end) {
        load_patch(c_begin);
        store_patch(pbuf0);
    }
    __syncthreads();

    const int64_t plane = int64_t(a.Ho) * a.Wo;
    int cur = 0;
    for (int c = c_begin; c < c_end; ++c) {
        const bool more = c + 1 < c_end;
        if (more) load_patch(c + 1);                // in flight while this tile is multiplied
        const uint16_t *pb = cur ? pbuf1 : pbuf0;
        int n, ho0, wo0;
        tile_origin(c, n, ho0, wo0);

        // this lane's column of each fragment: patch position at tap (0, 0)
        int qb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = wn * (NB / 2) + j * 16 + (lane & 15);
            const int i = col / a.WB;
            const int wl = col - i * a.WB;
            const bool ok = col < a.R * a.WB && ho0 + i < a.Ho && wo0 + wl < a.Wo;
            qb[j] = ok ? i * a.stride * a.IW + wl * a.stride : 0;
        }
        // the product is formed transposed, D = window^T x filter^T: the
        // patch fragment is the MFMA A operand (lane: column lane%16) and the
        // filter fragment the B operand (lane: output channel lane%16), so a
        // lane ends with 4 consecutive columns of one output channel
        floatx4_t acc[2][FN];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        // window fragments of one K step for every column fragment, read two
        // steps ahead of their MFMAs
        auto read_b = [&](int ks, uint4 (&b)[FN]) {
            const int gr = (ks & 1) * 4 + (lane >> 4);     // granule of this lane's 8 channels
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = qb[j] + dq[ks];
                b[j] = *reinterpret_cast<const uint4 *>(pb + row * KI + ((gr ^ (row & 7)) * 8));
            }
        };
        uint4 bb[3][FN];
        read_b(0, bb[0]);
        if (NKF > 1) read_b(1, bb[1]);
#pragma unroll
        for (int ks = 0; ks < NKF; ++ks) {
            if (ks + 2 < NKF) read_b(ks + 2, bb[(ks + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's MFMAs
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = mfma16x16x32<BF16>(bb[ks % 3][j], af[i][ks], acc[i][j]);
        }
        // outputs: lane holds D[4*(lane/16) + v][lane%16], i.e. columns
        // c0 .. c0+3 (c0 = fragment base + 4*(lane/16)) of output channel
        // m0 + 32*wm + 16*i + lane%16; one 16-byte store when the four are
        // consecutive outputs of one row and 16-byte aligned
        float *const yimg = a.y + int64_t(n) * a.Cout * plane;
        const bool quad = (a.Wo & 3) == 0 && (a.WB & 3) == 0;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c0 = wn * (NB / 2) + j * 16 + 4 * (lane >> 4);
            const int i0 = c0 / a.WB;
            const int wl0 = c0 - i0 * a.WB;
            const bool whole = quad && c0 + 3 < a.R * a.WB && ho0 + i0 < a.Ho && wo0 + wl0 + 3 < a.Wo;
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                const int co = m0 + 32 * wm + i2 * 16 + (lane & 15);
                if (co >= a.Cout) continue;
                float *ych = yimg + int64_t(co) * plane;
                if (whole) {
                    *reinterpret_cast<floatx4_t *>(ych + int64_t(ho0 + i0) * a.Wo + wo0 + wl0) = acc[i2][j];
                    continue;
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int col = c0 + v;
                    const int i = col / a.WB;
                    const int wl = col - i * a.WB;
                    if (col < a.R * a.WB && ho0 + i < a.Ho && wo0 + wl < a.Wo)
                        ych[int64_t(ho0 + i) * a.Wo + wo0 + wl] = acc[i2][j][v];
                }
            }
        }
        if (more) store_patch(cur ? pbuf0 : pbuf1);
        __syncthreads();
        cur ^= 1;
    }
}

template <int NKF, int FN, bool VEC>
hipError_t launch_fs(const ImplicitArgs &h, hipStream_t s)
{
    FsKArgs a{};
    a.x = static_cast<const uint16_t *>(h.x);
    a.wst = static_cast<const uint16_t *>(h.wst);
    a.y = h.y;
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
    a.kstage = h.kstage;
    a.R = h.R;
    a.WB = h.WB;
    a.IR = h.IR;
    a.IW = h.IW;
    a.tiles_ho = (h.Ho + h.R - 1) / h.R;
    a.tiles_wo = (h.Wo + h.WB - 1) / h.WB;
    a.tiles_m = (h.Cout + 63) / 64;
    const int64_t col_tiles = int64_t(h.N) * a.tiles_ho * a.tiles_wo;
    if (col_tiles < 1 || col_tiles > 0x7fffffff) return hipErrorInvalidValue;
    a.col_tiles = int(col_tiles);
    a.groups = int(std::min<int64_t>(col_tiles, std::max(1, h.fs_groups)));
    const int64_t grid = int64_t(a.groups) * a.tiles_m;
    const size_t lds = size_t(2) * (h.Cin / KI) * h.IR * h.IW * 128;
    auto kern = h.bf16 ? conv_implicit_fs_kernel<NKF, FN, true, VEC>
                       : conv_implicit_fs_kernel<NKF, FN, false, VEC>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_implicit_fs(const ImplicitArgs &h, hipStream_t s)
{
    const int64_t K = int64_t(h.KW) * h.KH * h.Cin;
    const int64_t V = int64_t(h.Cin / KI) * h.IR * h.IW * 8;
    if (h.Cin % KI != 0 || h.R < 1 || h.WB < 1 || h.IR < (h.R - 1) * h.stride + h.KH ||
        h.IW < (h.WB - 1) * h.stride + h.KW || h.kstage != K || h.tile_m != 64 ||
        h.tile_n < h.R * h.WB ||
        implicit_fs_lds_bytes(h.Cin, h.IR, h.IW) > kImplicitMaxLdsBytes)
        return hipErrorInvalidValue;
    if (h.W % 8 == 0) {
        // row-chunk patch loads: every unit of a tile held in registers
        const int64_t chunks = (int64_t(h.IW) + 7) / 8 + 1;
        if (int64_t(h.Cin / KI) * 8 * h.IR * chunks > 256 * kFsUnits) return hipErrorInvalidValue;
        if (K == 576 && h.tile_n == 64) return launch_fs<18, 2, true>(h, s);
        if (K == 64 && h.tile_n == 128) return launch_fs<2, 4, true>(h, s);
        if (K == 128 && h.tile_n == 128) return launch_fs<4, 4, true>(h, s);
        if (K == 256 && h.tile_n == 128) return launch_fs<8, 4, true>(h, s);
        return hipErrorInvalidValue;
    }
    if (V > 256 * kFsPrefetch) return hipErrorInvalidValue;
    if (K == 576 && h.tile_n == 64) return launch_fs<18, 2, false>(h, s);
    if (K == 64 && h.tile_n == 128) return launch_fs<2, 4, false>(h, s);
    if (K == 128 && h.tile_n == 128) return launch_fs<4, 4, false>(h, s);
    if (K == 256 && h.tile_n == 128) return launch_fs<8, 4, false>(h, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
