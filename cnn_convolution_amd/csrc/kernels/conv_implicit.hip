// fp16 / bf16 implicit im2win convolution on the CDNA4 matrix cores: the
// window rows are built in LDS straight from x, so the window tensor never
// goes through HBM and no pack kernel runs.
//
// Output tile: MB output channels x (R window rows (n, ho0 .. ho0+R-1) of one
// image) x (WB output columns wo0 .. wo0+WB-1), NB >= R*WB GEMM columns
// (c = i*WB + wl; the rest of the NB columns is padding whose results are
// never stored). The window rows of the tile are the im2win rows of Eq. (2)
// of "Enabling Memory-efficient Im2win Convolution ..." (Sec. III-B): window
// row ho holds the KH input rows ho*s - p .. ho*s - p + KH - 1 interleaved
// column by column. Consecutive window rows share KH - s of those input
// rows, so the tile's rows are held as one patch of IR = (R-1)*s + KH input
// rows x IW = (WB-1)*s + KW input columns, channels innermost: the window of
// column (i, wl) at filter tap (kh, kw) is patch position
// (i*s + kh, wl*s + kw), and the 64 channels of one block at a position are
// one 128-byte LDS row (granule g of position q in slot g ^ (q & 7), so the
// fragment reads of consecutive positions hit different bank groups). Zero
// padding is written into the patch where the input row or column lies
// outside x.
//
// K runs over channel blocks of 64 (outer) and the KH*KW taps (inner); each
// (block, tap) is one 64-element K stage. Its filter tile (MB rows of the
// staged filter, K order (kw, kh, ci), the order in which Sec. III-D of the
// same paper contracts a window) goes memory -> LDS with
// global_load_lds_dwordx4 through three stage buffers, as in the
// direct-to-LDS window-GEMM; the window fragments come from the patch. The
// patch of a channel block is loaded once and serves all KH*KW taps: 8
// channels of one position per 16-byte vector, gathered with 2-byte loads
// that are coalesced along the input row.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "epilogue.hpp"
#include "lds_dma.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

constexpr int KI = kStageK;
constexpr int kPatchBatch = 4;   // patch vectors per thread whose loads are in flight together

struct ImplicitKArgs {
    const uint16_t *x;
    const uint16_t *wst;
    OutSpec out;            // y and its epilogue
    int Cin, H, W, Cout, KH, KW, stride, pad, Ho, Wo;
    int kstage;
    int R, WB, IR, IW;
    int tiles_ho, tiles_wo, tiles_m;
};

template <int MB, int NB, int WM, int NS, bool BF16>
__global__ __launch_bounds__(256) void conv_implicit_kernel(const ImplicitKArgs a)
{
    constexpr int WN = 4 / WM;
    constexpr int FM = MB / WM / 16;
    constexpr int FN = NB / WN / 16;
    constexpr int AI = MB / 32;            // 1 KB filter blocks per wave per stage
    constexpr int D = AI;                  // copies per wave per stage
    static_assert(AI >= 1 && AI * 32 == MB, "tiling");
    static_assert(FM >= 1 && FN >= 1 && WM * WN == 4, "wave layout");
    static_assert(NS >= 3 && (NS - 2) * D < 64, "stage buffers");
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    auto sbuf = [&](int b) { return lds + b * MB * KI; };   // filter stage buffer b < NS
    uint16_t *const patch = lds + NS * MB * KI;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, a.tiles_m, tm, tn);
    const int m0 = tm * MB;
    const int two = tn % a.tiles_wo;
    const int t2 = tn / a.tiles_wo;
    const int tho = t2 % a.tiles_ho;
    const int n = t2 / a.tiles_ho;
    const int ho0 = tho * a.R;
    const int wo0 = two * a.WB;
    const int ih0 = ho0 * a.stride - a.pad;
    const int iw0 = wo0 * a.stride - a.pad;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int taps = a.KH * a.KW;
    const int nk = (a.Cin / KI) * taps;
    const int HW = a.H * a.W;
    const uint16_t *const ximg = a.x + int64_t(n) * a.Cin * HW;

    // filter copy sources: row (wave + 4i)*8 + (lane >> 3) of the tile, granule
    // (lane & 7) ^ (lane >> 3); rows past Cout read row Cout-1 (never stored)
    const int rib = lane >> 3;
    const int g8 = ((lane & 7) ^ rib) * 8;
    const uint16_t *asrc[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = (wave + 4 * i) * 8 + rib;
        asrc[i] = a.wst + int64_t(min(m0 + r, a.Cout - 1)) * a.kstage + g8;
    }
    auto issue = [&](int stage, uint16_t *sa) {
        const int blk = stage / taps;
        const int tap = stage - blk * taps;
        const int kh = tap / a.KW;
        const int kw = tap - kh * a.KW;
        const int off = (kw * a.KH + kh) * a.Cin + blk * KI;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            copy_to_lds(asrc[i] + off, __builtin_amdgcn_readfirstlane(lds_addr(sa + (wave + 4 * i) * 512)));
    };

    // patch of channel block blk: IR*IW positions x 8 granules of 8 channels;
    // vector v = g*P + q, so consecutive lanes take consecutive positions of
    // one input row. The 2-byte loads go through a buffer resource on the
    // image (one 32-bit offset register per vector, the channel step in a
    // scalar offset); a position outside x loads element 0 of the image and
    // stores zeros instead.
    const int P = a.IR * a.IW;
    const int V = P * 8;
    // (an image holds fewer than 2^31 elements: byte offsets fit 32 unsigned bits)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(ximg), short(0), int(unsigned(a.Cin) * unsigned(HW) * 2u), 0x00020000);
    auto build_patch = [&](int blk) {
        const int cbase = blk * KI;
        for (int v0 = 0; v0 < V; v0 += 256 * kPatchBatch) {
            uint32_t val[kPatchBatch][8];
            int dst[kPatchBatch];
            bool in[kPatchBatch];
#pragma unroll
            for (int u = 0; u < kPatchBatch; ++u) {
                const int v = v0 + u * 256 + int(threadIdx.x);
                const int g = v / P;
                const int q = v - g * P;
                const int ihl = q / a.IW;
                const int ih = ih0 + ihl;
                const int iw = iw0 + (q - ihl * a.IW);
                in[u] = v < V && unsigned(ih) < unsigned(a.H) && unsigned(iw) < unsigned(a.W);
                dst[u] = v < V ? q * KI + ((g ^ (q & 7)) << 3) : -1;
                const unsigned off = in[u] ? unsigned((cbase + g * 8) * HW + ih * a.W + iw) * 2u : 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    val[u][e] = __builtin_amdgcn_raw_buffer_load_b16(xr, int(off), int(unsigned(e * HW) * 2u), 0);
            }
#pragma unroll
            for (int u = 0; u < kPatchBatch; ++u) {
                if (dst[u] < 0) continue;
                uint4 o;
                o.x = in[u] ? (val[u][0] | (val[u][1] << 16)) : 0u;
                o.y = in[u] ? (val[u][2] | (val[u][3] << 16)) : 0u;
                o.z = in[u] ? (val[u][4] | (val[u][5] << 16)) : 0u;
                o.w = in[u] ? (val[u][6] | (val[u][7] << 16)) : 0u;
                *reinterpret_cast<uint4 *>(patch + dst[u]) = o;
            }
        }
    };

    floatx4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // this lane's B column of each fragment: patch position of its window at
    // tap (0, 0); padding columns and columns past the image use position 0
    int qb[FN];
    bool cok[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int c = wn * (NB / WN) + j * 16 + (lane & 15);
        const int i = c / a.WB;
        const int wl = c - i * a.WB;
        cok[j] = c < a.R * a.WB && ho0 + i < a.Ho && wo0 + wl < a.Wo;
        qb[j] = cok[j] ? i * a.stride * a.IW + wl * a.stride : 0;
    }
    const int arow = wm * (MB / WM) + (lane & 15);
    auto compute = [&](int stage, const uint16_t *sa) {
        const int tap = stage % taps;
        const int kh = tap / a.KW;
        const int dq = kh * a.IW + (tap - kh * a.KW);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int gr = kk * 4 + (lane >> 4);        // granule of this lane's 8 K values
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = arow + i * 16;
                af[i] = *reinterpret_cast<const uint4 *>(sa + r * KI + ((gr ^ (r & 7)) * 8));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int q = qb[j] + dq;
                bf[j] = *reinterpret_cast<const uint4 *>(patch + q * KI + ((gr ^ (q & 7)) * 8));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<BF16>(af[i], bf[j], acc[i][j]);
        }
    };

    // the filter pipeline of the direct-to-LDS window-GEMM with NS stage
    // buffers: NS-1 stages in flight, each wave waiting only for its own
    // oldest one (every step issues one group, the stage index clamped to the
    // last, so the count in flight is the same at every step); at the first
    // tap of a channel block (after the barrier that ends every wave's reads
    // of the previous block) the patch is rebuilt and published by a second
    // barrier
    build_patch(0);
#pragma unroll
    for (int b = 0; b < NS - 1; ++b) issue(min(b, nk - 1), sbuf(b));
    auto step = [&](int k, int b) {
        wait_vm<(NS - 2) * D>();
        stage_barrier();
        if (k > 0 && k % taps == 0) {
            build_patch(k / taps);
            stage_barrier();
        }
        issue(min(k + NS - 1, nk - 1), sbuf((b + NS - 1) % NS));   // the buffer stage k-1 used
        compute(k, sbuf(b));
        __builtin_amdgcn_sched_barrier(0);
    };
    // unrolled by NS so that every buffer is named statically; the exit test
    // is uniform and the accumulators stay in the same registers
    for (int k = 0; k < nk; k += NS) {
#pragma unroll
        for (int b = 0; b < NS; ++b)
            if (k + b < nk) step(k + b, b);
    }
    wait_vm<0>();

    // epilogue: lane holds D[4*(lane/16) + v][lane%16] of every 16x16 block
    const int64_t plane = int64_t(a.Ho) * a.Wo;
    with_ytype(a.out, [&](auto tc) {
        constexpr int T = decltype(tc)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if (!cok[j]) continue;
            const int c = wn * (NB / WN) + j * 16 + (lane & 15);
            const int i = c / a.WB;
            const int wl = c - i * a.WB;
            const int64_t p = int64_t(ho0 + i) * a.Wo + wo0 + wl;
#pragma unroll
            for (int i2 = 0; i2 < FM; ++i2) {
                const int co0 = m0 + wm * (MB / WM) + i2 * 16 + (lane >> 4) * 4;
                if (a.out.plain) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (co0 + v < a.Cout)
                            static_cast<float *>(a.out.y)[(int64_t(n) * a.Cout + co0 + v) * plane + p] =
                                acc[i2][j][v];
                } else {
                    out_store_cols4<T>(a.out, n, co0, p, acc[i2][j]);
                }
            }
        }
    });
}

template <int MB, int NB, int WM, int NS>
hipError_t launch_implicit_tile(const ImplicitArgs &h, hipStream_t s)
{
    ImplicitKArgs a{};
    a.x = static_cast<const uint16_t *>(h.x);
    a.wst = static_cast<const uint16_t *>(h.wst);
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
    a.kstage = h.kstage;
    a.R = h.R;
    a.WB = h.WB;
    a.IR = h.IR;
    a.IW = h.IW;
    a.tiles_ho = (h.Ho + h.R - 1) / h.R;
    a.tiles_wo = (h.Wo + h.WB - 1) / h.WB;
    a.tiles_m = (h.Cout + MB - 1) / MB;
    const int64_t tiles = int64_t(a.tiles_m) * h.N * a.tiles_ho * a.tiles_wo;
    if (tiles < 1 || tiles > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = implicit_lds_bytes(MB, h.IR, h.IW, NS);
    auto kern = h.bf16 ? conv_implicit_kernel<MB, NB, WM, NS, true> : conv_implicit_kernel<MB, NB, WM, NS, false>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(tiles)), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_implicit(const ImplicitArgs &h, hipStream_t s)
{
    // channel blocks of 64, a patch that holds every window of the tile
    if (h.Cin % KI != 0 || h.R < 1 || h.WB < 1 || h.IR < (h.R - 1) * h.stride + h.KH ||
        h.IW < (h.WB - 1) * h.stride + h.KW || h.kstage != h.KW * h.KH * h.Cin ||
        h.tile_n < h.R * h.WB || h.stages < 3 || h.stages > 5 ||
        implicit_lds_bytes(h.tile_m, h.IR, h.IW, h.stages) > kImplicitMaxLdsBytes)
        return hipErrorInvalidValue;
#define IM2WIN_IMPLICIT_TILE(M, N, W)                                                              \
    if (h.tile_m == M && h.tile_n == N && h.wm == W) {                                            \
        if (h.stages == 5) return launch_implicit_tile<M, N, W, 5>(h, s);                          \
        if (h.stages == 4) return launch_implicit_tile<M, N, W, 4>(h, s);                          \
        return launch_implicit_tile<M, N, W, 3>(h, s);                                             \
    }
    IM2WIN_IMPLICIT_TILE(64, 64, 1)
    IM2WIN_IMPLICIT_TILE(64, 128, 1)
    IM2WIN_IMPLICIT_TILE(128, 64, 2)
    IM2WIN_IMPLICIT_TILE(128, 128, 2)
#undef IM2WIN_IMPLICIT_TILE
    return hipErrorInvalidValue;
}

}  // namespace im2win
