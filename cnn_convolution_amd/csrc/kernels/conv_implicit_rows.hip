// fp16 / bf16 implicit im2win convolution, row-block form, for layers with
// 64 input channels, stride 1, input rows a multiple of 8 long and output
// rows of at most 64 columns (the ResNet-style 3x3 and 1x1 layers).
//
// A workgroup of eight waves owns a block of RW consecutive output rows
// (n, ho0 .. ho0+RW-1) of one image and a block of 64 output channels. The
// window rows of those output rows (Eq. (2) of "Enabling Memory-efficient
// Im2win Convolution with Multi-precision Support on GPU CUDA and Tensor
// Cores", Sec. III-B: window row ho interleaves input rows ho - pad .. ho -
// pad + KH - 1) share all but their first and last input rows, so the block
// holds the union once: SL = RW + KH - 1 input rows of IW = W + 2*pad
// positions (zero padding included), channels innermost, one 128-byte LDS
// row per position (8-channel granule g of position q in slot g ^ (q & 7),
// so reads of consecutive positions hit different bank groups). The window
// of output column wo of row i at filter tap (kh, kw) is position
// (i + kh, wo + kw).
//
// The filter block stays in LDS for the whole contraction: w[co][ci][kh][kw]
// is read as it is stored (8 channels x all taps of one output channel per
// thread, 16-byte loads), reordered in registers into one 64-channel run per
// tap (the window's K order of Sec. III-D: taps outer, channels inner), and
// written once. Nothing is staged in device memory.
//
// Every load of the block is issued before the first wait (the filter and
// the input rows, 16-byte loads of 8 consecutive columns of one channel,
// transposed 8 x 8 in registers with byte permutes into 8 channels of one
// position), then one barrier; after it wave i contracts output row i on its
// own (no further barrier): the product is formed transposed, D[column][co],
// so that a lane holds 4 consecutive output columns of one channel and
// stores them as one 16-byte vector.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "lds_dma.hpp"
#include "out_blocks.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

constexpr int kRowsThreads = 512;   // eight waves: one output row each

struct RowsKArgs {
    const uint16_t *x;
    const uint16_t *w;
    OutSpec out;            // y and its epilogue
    int Cin, H, W, Cout, pad, Ho, Wo;
    int RW;                 // output rows per workgroup
    int row_groups;         // ceil(Ho / RW)
    int co_blocks;          // ceil(Cout / 64)
    int IW;                 // W + 2*pad
};

// 16-bit element e (0..7) of a 16-byte vector, as the low half of a dword
__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

template <int KH, int KW, bool BF16>
__global__ __launch_bounds__(kRowsThreads) void conv_implicit_rows_kernel(const RowsKArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int CIN = 64;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *const fl = lds;                        // [TAPS][64 co][64 ci], 8 KB per tap
    uint16_t *const patch = lds + TAPS * 64 * CIN;   // [SL][IW][64 ci]

    int cb, tn;
    tile_coords(blockIdx.x, gridDim.x, a.co_blocks, cb, tn);
    const int rg = tn % a.row_groups;
    const int n = tn / a.row_groups;
    const int ho0 = rg * a.RW;
    const int rw = min(a.RW, a.Ho - ho0);            // rows of this block
    const int SL = rw + KH - 1;                      // input rows held
    const int ih0 = ho0 - a.pad;
    const int tid = threadIdx.x;
    const int HW = a.H * a.W;
    const uint16_t *const ximg = a.x + int64_t(n) * CIN * HW;

    // ---- issue every load of the block -------------------------------------
    // filter: thread = (output channel co_l, 8-channel group cg); its 8 x TAPS
    // halves w[co][cg*8 .. cg*8+7][taps] are contiguous (16*TAPS bytes)
    const int co_l = tid >> 3;
    const int cg = tid & 7;
    const int co_src = min(cb * 64 + co_l, a.Cout - 1);  // rows past Cout: never stored
    uint4 wraw[TAPS];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.w + (int64_t(co_src) * CIN + cg * 8) * TAPS);
#pragma unroll
        for (int i = 0; i < TAPS; ++i) wraw[i] = src[i];
    }
    // input rows: units of (input row i, chunk k of 8 columns, 8-channel group
    // g), g fastest so that the 8 lanes writing one position hit 8 different
    // bank groups; a wave's load of channel g*8+e covers 8 consecutive chunks
    const int CW = a.W >> 3;
    const int units = SL * CW * 8;
    auto unit_src = [&](int u, int &i, int &k, int &g, bool &in) {
        g = u & 7;
        const int r = u >> 3;
        i = r / CW;
        k = r - i * CW;
        in = unsigned(ih0 + i) < unsigned(a.H);
    };
    uint4 xraw[8];
    int ui, uk, ug;
    bool uin;
    {
        const int u = min(tid, units - 1);
        unit_src(u, ui, uk, ug, uin);
        const uint4 *src = reinterpret_cast<const uint4 *>(
            ximg + int64_t(ug * 8) * HW + int64_t(uin ? ih0 + ui : 0) * a.W + uk * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) xraw[e] = src[int64_t(e) * (HW >> 3)];
    }

    // ---- filter: one 16-byte vector per tap, 8 channels of co_l -------------
    // (element e of tap t is half e*TAPS + t of the 8*TAPS run)
#pragma unroll
    for (int t = 0; t < TAPS; ++t) {
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int p0 = (2 * d) * TAPS + t, p1 = (2 * d + 1) * TAPS + t;
            const uint32_t s0 = dword_of(wraw[p0 >> 3], (p0 & 7) >> 1);
            const uint32_t s1 = dword_of(wraw[p1 >> 3], (p1 & 7) >> 1);
            const uint32_t sel = ((p0 & 1) ? 0x0302u : 0x0100u) | ((p1 & 1) ? 0x07060000u : 0x05040000u);
            o[d] = __builtin_amdgcn_perm(s1, s0, sel);
        }
        *reinterpret_cast<uint4 *>(fl + t * 64 * CIN + co_l * CIN + ((cg ^ (co_l & 7)) << 3)) =
            uint4{o[0], o[1], o[2], o[3]};
    }

    // ---- input rows: 8 x 8 transpose into 8 positions of one granule ---------
    auto put_unit = [&](int i, int k, int g, bool in, const uint4 *raw) {
        const int qrow = i * a.IW + a.pad + k * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            uint4 o;
            o.x = in ? __builtin_amdgcn_perm(dword_of(raw[1], j >> 1), dword_of(raw[0], j >> 1), sel) : 0u;
            o.y = in ? __builtin_amdgcn_perm(dword_of(raw[3], j >> 1), dword_of(raw[2], j >> 1), sel) : 0u;
            o.z = in ? __builtin_amdgcn_perm(dword_of(raw[5], j >> 1), dword_of(raw[4], j >> 1), sel) : 0u;
            o.w = in ? __builtin_amdgcn_perm(dword_of(raw[7], j >> 1), dword_of(raw[6], j >> 1), sel) : 0u;
            const int q = qrow + j;
            *reinterpret_cast<uint4 *>(patch + q * CIN + ((g ^ (q & 7)) << 3)) = o;
        }
    };
    if (tid < units) put_unit(ui, uk, ug, uin, xraw);
    for (int u = tid + kRowsThreads; u < units; u += kRowsThreads) {
        int i, k, g;
        bool in;
        unit_src(u, i, k, g, in);
        const uint4 *src = reinterpret_cast<const uint4 *>(
            ximg + int64_t(g * 8) * HW + int64_t(in ? ih0 + i : 0) * a.W + k * 8);
        uint4 raw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[e] = src[int64_t(e) * (HW >> 3)];
        put_unit(i, k, g, in, raw);
    }
    // zero padding columns (positions < pad and >= pad + W) of every row
    const int pads = SL * 2 * a.pad * 8;
    for (int v = tid; v < pads; v += kRowsThreads) {
        const int g = v & 7;
        const int r = v >> 3;
        const int i = r / (2 * a.pad);
        const int c = r - i * 2 * a.pad;
        const int q = i * a.IW + (c < a.pad ? c : a.W + c);
        *reinterpret_cast<uint4 *>(patch + q * CIN + ((g ^ (q & 7)) << 3)) = uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    // ---- this wave's output blocks: up to 64 outputs x 64 channels -----------
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int outs = rw * a.Wo;
    int b0, nb;
    wave_blocks(wave, outs, b0, nb);
    floatx4_t acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    int qa[4];
    block_bases(qa, b0, lane, outs, a.Wo, a.IW);
    const int rb = lane & 15;                        // this lane's B column (co) in a block
    // one compiled contraction per block count, so the unrolled K loop holds
    // no run-time test
    auto contract = [&](auto nbc) {
        constexpr int NBW = decltype(nbc)::value;
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const uint16_t *ft = fl + (kh * KW + kw) * 64 * CIN;
                const int dq = kh * a.IW + kw;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int gr = kk * 4 + (lane >> 4);
                    uint4 af[NBW], bf[4];
#pragma unroll
                    for (int s = 0; s < NBW; ++s) {
                        const int q = qa[s] + dq;
                        af[s] = *reinterpret_cast<const uint4 *>(patch + q * CIN + ((gr ^ (q & 7)) << 3));
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = c * 16 + rb;
                        bf[c] = *reinterpret_cast<const uint4 *>(ft + r * CIN + ((gr ^ (r & 7)) << 3));
                    }
#pragma unroll
                    for (int s = 0; s < NBW; ++s)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(af[s], bf[c], acc[s][c]);
                }
            }
        }
    };
    if (nb >= 4) contract(std::integral_constant<int, 4>{});
    else if (nb == 3) contract(std::integral_constant<int, 3>{});
    else if (nb == 2) contract(std::integral_constant<int, 2>{});
    else if (nb == 1) contract(std::integral_constant<int, 1>{});
    // direct 16-byte stores for fp32 y of the 3x3 form (measured faster than the
    // LDS-staged whole-line stores there: 14.5 vs 16.5 us on the ResNet layer);
    // the 1x1 form, half-precision y and rows of other widths go through LDS
    if ((a.Wo & 3) == 0 && a.out.type == 0 && TAPS > 1) {
        if (nb > 0) store_blocks<4, true>(acc, nb, b0, lane, a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
    } else {
        __syncthreads();                             // patch and filter are dead: LDS is store scratch
        if (nb > 0)
            store_blocks_lds(acc, nb, b0, lane, reinterpret_cast<float *>(lds) + wave * kStoreScratchFloats,
                             a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
    }
}

// The half-precision row block over several 64-channel blocks and for any
// row width (the deep 3x3 layers: 128 - 512 channels on small images): the
// block's accumulators stay in registers while the channel blocks pass
// through LDS one at a time, each block's filter chunk (64 output channels x
// all taps x 64 channels, reordered from w as stored) and patch rows replacing
// the previous block's after a barrier. The next block's loads are issued
// before the current block is contracted and written after it, so they are
// in flight during the contraction. Rows whose width is a multiple of 8 are
// loaded as 16-byte row chunks and transposed in registers (as in the
// one-block kernel); other widths are gathered 2 bytes at a time, 8 channels
// of one position per unit with consecutive lanes on consecutive columns.
template <int KH, int KW, bool BF16, bool VEC8>
__global__ __launch_bounds__(kRowsThreads) void conv_implicit_rows_multi_kernel(const RowsKArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int CIN = 64;                          // channels per block
    constexpr int UG = 4;                            // gathered units per thread held per block
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *const fl = lds;                        // [TAPS][64 co][64 ci]
    uint16_t *const patch = lds + TAPS * 64 * CIN;   // [SL][IW][64 ci]

    int cb, tn;
    tile_coords(blockIdx.x, gridDim.x, a.co_blocks, cb, tn);
    const int rg = tn % a.row_groups;
    const int n = tn / a.row_groups;
    const int ho0 = rg * a.RW;
    const int rw = min(a.RW, a.Ho - ho0);
    const int SL = rw + KH - 1;
    const int ih0 = ho0 - a.pad;
    const int tid = threadIdx.x;
    const int HW = a.H * a.W;
    const int nblk = a.Cin / CIN;
    const uint16_t *const ximg = a.x + int64_t(n) * a.Cin * HW;
    const int co_l = tid >> 3;
    const int cg = tid & 7;
    const int co_src = min(cb * 64 + co_l, a.Cout - 1);
    // patch units of one block: VEC8: (row i, 8-column chunk k, group g), g
    // fastest; gather: (row i, group g, column c), c fastest
    const int units = VEC8 ? SL * (a.W >> 3) * 8 : SL * 8 * a.W;

    // ---- registers of one block's loads ------------------------------------
    uint4 wraw[TAPS];
    uint4 vraw[8];                                   // VEC8: the first unit
    uint32_t graw[UG][8];                            // gather: the first UG units
    // the patch units are prefetched; the filter chunk (from L2: w is small
    // and read by every workgroup of its 64-channel block) is loaded when the
    // block is written, which keeps the registers held across the contraction
    // to the patch units
    auto issue = [&](int blk) {
        const uint16_t *xb = ximg + int64_t(blk * CIN) * HW;
        if constexpr (VEC8) {
            const int CW = a.W >> 3;
            const int u = min(tid, units - 1);
            const int g = u & 7, r = u >> 3, i = r / CW, k = r - i * CW;
            const bool in = unsigned(ih0 + i) < unsigned(a.H);
            const uint4 *vs = reinterpret_cast<const uint4 *>(xb + int64_t(g * 8) * HW +
                                                              int64_t(in ? ih0 + i : 0) * a.W + k * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) vraw[e] = vs[int64_t(e) * (HW >> 3)];
        } else {
#pragma unroll
            for (int j = 0; j < UG; ++j) {
                const int u = min(tid + j * kRowsThreads, units - 1);
                const int c = u % a.W, r = u / a.W, g = r & 7, i = r >> 3;
                const bool in = unsigned(ih0 + i) < unsigned(a.H);
                const uint16_t *gs = xb + int64_t(g * 8) * HW + (in ? (ih0 + i) * a.W + c : 0);
#pragma unroll
                for (int e = 0; e < 8; ++e) graw[j][e] = gs[int64_t(e) * HW];
            }
        }
    };
    // 8 x 8 transpose of a VEC8 unit into 8 positions of one granule
    auto put_vec8 = [&](int i, int k, int g, bool in, const uint4 *raw) {
        const int qrow = i * a.IW + a.pad + k * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            uint4 o;
            o.x = in ? __builtin_amdgcn_perm(dword_of(raw[1], j >> 1), dword_of(raw[0], j >> 1), sel) : 0u;
            o.y = in ? __builtin_amdgcn_perm(dword_of(raw[3], j >> 1), dword_of(raw[2], j >> 1), sel) : 0u;
            o.z = in ? __builtin_amdgcn_perm(dword_of(raw[5], j >> 1), dword_of(raw[4], j >> 1), sel) : 0u;
            o.w = in ? __builtin_amdgcn_perm(dword_of(raw[7], j >> 1), dword_of(raw[6], j >> 1), sel) : 0u;
            const int q = qrow + j;
            *reinterpret_cast<uint4 *>(patch + q * CIN + ((g ^ (q & 7)) << 3)) = o;
        }
    };
    auto put_gather = [&](int u, const uint32_t *h) {
        const int c = u % a.W, r = u / a.W, g = r & 7, i = r >> 3;
        const bool in = unsigned(ih0 + i) < unsigned(a.H);
        const int q = i * a.IW + a.pad + c;
        *reinterpret_cast<uint4 *>(patch + q * CIN + ((g ^ (q & 7)) << 3)) =
            in ? uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)}
               : uint4{0u, 0u, 0u, 0u};
    };
    // write one block: the filter chunk from wraw, the patch from the held
    // units, the remaining units loaded and written here
    auto commit = [&](int blk) {
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(
                a.w + (int64_t(co_src) * a.Cin + blk * CIN + cg * 8) * TAPS);
#pragma unroll
            for (int i = 0; i < TAPS; ++i) wraw[i] = src[i];
        }
#pragma unroll
        for (int t = 0; t < TAPS; ++t) {
            uint32_t o[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int p0 = (2 * d) * TAPS + t, p1 = (2 * d + 1) * TAPS + t;
                const uint32_t s0 = dword_of(wraw[p0 >> 3], (p0 & 7) >> 1);
                const uint32_t s1 = dword_of(wraw[p1 >> 3], (p1 & 7) >> 1);
                const uint32_t sel = ((p0 & 1) ? 0x0302u : 0x0100u) | ((p1 & 1) ? 0x07060000u : 0x05040000u);
                o[d] = __builtin_amdgcn_perm(s1, s0, sel);
            }
            *reinterpret_cast<uint4 *>(fl + t * 64 * CIN + co_l * CIN + ((cg ^ (co_l & 7)) << 3)) =
                uint4{o[0], o[1], o[2], o[3]};
        }
        const uint16_t *xb = ximg + int64_t(blk * CIN) * HW;
        if constexpr (VEC8) {
            const int CW = a.W >> 3;
            auto unit = [&](int u, int &i, int &k, int &g, bool &in) {
                g = u & 7;
                const int r = u >> 3;
                i = r / CW;
                k = r - i * CW;
                in = unsigned(ih0 + i) < unsigned(a.H);
            };
            if (tid < units) {
                int i, k, g;
                bool in;
                unit(tid, i, k, g, in);
                put_vec8(i, k, g, in, vraw);
            }
            for (int u = tid + kRowsThreads; u < units; u += kRowsThreads) {
                int i, k, g;
                bool in;
                unit(u, i, k, g, in);
                const uint4 *vs = reinterpret_cast<const uint4 *>(xb + int64_t(g * 8) * HW +
                                                                  int64_t(in ? ih0 + i : 0) * a.W + k * 8);
                uint4 raw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) raw[e] = vs[int64_t(e) * (HW >> 3)];
                put_vec8(i, k, g, in, raw);
            }
        } else {
#pragma unroll
            for (int j = 0; j < UG; ++j)
                if (tid + j * kRowsThreads < units) put_gather(tid + j * kRowsThreads, graw[j]);
            for (int u = tid + UG * kRowsThreads; u < units; u += kRowsThreads) {
                const int c = u % a.W, r = u / a.W, g = r & 7, i = r >> 3;
                const bool in = unsigned(ih0 + i) < unsigned(a.H);
                const uint16_t *gs = xb + int64_t(g * 8) * HW + (in ? (ih0 + i) * a.W + c : 0);
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = gs[int64_t(e) * HW];
                put_gather(u, h);
            }
        }
    };

    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int outs = rw * a.Wo;
    int b0, nb;
    wave_blocks(wave, outs, b0, nb);
    floatx4_t acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    int qa[4];
    block_bases(qa, b0, lane, outs, a.Wo, a.IW);
    const int rb = lane & 15;
    auto contract = [&](auto nbc) {
        constexpr int NBW = decltype(nbc)::value;
        // the per-lane bases pass through an empty asm once per block, so the
        // compiler recomputes each step's LDS addresses instead of holding all
        // of them in registers across the channel-block loop
        int q0[NBW];
#pragma unroll
        for (int s = 0; s < NBW; ++s) {
            q0[s] = qa[s];
            asm volatile("" : "+v"(q0[s]));
        }
        int rbv = rb;
        asm volatile("" : "+v"(rbv));
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const uint16_t *ft = fl + (kh * KW + kw) * 64 * CIN;
                const int dq = kh * a.IW + kw;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int gr = kk * 4 + (lane >> 4);
                    uint4 af[NBW], bf[4];
#pragma unroll
                    for (int s = 0; s < NBW; ++s) {
                        const int q = q0[s] + dq;
                        af[s] = *reinterpret_cast<const uint4 *>(patch + q * CIN + ((gr ^ (q & 7)) << 3));
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = c * 16 + rbv;
                        bf[c] = *reinterpret_cast<const uint4 *>(ft + r * CIN + ((gr ^ (r & 7)) << 3));
                    }
#pragma unroll
                    for (int s = 0; s < NBW; ++s)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(af[s], bf[c], acc[s][c]);
                }
            }
        }
    };

    // zero padding columns of every row held (the same positions in every block)
    const int pads = SL * 2 * a.pad * 8;
    for (int v = tid; v < pads; v += kRowsThreads) {
        const int g = v & 7;
        const int r = v >> 3;
        const int i = r / (2 * a.pad);
        const int c = r - i * 2 * a.pad;
        const int q = i * a.IW + (c < a.pad ? c : a.W + c);
        *reinterpret_cast<uint4 *>(patch + q * CIN + ((g ^ (q & 7)) << 3)) = uint4{0u, 0u, 0u, 0u};
    }
    issue(0);
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk > 0) __syncthreads();                // every wave is done with the previous block
        commit(blk);
        __syncthreads();
        if (blk + 1 < nblk) issue(blk + 1);          // in flight during this block's contraction
        if (nb >= 4) contract(std::integral_constant<int, 4>{});
        else if (nb == 3) contract(std::integral_constant<int, 3>{});
        else if (nb == 2) contract(std::integral_constant<int, 2>{});
        else if (nb == 1) contract(std::integral_constant<int, 1>{});
    }
    if ((a.Wo & 3) == 0 && a.out.type == 0) {
        if (nb > 0) store_blocks(acc, nb, b0, lane, a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
    } else {
        __syncthreads();                             // patch and filter are dead: LDS is store scratch
        if (nb > 0)
            store_blocks_lds(acc, nb, b0, lane, reinterpret_cast<float *>(lds) + wave * kStoreScratchFloats,
                             a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
    }
}

// fp32 form of the same row block on the matrix cores' fp32 multiply
// (v_mfma_f32_16x16x4_f32: fp32 products, fp32 accumulation): the input
// channels are taken in blocks of 32 (128 bytes per position, the LDS
// geometry of the half-precision form), each block's filter slice (64
// output channels x all taps x 32 channels) and its input rows loaded,
// contracted, and replaced by the next block's after a barrier. Units of the
// input rows are 4 channels x 4 columns (16-byte loads of 4 columns of one
// channel), transposed by register moves. K of one MFMA step is 4 channels:
// lane group g = lane / 16 holds channels 4g .. 4g + 3 of a 16-channel slice
// as one 16-byte vector and feeds element j to step j, for the window rows
// and the filter alike.
struct RowsF32KArgs {
    const float *x;
    const float *w;
    OutSpec out;            // y and its epilogue
    int Cin, H, W, Cout, pad, Ho, Wo;
    int RW, row_groups, co_blocks, IW;
};

// VEC4: rows of 4k floats, loaded as 16-byte row chunks of one channel and
// transposed in registers; otherwise (any row width) each unit gathers the 4
// channels of one position with 4-byte loads, consecutive lanes on
// consecutive positions of the block's input rows (one contiguous run of
// every channel plane), and the rows outside the image are zeroed once.
template <int KH, int KW, bool VEC4>
__global__ __launch_bounds__(kRowsThreads) void conv_implicit_rows_f32_kernel(const RowsF32KArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int CB = 32;                           // channels per block: 128 bytes per position
    extern __shared__ __attribute__((aligned(16))) float ldsf[];
    float *const fl = ldsf;                          // [TAPS][64 co][32 ci], 8 KB per tap
    float *const patch = ldsf + TAPS * 64 * CB;      // [SL][IW][32 ci]

    int cb, tn;
    tile_coords(blockIdx.x, gridDim.x, a.co_blocks, cb, tn);
    const int rg = tn % a.row_groups;
    const int n = tn / a.row_groups;
    const int ho0 = rg * a.RW;
    const int rw = min(a.RW, a.Ho - ho0);
    const int SL = rw + KH - 1;
    const int ih0 = ho0 - a.pad;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int HW = a.H * a.W;
    const float *const ximg = a.x + int64_t(n) * a.Cin * HW;
    const int nblk = a.Cin / CB;
    const int CW = a.W >> 2;                         // chunks of 4 columns
    // VEC4: (input row, chunk, 4-channel group); else (4-channel group,
    // position of the block's rows in the image), position fastest
    const int r_lo = max(ih0, 0), r_hi = max(min(ih0 + SL, a.H), r_lo);
    const int npos = (r_hi - r_lo) * a.W;
    const int units = VEC4 ? SL * CW * 8 : 8 * npos;
    const int co_l = tid >> 3;
    const int cg = tid & 7;                          // 4-channel group of the block
    const int co_src = min(cb * 64 + co_l, a.Cout - 1);

    // zero padding columns of every row held (the same positions for every block)
    const int pads = SL * 2 * a.pad * 8;
    for (int v = tid; v < pads; v += kRowsThreads) {
        const int g = v & 7;
        const int r = v >> 3;
        const int i = r / (2 * a.pad);
        const int c = r - i * 2 * a.pad;
        const int q = i * a.IW + (c < a.pad ? c : a.W + c);
        *reinterpret_cast<float4 *>(patch + q * CB + ((g ^ (q & 7)) << 2)) = float4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (!VEC4) {
        // rows of the block outside the image (the same in every channel block)
        const int top = r_lo - ih0;                  // rows 0 .. top-1
        const int bot = SL - (r_hi - ih0);           // the last bot rows
        for (int v = tid; v < (top + bot) * a.IW * 8; v += kRowsThreads) {
            const int g = v & 7, e = v >> 3;
            const int zr = e / a.IW, c = e - zr * a.IW;
            const int i = zr < top ? zr : (r_hi - ih0) + (zr - top);
            const int q = i * a.IW + c;
            *reinterpret_cast<float4 *>(patch + q * CB + ((g ^ (q & 7)) << 2)) = float4{0.f, 0.f, 0.f, 0.f};
        }
    }

    floatx4_t acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const int outs = rw * a.Wo;
    int b0, nb;
    wave_blocks(wave, outs, b0, nb);
    int qa[4];
    block_bases(qa, b0, lane, outs, a.Wo, a.IW);
    const int rbl = lane & 15;

    for (int blk = 0; blk < nblk; ++blk) {
        if (blk > 0) __syncthreads();                // every wave is done with the previous block
        // filter slice: thread (co_l, cg) reads w[co][blk*32 + cg*4 .. +3][taps]
        // (4*TAPS contiguous floats) and writes one 4-channel vector per tap
        float4 wraw[TAPS];
        {
            const float4 *src = reinterpret_cast<const float4 *>(
                a.w + (int64_t(co_src) * a.Cin + blk * CB + cg * 4) * TAPS);
#pragma unroll
            for (int i = 0; i < TAPS; ++i) wraw[i] = src[i];
        }
        auto load_unit = [&](int u, float4 *raw, int &q0, int &g, bool &in) {
            g = u & 7;
            const int r = u >> 3;
            const int i = r / CW;
            const int k = r - i * CW;
            in = unsigned(ih0 + i) < unsigned(a.H);
            q0 = i * a.IW + a.pad + k * 4;
            const float4 *src = reinterpret_cast<const float4 *>(
                ximg + int64_t(blk * CB + g * 4) * HW + int64_t(in ? ih0 + i : 0) * a.W + k * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) raw[e] = src[int64_t(e) * (HW >> 2)];
        };
        auto put_unit = [&](int q0, int g, bool in, const float4 *raw) {
            const float4 z{0.f, 0.f, 0.f, 0.f};
            const float4 o0 = in ? float4{raw[0].x, raw[1].x, raw[2].x, raw[3].x} : z;
            const float4 o1 = in ? float4{raw[0].y, raw[1].y, raw[2].y, raw[3].y} : z;
            const float4 o2 = in ? float4{raw[0].z, raw[1].z, raw[2].z, raw[3].z} : z;
            const float4 o3 = in ? float4{raw[0].w, raw[1].w, raw[2].w, raw[3].w} : z;
            *reinterpret_cast<float4 *>(patch + q0 * CB + ((g ^ (q0 & 7)) << 2)) = o0;
            *reinterpret_cast<float4 *>(patch + (q0 + 1) * CB + ((g ^ ((q0 + 1) & 7)) << 2)) = o1;
            *reinterpret_cast<float4 *>(patch + (q0 + 2) * CB + ((g ^ ((q0 + 2) & 7)) << 2)) = o2;
            *reinterpret_cast<float4 *>(patch + (q0 + 3) * CB + ((g ^ ((q0 + 3) & 7)) << 2)) = o3;
        };
        // the first two units of this thread are in flight with the filter slice
        float4 r0[4], r1[4];
        int q0a = 0, g0a = 0, q0b = 0, g0b = 0;
        bool i0a = false, i0b = false;
        if constexpr (VEC4) {
            load_unit(min(tid, units - 1), r0, q0a, g0a, i0a);
            load_unit(min(tid + kRowsThreads, units - 1), r1, q0b, g0b, i0b);
        }
#pragma unroll
        for (int t = 0; t < TAPS; ++t) {
            // element e of tap t is float e*TAPS + t of the 4*TAPS run
            const float *f = reinterpret_cast<const float *>(wraw);
            *reinterpret_cast<float4 *>(fl + t * 64 * CB + co_l * CB + ((cg ^ (co_l & 7)) << 2)) =
                float4{f[t], f[TAPS + t], f[2 * TAPS + t], f[3 * TAPS + t]};
        }
        if constexpr (VEC4) {
            if (tid < units) put_unit(q0a, g0a, i0a, r0);
            if (tid + kRowsThreads < units) put_unit(q0b, g0b, i0b, r1);
            for (int u = tid + 2 * kRowsThreads; u < units; u += kRowsThreads) {
                float4 raw[4];
                int q0, g;
                bool in;
                load_unit(u, raw, q0, g, in);
                put_unit(q0, g, in, raw);
            }
        } else {
            const float *xb = ximg + int64_t(blk * CB) * HW + int64_t(r_lo) * a.W;
            for (int u = tid; u < units; u += kRowsThreads) {
                const int g = u / npos, p = u - g * npos;
                const float *src = xb + int64_t(g * 4) * HW + p;
                const float v0 = src[0], v1 = src[HW], v2 = src[2 * HW], v3 = src[3 * HW];
                const int r = p / a.W;
                const int q = (r_lo - ih0 + r) * a.IW + a.pad + (p - r * a.W);
                *reinterpret_cast<float4 *>(patch + q * CB + ((g ^ (q & 7)) << 2)) = float4{v0, v1, v2, v3};
            }
        }
        __syncthreads();

        // (fp32 MFMAs are long enough that the run-time block tests cost
        // nothing; specialising per block count spills registers here)
        if (nb > 0) {
#pragma unroll
            for (int t = 0; t < TAPS; ++t) {
                const float *ft = fl + t * 64 * CB;
                const int dq = (t / KW) * a.IW + (t % KW);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int gr = h * 4 + (lane >> 4);
                    floatx4_t af[4], bf[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int q = qa[s] + dq;
                        if (s < nb) af[s] = *reinterpret_cast<const floatx4_t *>(patch + q * CB + ((gr ^ (q & 7)) << 2));
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = c * 16 + rbl;
                        bf[c] = *reinterpret_cast<const floatx4_t *>(ft + r * CB + ((gr ^ (r & 7)) << 2));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            if (s >= nb) break;
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                acc[s][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[s][j], bf[c][j], acc[s][c], 0, 0, 0);
                        }
                }
            }
        }
    }
    if ((a.Wo & 3) == 0 && a.out.type == 0) {
        if (nb > 0) store_blocks<4, true>(acc, nb, b0, lane, a.out, n, a.Cout, cb, a.Ho, a.Wo, ho0, outs);
    } else {
        __syncthreads();                             // patch and filter are dead: LDS is store scratch
        if (nb > 0)
            store_blocks_lds(acc, nb, b0, lane, ldsf + wave * kStoreScratchFloats, a.out, n, a.Cout, cb, a.Ho,
                             a.Wo, ho0, outs);
    }
}

template <int KH, int KW>
hipError_t launch_rows_f32(const ImplicitArgs &h, hipStream_t s)
{
    RowsF32KArgs a{};
    a.x = static_cast<const float *>(h.x);
    a.w = static_cast<const float *>(h.wst);
    a.out = h.out;
    a.Cin = h.Cin;
    a.H = h.H;
    a.W = h.W;
    a.Cout = h.Cout;
    a.pad = h.pad;
    a.Ho = h.Ho;
    a.Wo = h.Wo;
    a.RW = h.R;
    a.row_groups = (h.Ho + h.R - 1) / h.R;
    a.co_blocks = (h.Cout + 63) / 64;
    a.IW = h.W + 2 * h.pad;
    const int64_t blocks = int64_t(a.co_blocks) * h.N * a.row_groups;
    if (blocks < 1 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = implicit_rows_lds_bytes(KH * KW, h.R + KH - 1, a.IW);
    auto kern = h.W % 4 == 0 ? conv_implicit_rows_f32_kernel<KH, KW, true> : conv_implicit_rows_f32_kernel<KH, KW, false>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kRowsThreads), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW>
hipError_t launch_rows(const ImplicitArgs &h, hipStream_t s)
{
    RowsKArgs a{};
    a.x = static_cast<const uint16_t *>(h.x);
    a.w = static_cast<const uint16_t *>(h.wst);
    a.out = h.out;
    a.Cin = h.Cin;
    a.H = h.H;
    a.W = h.W;
    a.Cout = h.Cout;
    a.pad = h.pad;
    a.Ho = h.Ho;
    a.Wo = h.Wo;
    a.RW = h.R;
    a.row_groups = (h.Ho + h.R - 1) / h.R;
    a.co_blocks = (h.Cout + 63) / 64;
    a.IW = h.W + 2 * h.pad;
    const int64_t blocks = int64_t(a.co_blocks) * h.N * a.row_groups;
    if (blocks < 1 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = implicit_rows_lds_bytes(KH * KW, h.R + KH - 1, a.IW);
    // one 64-channel block with 8-column rows: the one-block kernel; else the
    // channel-block loop (16-byte row chunks or 2-byte gathers)
    const bool one = h.Cin == 64 && h.W % 8 == 0;
    auto kern = one ? (h.bf16 ? conv_implicit_rows_kernel<KH, KW, true> : conv_implicit_rows_kernel<KH, KW, false>)
          : h.W % 8 == 0
              ? (h.bf16 ? conv_implicit_rows_multi_kernel<KH, KW, true, true>
                        : conv_implicit_rows_multi_kernel<KH, KW, false, true>)
              : (h.bf16 ? conv_implicit_rows_multi_kernel<KH, KW, true, false>
                        : conv_implicit_rows_multi_kernel<KH, KW, false, false>);
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kRowsThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_implicit_rows(const ImplicitArgs &h, hipStream_t s)
{
    // the kernel's assumptions, checked again here (the planner only picks it
    // for such layers): 64 input channels, stride 1, whole rows of W % 8 == 0
    // elements, at most 64 output columns, one output row per wave
    if (h.f32) {
        // fp32: channel blocks of 32, rows of any width (row chunks where W % 4 == 0)
        if (h.Cin % 32 != 0 || h.Cin < 32 || h.stride != 1 || h.W < 1 || h.Wo < 1 ||
            h.Wo > 64 || h.Wo != h.W + 2 * h.pad - h.KW + 1 || h.R < 1 || int64_t(h.R) * h.Wo > 512 ||
            h.Ho != h.H + 2 * h.pad - h.KH + 1 ||
            implicit_rows_lds_bytes(h.KH * h.KW, h.R + h.KH - 1, h.W + 2 * h.pad) > kImplicitMaxLdsBytes)
            return hipErrorInvalidValue;
        if (h.KH == 3 && h.KW == 3) return launch_rows_f32<3, 3>(h, s);
        if (h.KH == 1 && h.KW == 1) return launch_rows_f32<1, 1>(h, s);
        return hipErrorInvalidValue;
    }
    if (h.Cin % 64 != 0 || h.Cin < 64 || h.stride != 1 || h.W < 1 || h.Wo < 1 || h.Wo > 64 ||
        int64_t(h.Cin) * h.H * h.W >= (int64_t(1) << 31) ||
        h.Wo != h.W + 2 * h.pad - h.KW + 1 || h.R < 1 || int64_t(h.R) * h.Wo > 512 ||
        h.Ho != h.H + 2 * h.pad - h.KH + 1 ||
        implicit_rows_lds_bytes(h.KH * h.KW, h.R + h.KH - 1, h.W + 2 * h.pad) > kImplicitMaxLdsBytes)
        return hipErrorInvalidValue;
    if (h.KH == 3 && h.KW == 3) return launch_rows<3, 3>(h, s);
    if (h.KH == 1 && h.KW == 1) return launch_rows<1, 1>(h, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
