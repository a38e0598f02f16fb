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

#include <cstdint>

#include "../launch.hpp"

namespace im2win {
namespace {

// ---------------------------------------------------------------- row-interleaved
// One wave per (window row, channel): the wave reads the KH input rows
// coalesced along w and writes the channel's interleaved run of pos_pad
// elements (tail past W_win*KH zero-filled). 4 waves per workgroup.
template <typename E>
__global__ __launch_bounds__(256) void pack_row_kernel(
    const E *__restrict__ x, E *__restrict__ out, int Cin, int H, int W, int KH, int stride,
    int pad, int Ho, int Wwin, int pos_pad, int row_elems, int row0, int rows)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t task = int64_t(blockIdx.x) * 4 + wave;      // (local row, channel)
    if (task >= int64_t(rows) * Cin) return;
    const int rl = int(task / Cin);
    const int ci = int(task - int64_t(rl) * Cin);
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const E *xc = x + (int64_t(n) * Cin + ci) * H * W;
    E *o = out + int64_t(rl) * row_elems + int64_t(ci) * pos_pad;
    for (int kh = 0; kh < KH; ++kh) {
        const int ih = ho * stride + kh - pad;
        const bool row_ok = ih >= 0 && ih < H;
        const E *xr = xc + int64_t(row_ok ? ih : 0) * W;
        for (int w = lane; w < Wwin; w += 64) {
            const int iw = w - pad;
            E v = E(0);
            if (row_ok && iw >= 0 && iw < W) v = xr[iw];
            o[w * KH + kh] = v;
        }
    }
    for (int q = Wwin * KH + lane; q < pos_pad; q += 64) o[q] = E(0);
}

// ---------------------------------------------------------------- channels-last
// Workgroup = (window row r, block of PW padded columns, block of CB channels).
// Phase 1 stages T[ci][kh][w] in LDS with coalesced reads along w; phase 2
// reads CG x 8 blocks (CG channels x 8 columns) as 16-byte LDS rows, transposes
// them in registers and writes CG-channel vectors, so that global writes run
// along ci, the innermost dimension of the window tensor.
constexpr int PW = 32;           // padded columns per workgroup
constexpr int CB = 64;           // channels per workgroup
constexpr int LDS_PITCH = PW + 8;  // elements per (ci, kh) LDS row (16-byte multiple)

template <int CG>
struct Vec;
template <> struct Vec<8> { using T = uint4; };
template <> struct Vec<4> { using T = uint2; };

// 16-bit lanes of a 32-bit word
__device__ __forceinline__ uint32_t lo16(uint32_t v) { return v & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t v) { return v >> 16; }

template <int CG>
__global__ __launch_bounds__(256) void pack_cl_kernel(
    const uint16_t *__restrict__ x, uint16_t *__restrict__ out, int Cin, int H, int W, int KH,
    int stride, int pad, int Ho, int Wwin, int Cin_pad, int row_elems, int row0, int wblocks,
    int cblocks)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[CB * 8 * LDS_PITCH];  // KH <= 8 per pass
    int b = blockIdx.x;
    const int cbk = b % cblocks;
    b /= cblocks;
    const int wbk = b % wblocks;
    const int rl = b / wblocks;
    const int r = row0 + rl;
    const int n = r / Ho;
    const int ho = r - n * Ho;
    const int c0 = cbk * CB;
    const int w0 = wbk * PW;
    const int cb = min(CB, Cin_pad - c0);                  // channels in this block (multiple of CG)
    uint16_t *orow = out + int64_t(rl) * row_elems;

    for (int kh0 = 0; kh0 < KH; kh0 += 8) {
        const int khn = min(8, KH - kh0);
        // phase 1: tile[(ci*8 + kh)*LDS_PITCH + w] = xp value (0 outside / padded channel)
        const int items1 = cb * khn * PW;
        for (int i = threadIdx.x; i < items1; i += blockDim.x) {
            const int wl = i % PW;
            const int t = i / PW;
            const int kh = t % khn;
            const int ci = t / khn;
            const int c = c0 + ci;
            const int ih = ho * stride + kh0 + kh - pad;
            const int iw = w0 + wl - pad;
            uint16_t v = 0;
            if (c < Cin && ih >= 0 && ih < H && iw >= 0 && iw < W)
                v = x[((int64_t(n) * Cin + c) * H + ih) * W + iw];
            tile[(ci * 8 + kh) * LDS_PITCH + wl] = v;
        }
        __syncthreads();
        // phase 2: (kh, column group of 8, channel group of CG)
        const int cgroups = cb / CG;
        const int items2 = khn * (PW / 8) * cgroups;
        for (int i = threadIdx.x; i < items2; i += blockDim.x) {
            const int cg = i % cgroups;
            const int t = i / cgroups;
            const int wg = t % (PW / 8);
            const int kh = t / (PW / 8);
            uint32_t rowv[CG][4];
#pragma unroll
            for (int e = 0; e < CG; ++e) {
                const uint4 q = *reinterpret_cast<const uint4 *>(
                    &tile[((cg * CG + e) * 8 + kh) * LDS_PITCH + wg * 8]);
                rowv[e][0] = q.x; rowv[e][1] = q.y; rowv[e][2] = q.z; rowv[e][3] = q.w;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = w0 + wg * 8 + j;
                if (w >= Wwin) break;
                uint32_t o[CG / 2];
#pragma unroll
                for (int q = 0; q < CG / 2; ++q) {
                    const uint32_t a = rowv[2 * q][j >> 1];
                    const uint32_t c = rowv[2 * q + 1][j >> 1];
                    o[q] = (j & 1) ? (hi16(a) | (c & 0xffff0000u)) : (lo16(a) | (c << 16));
                }
                uint16_t *dst = orow + (int64_t(w) * KH + kh0 + kh) * Cin_pad + c0 + cg * CG;
                if constexpr (CG == 8) {
                    *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
                } else {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
                }
            }
        }
        __syncthreads();
    }
    // zero the row tail past W_win*KH*Cin_pad (alignment padding), once per row
    if (wbk == 0 && cbk == 0) {
        const int used = Wwin * KH * Cin_pad;
        for (int q = used + threadIdx.x; q < row_elems; q += blockDim.x) orow[q] = 0;
    }
}

}  // namespace

hipError_t launch_pack_row(const PackArgs &a, hipStream_t s)
{
    const int64_t tasks = int64_t(a.rows) * a.Cin;
    const dim3 grid(static_cast<unsigned>((tasks + 3) / 4));
    if (a.esize == 4)
        hipLaunchKernelGGL(pack_row_kernel<uint32_t>, grid, dim3(256), 0, s,
                           static_cast<const uint32_t *>(a.x), static_cast<uint32_t *>(a.out),
                           a.Cin, a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.pos_pad,
                           a.row_elems, a.row0, a.rows);
    else
        hipLaunchKernelGGL(pack_row_kernel<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.x), static_cast<uint16_t *>(a.out),
                           a.Cin, a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.pos_pad,
                           a.row_elems, a.row0, a.rows);
    return hipGetLastError();
}

hipError_t launch_pack_cl(const PackArgs &a, hipStream_t s)
{
    if (a.esize != 2) return hipErrorInvalidValue;
    const int wblocks = (a.Wwin + PW - 1) / PW;
    const int cblocks = (a.Cin_pad + CB - 1) / CB;
    const int64_t blocks = int64_t(a.rows) * wblocks * cblocks;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (a.Cin_pad % 8 == 0)
        hipLaunchKernelGGL(pack_cl_kernel<8>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.x), static_cast<uint16_t *>(a.out),
                           a.Cin, a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad,
                           a.row_elems, a.row0, wblocks, cblocks);
    else if (a.Cin_pad == 4)
        hipLaunchKernelGGL(pack_cl_kernel<4>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t *>(a.x), static_cast<uint16_t *>(a.out),
                           a.Cin, a.H, a.W, a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad,
                           a.row_elems, a.row0, wblocks, cblocks);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace im2win
