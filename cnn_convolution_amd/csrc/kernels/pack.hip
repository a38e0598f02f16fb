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
    int pad, int Ho, int Wwin, int pos_pad, int row_elems, int row0, int rows, int cgroups)
{
    const int KH = KHT > 0 ? KHT : KH_rt;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int task = blockIdx.x * 4 + wave;
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

}  // namespace

template <typename E>
hipError_t launch_pack_row_t(const PackArgs &a, hipStream_t s)
{
    const int cgroups = (a.Cin + CPW - 1) / CPW;
    const int64_t tasks = int64_t(a.rows) * cgroups;
    const dim3 grid(static_cast<unsigned>((tasks + 3) / 4));
    const E *x = static_cast<const E *>(a.x);
    E *out = static_cast<E *>(a.out);
#define IM2WIN_PACK_ROW(K)                                                                       \
    hipLaunchKernelGGL((pack_row_kernel<E, K>), grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W,   \
                       a.KH, a.stride, a.pad, a.Ho, a.Wwin, a.pos_pad, a.row_elems, a.row0,       \
                       a.rows, cgroups)
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

hipError_t launch_pack_row(const PackArgs &a, hipStream_t s)
{
    return a.esize == 4 ? launch_pack_row_t<uint32_t>(a, s) : launch_pack_row_t<uint16_t>(a, s);
}

hipError_t launch_pack_cl(const PackArgs &a, hipStream_t s)
{
    if (a.esize != 2) return hipErrorInvalidValue;
    const int cblocks = (a.Cin_pad + CB - 1) / CB;
    const dim3 grid(static_cast<unsigned>(int64_t(a.rows) * cblocks));
    const auto *x = static_cast<const uint16_t *>(a.x);
    auto *out = static_cast<uint16_t *>(a.out);
    if (a.Cin_pad % 8 == 0)
        hipLaunchKernelGGL(pack_cl_kernel<8>, grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W, a.KH,
                           a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad, a.row_elems, a.row0, cblocks);
    else if (a.Cin_pad == 4)
        hipLaunchKernelGGL(pack_cl_kernel<4>, grid, dim3(256), 0, s, x, out, a.Cin, a.H, a.W, a.KH,
                           a.stride, a.pad, a.Ho, a.Wwin, a.Cin_pad, a.row_elems, a.row0, cblocks);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace im2win
