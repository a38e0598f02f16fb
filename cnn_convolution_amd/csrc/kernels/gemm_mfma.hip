// fp16 / bf16 window-GEMM on the CDNA4 matrix cores, fp32 accumulation
// (the half-precision im2win kernel of "Enabling Memory-efficient Im2win
// Convolution ...", Sec. III-D, Algorithm 1, re-designed for gfx950).
//
// GEMM view of one chunk of window rows: M = Cout, N = rows*Wo columns
// n = (r, wo), K = KW*KH*Cin_pad. In the channels-last window tensor the
// window of column n is ONE contiguous run of K elements starting at
//     base(n) = r*row_elems + wo*stride*KH*Cin_pad,
// so B[k][n] = T[base(n) + k], and the staged filter A[co][k] uses the same
// K order (kw outer, kh, channel inner). Overlapping windows of neighbouring
// columns are the same bytes of T, served by L1/L2.
//
// Tiles. A workgroup of 4 waves computes an MB x NB tile; K advances in
// slices of 32 through two LDS buffers (ping-pong: the global loads of slice
// k+1 are in flight while slice k is multiplied). Each wave multiplies
// (MB/WM) x (NB/WN) with v_mfma_f32_16x16x32_{f16,bf16}: A and B fragments
// are 8 consecutive K values per lane (one 16-byte LDS read), so any
// consistent K order is valid. LDS rows are padded by 16 bytes so that the
// fragment reads hit 32 distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int KB = 32;           // K slice per LDS stage (one MFMA K step)
constexpr int PITCH = KB + 8;    // halves per LDS row: 80 bytes

template <bool BF16>
__device__ __forceinline__ floatx4 mfma16(const uint4 &a, const uint4 &b, const floatx4 &c)
{
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
}

template <int MB, int NB, int WM, int WN, bool BF16>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const uint16_t *__restrict__ win, const uint16_t *__restrict__ wst, float *__restrict__ y,
    int rows, int row0, int row_elems, int col_step, int krun, int kstage, int Ho, int Wo,
    int Cout, int tiles_m)
{
    constexpr int FM = MB / WM / 16;
    constexpr int FN = NB / WN / 16;
    constexpr int AV = MB * KB / 8 / 256;   // 16-byte A vectors per thread per slice
    constexpr int BV = NB * KB / 8 / 256;
    static_assert(AV >= 1 && BV >= 1, "tile too small for 256 threads");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][MB * PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][NB * PITCH];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int m0 = tm * MB;
    const int n0 = tn * NB;
    const int ncols = rows * Wo;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // per-thread load descriptors (index precomputation: once per tile)
    const uint16_t *ap[AV];
    bool aok[AV];
    const uint16_t *bp[BV];
    int bk[BV];       // window-relative K offset of this vector; -1: column outside the chunk
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int v = tid + i * 256;
        const int co = m0 + (v >> 2);
        aok[i] = co < Cout;
        ap[i] = wst + int64_t(aok[i] ? co : 0) * kstage + (v & 3) * 8;
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int v = tid + i * 256;
        const int n = n0 + (v >> 2);
        const bool ok = n < ncols;
        const int rl = ok ? n / Wo : 0;
        const int wo = ok ? n - rl * Wo : 0;
        bp[i] = win + int64_t(rl) * row_elems + int64_t(wo) * col_step + (v & 3) * 8;
        bk[i] = ok ? (v & 3) * 8 : -1;
    }

    uint4 ra[AV], rb[BV];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AV; ++i)
            ra[i] = aok[i] ? *reinterpret_cast<const uint4 *>(ap[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int left = krun - (k0 + bk[i]);   // window elements left from this vector
            uint4 q = make_uint4(0, 0, 0, 0);
            if (bk[i] >= 0 && left >= 8) {
                q = *reinterpret_cast<const uint4 *>(bp[i] + k0);
            } else if (bk[i] >= 0 && left >= 4) {
                const uint2 h = *reinterpret_cast<const uint2 *>(bp[i] + k0);
                q = make_uint4(h.x, h.y, 0, 0);
            }
            rb[i] = q;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int v = tid + i * 256;
            *reinterpret_cast<uint4 *>(&As[buf][(v >> 2) * PITCH + (v & 3) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int v = tid + i * 256;
            *reinterpret_cast<uint4 *>(&Bs[buf][(v >> 2) * PITCH + (v & 3) * 8]) = rb[i];
        }
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk = kstage / KB;
    gload(0);
    sstore(0);
    __syncthreads();
    const int arow = wm * (MB / WM) + (lane & 15);
    const int brow = wn * (NB / WN) + (lane & 15);
    const int kofs = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * KB);
        uint4 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *reinterpret_cast<const uint4 *>(&As[buf][(arow + i * 16) * PITCH + kofs]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = *reinterpret_cast<const uint4 *>(&Bs[buf][(brow + j * 16) * PITCH + kofs]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<BF16>(af[i], bf[j], acc[i][j]);
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds D[4*(lane/16) + v][lane%16] of every 16x16 block
    const int64_t plane = int64_t(Ho) * Wo;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + brow + j * 16;
        if (n >= ncols) continue;
        const int rl = n / Wo;
        const int wo = n - rl * Wo;
        const int r = row0 + rl;
        const int img = r / Ho;
        const int ho = r - img * Ho;
        float *yb = y + int64_t(img) * Cout * plane + int64_t(ho) * Wo + wo;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = m0 + wm * (MB / WM) + i * 16 + (lane >> 4) * 4 + v;
                if (co < Cout) yb[int64_t(co) * plane] = acc[i][j][v];
            }
        }
    }
}

template <int MB, int NB, int WM, int WN>
hipError_t launch_tile(const MfmaGemmArgs &a, hipStream_t s)
{
    const int tiles_m = (a.Cout + MB - 1) / MB;
    const int64_t ncols = int64_t(a.rows) * a.Wo;
    const int64_t tiles_n = (ncols + NB - 1) / NB;
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    const auto *win = static_cast<const uint16_t *>(a.win);
    const auto *wst = static_cast<const uint16_t *>(a.wst);
    if (a.bf16)
        hipLaunchKernelGGL((gemm_mfma_kernel<MB, NB, WM, WN, true>), grid, dim3(256), 0, s, win,
                           wst, a.y, a.rows, a.row0, a.row_elems, a.col_step, a.krun, a.kstage,
                           a.Ho, a.Wo, a.Cout, tiles_m);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<MB, NB, WM, WN, false>), grid, dim3(256), 0, s, win,
                           wst, a.y, a.rows, a.row0, a.row_elems, a.col_step, a.krun, a.kstage,
                           a.Ho, a.Wo, a.Cout, tiles_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const MfmaGemmArgs &a, hipStream_t s)
{
    if (a.kstage % KB != 0 || a.krun % 4 != 0 || a.col_step % 8 != 0 || a.row_elems % 8 != 0)
        return hipErrorInvalidValue;
    if (a.tile_m == 64 && a.tile_n == 128) return launch_tile<64, 128, 2, 2>(a, s);
    if (a.tile_m == 128 && a.tile_n == 128) return launch_tile<128, 128, 2, 2>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
