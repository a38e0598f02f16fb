// fp16 / bf16 window-GEMM on the CDNA4 matrix cores, register-direct form.
//
// Same contraction as gemm_mfma.hip (M = Cout, N = window columns n = (r, wo),
// K = KW*KH*Cin_pad in the channels-last window tensor, where the window of
// column n is one contiguous run of K elements at
// base(n) = r*row_elems + wo*stride*KH*Cin_pad), but without LDS: every wave
// owns a (16*FM) x (16*FN) output tile and loads its MFMA fragments straight
// from memory into registers, 8 consecutive K values (16 bytes) per lane.
//  - the filter fragments are the same for every wave of an M block, so they
//    are served by the L1 of the CU and the L2;
//  - the window fragments of neighbouring columns are the same bytes of the
//    window tensor shifted by stride*KH*Cin_pad (the overlapping windows of
//    the im2win transform), so most of them are L1 hits as well.
// Waves never wait for each other (no barrier, no LDS); the loads of the next
// PF K steps are in flight while the current one is multiplied.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../launch.hpp"

namespace im2win {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ uint4 mask4(const uint4 &q, bool lo, bool hi)
{
    const uint32_t ml = lo ? 0xffffffffu : 0u, mh = hi ? 0xffffffffu : 0u;
    return make_uint4(q.x & ml, q.y & ml, q.z & mh, q.w & mh);
}

template <int FM, int FN, int PF, bool BF16>
__global__ __launch_bounds__(256) void gemm_mfma_direct_kernel(
    const uint16_t *__restrict__ win, const uint16_t *__restrict__ wst, float *__restrict__ y,
    int rows, int row0, int row_elems, int col_step, int krun, int kstage, int Ho, int Wo,
    int Cout, int tiles_m, int tiles_total)
{
    constexpr int MW = 16 * FM, NW = 16 * FN;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + int(threadIdx.x >> 6);   // wave tile, M index fastest
    if (t >= tiles_total) return;                           // no barriers in this kernel
    const int tn = t / tiles_m;
    const int tm = t - tn * tiles_m;
    const int m0 = tm * MW;
    const int n0 = tn * NW;
    const int ncols = rows * Wo;
    const int kl = (lane >> 4) * 8;                          // this lane's K offset in a step

    // fragment sources (index precomputation, once per tile)
    const uint16_t *ap[FM];
    bool aok[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int co = m0 + i * 16 + (lane & 15);
        aok[i] = co < Cout;
        ap[i] = wst + int64_t(aok[i] ? co : 0) * kstage + kl;
    }
    const uint16_t *bp[FN];
    bool bok[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + j * 16 + (lane & 15);
        bok[j] = n < ncols;
        const int rl = bok[j] ? n / Wo : 0;
        const int wo = bok[j] ? n - rl * Wo : 0;
        bp[j] = win + int64_t(rl) * row_elems + int64_t(wo) * col_step + kl;
    }

    struct Frags {
        uint4 a[FM], b[FN];
    };
    Frags f[PF];
    const int nk = kstage / 32;
    const int last = (nk - 1) * 32;
    // loads are unconditional: K steps past the window end read its start
    // (and are masked to zero when used)
    auto load = [&](int k0, Frags &d) {
        const int kb = min(k0, last);
        const int kw = kb + kl < krun ? kb : 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) d.a[i] = *reinterpret_cast<const uint4 *>(ap[i] + kb);
#pragma unroll
        for (int j = 0; j < FN; ++j) d.b[j] = *reinterpret_cast<const uint4 *>(bp[j] + kw);
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](int k0, const Frags &d) {
        const int left = krun - (k0 + kl);                   // window elements left for this lane
        const bool lo = left > 0, hi = left >= 8;            // 4-element tail or nothing
        uint4 a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = mask4(d.a[i], aok[i], aok[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = mask4(d.b[j], bok[j] && lo, bok[j] && hi);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<BF16>(a[i], b[j], acc[i][j]);
    };

#pragma unroll
    for (int p = 0; p < PF; ++p) load(p * 32, f[p]);
    // steady state unrolled PF times (every fragment set named statically,
    // no branch inside), then the remaining K steps without further loads
    int k = 0;
    for (; k + PF <= nk; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            mma((k + p) * 32, f[p]);
            load((k + p + PF) * 32, f[p]);
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (k + p < nk) mma((k + p) * 32, f[p]);

    // epilogue: lane holds D[4*(lane/16) + v][lane%16] of every 16x16 block
    const int64_t plane = int64_t(Ho) * Wo;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + j * 16 + (lane & 15);
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
                const int co = m0 + i * 16 + (lane >> 4) * 4 + v;
                if (co < Cout) yb[int64_t(co) * plane] = acc[i][j][v];
            }
        }
    }
}

template <int FM, int FN>
hipError_t launch_direct(const MfmaGemmArgs &a, hipStream_t s)
{
    const int tiles_m = (a.Cout + 16 * FM - 1) / (16 * FM);
    const int64_t ncols = int64_t(a.rows) * a.Wo;
    const int64_t tiles_n = (ncols + 16 * FN - 1) / (16 * FN);
    const int64_t tiles = tiles_m * tiles_n;
    const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
    const auto *win = static_cast<const uint16_t *>(a.win);
    const auto *wst = static_cast<const uint16_t *>(a.wst);
    if (a.bf16)
        hipLaunchKernelGGL((gemm_mfma_direct_kernel<FM, FN, 2, true>), grid, dim3(256), 0, s, win,
                           wst, a.y, a.rows, a.row0, a.row_elems, a.col_step, a.krun, a.kstage,
                           a.Ho, a.Wo, a.Cout, tiles_m, int(tiles));
    else
        hipLaunchKernelGGL((gemm_mfma_direct_kernel<FM, FN, 2, false>), grid, dim3(256), 0, s, win,
                           wst, a.y, a.rows, a.row0, a.row_elems, a.col_step, a.krun, a.kstage,
                           a.Ho, a.Wo, a.Cout, tiles_m, int(tiles));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma_direct(const MfmaGemmArgs &a, hipStream_t s)
{
    if (a.kstage % 32 != 0 || a.krun % 4 != 0 || a.col_step % 8 != 0 || a.row_elems % 8 != 0)
        return hipErrorInvalidValue;
    // tile_m / tile_n are the wave tile here
    if (a.tile_m == 64 && a.tile_n == 64) return launch_direct<4, 4>(a, s);
    if (a.tile_m == 64 && a.tile_n == 32) return launch_direct<4, 2>(a, s);
    if (a.tile_m == 32 && a.tile_n == 64) return launch_direct<2, 4>(a, s);
    if (a.tile_m == 32 && a.tile_n == 32) return launch_direct<2, 2>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
