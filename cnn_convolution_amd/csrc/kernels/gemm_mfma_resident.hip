// fp16 / bf16 window-GEMM on the CDNA4 matrix cores, filter-resident form,
// for layers whose staged filter rows are short (small Cin*KH*KW).
//
// Same contraction as gemm_mfma.hip: M = Cout, N = window columns n = (r, wo),
// K = KW*KH*Cin_pad; in the channels-last window tensor the window of column
// n is one contiguous run of K elements at base(n) = r*row_elems +
// wo*stride*KH*Cin_pad, and the staged filter A[co][k] uses the same K order
// (the window contraction of "Enabling Memory-efficient Im2win Convolution
// ...", Sec. III-C Eq. (3) and Sec. III-D).
//
// When a 64-row block of the staged filter fits in LDS for the whole K
// (64 x K_stage halves), a workgroup copies it there once and its four waves
// never synchronise again: every wave owns a 64 x (16*FN) output tile, reads
// its A fragments from the resident block and loads its B fragments straight
// from the window tensor into registers, eight consecutive K values (16
// bytes) per lane, PF K steps ahead of their use. The window bytes pass
// through LDS zero times (the tiled kernel stages them every K step), which
// is what bounds that kernel on these layers: LDS traffic per CU drops to the
// A fragment reads alone.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../launch.hpp"
#include "tile_map.hpp"

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

constexpr int MR = 64;       // filter rows per workgroup (all waves share them)
constexpr int AU = 8;        // 16-byte A loads in flight per thread while filling LDS

template <int FN, int PF, bool BF16>
__global__ __launch_bounds__(256) void gemm_mfma_resident_kernel(
    const uint16_t *__restrict__ win, const uint16_t *__restrict__ wst, float *__restrict__ y,
    int rows, int row0, int row_elems, int col_step, int krun, int kstage, int Ho, int Wo,
    int Cout, int tiles_m)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t As[];   // [MR][kstage + 8]
    constexpr int NW = 16 * FN;           // columns per wave
    constexpr int NB = 4 * NW;            // columns per workgroup
    const int pitch = kstage + 8;         // 16-byte row pad: conflict-free fragment reads
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int m0 = tm * MR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ncols = rows * Wo;
    const int kl = (lane >> 4) * 8;       // this lane's K offset inside a 32-wide K step
    const int nk = kstage / 32;

    // B fragment sources: column n0 + j*16 + lane%16 of this wave
    const uint16_t *bp[FN];
    bool bok[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = tn * NB + wave * NW + j * 16 + (lane & 15);
        bok[j] = n < ncols;
        const int rl = bok[j] ? n / Wo : 0;
        const int wo = bok[j] ? n - rl * Wo : 0;
        bp[j] = win + int64_t(rl) * row_elems + int64_t(wo) * col_step + kl;
    }
    // Loads are unconditional: a K step whose 8 values start past the window
    // reads the window start instead (masked to zero when used); a step that
    // holds the last 4 values of a window reads 4 more halves, which stay
    // inside the row (row_elems keeps that slack).
    auto load_b = [&](int s, uint4 (&f)[FN]) {
        const int k0 = 32 * min(s, nk - 1);
        const int kk = k0 + kl < krun ? k0 : 0;
#pragma unroll
        for (int j = 0; j < FN; ++j) f[j] = *reinterpret_cast<const uint4 *>(bp[j] + kk);
    };
    uint4 fb[PF][FN];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_b(p, fb[p]);

    // copy this workgroup's filter rows into LDS (rows past Cout are zero)
    const int gpr = kstage / 8;           // 16-byte granules per row
    const int total = MR * gpr;
    for (int v0 = tid; v0 < total; v0 += 256 * AU) {
        uint4 q[AU];
        int dst[AU];
#pragma unroll
        for (int u = 0; u < AU; ++u) {
            const int v = v0 + u * 256;
            const int r = v / gpr;
            const int g = v - r * gpr;
            const bool ok = v < total && m0 + r < Cout;
            q[u] = *reinterpret_cast<const uint4 *>(wst + (ok ? int64_t(m0 + r) * kstage + g * 8 : 0));
            if (!ok) q[u] = make_uint4(0u, 0u, 0u, 0u);
            dst[u] = v < total ? r * pitch + g * 8 : -1;
        }
#pragma unroll
        for (int u = 0; u < AU; ++u)
            if (dst[u] >= 0) *reinterpret_cast<uint4 *>(As + dst[u]) = q[u];
    }
    __syncthreads();

    floatx4 acc[4][FN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *arow = As + (lane & 15) * pitch + kl;
    auto load_a = [&](int s, uint4 (&a)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const uint4 *>(arow + i * 16 * pitch + 32 * s);
    };
    auto mma = [&](int s, const uint4 (&a)[4], const uint4 (&f)[FN]) {
        const int left = krun - (32 * s + kl);        // window values left for this lane
        const bool lo = left > 0, hi = left >= 8;     // 8 values, a 4-value tail, or none
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint32_t ml = (bok[j] && lo) ? 0xffffffffu : 0u;
            const uint32_t mh = (bok[j] && hi) ? 0xffffffffu : 0u;
            const uint4 b = make_uint4(f[j].x & ml, f[j].y & ml, f[j].z & mh, f[j].w & mh);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] = mfma16<BF16>(a[i], b, acc[i][j]);
        }
    };

    // steady state: PF steps per trip, every register set named statically,
    // no data-dependent branch; then the remaining steps without loads
    uint4 a0[4], a1[4];
    load_a(0, a0);
    int s = 0;
    for (; s + PF <= nk; s += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            uint4(&cur)[4] = (p & 1) ? a1 : a0;
            uint4(&nxt)[4] = (p & 1) ? a0 : a1;
            load_a(min(s + p + 1, nk - 1), nxt);
            mma(s + p, cur, fb[p]);
            load_b(s + p + PF, fb[p]);
        }
        if constexpr (PF & 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a0[i] = a1[i];
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        if (s + p < nk) {
            uint4(&cur)[4] = (p & 1) ? a1 : a0;
            uint4(&nxt)[4] = (p & 1) ? a0 : a1;
            load_a(min(s + p + 1, nk - 1), nxt);
            mma(s + p, cur, fb[p]);
        }
    }

    // epilogue: lane holds D[4*(lane/16) + v][lane%16] of every 16x16 block
    const int64_t plane = int64_t(Ho) * Wo;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = tn * NB + wave * NW + j * 16 + (lane & 15);
        if (n >= ncols) continue;
        const int rl = n / Wo;
        const int wo = n - rl * Wo;
        const int r = row0 + rl;
        const int img = r / Ho;
        const int ho = r - img * Ho;
        float *yb = y + int64_t(img) * Cout * plane + int64_t(ho) * Wo + wo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = m0 + i * 16 + (lane >> 4) * 4 + v;
                if (co < Cout) yb[int64_t(co) * plane] = acc[i][j][v];
            }
        }
    }
}

template <int FN, int PF, bool BF16>
hipError_t launch_resident_t(const MfmaGemmArgs &a, hipStream_t s)
{
    const void *kern = reinterpret_cast<const void *>(&gemm_mfma_resident_kernel<FN, PF, BF16>);
    const size_t lds = size_t(MR) * (a.kstage + 8) * 2;
    // a workgroup may hold more than 64 KB of LDS on gfx950: raise the
    // per-kernel limit once, to the largest block this form accepts
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [&] {
        attr = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   static_cast<int>(kResidentMaxLdsBytes));
    });
    if (attr != hipSuccess) return attr;
    const int tiles_m = (a.Cout + MR - 1) / MR;
    const int64_t ncols = int64_t(a.rows) * a.Wo;
    const int64_t tiles_n = (ncols + 64 * FN - 1) / (64 * FN);
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    hipLaunchKernelGGL((gemm_mfma_resident_kernel<FN, PF, BF16>), grid, dim3(256), lds, s,
                       static_cast<const uint16_t *>(a.win), static_cast<const uint16_t *>(a.wst),
                       a.y, a.rows, a.row0, a.row_elems, a.col_step, a.krun, a.kstage, a.Ho, a.Wo,
                       a.Cout, tiles_m);
    return hipGetLastError();
}

template <int FN, bool BF16>
hipError_t launch_resident_pf(const MfmaGemmArgs &a, hipStream_t s)
{
    // K steps of window fragments in flight per wave (kslice carries it)
    switch (a.kb) {
    case 4: return launch_resident_t<FN, 4, BF16>(a, s);
    case 8: return launch_resident_t<FN, 8, BF16>(a, s);
    case 16: return launch_resident_t<FN, 16, BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm_mfma_resident(const MfmaGemmArgs &a, hipStream_t s)
{
    if (a.kstage % 32 != 0 || a.krun % 4 != 0 || a.col_step % 8 != 0 || a.row_elems % 8 != 0)
        return hipErrorInvalidValue;
    if (int64_t(MR) * (a.kstage + 8) * 2 > kResidentMaxLdsBytes) return hipErrorInvalidValue;
    // tile_n is the workgroup's column count: 4 waves x 16*FN
    if (a.tile_n == 128) return a.bf16 ? launch_resident_pf<2, true>(a, s) : launch_resident_pf<2, false>(a, s);
    if (a.tile_n == 256) return a.bf16 ? launch_resident_pf<4, true>(a, s) : launch_resident_pf<4, false>(a, s);
    if (a.tile_n == 64) return a.bf16 ? launch_resident_pf<1, true>(a, s) : launch_resident_pf<1, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
