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
// Tiles. A workgroup computes an MB x NB tile; K advances in stages of
// KS*KB through two LDS buffers (ping-pong: the global loads of stage k+1 are
// in flight while stage k is multiplied). KS groups of 4 waves split every
// stage (intra-workgroup split-K) and are summed through LDS at the end.
// Each wave multiplies (MB/WM) x (NB/WN) with v_mfma_f32_16x16x32_{f16,bf16}:
// A and B fragments are 8 consecutive K values per lane (one 16-byte LDS
// read), so any consistent K order is valid. LDS rows are padded by 16 bytes
// so that the fragment reads hit 32 distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../launch.hpp"
#include "epilogue.hpp"
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

template <int MB, int NB, int KB, int KS, int WM, int WN, bool BF16>
__global__ __launch_bounds__(256 * KS) void gemm_mfma_kernel(
    const uint16_t *__restrict__ win, const uint16_t *__restrict__ wst, const OutSpec o,
    int rows, int row0, int row_elems, int col_step, int krun, int kstage, int Ho, int Wo,
    int Cout, int tiles_m)
{
    constexpr int NTH = 256 * KS;
    constexpr int KI = KB * KS;              // K per stage
    constexpr int PITCH = KI + 8;            // halves per LDS row (16-byte pad: conflict-free)
    constexpr int GPR = KI / 8;              // 16-byte granules per row
    constexpr int FM = MB / WM / 16;
    constexpr int FN = NB / WN / 16;
    constexpr int AV = MB * GPR / NTH;       // 16-byte A vectors per thread per stage
    constexpr int BV = NB * GPR / NTH;
    static_assert(AV >= 1 && BV >= 1 && AV * NTH == MB * GPR && BV * NTH == NB * GPR, "tiling");
    static_assert(WM * WN == 4, "4 waves per group");
    static_assert(KS == 1 || MB * NB * 4 <= 2 * (MB + NB) * PITCH * 2, "reduction fits LDS");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (MB + NB) * PITCH];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    const int m0 = tm * MB;
    const int n0 = tn * NB;
    const int ncols = rows * Wo;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 2;               // K group
    const int wig = wave & 3;
    const int wm = wig % WM;
    const int wn = wig / WM;

    // per-thread load descriptors (index precomputation: once per tile)
    const uint16_t *ap[AV];
    bool aok[AV];
    const uint16_t *bp[BV];
    int bk[BV];       // window-relative K offset of this vector; -1: column outside the chunk
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int v = tid + i * NTH;
        const int co = m0 + v / GPR;
        aok[i] = co < Cout;
        ap[i] = wst + int64_t(aok[i] ? co : 0) * kstage + (v % GPR) * 8;
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int v = tid + i * NTH;
        const int n = n0 + v / GPR;
        const bool ok = n < ncols;
        const int rl = ok ? n / Wo : 0;
        const int wo = ok ? n - rl * Wo : 0;
        bp[i] = win + int64_t(rl) * row_elems + int64_t(wo) * col_step + (v % GPR) * 8;
        bk[i] = ok ? (v % GPR) * 8 : -1;
    }

    // NS register sets of global loads. Loads are unconditional (clamped to a
    // valid address); the masks that zero what lies outside the window are
    // applied only when a set is written to LDS, so nothing waits for a load
    // before its data is needed.
    constexpr int NS = (AV + BV <= 4) ? 4 : 2;   // pipeline depth: NS + 1 stages
    struct Set {
        uint4 a[AV], b[BV];
        bool blo[BV], bhi[BV];
    };
    Set sets[NS];
    auto gload = [&](int k0, Set &st) {
#pragma unroll
        for (int i = 0; i < AV; ++i) st.a[i] = *reinterpret_cast<const uint4 *>(ap[i] + k0);
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int left = krun - (k0 + bk[i]);   // window elements left from this vector
            const bool any = bk[i] >= 0 && left > 0;
            st.blo[i] = any;
            st.bhi[i] = any && left >= 8;           // else a 4-element tail (or nothing)
            st.b[i] = *reinterpret_cast<const uint4 *>(bp[i] + (any ? k0 : 0));
        }
    };
    auto sstore = [&](int buf, const Set &st) {
        uint16_t *As = smem + buf * (MB + NB) * PITCH;
        uint16_t *Bs = As + MB * PITCH;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int v = tid + i * NTH;
            const uint32_t m = aok[i] ? 0xffffffffu : 0u;
            const uint4 q = st.a[i];
            *reinterpret_cast<uint4 *>(&As[(v / GPR) * PITCH + (v % GPR) * 8]) =
                make_uint4(q.x & m, q.y & m, q.z & m, q.w & m);
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int v = tid + i * NTH;
            const uint32_t lo = st.blo[i] ? 0xffffffffu : 0u;
            const uint32_t hi = st.bhi[i] ? 0xffffffffu : 0u;
            const uint4 q = st.b[i];
            *reinterpret_cast<uint4 *>(&Bs[(v / GPR) * PITCH + (v % GPR) * 8]) =
                make_uint4(q.x & lo, q.y & lo, q.z & hi, q.w & hi);
        }
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int arow = wm * (MB / WM) + (lane & 15);
    const int brow = wn * (NB / WN) + (lane & 15);
    const int kofs = grp * KB + (lane >> 4) * 8;
    auto compute = [&](int buf) {
        const uint16_t *As = smem + buf * (MB + NB) * PITCH;
        const uint16_t *Bs = As + MB * PITCH;
#pragma unroll
        for (int kk = 0; kk < KB; kk += 32) {
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(&As[(arow + i * 16) * PITCH + kofs + kk]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const uint4 *>(&Bs[(brow + j * 16) * PITCH + kofs + kk]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<BF16>(af[i], bf[j], acc[i][j]);
        }
    };

    // Software pipeline, NS + 1 stages deep: at step k the register set that
    // holds stage k+1 is written to LDS and immediately reused for the loads
    // of stage k+1+NS, then stage k is multiplied from the other LDS buffer.
    // Every load has NS steps to land, and the wait before a store only
    // covers the oldest set in flight. The body has no data-dependent
    // branches: loads past the end re-read the last stage. The loop is
    // unrolled NS times so that every register set is named statically.
    const int nk = kstage / KI;
    const int last = (nk - 1) * KI;
#pragma unroll
    for (int i = 0; i < NS; ++i) gload(min(i * KI, last), sets[i]);
    sstore(0, sets[0]);
    gload(min(NS * KI, last), sets[0]);
    __syncthreads();
    bool done = false;
    auto step = [&](int k, auto J) {
        constexpr int j = decltype(J)::value;        // k % NS
        constexpr int nxt = (j + 1) % NS;
        sstore((j + 1) & 1, sets[nxt]);              // stage k+1
        gload(min((k + 1 + NS) * KI, last), sets[nxt]);
        compute(j & 1);                              // stage k
        __syncthreads();
        done = k + 1 >= nk;
    };
    for (int kt = 0;; kt += NS) {
        step(kt, std::integral_constant<int, 0>{});
        if (done) break;
        step(kt + 1, std::integral_constant<int, 1>{});
        if (done) break;
        if constexpr (NS == 4) {
            step(kt + 2, std::integral_constant<int, 2>{});
            if (done) break;
            step(kt + 3, std::integral_constant<int, 3>{});
            if (done) break;
        }
    }

    if constexpr (KS > 1) {
        // wave-level reduction of the K groups through LDS (the stage buffers
        // are free after the last barrier): group g > 0 parks its partial
        // tile, group 0 adds the partials in a fixed order.
        float *red = reinterpret_cast<float *>(smem);
        constexpr int PER = FM * FN * 4;     // floats per lane
        for (int g = 1; g < KS; ++g) {
            if (grp == g) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            red[((wig * PER) + (i * FN + j) * 4 + v) * 64 + lane] = acc[i][j][v];
            }
            __syncthreads();
            if (grp == 0) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[i][j][v] += red[((wig * PER) + (i * FN + j) * 4 + v) * 64 + lane];
            }
            __syncthreads();
        }
        if (grp != 0) return;
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
        const int64_t p = int64_t(ho) * Wo + wo;
        if (o.plain) {
            float *yb = static_cast<float *>(o.y) + int64_t(img) * Cout * plane + p;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int co = m0 + wm * (MB / WM) + i * 16 + (lane >> 4) * 4 + v;
                    if (co < Cout) yb[int64_t(co) * plane] = acc[i][j][v];
                }
            }
        } else {
            with_ytype(o, [&](auto tc) {
                constexpr int T = decltype(tc)::value;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    out_store_cols4<T>(o, img, m0 + wm * (MB / WM) + i * 16 + (lane >> 4) * 4, p, acc[i][j]);
            });
        }
    }
}

template <int MB, int NB, int KB, int KS, int WM, int WN>
hipError_t launch_tile(const MfmaGemmArgs &a, hipStream_t s)
{
    if (a.kstage % (KB * KS) != 0) return hipErrorInvalidValue;
    const int tiles_m = (a.Cout + MB - 1) / MB;
    const int64_t ncols = int64_t(a.rows) * a.Wo;
    const int64_t tiles_n = (ncols + NB - 1) / NB;
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    const auto *win = static_cast<const uint16_t *>(a.win);
    const auto *wst = static_cast<const uint16_t *>(a.wst);
    if (a.bf16)
        hipLaunchKernelGGL((gemm_mfma_kernel<MB, NB, KB, KS, WM, WN, true>), grid, dim3(256 * KS),
                           0, s, win, wst, a.out, a.rows, a.row0, a.row_elems, a.col_step, a.krun,
                           a.kstage, a.Ho, a.Wo, a.Cout, tiles_m);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<MB, NB, KB, KS, WM, WN, false>), grid, dim3(256 * KS),
                           0, s, win, wst, a.out, a.rows, a.row0, a.row_elems, a.col_step, a.krun,
                           a.kstage, a.Ho, a.Wo, a.Cout, tiles_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const MfmaGemmArgs &a, hipStream_t s)
{
    if (a.krun % 4 != 0 || a.col_step % 8 != 0 || a.row_elems % 8 != 0) return hipErrorInvalidValue;
#define IM2WIN_TILE(M, N, KB, KS, WM)                                                            \
    if (a.tile_m == M && a.tile_n == N && a.kb == KB && a.ks == KS && a.wm == WM)                 \
        return launch_tile<M, N, KB, KS, WM, 4 / WM>(a, s);
    IM2WIN_TILE(64, 64, 64, 1, 2)
    IM2WIN_TILE(64, 64, 32, 1, 2)
    IM2WIN_TILE(64, 64, 32, 2, 2)
    IM2WIN_TILE(64, 128, 64, 1, 2)
    IM2WIN_TILE(64, 128, 32, 1, 2)
    IM2WIN_TILE(64, 128, 32, 2, 2)
    IM2WIN_TILE(128, 64, 64, 1, 2)
    IM2WIN_TILE(128, 64, 32, 1, 2)
    IM2WIN_TILE(128, 64, 32, 2, 2)
    IM2WIN_TILE(128, 128, 64, 1, 2)
    IM2WIN_TILE(128, 128, 32, 1, 2)
    IM2WIN_TILE(128, 128, 32, 2, 2)
    IM2WIN_TILE(64, 128, 64, 1, 1)
    IM2WIN_TILE(64, 256, 64, 1, 1)
    IM2WIN_TILE(64, 256, 32, 1, 1)
    IM2WIN_TILE(128, 256, 64, 1, 2)
    IM2WIN_TILE(128, 128, 64, 1, 1)
#undef IM2WIN_TILE
    return hipErrorInvalidValue;
}

}  // namespace im2win
