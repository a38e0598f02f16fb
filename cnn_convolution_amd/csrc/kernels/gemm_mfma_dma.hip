// fp16 / bf16 window-GEMM on the CDNA4 matrix cores, direct-to-LDS form.
//
// Same contraction as gemm_mfma.hip (M = Cout, N = window columns n = (r, wo),
// K = KW*KH*Cin_pad; the window of column n is one contiguous run of K
// elements of the channels-last window tensor at base(n) = r*row_elems +
// wo*stride*KH*Cin_pad; "Enabling Memory-efficient Im2win Convolution ...",
// Sec. III-C Eq. (3), Sec. III-D), for windows whose length is a multiple of
// the 64-element K stage (no K tail to mask).
//
// The filter and window tiles of a K stage go from memory straight into LDS
// with global_load_lds_dwordx4 (gfx950): a wave instruction fills one 1 KB
// block, lane l writing bytes [16l, 16l+16). A block holds 8 rows of 128 bytes
// (64 halves); lane l fetches granule g = (l & 7) ^ (l >> 3) of row l >> 3,
// so granule g of a row r sits in slot g ^ (r & 7): the fragment reads of 8
// consecutive rows hit 8 different 16-byte bank groups. There is no register
// staging and no LDS store instruction. Three stage buffers: while stage k is
// multiplied, stages k+1 and k+2 are in flight; each wave waits only for its
// own oldest stage (s_waitcnt vmcnt) and the workgroup barrier then makes all
// waves' copies visible. The barrier is the raw s_barrier, fenced for the
// compiler only: a workgroup memory fence would make every wave wait for all
// its copies in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "epilogue.hpp"
#include "lds_dma.hpp"
#include "tile_map.hpp"

namespace im2win {
namespace {

constexpr int KI = kStageK;

// Ablation switches (ABL, a bit mask; 0 is the kernel as planned), for
// measuring what each of the page's three optimisations gives on MI355X
// ("Enabling Memory-efficient Im2win Convolution ...", Sec. III-E; the
// ablation of Sec. IV-E, Fig. 4): no serpentine tile order (plain row-major tiles), no
// direct-to-LDS copies (global loads into registers, then LDS stores), one
// stage buffer instead of three (each stage loaded, waited for, then
// multiplied).
constexpr int kAblateSerpentine = 1;
constexpr int kAblateDma = 2;
constexpr int kAblateBuffers = 4;

template <int MB, int NB, int WM, bool BF16, int ABL>
__global__ __launch_bounds__(256) void gemm_mfma_dma_kernel(
    const uint16_t *__restrict__ win, const uint16_t *__restrict__ wst, const OutSpec o,
    int rows, int row0, int row_elems, int col_step, int kstage, int Ho, int Wo, int Cout,
    int tiles_m)
{
    constexpr bool SERP = !(ABL & kAblateSerpentine);
    constexpr bool DMA = !(ABL & kAblateDma);
    constexpr int NBUF = (ABL & kAblateBuffers) ? 1 : 3;
    constexpr int WN = 4 / WM;
    constexpr int FM = MB / WM / 16;
    constexpr int FN = NB / WN / 16;
    constexpr int AI = MB / 32;            // 1 KB filter blocks per wave per stage
    constexpr int BI = NB / 32;            // 1 KB window blocks per wave per stage
    constexpr int D = AI + BI;             // copies per wave per stage
    static_assert(AI >= 1 && BI >= 1 && AI * 32 == MB && BI * 32 == NB, "tiling");
    static_assert(FM >= 1 && FN >= 1 && WM * WN == 4, "wave layout");
    __shared__ __attribute__((aligned(16))) uint16_t sa0[MB * KI], sb0[NB * KI];
    __shared__ __attribute__((aligned(16))) uint16_t sa1[NBUF > 1 ? MB * KI : 8], sb1[NBUF > 1 ? NB * KI : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sa2[NBUF > 1 ? MB * KI : 8], sb2[NBUF > 1 ? NB * KI : 8];

    int tm, tn;
    if constexpr (SERP) {
        tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
    } else {
        tm = blockIdx.x % tiles_m;
        tn = blockIdx.x / tiles_m;
    }
    const int m0 = tm * MB;
    const int n0 = tn * NB;
    const int ncols = rows * Wo;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int nk = kstage / KI;

    // copy sources: row (or column) blk*8 + (lane >> 3) of the tile, granule g.
    // Filter rows past Cout read row Cout-1 and columns past the chunk read
    // column 0: they only feed outputs the epilogue never stores.
    const int rib = lane >> 3;
    const int g8 = ((lane & 7) ^ rib) * 8;
    const uint16_t *asrc[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = (wave + 4 * i) * 8 + rib;
        asrc[i] = wst + int64_t(min(m0 + r, Cout - 1)) * kstage + g8;
    }
    const uint16_t *bsrc[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int n = n0 + (wave + 4 * i) * 8 + rib;
        const bool ok = n < ncols;
        const int rl = ok ? n / Wo : 0;
        const int wo = ok ? n - rl * Wo : 0;
        bsrc[i] = win + int64_t(rl) * row_elems + int64_t(wo) * col_step + g8;
    }
    auto issue = [&](int stage, uint16_t *sa, uint16_t *sb) {
        const int k0 = stage * KI;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            copy_to_lds(asrc[i] + k0, __builtin_amdgcn_readfirstlane(lds_addr(sa + (wave + 4 * i) * 512)));
#pragma unroll
        for (int i = 0; i < BI; ++i)
            copy_to_lds(bsrc[i] + k0, __builtin_amdgcn_readfirstlane(lds_addr(sb + (wave + 4 * i) * 512)));
    };
    // the same copies through registers (ablation): lane l's 16 bytes land
    // at bytes [16l, 16l+16) of the same 1 KB block
    uint4 stg[D];
    auto load_regs = [&](int stage) {
        const int k0 = stage * KI;
#pragma unroll
        for (int i = 0; i < AI; ++i) stg[i] = *reinterpret_cast<const uint4 *>(asrc[i] + k0);
#pragma unroll
        for (int i = 0; i < BI; ++i) stg[AI + i] = *reinterpret_cast<const uint4 *>(bsrc[i] + k0);
    };
    auto store_regs = [&](uint16_t *sa, uint16_t *sb) {
#pragma unroll
        for (int i = 0; i < AI; ++i) *reinterpret_cast<uint4 *>(sa + (wave + 4 * i) * 512 + lane * 8) = stg[i];
#pragma unroll
        for (int i = 0; i < BI; ++i) *reinterpret_cast<uint4 *>(sb + (wave + 4 * i) * 512 + lane * 8) = stg[AI + i];
    };

    floatx4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int arow = wm * (MB / WM) + (lane & 15);
    const int bcol = wn * (NB / WN) + (lane & 15);
    auto compute = [&](const uint16_t *sa, const uint16_t *sb) {
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
                const int c = bcol + j * 16;
                bf[j] = *reinterpret_cast<const uint4 *>(sb + c * KI + ((gr ^ (c & 7)) * 8));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<BF16>(af[i], bf[j], acc[i][j]);
        }
    };

    // three-buffer pipeline, unrolled by three so that every buffer is named
    // statically (the compiler then tracks the copies into each one apart).
    // Every step issues one stage group (the stage index clamped to the last
    // one, so the final two steps re-copy it into buffers already read), so
    // each wave always has exactly two groups in flight at the top of a step
    // and waits for the older one: no data-dependent branch in the loop.
    if constexpr (NBUF == 1) {
        // ablation: one buffer, each stage loaded and waited for before it is
        // multiplied, and multiplied by every wave before the next is loaded
        for (int k = 0; k < nk; ++k) {
            if (k > 0) stage_barrier();
            if constexpr (DMA) {
                issue(k, sa0, sb0);
                wait_vm<0>();
            } else {
                load_regs(k);
                store_regs(sa0, sb0);
            }
            stage_barrier();
            compute(sa0, sb0);
        }
    } else if constexpr (!DMA) {
        // ablation: the three-buffer pipeline with register-staged copies:
        // stage k+2 is loaded while stage k is multiplied and stored after it,
        // into the buffer stage k-1 used (read by every wave before this
        // step's barrier)
        load_regs(0);
        store_regs(sa0, sb0);
        load_regs(min(1, nk - 1));
        store_regs(sa1, sb1);
        auto rstep = [&](int k, uint16_t *ca, uint16_t *cb, uint16_t *na, uint16_t *nb) {
            stage_barrier();
            load_regs(min(k + 2, nk - 1));
            compute(ca, cb);
            store_regs(na, nb);
        };
        for (int k = 0;; k += 3) {
            rstep(k, sa0, sb0, sa2, sb2);
            if (k + 1 >= nk) break;
            rstep(k + 1, sa1, sb1, sa0, sb0);
            if (k + 2 >= nk) break;
            rstep(k + 2, sa2, sb2, sa1, sb1);
            if (k + 3 >= nk) break;
        }
    } else {
        issue(0, sa0, sb0);
        issue(min(1, nk - 1), sa1, sb1);
        auto step = [&](int k, uint16_t *ca, uint16_t *cb, uint16_t *na, uint16_t *nb) {
            wait_vm<D>();                      // own copies of stage k landed (k+1 may fly)
            stage_barrier();                   // everyone's copies of stage k landed; stage k-1 read
            issue(min(k + 2, nk - 1), na, nb); // into the buffer stage k-1 used
            compute(ca, cb);
            __builtin_amdgcn_sched_barrier(0); // keep each step's work inside its step
        };
        // the loop may leave after any step (uniform test): the accumulators then
        // stay in the same registers from one step to the next
        for (int k = 0;; k += 3) {
            step(k, sa0, sb0, sa2, sb2);
            if (k + 1 >= nk) break;
            step(k + 1, sa1, sb1, sa0, sb0);
            if (k + 2 >= nk) break;
            step(k + 2, sa2, sb2, sa1, sb1);
            if (k + 3 >= nk) break;
        }
    }
    wait_vm<0>();                          // no copy may still be writing LDS at the end

    // epilogue: lane holds D[4*(lane/16) + v][lane%16] of every 16x16 block
    const int64_t plane = int64_t(Ho) * Wo;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + bcol + j * 16;
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

template <int MB, int NB, int WM, int ABL>
hipError_t launch_dma_variant(const MfmaGemmArgs &a, hipStream_t s)
{
    const int tiles_m = (a.Cout + MB - 1) / MB;
    const int64_t ncols = int64_t(a.rows) * a.Wo;
    const int64_t tiles_n = (ncols + NB - 1) / NB;
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    const auto *win = static_cast<const uint16_t *>(a.win);
    const auto *wst = static_cast<const uint16_t *>(a.wst);
    if (a.bf16)
        hipLaunchKernelGGL((gemm_mfma_dma_kernel<MB, NB, WM, true, ABL>), grid, dim3(256), 0, s, win, wst,
                           a.out, a.rows, a.row0, a.row_elems, a.col_step, a.kstage, a.Ho, a.Wo,
                           a.Cout, tiles_m);
    else
        hipLaunchKernelGGL((gemm_mfma_dma_kernel<MB, NB, WM, false, ABL>), grid, dim3(256), 0, s, win,
                           wst, a.out, a.rows, a.row0, a.row_elems, a.col_step, a.kstage, a.Ho, a.Wo,
                           a.Cout, tiles_m);
    return hipGetLastError();
}

template <int MB, int NB, int WM>
hipError_t launch_dma_tile(const MfmaGemmArgs &a, hipStream_t s)
{
    switch (a.ablate) {
    case 0: return launch_dma_variant<MB, NB, WM, 0>(a, s);
    case 1: return launch_dma_variant<MB, NB, WM, 1>(a, s);
    case 2: return launch_dma_variant<MB, NB, WM, 2>(a, s);
    case 3: return launch_dma_variant<MB, NB, WM, 3>(a, s);
    case 4: return launch_dma_variant<MB, NB, WM, 4>(a, s);
    case 5: return launch_dma_variant<MB, NB, WM, 5>(a, s);
    case 6: return launch_dma_variant<MB, NB, WM, 6>(a, s);
    case 7: return launch_dma_variant<MB, NB, WM, 7>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm_mfma_dma(const MfmaGemmArgs &a, hipStream_t s)
{
    // whole K stages only: the window length is the staged filter row length
    if (a.krun != a.kstage || a.kstage % KI != 0 || a.col_step % 8 != 0 || a.row_elems % 8 != 0)
        return hipErrorInvalidValue;
    if (a.tile_m == 64 && a.tile_n == 128 && a.wm == 1) return launch_dma_tile<64, 128, 1>(a, s);
    if (a.tile_m == 64 && a.tile_n == 64 && a.wm == 2) return launch_dma_tile<64, 64, 2>(a, s);
    if (a.tile_m == 128 && a.tile_n == 64 && a.wm == 2) return launch_dma_tile<128, 64, 2>(a, s);
    if (a.tile_m == 128 && a.tile_n == 128 && a.wm == 2) return launch_dma_tile<128, 128, 2>(a, s);
    if (a.tile_m == 128 && a.tile_n == 128 && a.wm == 1) return launch_dma_tile<128, 128, 1>(a, s);
    if (a.tile_m == 64 && a.tile_n == 256 && a.wm == 1) return launch_dma_tile<64, 256, 1>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace im2win
