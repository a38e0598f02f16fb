// fp16 / bf16 implicit im2win convolution, split-K row-block form, for
// layers with a multiple of 128 input channels (3x3, 5x5 or 1x1 filters,
// stride 1 or 2) and tasks of at most 208 outputs.
//
// A task is RW whole output rows of one image (or IMG whole images) times 64
// output channels, and its window rows are built in LDS from NCHW x one
// 32-channel K chunk at a time, as in the pipelined row-block kernel (the
// window rows of Eq. (2) of "Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores", Sec. III-B, held once
// for all the task's output rows; the contraction of Sec. III-C Eq. (3) and
// Sec. III-D over K = channels x taps).
//
// The eight waves of a workgroup, two per SIMD (one wave per SIMD issues
// the matrix products at little over half their peak rate, two near 90%),
// are four K groups x two output halves. K group g contracts the chunks g,
// g + 4, g + 8, ... of the input channels; within it, each wave takes half of
// the task's 16-output blocks times all 64 output channels (up to 7 x 4
// blocks of 16 x 16). Per tap a wave reads one 16-byte window fragment per
// block from LDS and four filter fragments from memory, so LDS carries only
// the windows (a quarter of a kilobyte per product, half of what a wave
// tile of 64 x 64 reads with the filter in LDS as well). The two waves of a K
// group share two LDS slots (the patch granule-major, see ks_put_unit):
// while they contract one chunk they have the next one's loads in flight and
// write it into the other slot afterwards, one barrier per chunk. The filter
// is read pre-arranged in fragment order (a staging launch writes it into the
// workspace), one 1-KB run per 16 output channels and tap, straight into
// registers one tap ahead of its use; the loop over (chunk, tap) stays
// rolled, so that each accumulator is updated in place (an unrolled tap loop
// had the compiler alternate accumulator registers, twice the register
// file). At the end the four K groups' partial sums meet in LDS: the wave of
// group c adds the other groups' sums of output channels 16c .. 16c+15 of
// its blocks to its own and stores them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../launch.hpp"
#include "epilogue.hpp"
#include "lds_dma.hpp"
#include "pipe_patch.hpp"

namespace im2win {
namespace {

constexpr int kKsGroups = int(kKsplitGroups);   // K groups
constexpr int kKsThreads = 512;                  // 8 waves: K group x output half

// patch units a lane holds in registers between a chunk's global loads and
// its LDS writes (32 registers for any vector width); none for filters of
// more than 9 taps, whose longer contraction keeps more registers live (the
// units then go straight from memory to LDS at the end of a chunk), nor for
// the 3x3 form with 8-position vectors and 7 blocks per wave, whose registers
// spilled with them (14 registers; the 28x28 stride-2 layer 57.7 -> 54.6 us
// without)
template <int V, int TAPS, int NBW>
constexpr int ks_units_held()
{
    return TAPS > 9 || (TAPS == 9 && V == 8 && NBW == 7) ? 0 : V == 8 ? 1 : V == 4 ? 2 : 4;
}

// Staged filter, fragment order: fragment (cb, blk, t, c4) is 64 lanes x 8
// halves, lane l holding the 8 input channels blk*32 + (l >> 4)*8 .. +7 of
// output channel cb*64 + c4*16 + (l & 15) at tap t (zero past Cout).
__device__ __forceinline__ const uint4 *ks_frag(const uint16_t *wf, int nch, int taps, int cb, int blk, int t)
{
    return reinterpret_cast<const uint4 *>(wf) + ((int64_t(cb) * nch + blk) * taps + t) * (4 * 64);
}

// One workgroup per (cb, blk, c4): the 16 output channels cb*64 + c4*16 ..
// +15 each hold their 32 input channels blk*32 .. +31 over all taps as one
// contiguous run of 64*TAPS bytes of w. The workgroup copies the 16 runs into
// LDS with 16-byte loads (consecutive lanes on consecutive bytes of a run),
// then writes the TAPS fragments (cb, blk, t, c4), each 1 KB contiguous, one
// 16-byte lane slot per thread: lane l's 8 halves are channels (l >> 4)*8 ..
// +7 of output channel l & 15 at tap t, gathered from LDS 2 bytes at a time.
// Output channels past Cout are written as zeros.
constexpr int kStageThreads = 256;
template <int TAPS>
__global__ __launch_bounds__(kStageThreads) void ks_stage_kernel(const uint16_t *__restrict__ w,
                                                                uint4 *__restrict__ wf, int Cout, int Cin)
{
    constexpr int RUN = kChunkC * TAPS;              // halves of one output channel's run
    constexpr int RUNV = RUN / 8;                    // 16-byte vectors of a run (4 * TAPS)
    __shared__ uint4 runs[16 * RUNV];
    const int nch = Cin / kChunkC;
    const int c4 = blockIdx.x & 3;
    const int r = blockIdx.x >> 2;
    const int blk = r % nch;
    const int cb = r / nch;
    const int co0 = cb * 64 + c4 * 16;
    // every load of the thread in flight before the first LDS write
    constexpr int PER = (16 * RUNV + kStageThreads - 1) / kStageThreads;
    uint4 v4[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int v = threadIdx.x + j * kStageThreads;
        const int col = v / RUNV;                    // output channel of the block
        const int k = v - col * RUNV;
        const int co = co0 + col;
        v4[j] = v < 16 * RUNV && co < Cout
                    ? reinterpret_cast<const uint4 *>(w + (int64_t(co) * Cin + blk * kChunkC) * TAPS)[k]
                    : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int v = threadIdx.x + j * kStageThreads;
        if (v < 16 * RUNV) runs[v] = v4[j];
    }
    __syncthreads();
    const uint16_t *h = reinterpret_cast<const uint16_t *>(runs);
    uint4 *const dst = wf + ((int64_t(cb) * nch + blk) * TAPS * 4 + c4) * 64;
    for (int o = threadIdx.x; o < TAPS * 64; o += kStageThreads) {
        const int t = o >> 6, lane = o & 63;
        // channel e of the lane's 8 at tap t: half ((lane >> 4)*8 + e)*TAPS + t of run lane & 15
        const uint16_t *src = h + (lane & 15) * RUN + ((lane >> 4) * 8) * TAPS + t;
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = uint32_t(src[(2 * e) * TAPS]) | (uint32_t(src[(2 * e + 1) * TAPS]) << 16);
        dst[int64_t(t) * 4 * 64 + lane] = uint4{d[0], d[1], d[2], d[3]};
    }
}

// The slots hold a patch granule-major: the 8 channels of granule g (0..3) at
// patch position q are the 16 bytes at (g * NP + q) * 16, NP positions per
// granule plane. Sixteen lanes that read one granule at consecutive
// positions hit consecutive 16-byte slots (no bank conflict), and a tap's
// window is the same address plus one uniform offset. NP is 1 modulo 8, so
// that the four granules of one position fall in different bank groups when
// the loads write them.
template <int V, bool MI>
__device__ __forceinline__ void ks_put_unit(uint16_t *patch, int NP, const PipeKArgs &a, const PipeTask &tk,
                                            const ChunkGeom &cg, int u, const PlaneVec<V> *raw)
{
    const int im = MI ? u / cg.units1 : 0, u1 = u - im * cg.units1;
    const int g = u1 & 3;
    const int p0 = (cg.j_lo + (u1 >> 2)) * V;
    const int row0 = im * tk.SL - tk.ih0;            // patch row of input row 0 of this image
    uint16_t *const gp = patch + g * NP * 8;
    {
        int r = p0 / a.W;
        int col = p0 - r * a.W;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int p = p0 + v;
            if (p >= cg.p_lo && p < cg.p_hi)
                *reinterpret_cast<uint4 *>(gp + ((row0 + r) * a.IW + a.pad + col) * 8) = position_of<V>(raw, v);
            if (++col == a.W) { col = 0; ++r; }
        }
    }
}

// zeros at the positions no load writes: the padding columns of every row
// and the rows of the task outside the image (thread t0 of nt)
template <bool MI>
__device__ __forceinline__ void ks_zero(uint16_t *patch, int NP, const PipeKArgs &a, const PipeTask &tk, int t0,
                                        int nt)
{
    const uint4 z{0u, 0u, 0u, 0u};
    const int rows = tk.nimg * tk.SL;
    const int pc = 2 * a.pad;
    for (int v = t0; v < 4 * rows * pc; v += nt) {
        const int g = v & 3, e = v >> 2;
        const int i = e / pc, c = e - i * pc;
        *reinterpret_cast<uint4 *>(patch + (g * NP + i * a.IW + (c < a.pad ? c : a.W + c)) * 8) = z;
    }
    const int top = min(max(-tk.ih0, 0), tk.SL);
    const int bot0 = max(min(a.H - tk.ih0, tk.SL), top);
    const int run = (top + (tk.SL - bot0)) * a.IW;   // zero positions per image (whole rows)
    for (int v = t0; v < 4 * run * tk.nimg; v += nt) {
        const int g = v & 3, e = v >> 2;
        const int im = MI ? e / run : 0, k = e - im * run;
        const int q = im * tk.SL * a.IW + (k < top * a.IW ? k : bot0 * a.IW + (k - top * a.IW));
        *reinterpret_cast<uint4 *>(patch + (g * NP + q) * 8) = z;
    }
}

template <int KH, int KW, bool BF16, int V, bool MI, int NBW>
__global__ __launch_bounds__(kKsThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv_implicit_ksplit_kernel(
    const PipeKArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int UH = ks_units_held<V, TAPS, NBW>();
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int kg = wave & (kKsGroups - 1);         // K group: chunks kg + 4 j
    const int half = wave >> 2;                    // output half of the task
    const int gl = half * 64 + lane;               // thread of the K group (0..127)
    const PipeTask tk = pipe_task<KH, MI>(a, xcd_logical(blockIdx.x, gridDim.x));
    const ChunkGeom cg = chunk_geom<V, MI>(a, tk);
    const int nch = a.Cin / kChunkC;
    const int steps = nch / kKsGroups;
    const int spw = steps > 1 ? a.slots : 1;       // LDS slots per K group
    const int NP = a.slot_halves / 32;             // positions per granule plane
    // this wave's 64 output channels: the task's (co_split 1) or its half of
    // the task's 128 (co_split 2); the filter is read from the last block
    // that exists where the half lies past Cout (nothing of it is stored)
    const int cbw = a.co_split == 2 ? tk.cb * 2 + half : tk.cb;
    const int cba = min(cbw, (a.Cout - 1) >> 6);
    uint16_t *const slot0 = lds + spw * kg * a.slot_halves;
    uint16_t *const slot1 = slot0 + (spw - 1) * a.slot_halves;

    PlaneVec<V> raw[UH > 0 ? UH : 1][8];
    auto fetch = [&](int j) {
        const int blk = kg + kKsGroups * j;
#pragma unroll
        for (int k = 0; k < UH; ++k) {
            const int u = gl + 128 * k;
            if (u < cg.units) load_patch_unit<V, MI>(a, tk, blk, cg, u, raw[k]);
        }
    };
    auto put = [&](int j, uint16_t *patch) {
        const int blk = kg + kKsGroups * j;
#pragma unroll
        for (int k = 0; k < UH; ++k) {
            const int u = gl + 128 * k;
            if (u < cg.units) ks_put_unit<V, MI>(patch, NP, a, tk, cg, u, raw[k]);
        }
        for (int u = gl + 128 * UH; u < cg.units; u += 128) {   // beyond the held units
            PlaneVec<V> r1[8];
            load_patch_unit<V, MI>(a, tk, blk, cg, u, r1);
            ks_put_unit<V, MI>(patch, NP, a, tk, cg, u, r1);
        }
    };
    // the first chunk's loads go out first; the set-up below runs under them
    fetch(0);

    ks_zero<MI>(slot0, NP, a, tk, gl, 128);
    if (spw > 1) ks_zero<MI>(slot1, NP, a, tk, gl, 128);

    // output m of the task (row-major over its rows, image after image) is in
    // block m / 16; this wave takes blocks [b0, b0 + nbs). The window of its
    // block s at tap (0, 0) is at halves offset bb[s] of a slot (lane's granule)
    const int outs = tk.nimg * tk.rw * a.Wo;
    const int opi = tk.rw * a.Wo;
    const int nbt = (outs + 15) >> 4;
    const bool split_out = a.co_split == 1;
    const int b0 = split_out && half ? (nbt + 1) >> 1 : 0;
    const int nbs = !split_out ? nbt : half ? nbt - b0 : (nbt + 1) >> 1;
    const int gr = lane >> 4;
    int bb[NBW];
#pragma unroll
    for (int s = 0; s < NBW; ++s) {
        const int m = min((b0 + s) * 16 + (lane & 15), outs - 1);
        const int im = MI ? m / opi : 0, rem = m - im * opi;
        const int i = rem / a.Wo;
        bb[s] = (gr * NP + (im * tk.SL + i * a.stride) * a.IW + (rem - i * a.Wo) * a.stride) * 8;
    }

    // filter fragments of iteration it (chunk it / TAPS, tap it % TAPS): fa0
    // for this iteration, fa1 for the next, loaded during this one
    auto load_a = [&](int it, uint4 *f) {
        const int j = it / TAPS, t = it - j * TAPS;
        const uint4 *p = ks_frag(a.w, nch, TAPS, cba, kg + kKsGroups * j, t) + lane;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) f[c4] = p[c4 * 64];
    };
    const int iters = steps * TAPS;
    uint4 fa0[4], fa1[4];
    load_a(0, fa0);
    put(0, slot0);
    stage_barrier();

    floatx4_t acc[NBW][4];
#pragma unroll
    for (int s = 0; s < NBW; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    uint4 bf[NBW];
    int j = 0, t = 0;
    for (int it = 0; it < iters; ++it) {
        const uint16_t *const cur = (j & 1) ? slot1 : slot0;
        if (it + 1 < iters) load_a(it + 1, fa1);
        if (t == 0) {
            if (j + 1 < steps) fetch(j + 1);
#pragma unroll
            for (int s = 0; s < NBW; ++s) bf[s] = *reinterpret_cast<const uint4 *>(cur + bb[s]);
        }
        // the next tap's windows, read as each block's products issue (after
        // the last tap: tap 0 again, a harmless read that keeps the loop
        // free of branches)
        const int tn = t + 1 < TAPS ? t + 1 : 0;
        const int dq = ((tn / KW) * a.IW + (tn - (tn / KW) * KW)) * 8;
#pragma unroll
        for (int s = 0; s < NBW; ++s) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(bf[s], fa0[c], acc[s][c]);
            bf[s] = *reinterpret_cast<const uint4 *>(cur + bb[s] + dq);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) fa0[c] = fa1[c];
        if (t + 1 == TAPS) {
            if (j + 1 < steps) {
                // the other slot was last read in the previous chunk, which
                // every wave finished before the last barrier; with one slot,
                // every wave first finishes reading this chunk
                if (spw == 1) stage_barrier();
                put(j + 1, (j & 1) ? slot0 : slot1);
                stage_barrier();
            }
            t = 0;
            ++j;
        } else {
            ++t;
        }
    }

    // the K groups' partial sums, in two rounds of two 16-channel blocks c:
    // the waves of the other groups put their sums of block c of their
    // output blocks into LDS ([c - 2r][3 givers][half][NBW][64 lanes] of
    // 16-byte vectors), the wave of group c adds them to its own
    floatx4_t own[NBW];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (c == kg)
#pragma unroll
            for (int s = 0; s < NBW; ++s) own[s] = acc[s][c];
    floatx4_t *const red = reinterpret_cast<floatx4_t *>(lds);
    stage_barrier();                               // the slots are dead: LDS holds the sums
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * r + cc;
            if (c == kg) continue;
            const int k = kg < c ? kg : kg - 1;
#pragma unroll
            for (int s = 0; s < NBW; ++s) red[(((cc * 3 + k) * 2 + half) * NBW + s) * 64 + lane] = acc[s][c];
        }
        stage_barrier();
        if ((kg >> 1) == r) {
            const int cc = kg & 1;
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int s = 0; s < NBW; ++s) own[s] += red[(((cc * 3 + k) * 2 + half) * NBW + s) * 64 + lane];
        }
        if (r == 0) stage_barrier();
    }

    // lane l holds outputs m0 .. m0+3 (m0 = 16 (b0 + s) + 4 (l >> 4)) of
    // output channel co: consecutive elements of one plane unless they cross
    // an image (several images per task) or the task's end
    const int co = cbw * 64 + kg * 16 + (lane & 15);
    if (co >= a.Cout) return;
    const OutSpec &o = a.out;
    const int64_t plane = o.plane;
    const ChanEpi ep = chan_epi(o, co);
    with_ytype(o, [&](auto tc) {
        constexpr int T = decltype(tc)::value;
#pragma unroll
        for (int s = 0; s < NBW; ++s) {
            const int m0 = (b0 + s) * 16 + 4 * (lane >> 4);
            if (s >= nbs || m0 >= outs) continue;
            const int im = MI ? m0 / opi : 0;
            const int64_t p = MI ? int64_t(m0 - im * opi) : int64_t(tk.ho0) * a.Wo + m0;
            const int64_t off = (int64_t(tk.n + im) * a.Cout + co) * plane + p;
            if (m0 + 3 < outs && p + 3 < plane && (off & 3) == 0) {
                put4<T>(o.y, off, epi_apply(ep, own[s][0]), epi_apply(ep, own[s][1]), epi_apply(ep, own[s][2]),
                        epi_apply(ep, own[s][3]));
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = m0 + v;
                    if (m >= outs) break;
                    const int iv = MI ? m / opi : 0;
                    const int64_t pv = MI ? int64_t(m - iv * opi) : int64_t(tk.ho0) * a.Wo + m;
                    put1<T>(o.y, (int64_t(tk.n + iv) * a.Cout + co) * plane + pv, epi_apply(ep, own[s][v]));
                }
            }
        }
    });
}

}  // namespace

hipError_t launch_ksplit_stage(const void *w, void *wf, int Cout, int Cin, int taps, hipStream_t s)
{
    if (Cin % kChunkC != 0 || Cout < 1 || !(taps == 1 || taps == 9 || taps == 25)) return hipErrorInvalidValue;
    // one workgroup per 1 KB x taps fragment group (cb, blk, c4)
    const int64_t groups = ksplit_stage_bytes(Cout, Cin, taps) / (1024 * int64_t(taps));
    if (groups > 0x7fffffff) return hipErrorInvalidValue;
    void *args[] = {&w, &wf, &Cout, &Cin};
    const void *k = taps == 9    ? reinterpret_cast<const void *>(ks_stage_kernel<9>)
                    : taps == 25 ? reinterpret_cast<const void *>(ks_stage_kernel<25>)
                                 : reinterpret_cast<const void *>(ks_stage_kernel<1>);
    return hipLaunchKernel(k, dim3(unsigned(groups)), dim3(kStageThreads), args, 0, s);
}

hipError_t launch_conv_implicit_ksplit(const ImplicitArgs &h, hipStream_t s)
{
    const int img = std::max(h.images, 1);
    const int64_t outs = int64_t(img) * h.R * h.Wo;
    // tile_m 128: the two waves of a K group split 128 output channels, each
    // over all of the task's blocks
    const int cos = h.tile_m == 128 ? 2 : 1;
    const int nbw = int(ksplit_nbw(outs, cos));
    const int slots = h.stages == 1 ? 1 : 2;
    if (h.f32 || h.Cin % (kChunkC * kKsGroups) != 0 || h.stride < 1 || h.stride > 2 || h.W < 1 || h.H < 1 ||
        h.Wo < 1 || h.Ho < 1 || h.R < 1 || outs > kKsplitMaxOuts / cos || h.IW != h.W + 2 * h.pad ||
        (h.Wo - 1) * h.stride + h.KW > h.IW || h.IR != img * ((h.R - 1) * h.stride + h.KH) ||
        (img > 1 && h.R != h.Ho) || int64_t(h.Cin) * h.H * h.W >= (int64_t(1) << 31) ||
        !((h.KH == 3 && h.KW == 3) || (h.KH == 1 && h.KW == 1) || (h.KH == 5 && h.KW == 5)))
        return hipErrorInvalidValue;
    PipeKArgs a{};
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
    a.co_blocks = (h.Cout + 64 * cos - 1) / (64 * cos);
    a.co_split = cos;
    a.slots = slots;
    a.IW = h.IW;
    a.N = h.N;
    a.IMG = img;
    a.stride = h.stride;
    const int64_t ntasks = img > 1 ? int64_t(a.co_blocks) * ((h.N + img - 1) / img)
                                   : int64_t(a.co_blocks) * h.N * a.row_groups;
    if (ntasks > 0x7fffffff) return hipErrorInvalidValue;
    a.ntasks = int(ntasks);
    a.SLmax = h.IR;
    a.slot_halves = int(ksplit_plane(h.IR, h.IW)) * 4 * 8;
    const int64_t lds = ksplit_lds_bytes(h.IR, h.IW, h.Cin, nbw, slots);
    if (lds > kImplicitMaxLdsBytes) return hipErrorInvalidValue;
    const int hw = h.H * h.W;
    void *args[] = {&a};
#define IM2WIN_KS_K(KH, B, V, M)                                                                             \
    (nbw == 4 ? reinterpret_cast<const void *>(conv_implicit_ksplit_kernel<KH, KH, B, V, M, 4>)               \
              : reinterpret_cast<const void *>(conv_implicit_ksplit_kernel<KH, KH, B, V, M, 7>))
#define IM2WIN_KS_V(KH, B, M)                                                                                \
    (hw % 8 == 0 ? IM2WIN_KS_K(KH, B, 8, M) : hw % 4 == 0 ? IM2WIN_KS_K(KH, B, 4, M) : IM2WIN_KS_K(KH, B, 1, M))
#define IM2WIN_KS_M(KH, B) (img > 1 ? IM2WIN_KS_V(KH, B, true) : IM2WIN_KS_V(KH, B, false))
#define IM2WIN_KS_B(KH) (h.bf16 ? IM2WIN_KS_M(KH, true) : IM2WIN_KS_M(KH, false))
    const void *kern = h.KH == 3 ? IM2WIN_KS_B(3) : h.KH == 5 ? IM2WIN_KS_B(5) : IM2WIN_KS_B(1);
#undef IM2WIN_KS_B
#undef IM2WIN_KS_M
#undef IM2WIN_KS_V
#undef IM2WIN_KS_K
    return hipLaunchKernel(kern, dim3(unsigned(ntasks)), dim3(kKsThreads), args, size_t(lds), s);
}

}  // namespace im2win
