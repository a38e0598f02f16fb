// fp16 / bf16 implicit im2win convolution, pipelined row-block form, for
// 3x3 and 1x1 layers with a multiple of 32 input channels and output rows of
// at most 256 columns.
//
// A task is a block of RW whole output rows (n, ho0 .. ho0+RW-1) of one image
// and 64 output channels, as in the row-block kernel: the window rows of those
// output rows (Eq. (2) of "Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores", Sec. III-B) share all
// but their first and last input rows, so a task holds the union once, SL =
// (RW - 1) * s + KH input rows of IW = W + 2*pad positions, channels
// innermost; the window of output (i, wo) at tap (kh, kw) is position
// (i * s + kh, wo * s + kw) for stride s.
//
// The contraction runs over K chunks of 32 input channels x all taps (the
// window's K order of Sec. III-D, taps outer and channels inner within a
// chunk). Each workgroup is persistent and walks its tasks chunk by chunk,
// with two LDS slots, each holding one chunk: the filter block
// [TAPS][64 co][32 ci] and the patch [SL][IW][32 ci], 64 bytes per row or
// position (16-byte granule g of row q in slot g ^ ((q >> 1) & 3), so that
// eight consecutive rows read at one granule hit eight different bank groups).
//
// The eight waves have two roles. Waves 0-3 contract: each owns up to four
// 16-output MFMA blocks of the task (the task's outputs flattened row-major)
// times the 64 output channels, reads chunk c from slot c & 1 and, after a
// task's last chunk, stores its results and starts the next task. Waves 4-7
// load: while chunk c is contracted they write chunk c + 1 (loaded into
// registers one step earlier) into the other slot and issue the global loads
// of chunk c + 2. One barrier per chunk, which waits for LDS accesses only,
// so the loads in flight cross it. The filter is read from w as stored (8
// channels x all taps of one output channel per loader lane, reordered in
// registers), the input as 8 channels x V consecutive positions of a channel
// plane (V = 8, 4 or 1 by how the plane is aligned), transposed in registers
// into V positions of 8 channels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../launch.hpp"
#include "lds_dma.hpp"
#include "out_blocks.hpp"
#include "pipe_patch.hpp"

namespace im2win {
namespace {

constexpr int kPipeThreads = 512;
constexpr int kComputeWaves = 4;
constexpr int kLoaderThreads = kPipeThreads - 64 * kComputeWaves;
constexpr int kUnitsHeld = 2;     // patch units per loader lane held in registers

// filter chunk: lane (output channel co_l of the task's block, granule fg)
// reads the 8 x TAPS halves w[co][blk*32 + fg*8 .. +7][taps] as stored
template <int TAPS>
__device__ __forceinline__ void load_filter_unit(const PipeKArgs &a, const PipeTask &tk, int blk, int co_l,
                                                 int fg, uint4 *wraw)
{
    const int co_src = min(tk.cb * 64 + co_l, a.Cout - 1);   // rows past Cout: never stored
    const uint4 *ws = reinterpret_cast<const uint4 *>(a.w + (int64_t(co_src) * a.Cin + blk * kChunkC + fg * 8) * TAPS);
#pragma unroll
    for (int i = 0; i < TAPS; ++i) wraw[i] = ws[i];
}

// ... and writes one 16-byte vector per tap (element (channel e, tap t) is
// half e*TAPS + t of the run) into row co_l of the tap's block
template <int TAPS>
__device__ __forceinline__ void put_filter_unit(uint16_t *fl, int co_l, int fg, const uint4 *wraw)
{
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
        *reinterpret_cast<uint4 *>(fl + t * 64 * kChunkC + co_l * kChunkC + (gslot(fg, co_l) << 3)) =
            uint4{o[0], o[1], o[2], o[3]};
    }
}

// Patch position of the window at tap (0, 0) of each of a lane's output
// blocks: output m of the task is image m / opi, row i and column wo of the
// rest (opi = rw * Wo outputs per image), at patch row im * SL + i * st and
// column wo * st.
template <bool MI>
__device__ __forceinline__ void task_bases(int *qa, int b0, int lane, int outs, int Wo, int IW, int opi, int SL,
                                           int st)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int m = min((b0 + s) * 16 + (lane & 15), outs - 1);
        const int im = MI ? m / opi : 0, rem = m - im * opi;
        const int i = rem / Wo;
        qa[s] = (im * SL + i * st) * IW + (rem - i * Wo) * st;
    }
}

// Stores of a task of several whole images through the wave's LDS scratch
// (as store_blocks_lds): lane l stores output m = 16*b0 + l of each channel
// row, at its image's plane.
template <int MAXB>
__device__ __forceinline__ void store_blocks_images(const floatx4_t (*acc)[4], int nb, int b0, int lane,
                                                   float *scratch, const OutSpec &o, int n, int Cout, int cb,
                                                   int plane, int outs)
{
    const int nout = min(nb * 16, outs - b0 * 16);
    const int m = b0 * 16 + lane;
    const int im = m / plane;
    const int p = m - im * plane;
    float *const srow = scratch + (lane & 15) * kStoreRow + 4 * (lane >> 4);
    with_ytype(o, [&](auto tc) {
        constexpr int T = decltype(tc)::value;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int s = 0; s < MAXB; ++s)
                if (s < nb) *reinterpret_cast<floatx4_t *>(srow + s * 16) = acc[s][c];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = cb * 64 + c * 16 + r;
                const float v = scratch[r * kStoreRow + lane];
                if (co < Cout && lane < nout) {
                    if (o.plain)
                        static_cast<float *>(o.y)[(int64_t(n + im) * Cout + co) * plane + p] = v;
                    else
                        out_store<T>(o, n + im, co, p, v);
                }
            }
        }
    });
}

// One K chunk (32 channels x TAPS taps) of a wave's NBW output blocks x 64
// output channels: per tap, lane l reads the 8 channels of granule l / 16 of
// the window position of output row l % 16 of each block (A) and of output
// channel l % 16 of each 16-channel block (B). PREFETCH: the fragments of
// tap t + 1 are read while the products of tap t issue (two register sets,
// the order pinned for the scheduler), for a wave that has its SIMD to itself.
template <int KH, int KW, bool BF16, int NBW, bool PREFETCH>
__device__ __forceinline__ void contract_chunk(floatx4_t (*acc)[4], const int *qa, const uint16_t *fl, int IW,
                                               int lane)
{
    constexpr int TAPS = KH * KW;
    const uint16_t *patch = fl + TAPS * 64 * kChunkC;
    const int gr = lane >> 4;
    // the per-lane bases pass through an empty asm once per chunk, so the
    // compiler recomputes each tap's LDS addresses instead of holding all of
    // them in registers across the chunk loop
    int q0[NBW];
#pragma unroll
    for (int s = 0; s < NBW; ++s) {
        q0[s] = qa[s];
        asm volatile("" : "+v"(q0[s]));
    }
    int rbv = lane & 15;
    asm volatile("" : "+v"(rbv));
    auto fetch_tap = [&](int t, uint4 *fa, uint4 *fb) {
        const int kh = t / KW, kw = t - (t / KW) * KW;
        const uint16_t *ft = fl + t * 64 * kChunkC;
        const int dq = kh * IW + kw;
#pragma unroll
        for (int s = 0; s < NBW; ++s) {
            const int q = q0[s] + dq;
            fa[s] = *reinterpret_cast<const uint4 *>(patch + q * kChunkC + (gslot(gr, q) << 3));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = c * 16 + rbv;
            fb[c] = *reinterpret_cast<const uint4 *>(ft + r * kChunkC + (gslot(gr, r) << 3));
        }
    };
    if constexpr (PREFETCH) {
        uint4 af[2][NBW], bf[2][4];
        fetch_tap(0, af[0], bf[0]);
        __builtin_amdgcn_sched_group_barrier(0x100, NBW + 4, 0);
#pragma unroll
        for (int t = 0; t < TAPS; ++t) {
            if (t + 1 < TAPS) fetch_tap(t + 1, af[(t + 1) & 1], bf[(t + 1) & 1]);
#pragma unroll
            for (int s = 0; s < NBW; ++s)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(af[t & 1][s], bf[t & 1][c], acc[s][c]);
            if (t + 1 < TAPS) __builtin_amdgcn_sched_group_barrier(0x100, NBW + 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NBW * 4, 0);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TAPS; ++t) {
            uint4 af[NBW], bf[4];
            fetch_tap(t, af, bf);
#pragma unroll
            for (int s = 0; s < NBW; ++s)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[s][c] = mfma16x16x32<BF16>(af[s], bf[c], acc[s][c]);
        }
    }
}

// nb (<= MAXB) blocks, one compiled contraction per block count
template <int KH, int KW, bool BF16, bool PREFETCH, int MAXB = 4>
__device__ __forceinline__ void contract_blocks(floatx4_t (*acc)[4], int nb, const int *qa, const uint16_t *fl,
                                                int IW, int lane)
{
    if constexpr (MAXB >= 4) {
        if (nb >= 4) { contract_chunk<KH, KW, BF16, 4, PREFETCH>(acc, qa, fl, IW, lane); return; }
    }
    if constexpr (MAXB >= 3) {
        if (nb == 3) { contract_chunk<KH, KW, BF16, 3, PREFETCH>(acc, qa, fl, IW, lane); return; }
    }
    if (nb >= 2) contract_chunk<KH, KW, BF16, 2, PREFETCH>(acc, qa, fl, IW, lane);
    else if (nb == 1) contract_chunk<KH, KW, BF16, 1, PREFETCH>(acc, qa, fl, IW, lane);
}

template <int KH, int KW, bool BF16, int V, bool MI>
__global__ __launch_bounds__(kPipeThreads) void conv_implicit_pipe_kernel(const PipeKArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int FILT = TAPS * 64 * kChunkC;        // halves of a slot's filter block
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    float *const scratch = reinterpret_cast<float *>(lds + 2 * a.slot_halves);

    const int tid = threadIdx.x;
    const int G = gridDim.x;
    // in each round of G tasks, the tasks of one XCD are consecutive
    const int L = xcd_logical(blockIdx.x, G);
    const int my_tasks = L < a.ntasks ? (a.ntasks - L + G - 1) / G : 0;
    const int nch = a.Cin / kChunkC;
    const int total = my_tasks * nch;

    // loads write only columns pad .. pad + W - 1 (and whole rows of zeros)
    zero_pad_columns(lds + FILT, a, a.SLmax, tid, kPipeThreads);
    zero_pad_columns(lds + a.slot_halves + FILT, a, a.SLmax, tid, kPipeThreads);

    if (tid >= 64 * kComputeWaves) {
        // ================= loader waves =================
        const int lt = tid - 64 * kComputeWaves;
        const int co_l = lt >> 2;                    // filter row of this lane
        const int fg = lt & 3;                       // its 8-channel granule
        uint4 wraw[TAPS];
        PlaneVec<V> praw[kUnitsHeld][8];
        auto fetch = [&](int c) {
            const PipeTask tk = pipe_task<KH, MI>(a, L + (c / nch) * G);
            const int blk = c - (c / nch) * nch;
            const ChunkGeom cg = chunk_geom<V, MI>(a, tk);
            load_filter_unit<TAPS>(a, tk, blk, co_l, fg, wraw);
#pragma unroll
            for (int k = 0; k < kUnitsHeld; ++k) {
                const int u = lt + k * kLoaderThreads;
                if (u < cg.units) load_patch_unit<V, MI>(a, tk, blk, cg, u, praw[k]);
            }
        };
        auto put = [&](int c) {
            const PipeTask tk = pipe_task<KH, MI>(a, L + (c / nch) * G);
            const int blk = c - (c / nch) * nch;
            const ChunkGeom cg = chunk_geom<V, MI>(a, tk);
            uint16_t *const fl = lds + (c & 1) * a.slot_halves;
            uint16_t *const patch = fl + FILT;
            put_filter_unit<TAPS>(fl, co_l, fg, wraw);
#pragma unroll
            for (int k = 0; k < kUnitsHeld; ++k) {
                const int u = lt + k * kLoaderThreads;
                if (u < cg.units) put_patch_unit<V, MI>(patch, a, tk, cg, u, praw[k]);
            }
            for (int u = lt + kUnitsHeld * kLoaderThreads; u < cg.units; u += kLoaderThreads) {
                PlaneVec<V> raw[8];
                load_patch_unit<V, MI>(a, tk, blk, cg, u, raw);
                put_patch_unit<V, MI>(patch, a, tk, cg, u, raw);
            }
            // rows outside the image: zero in each slot once per task (the
            // task's first two chunks, one per slot); the loads of its later
            // chunks write only rows inside the image
            if (blk < 2) zero_rows<MI>(patch, a, tk, lt, kLoaderThreads);
        };
        if (total > 0) {
            fetch(0);
            put(0);
            if (total > 1) fetch(1);
        }
        stage_barrier();
        for (int c = 0; c < total; ++c) {
            if (c + 1 < total) put(c + 1);
            if (c + 2 < total) fetch(c + 2);
            stage_barrier();
        }
    } else {
        // ================= computing waves =================
        const int wave = tid >> 6;
        const int lane = tid & 63;
        floatx4_t acc[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        PipeTask tk{};
        int outs = 0, b0 = 0, nb = 0;
        int qa[4] = {0, 0, 0, 0};
        stage_barrier();
        for (int c = 0; c < total; ++c) {
            const int blk = c - (c / nch) * nch;
            if (blk == 0) {
                tk = pipe_task<KH, MI>(a, L + (c / nch) * G);
                outs = tk.nimg * tk.rw * a.Wo;
                wave_blocks_of(wave, kComputeWaves, outs, b0, nb);
                task_bases<MI>(qa, b0, lane, outs, a.Wo, a.IW, tk.rw * a.Wo, tk.SL, a.stride);
            }
            contract_blocks<KH, KW, BF16, true>(acc, nb, qa, lds + (c & 1) * a.slot_halves, a.IW, lane);
            if (blk == nch - 1) {
                if (nb > 0) {
                    if (MI)
                        store_blocks_images<4>(acc, nb, b0, lane, scratch + wave * kStoreScratchFloats, a.out,
                                               tk.n, a.Cout, tk.cb, a.Ho * a.Wo, outs);
                    else if ((a.Wo & 3) == 0 && a.out.type == 0)
                        store_blocks(acc, nb, b0, lane, a.out, tk.n, a.Cout, tk.cb, a.Ho, a.Wo, tk.ho0, outs);
                    else
                        store_blocks_lds(acc, nb, b0, lane, scratch + wave * kStoreScratchFloats, a.out, tk.n,
                                         a.Cout, tk.cb, a.Ho, a.Wo, tk.ho0, outs);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) acc[s][cc] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
            stage_barrier();
        }
    }
}

// The paired form: one task per workgroup and a single LDS slot, small
// enough (at most 80 KB) that two workgroups share a CU, so that one's loads
// and stores overlap the other's contraction. All eight waves load a chunk
// (filter block by the first four, patch units by all), then the fewest
// waves that hold two 16-output blocks each contract it (R * Wo <= 256).
template <int KH, int KW, bool BF16, int V, bool MI>
__global__ __launch_bounds__(kPipeThreads) __attribute__((amdgpu_waves_per_eu(4))) void conv_implicit_pair_kernel(const PipeKArgs a)
{
    constexpr int TAPS = KH * KW;
    constexpr int FILT = TAPS * 64 * kChunkC;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *const fl = lds;
    uint16_t *const patch = lds + FILT;

    const int tid = threadIdx.x;
    const PipeTask tk = pipe_task<KH, MI>(a, xcd_logical(blockIdx.x, gridDim.x));
    const int nch = a.Cin / kChunkC;
    const ChunkGeom cg = chunk_geom<V, MI>(a, tk);
    zero_pad_columns(patch, a, tk.SL * tk.nimg, tid, kPipeThreads);

    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int outs = tk.nimg * tk.rw * a.Wo;
    // blocks two to a wave over as few waves as that takes: a wave reads the
    // same four filter fragments per tap for one block or two, and LDS reads,
    // not products, bound this form; the idle waves still load
    const int busy = min((((outs + 15) >> 4) + 1) >> 1, 8);
    int b0 = 0, nb = 0;
    if (wave < busy) wave_blocks_of(wave, busy, outs, b0, nb);
    int qa[4];
    task_bases<MI>(qa, b0, lane, outs, a.Wo, a.IW, tk.rw * a.Wo, tk.SL, a.stride);
    constexpr int MAXB = 2;                          // R * Wo <= 256: at most 2 blocks per wave
    floatx4_t acc[MAXB][4];
#pragma unroll
    for (int s = 0; s < MAXB; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int blk = 0; blk < nch; ++blk) {
        if (blk > 0) __syncthreads();                // every wave is done with the previous chunk
        if (tid < 256) {
            uint4 wraw[TAPS];
            load_filter_unit<TAPS>(a, tk, blk, tid >> 2, tid & 3, wraw);
            put_filter_unit<TAPS>(fl, tid >> 2, tid & 3, wraw);
        }
        // the filter's registers are dead before the patch's are loaded (at
        // most 128 registers per lane for two workgroups per CU)
        asm volatile("" ::: "memory");
        for (int u = tid; u < cg.units; u += kPipeThreads) {
            PlaneVec<V> raw[8];
            load_patch_unit<V, MI>(a, tk, blk, cg, u, raw);
            put_patch_unit<V, MI>(patch, a, tk, cg, u, raw);
        }
        // rows outside the image: zeroed once (the chunks' loads write only
        // rows inside it)
        if (blk == 0) zero_rows<MI>(patch, a, tk, tid, kPipeThreads);
        __syncthreads();
        contract_blocks<KH, KW, BF16, false, MAXB>(acc, nb, qa, fl, a.IW, lane);
    }
    if ((a.Wo & 3) == 0 && a.out.type == 0 && !MI) {
        if (nb > 0) store_blocks<MAXB>(acc, nb, b0, lane, a.out, tk.n, a.Cout, tk.cb, a.Ho, a.Wo, tk.ho0, outs);
    } else if (MI) {
        __syncthreads();                             // the chunk is dead: LDS is store scratch
        if (nb > 0)
            store_blocks_images<MAXB>(acc, nb, b0, lane, reinterpret_cast<float *>(lds) + wave * kStoreScratchFloats,
                                      a.out, tk.n, a.Cout, tk.cb, a.Ho * a.Wo, outs);
    } else {
        __syncthreads();                             // the chunk is dead: LDS is store scratch
        if (nb > 0)
            store_blocks_lds<MAXB>(acc, nb, b0, lane, reinterpret_cast<float *>(lds) + wave * kStoreScratchFloats,
                                   a.out, tk.n, a.Cout, tk.cb, a.Ho, a.Wo, tk.ho0, outs);
    }
}

}  // namespace

hipError_t launch_conv_implicit_pipe(const ImplicitArgs &h, hipStream_t s)
{
    // stages: 2 for the pipelined form (two LDS slots, persistent workgroups),
    // 1 for the paired form (one slot, one task per workgroup)
    const bool pair = h.stages == 1;
    const int img = std::max(h.images, 1);
    if (h.f32 || h.Cin % kChunkC != 0 || h.stride < 1 || h.W < 1 || h.H < 1 || h.Wo < 1 || h.Ho < 1 ||
        h.R < 1 || int64_t(img) * h.R * h.Wo > 256 || h.IW != h.W + 2 * h.pad ||
        (h.Wo - 1) * h.stride + h.KW > h.IW || h.IR != img * ((h.R - 1) * h.stride + h.KH) ||
        (img > 1 && h.R != h.Ho) ||
        int64_t(h.Cin) * h.H * h.W >= (int64_t(1) << 31) ||
        (!pair && h.groups < 1) || (h.stages != 1 && h.stages != 2) ||
        !((h.KH == 3 && h.KW == 3) || (h.KH == 1 && h.KW == 1)))
        return hipErrorInvalidValue;
    PipeKArgs a;
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
    a.IW = h.IW;
    a.N = h.N;
    a.IMG = img;
    a.stride = h.stride;
    const int64_t ntasks = img > 1 ? int64_t(a.co_blocks) * ((h.N + img - 1) / img)
                                   : int64_t(a.co_blocks) * h.N * a.row_groups;
    if (ntasks > 0x7fffffff) return hipErrorInvalidValue;
    a.ntasks = int(ntasks);
    a.SLmax = h.IR;
    const int taps = h.KH * h.KW;
    a.slot_halves = taps * 64 * kChunkC + a.SLmax * a.IW * kChunkC;
    const size_t lds = size_t(pair ? pair_lds_bytes(taps, a.SLmax, a.IW) : pipe_lds_bytes(taps, a.SLmax, a.IW));
    if (lds > size_t(kImplicitMaxLdsBytes)) return hipErrorInvalidValue;
    const int groups = pair ? a.ntasks : int(std::min<int64_t>(h.groups, ntasks));
    const int hw = h.H * h.W;
    void *args[] = {&a};
    const bool k3 = h.KH == 3;
#define IM2WIN_PIPE_PICK(K, V, M)                                                                            \
    (k3 ? (h.bf16 ? reinterpret_cast<const void *>(K<3, 3, true, V, M>)                                      \
                  : reinterpret_cast<const void *>(K<3, 3, false, V, M>))                                    \
        : (h.bf16 ? reinterpret_cast<const void *>(K<1, 1, true, V, M>)                                      \
                  : reinterpret_cast<const void *>(K<1, 1, false, V, M>)))
#define IM2WIN_PIPE_FORM(K, M)                                                                               \
    (hw % 8 == 0 ? IM2WIN_PIPE_PICK(K, 8, M) : hw % 4 == 0 ? IM2WIN_PIPE_PICK(K, 4, M) : IM2WIN_PIPE_PICK(K, 1, M))
    const void *kern = pair ? (img > 1 ? IM2WIN_PIPE_FORM(conv_implicit_pair_kernel, true)
                                       : IM2WIN_PIPE_FORM(conv_implicit_pair_kernel, false))
                            : (img > 1 ? IM2WIN_PIPE_FORM(conv_implicit_pipe_kernel, true)
                                       : IM2WIN_PIPE_FORM(conv_implicit_pipe_kernel, false));
#undef IM2WIN_PIPE_FORM
#undef IM2WIN_PIPE_PICK
    return hipLaunchKernel(kern, dim3(groups), dim3(kPipeThreads), args, lds, s);
}

}  // namespace im2win
