// Patches of the pipelined and split-K row-block kernels: the chunk-wise
// construction of a task's window rows in LDS straight from NCHW x.
//
// A task is a block of RW whole output rows (n, ho0 .. ho0+RW-1) of one image
// (or of IMG whole images) and 64 output channels. The window rows of those
// output rows (Eq. (2) of "Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores", Sec. III-B) share all
// but their first and last input rows, so a task holds the union once, SL =
// (RW - 1) * s + KH input rows of IW = W + 2*pad positions, channels
// innermost, one K chunk of 32 input channels at a time: 64 bytes per
// position (16-byte granule g of row q in slot g ^ ((q >> 1) & 3)). The
// window of output (i, wo) at tap (kh, kw) is position (i * s + kh, wo * s +
// kw) for stride s.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"

namespace im2win {
namespace {

constexpr int kChunkC = 32;       // input channels per K chunk (64 bytes per position)

struct PipeKArgs {
    const uint16_t *x;
    const uint16_t *w;
    OutSpec out;            // y and its epilogue
    int Cin, H, W, Cout, pad, Ho, Wo;
    int RW;             // output rows per task
    int row_groups;     // ceil(Ho / RW)
    int co_blocks;      // ceil(Cout / 64)
    int IW;             // W + 2*pad
    int ntasks;         // co_blocks * N * row_groups, or co_blocks * ceil(N / IMG)
    int SLmax;          // patch rows: RW + KH - 1, or IMG * (Ho + KH - 1)
    int slot_halves;    // one LDS slot: filter block + SLmax * IW * 32
    int N;
    int IMG;            // 1: tasks of RW output rows of one image; > 1: tasks of
                        // IMG whole images (RW = Ho), their patches stacked
    int stride;
    int slots;          // split-K kernel: LDS slots per K group (1 or 2)
    int co_split;       // split-K kernel: 1, the two waves of a K group take
                        // halves of the task's outputs; 2, one 64-channel half
                        // each of a task of 128 output channels
};

// LDS slot of 16-byte granule g (0..3) of 64-byte row q. A 16-byte LDS read
// serves 8 consecutive lanes per cycle without conflict when their addresses
// fall in 8 different 16-byte slots of a 128-byte window: 8 consecutive rows
// read at one granule are 4 even and 4 odd rows (the two halves of the
// window), and within each parity (q >> 1) & 3 takes 4 different values.
__device__ __forceinline__ int gslot(int g, int q)
{
    return g ^ ((q >> 1) & 3);
}

__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// V consecutive halves of one channel plane: a 16-byte, 8-byte or 2-byte load
template <int V> struct PlaneVec;
template <> struct PlaneVec<8> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ uint32_t dw(int d) const { return dword_of(v, d); }
};
template <> struct PlaneVec<4> {
    uint2 v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ uint32_t dw(int d) const { return d == 0 ? v.x : v.y; }
};
template <> struct PlaneVec<1> {
    uint32_t v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *p; }
    __device__ __forceinline__ uint32_t dw(int) const { return v; }
};

// 8 channels x V positions -> the 8 channels of position j (16 bytes)
template <int V>
__device__ __forceinline__ uint4 position_of(const PlaneVec<V> *raw, int j)
{
    if constexpr (V == 1) {
        return uint4{raw[0].v | (raw[1].v << 16), raw[2].v | (raw[3].v << 16),
                     raw[4].v | (raw[5].v << 16), raw[6].v | (raw[7].v << 16)};
    } else {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        return uint4{__builtin_amdgcn_perm(raw[1].dw(j >> 1), raw[0].dw(j >> 1), sel),
                     __builtin_amdgcn_perm(raw[3].dw(j >> 1), raw[2].dw(j >> 1), sel),
                     __builtin_amdgcn_perm(raw[5].dw(j >> 1), raw[4].dw(j >> 1), sel),
                     __builtin_amdgcn_perm(raw[7].dw(j >> 1), raw[6].dw(j >> 1), sel)};
    }
}

// A task: 64 output channels (block cb) of rw output rows from ho0 of nimg
// consecutive images from n (nimg > 1 only for whole images); image j's
// patch is rows j*SL .. j*SL + SL - 1 of the task's patch.
struct PipeTask {
    int cb, n, nimg, ho0, rw, ih0, SL;
};

// MI: the launch takes tasks of several whole images (a.IMG > 1); the
// kernels are compiled apart for it, so that row tasks pay nothing for it
template <int KH, bool MI>
__device__ __forceinline__ PipeTask pipe_task(const PipeKArgs &a, int t)
{
    PipeTask k;
    k.cb = t % a.co_blocks;
    const int r = t / a.co_blocks;
    if constexpr (MI) {
        k.n = r * a.IMG;
        k.nimg = min(a.IMG, a.N - k.n);
        k.ho0 = 0;
        k.rw = a.Ho;
    } else {
        const int rg = r % a.row_groups;
        k.n = r / a.row_groups;
        k.nimg = 1;
        k.ho0 = rg * a.RW;
        k.rw = min(a.RW, a.Ho - k.ho0);
    }
    k.ih0 = k.ho0 * a.stride - a.pad;
    k.SL = (k.rw - 1) * a.stride + KH;
    return k;
}

// Patch loads of one K chunk of a task: the task's input rows that lie in
// the image are a contiguous run [p_lo, p_hi) of every channel plane; unit u
// is (image u / units1 of the task, then 8-channel granule u1 & 3 and V
// positions from flat index (j_lo + u1/4) * V, u1 = u mod units1).
struct ChunkGeom {
    int p_lo, p_hi, j_lo, units1, units;
};

template <int V, bool MI>
__device__ __forceinline__ ChunkGeom chunk_geom(const PipeKArgs &a, const PipeTask &tk)
{
    ChunkGeom g;
    // rows [r_lo, r_hi) of the image; both clamped into [0, H], so a task that
    // lies wholly in the padding below the image (pad > KH) gets the empty run
    // [H*W, H*W), which is a whole number of V-position units (H*W % V == 0):
    // no unit is loaded
    const int r_lo = min(max(tk.ih0, 0), a.H);
    const int r_hi = max(min(tk.ih0 + tk.SL, a.H), r_lo);
    g.p_lo = r_lo * a.W;
    g.p_hi = r_hi * a.W;
    g.j_lo = g.p_lo / V;
    g.units1 = 4 * ((g.p_hi + V - 1) / V - g.j_lo);
    g.units = MI ? g.units1 * tk.nimg : g.units1;
    return g;
}

template <int V, bool MI>
__device__ __forceinline__ void load_patch_unit(const PipeKArgs &a, const PipeTask &tk, int blk,
                                                const ChunkGeom &cg, int u, PlaneVec<V> *raw)
{
    const int HW = a.H * a.W;
    const int im = MI ? u / cg.units1 : 0, u1 = u - im * cg.units1;
    const int g = u1 & 3, j = cg.j_lo + (u1 >> 2);
    const uint16_t *src =
        a.x + (int64_t(tk.n + im) * a.Cin + blk * kChunkC + g * 8) * HW + int64_t(j) * V;
#pragma unroll
    for (int e = 0; e < 8; ++e) raw[e].load(src + int64_t(e) * HW);
}

// the unit's positions inside [p_lo, p_hi), 8 channels each, into the patch
template <int V, bool MI>
__device__ __forceinline__ void put_patch_unit(uint16_t *patch, const PipeKArgs &a, const PipeTask &tk,
                                               const ChunkGeom &cg, int u, const PlaneVec<V> *raw)
{
    const int im = MI ? u / cg.units1 : 0, u1 = u - im * cg.units1;
    const int g = u1 & 3;
    const int p0 = (cg.j_lo + (u1 >> 2)) * V;
    const int row0 = im * tk.SL - tk.ih0;            // patch row of input row 0 of this image
    int r = p0 / a.W;
    int col = p0 - r * a.W;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int p = p0 + v;
        if (p >= cg.p_lo && p < cg.p_hi) {
            const int q = (row0 + r) * a.IW + a.pad + col;
            *reinterpret_cast<uint4 *>(patch + q * kChunkC + (gslot(g, q) << 3)) = position_of<V>(raw, v);
        }
        if (++col == a.W) { col = 0; ++r; }
    }
}

// rows of the task outside the image: zeros, in every image's patch (thread
// t0 of nt)
template <bool MI>
__device__ __forceinline__ void zero_rows(uint16_t *patch, const PipeKArgs &a, const PipeTask &tk, int t0, int nt)
{
    const int top = min(max(-tk.ih0, 0), tk.SL);
    const int bot0 = max(min(a.H - tk.ih0, tk.SL), top);
    const int zrows = top + (tk.SL - bot0);
    const int per = zrows * a.IW * 4;
    for (int v = t0; v < (MI ? per * tk.nimg : per); v += nt) {
        const int im = MI ? v / per : 0, w = v - im * per;
        const int g = w & 3, e = w >> 2;
        const int zr = e / a.IW, col = e - zr * a.IW;
        const int i = zr < top ? zr : bot0 + (zr - top);
        const int q = (im * tk.SL + i) * a.IW + col;
        *reinterpret_cast<uint4 *>(patch + q * kChunkC + (gslot(g, q) << 3)) = uint4{0u, 0u, 0u, 0u};
    }
}

// zero the padding columns (positions < pad and >= pad + W) of rows 0 .. SL-1
__device__ __forceinline__ void zero_pad_columns(uint16_t *patch, const PipeKArgs &a, int SL, int t0, int nt)
{
    const int n = SL * 2 * a.pad * 4;
    for (int v = t0; v < n; v += nt) {
        const int g = v & 3, e = v >> 2;
        const int i = e / (2 * a.pad), c = e - i * 2 * a.pad;
        const int q = i * a.IW + (c < a.pad ? c : a.W + c);
        *reinterpret_cast<uint4 *>(patch + q * kChunkC + (gslot(g, q) << 3)) = uint4{0u, 0u, 0u, 0u};
    }
}

// logical workgroup index, contiguous per XCD (workgroups are dispatched
// round-robin over the 8 XCDs): consecutive tasks, which share input rows
// (the 64-channel blocks of one row block) and neighbouring rows, run on one
// XCD and its L2
__device__ __forceinline__ int xcd_logical(int b, int G)
{
    const int per = G >> 3, rem = G & 7, x = b & 7;
    return x * per + min(x, rem) + (b >> 3);
}


}  // namespace
}  // namespace im2win
