// Output blocks of the implicit kernels that take whole output rows per
// workgroup (row-block and narrow-channel forms): the workgroup's outputs,
// flattened row-major, are cut into 16-output MFMA blocks shared over eight
// waves, and a block's results are stored as 16-byte vectors of 4
// consecutive outputs of one output channel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "epilogue.hpp"
#include "lds_dma.hpp"

namespace im2win {

// The rw x Wo outputs of a workgroup, flattened (i * Wo + wo, which is also
// their order inside each output plane), are cut into MFMA blocks of 16 and
// shared out over the workgroup's computing waves (eight, or four in the
// pipelined kernel) in contiguous ranges of at most 4 blocks.
// Lane l of a block works on output m = 16 * block + l % 16 (clamped to the
// last output: such lanes read a valid window and store nothing).
__device__ __forceinline__ void wave_blocks_of(int wave, int waves, int outs, int &b0, int &nb)
{
    const int total = (outs + 15) >> 4;
    b0 = wave * total / waves;
    nb = (wave + 1) * total / waves - b0;
}

__device__ __forceinline__ void wave_blocks(int wave, int outs, int &b0, int &nb)
{
    wave_blocks_of(wave, 8, outs, b0, nb);
}

// Patch position of the window at tap (0, 0) of each of a lane's output
// blocks (output m = i * Wo + wo: input row i, column wo of a patch of rows
// IW positions long; stride 1).
__device__ __forceinline__ void block_bases(int *qa, int b0, int lane, int outs, int Wo, int IW)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int m = min((b0 + s) * 16 + (lane & 15), outs - 1);
        const int i = m / Wo;
        qa[s] = i * IW + (m - i * Wo);
    }
}

// THROUGH: output lines (128 bytes) that one workgroup writes whole are
// stored at device scope (sc1). Each XCD's L2 keeps ordinary stores dirty
// until the kernel ends and then writes them all back, a tail the whole chip
// waits for; device-scope stores go through to memory as they are issued, in
// the shadow of the other waves' work. A line shared with a neighbouring
// workgroup keeps the ordinary store: written through in pieces from two
// XCDs it costs more than the tail. Measured on the ResNet 3x3 layer (fp16 x,
// fp32 y): 14.1 us with ordinary stores; 12.1 us with 8-row blocks, whose
// plane segments are whole lines, written through; 13.85 us with 7-row
// blocks written through regardless of lines. The same stores from the
// LDS-staged path measured slower (deep 3x3 layer 25.2 -> 27.0 us, the 1x1
// layer 42.0 -> 46.5 us), so only the direct stores of the row-block and
// narrow-channel kernels take it.
//
// The store is a buffer store with the sc1 cache policy from a wave-uniform
// base, written with the compiler's builtin rather than as inline asm, so
// that the compiler keeps the wait rules around it: a store of more than 8
// bytes reads its data registers after it issues (a vector-ALU write to them
// needs a wait state), and the data comes straight from matrix-core
// accumulators (a vector-memory read of them needs wait states after the
// product). An earlier inline-asm form kept neither, and now and then
// stored whatever the next instruction had put into the data registers.
constexpr int kCachePolicySc1 = 16;                  // buffer-store cache policy: sc1
constexpr int kBufferWord3 = 0x00020000;             // raw-buffer descriptor word 3 on gfx9

__device__ __forceinline__ void store16_through(void *base, uint32_t off, const floatx4_t &v)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, -1, kBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(off), 0, kCachePolicySc1);
}

// Whether the 128-byte line holding byte address p lies inside [lo, hi).
__device__ __forceinline__ bool whole_line(const void *p, uintptr_t lo, uintptr_t hi)
{
    const uintptr_t l = reinterpret_cast<uintptr_t>(p) & ~uintptr_t(127);
    return l >= lo && l + 128 <= hi;
}

// Lane l holds D[4*(l/16) + v][l % 16] of each 16 x 16 block: 4 consecutive
// outputs m of output channel co = block column l % 16, which are 4
// consecutive elements of the plane (one 16-byte fp32 or 8-byte half store
// when Wo % 4 == 0 and y is NCHW). acc holds MAXB blocks, nb <= MAXB of them
// in use. Outputs through the epilogue of o (y type, scale, bias, layout).
template <int MAXB = 4, bool THROUGH = false>
__device__ __forceinline__ void store_blocks(const floatx4_t (*acc)[4], int nb, int b0, int lane,
                                             const OutSpec &o, int n, int Cout, int cb, int Ho, int Wo,
                                             int ho0, int outs)
{
    const int64_t plane = int64_t(Ho) * Wo;
    if (o.plain) {
        float *const y = static_cast<float *>(o.y);
        // the write-through stores address the workgroup's 64 channel planes
        // from one wave-uniform base with 32-bit byte offsets
        float *const yw = y + (int64_t(n) * Cout + cb * 64) * plane + int64_t(ho0) * Wo;
        const bool through = THROUGH && 64 * plane * 4 < (int64_t(1) << 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int co = cb * 64 + c * 16 + (lane & 15);
            if (co >= Cout) continue;
            float *yb = y + (int64_t(n) * Cout + co) * plane + int64_t(ho0) * Wo;
            const int64_t cbase = int64_t(c * 16 + (lane & 15)) * plane;   // yb - yw, in floats
            // this workgroup's segment of the channel's plane
            const uintptr_t lo = reinterpret_cast<uintptr_t>(yb);
            const uintptr_t hi = reinterpret_cast<uintptr_t>(yb + outs);
#pragma unroll
            for (int s = 0; s < MAXB; ++s) {
                if (s >= nb) break;
                const int m = (b0 + s) * 16 + (lane >> 4) * 4;
                if ((Wo & 3) == 0) {
                    if (m < outs) {
                        if (through && whole_line(yb + m, lo, hi))
                            store16_through(yw, uint32_t((cbase + m) * 4), acc[s][c]);
                        else
                            *reinterpret_cast<floatx4_t *>(yb + m) = acc[s][c];
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (m + v < outs) yb[m + v] = acc[s][c][v];
                }
            }
        }
        return;
    }
    with_ytype(o, [&](auto tc) {
        constexpr int T = decltype(tc)::value;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int co = cb * 64 + c * 16 + (lane & 15);
            if (co >= Cout) continue;
            const ChanEpi e = chan_epi(o, co);
#pragma unroll
            for (int s = 0; s < MAXB; ++s) {
                if (s >= nb) break;
                const int m = (b0 + s) * 16 + (lane >> 4) * 4;
                const int64_t p = int64_t(ho0) * Wo + m;
                if ((Wo & 3) == 0 && !o.nhwc) {
                    if (m < outs)
                        put4<T>(o.y, out_offset(o, n, co, p), epi_apply(e, acc[s][c][0]), epi_apply(e, acc[s][c][1]),
                                epi_apply(e, acc[s][c][2]), epi_apply(e, acc[s][c][3]));
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (m + v < outs) put1<T>(o.y, out_offset(o, n, co, p + v), epi_apply(e, acc[s][c][v]));
                }
            }
        }
    });
}

// Per-wave LDS scratch of store_blocks_lds: 16 rows (output channels) of 64
// outputs, each row 4 floats longer so that the 16 rows fall in different
// bank groups.
constexpr int kStoreRow = 68;
constexpr int kStoreScratchFloats = 16 * kStoreRow;

// The same stores for any Wo, through a per-wave LDS scratch of
// kStoreScratchFloats floats: one 16-channel block at a time, a lane's 4
// outputs are written to the scratch row of its channel, then read back one
// channel row per instruction, so that each store instruction writes up to 64
// consecutive floats of one output plane (the wave's outputs are consecutive
// in every plane). For rows whose length is not a multiple of 4, where the
// 16-byte stores of store_blocks do not apply. LDS operations of one wave
// complete in order, so no barrier is needed between the 4 blocks.
template <int MAXB = 4>
__device__ __forceinline__ void store_blocks_lds(const floatx4_t (*acc)[4], int nb, int b0, int lane,
                                                 float *scratch, const OutSpec &o, int n, int Cout, int cb,
                                                 int Ho, int Wo, int ho0, int outs)
{
    const int64_t plane = int64_t(Ho) * Wo;
    const int nout = min(nb * 16, outs - b0 * 16);   // this wave's outputs
    const int64_t p0 = int64_t(ho0) * Wo + b0 * 16;   // their first position in the plane
    float *const srow = scratch + (lane & 15) * kStoreRow + 4 * (lane >> 4);
    with_ytype(o, [&](auto tc) {
        constexpr int T = decltype(tc)::value;
        // NCHW y with whole 4-output groups: lane (row group lane / 16, column
        // quad lane % 16) reads 4 consecutive outputs of a channel row and
        // stores them as one vector (16 bytes fp32, 8 bytes half), so that each
        // store instruction writes 4 channels x 64 consecutive outputs (whole
        // 128-byte lines) instead of one channel row of 4-byte pieces
        // (measured: deep 3x3 layer 29 -> 27 us, the 1x1 layer 47 -> 45 us)
        const bool quads = !o.nhwc && (p0 & 3) == 0 && (nout & 3) == 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int s = 0; s < MAXB; ++s)
                if (s < nb) *reinterpret_cast<floatx4_t *>(srow + s * 16) = acc[s][c];
            if (quads) {
                const int col = 4 * (lane & 15);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = (lane >> 4) + 4 * j;
                    const int co = cb * 64 + c * 16 + r;
                    if (co < Cout && col < nout) {
                        const floatx4_t v = *reinterpret_cast<const floatx4_t *>(scratch + r * kStoreRow + col);
                        const ChanEpi e = chan_epi(o, co);
                        put4<T>(o.y, (int64_t(n) * Cout + co) * plane + p0 + col, epi_apply(e, v[0]),
                                epi_apply(e, v[1]), epi_apply(e, v[2]), epi_apply(e, v[3]));
                    }
                }
                continue;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = cb * 64 + c * 16 + r;
                const float v = scratch[r * kStoreRow + lane];
                if (co < Cout && lane < nout) {
                    if (o.plain)
                        static_cast<float *>(o.y)[(int64_t(n) * Cout + co) * plane + p0 + lane] = v;
                    else
                        out_store<T>(o, n, co, p0 + lane, v);
                }
            }
        }
    });
}

}  // namespace im2win
