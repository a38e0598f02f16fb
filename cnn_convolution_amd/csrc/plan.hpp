// Host planner for the im2win forward convolution (no HIP dependency).
//
// Decides, for a layer descriptor: the output extent, the window-tensor
// layout and its padding, the chunking of window rows that keeps the
// workspace within 1/KW of the im2col buffer, the staged filter, and the
// GEMM tiling. Window rows are r = n*Ho + ho; a window row holds
// W_win = (Wo-1)*stride + KW padded input columns times KH filter rows
// ("Enabling Memory-efficient Im2win Convolution ...", Sec. III-B, Eq. (2)).
#pragma once

#include <algorithm>
#include <cstdint>

#include "im2win_conv2d.h"

namespace im2win {

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

// fp32 vector-ALU window-GEMM: each lane computes kValuMt output channels
// times kValuNt consecutive output columns of one window row.
constexpr int kValuMt = 16;
constexpr int kValuNt = 4;
constexpr int kValuThreads = 256;

// implicit matrix-core convolution: LDS of one workgroup = ns filter stage
// buffers of mb rows x 128 bytes + a patch of ir x iw positions x 128 bytes
inline int64_t implicit_lds_bytes(int64_t mb, int64_t ir, int64_t iw, int64_t ns) {
    return (ns * mb + ir * iw) * 128;
}
constexpr int64_t kImplicitMaxLdsBytes = 160 * 1024;   // one workgroup per CU
constexpr int64_t kImplicitPairLdsBytes = 80 * 1024;   // two workgroups per CU
// row-block implicit form: the filter block (8 KB per tap) + sl input rows of
// iw positions x 128 bytes
// (at least the per-wave store scratch: 8 waves x 16 x 68 floats)
constexpr int64_t kImplicitStoreScratchBytes = 8 * 16 * 68 * 4;
inline int64_t implicit_rows_lds_bytes(int64_t taps, int64_t sl, int64_t iw) {
    return std::max<int64_t>(taps * 8192 + sl * iw * 128, kImplicitStoreScratchBytes);
}
// pipelined row-block implicit form: two slots, each a 32-channel filter
// block (4 KB per tap) + sl input rows of iw positions x 64 bytes, and the
// store scratch of its four computing waves (16 x 68 floats each)
inline int64_t pipe_lds_bytes(int64_t taps, int64_t sl, int64_t iw) {
    return 2 * (taps * 4096 + sl * iw * 64) + 4 * 16 * 68 * 4;
}
// paired row-block implicit form: one such slot, which after the last chunk
// holds the store scratch of its eight waves
inline int64_t pair_lds_bytes(int64_t taps, int64_t sl, int64_t iw) {
    return std::max<int64_t>(taps * 4096 + sl * iw * 64, kImplicitStoreScratchBytes);
}
// split-K row-block implicit form: four K groups (two waves each), each with
// two LDS slots (one when it has a single chunk) of sl input rows of iw
// positions x 64 bytes; after the contraction the same LDS holds the partial
// sums that the groups exchange, two rounds of 12 KB per 16-output block of a
// wave (nbw blocks)
constexpr int64_t kKsplitGroups = 4;
constexpr int64_t kKsplitMaxOuts = 14 * 16;    // two waves of at most 7 blocks
// positions per granule plane of a slot: sl * iw rounded up to 1 modulo 8
inline int64_t ksplit_plane(int64_t sl, int64_t iw) { return ((sl * iw + 6) / 8) * 8 + 1; }
inline int64_t ksplit_lds_bytes(int64_t sl, int64_t iw, int64_t cin, int64_t nbw, int64_t slots = 2) {
    const int64_t spw = cin / (32 * kKsplitGroups) > 1 ? slots : 1;
    return std::max<int64_t>(kKsplitGroups * spw * ksplit_plane(sl, iw) * 64, 12 * nbw * 1024);
}
// blocks per wave as compiled, 4 or 7: the two waves of a K group split a
// task of at most 128 (or 224) outputs (co_split 1), or each takes all of a
// task of at most 64 (or 112) outputs (co_split 2)
inline int64_t ksplit_nbw(int64_t outs, int64_t co_split = 1) {
    return outs <= (co_split == 2 ? 4 : 8) * 16 ? 4 : 7;
}
// the filter staged in fragment order: 64-row output-channel blocks x Cin x taps
inline int64_t ksplit_stage_bytes(int64_t cout, int64_t cin, int64_t taps) {
    return ((cout + 63) / 64) * 64 * cin * taps * 2;
}
// narrow-channel implicit form: the filter block (64 rows of kp elements + 16
// bytes) + r window rows of lp elements, es bytes per element (the window rows'
// space holds at least the store scratch)
// The narrow-channel kernel gathers its filter block from w as stored when
// its launch has at most one workgroup per CU (each gather is paid once per
// workgroup); larger launches read the filter staged in the workspace.
inline bool narrow_gathers_filter(int64_t workgroups) { return workgroups <= 256; }

inline int64_t implicit_narrow_lds_bytes(int64_t es, int64_t kp, int64_t lp, int64_t r) {
    return 64 * (kp + 16 / es) * es + std::max<int64_t>(r * lp * es, kImplicitStoreScratchBytes);
}

// fp32 vector-ALU kernel: output columns per lane for this filter shape.
int valu_cols_per_lane(const conv2d_desc_t &d);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline int64_t elem_size(int32_t dtype) { return dtype == CONV2D_F32 ? 4 : 2; }

inline int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p) {
    const int64_t span = in + 2 * p - k;
    if (s < 1 || k < 1 || p < 0 || span < 0) return 0;
    return span / s + 1;
}

// Validate the descriptor alone (shapes, dtype, element-count limits).
conv2d_status_t check_desc(const conv2d_desc_t &d);

// Geometry of one layout (no chunking): Cin_pad, pos_pad, row_elems.
struct LayoutGeom {
    int64_t Cin_pad, pos_pad, row_elems;
};
LayoutGeom layout_geom(const conv2d_desc_t &d, int32_t layout);

// Staged-filter geometry for one layout: rows and row length (elements).
struct StageGeom {
    int64_t rows, row_len;
    bool needed;   // false when w is already in the staged order
};
StageGeom stage_geom(const conv2d_desc_t &d, int32_t layout, int tile_m);


// Full plan (fills the C struct). Returns CONV2D_OK or a validation error.
conv2d_status_t make_plan(const conv2d_desc_t &d, conv2d_plan_t *p);

// Plan of the implicit form; CONV2D_ERR_UNSUPPORTED when the layer does not
// qualify (fp32, Cin not a multiple of 64, or no tile whose patch fits LDS).
conv2d_status_t make_implicit_plan(const conv2d_desc_t &d, conv2d_implicit_plan_t *p);

}  // namespace im2win
