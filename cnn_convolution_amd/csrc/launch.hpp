// Host-side launchers of the HIP kernels (one per kernel family). Plain
// pointers and sizes only; every launcher enqueues on `stream` and returns
// hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace im2win {

// Output of every convolution kernel: y = scale[co] * (conv + bias[co]) (each
// factor optional), rounded once to the storage type of y, at its NCHW or
// NHWC offset. `plain` marks fp32 NCHW y with neither factor, the kernels'
// own fp32 store path.
struct OutSpec {
    void *y;
    const float *scale;     // [Cout] or nullptr (a factor of 1)
    const float *bias;      // [Cout] or nullptr (no bias)
    int type;               // 0 fp32, 1 fp16, 2 bf16
    int nhwc;               // 1: y [N][Ho][Wo][Cout]; 0: y [N][Cout][Ho][Wo]
    int plain;              // type 0, NCHW, no scale, no bias
    int Cout;
    int64_t plane;          // Ho * Wo
};

struct PackArgs {
    const void *x;          // NCHW input
    void *out;              // window rows [rows][row_elems]
    int N, Cin, H, W, KH, stride, pad, Ho, Wwin;
    int Cin_pad, pos_pad, row_elems;
    int row0, rows;         // window rows r in [row0, row0 + rows)
    int esize;              // 2 or 4 bytes
    int nhwc;               // x is [N][H][W][Cin] (channels-last window layout only)
};
struct StageArgs;
// A pack launch can carry the filter staging along, as extra workgroups
// ahead of the pack's own: pass `fold`; *folded tells whether it was taken
// (the tiled channels-last form, for rows too long to stage, does not).
hipError_t launch_pack_row(const PackArgs &a, hipStream_t s, const StageArgs *fold = nullptr,
                           bool *folded = nullptr);
hipError_t launch_pack_cl(const PackArgs &a, hipStream_t s, const StageArgs *fold = nullptr,
                          bool *folded = nullptr);

struct StageArgs {
    const void *w;          // [Cout][Cin][KH][KW]
    void *out;
    int Cout, Cin, KH, KW;
    int Cin_pad, rows, row_len;  // staged geometry
    int esize;
    int ohwi;               // w is [Cout][KH][KW][Cin] (channels-last order only)
};
hipError_t launch_stage_row(const StageArgs &a, hipStream_t s);
hipError_t launch_stage_cl(const StageArgs &a, hipStream_t s);

struct ValuGemmArgs {
    const float *win;       // window chunk [rows][Cin][pos_pad]
    const float *wst;       // staged filter [Cout_stage/16][Cin][KH][KW][16]
    OutSpec out;            // y and its epilogue
    int rows, row0, Cin, pos_pad, row_elems;
    int KH, KW, stride;
    int Ho, Wo, Cout, Cout_stage;
    int ksplit;             // waves of a workgroup splitting the channels (1, 2 or 4)
};
hipError_t launch_gemm_valu_f32(const ValuGemmArgs &a, hipStream_t s);

struct MfmaGemmArgs {
    const void *win;        // window chunk [rows][row_elems] (channels-last)
    const void *wst;        // staged filter [Cout][K_stage]
    OutSpec out;            // y and its epilogue
    int rows, row0, row_elems;
    int col_step;           // stride*KH*Cin_pad: window start step between columns
    int krun;               // KW*KH*Cin_pad: window length
    int kstage;             // staged filter row length (multiple of the K slice)
    int Ho, Wo, Cout;
    int tile_m, tile_n;     // output tile
    int kb, ks;             // K per wave group per LDS stage; wave groups splitting K
    int wm;                 // waves along M in a wave group (4 / wm along N)
    int bf16;               // 0: fp16, 1: bf16
    int ablate;             // direct-to-LDS kernel: ablation bits (0: as planned)
};
hipError_t launch_gemm_mfma(const MfmaGemmArgs &a, hipStream_t s);
// direct-to-LDS form: tile_m x tile_n with wm waves along M, K stages of 64;
// only for windows whose length krun equals kstage, a multiple of 64
hipError_t launch_gemm_mfma_dma(const MfmaGemmArgs &a, hipStream_t s);

// implicit form: window rows built in LDS straight from NCHW x (no window
// tensor); tile_m x tile_n output tile over R window rows x WB columns of
// one image, a patch of IR x IW input positions per 64-channel block
struct ImplicitArgs {
    const void *x;          // NCHW input
    const void *wst;        // staged filter [Cout][kstage], K order (kw, kh, ci)
    OutSpec out;            // y and its epilogue
    int N, Cin, H, W, Cout, KH, KW, stride, pad, Ho, Wo;
    int kstage;             // KW*KH*Cin
    int R, WB, IR, IW;
    int tile_m, tile_n, wm;
    int stages;             // filter stage buffers (3, 4 or 5)
    int bf16;
    int f32;                // fp32 x, w (row-block and narrow kernels)
    int narrow_cp;          // narrow kernel: channels per window position (4 or 8)
    int groups;             // persistent forms (narrow, pipelined row-block): workgroups
    int images;             // pipelined row-block form: whole images per task (0 or 1: row tasks)
};
hipError_t launch_conv_implicit(const ImplicitArgs &a, hipStream_t s);
// row-block form (fp16/bf16: Cin = 64, W % 8 == 0; fp32: Cin % 32 == 0,
// W % 4 == 0; stride 1, Wo <= 64, 1x1 or 3x3): R whole output rows of one
// image per workgroup, raw filter and input rows resident in LDS; wst is w
// itself
hipError_t launch_conv_implicit_rows(const ImplicitArgs &a, hipStream_t s);
// narrow-channel form (Cin <= 8, any filter and stride, Wo <= 512): R output
// rows of one image per workgroup, their channels-last window rows and the
// filter in LDS; wst is w itself
hipError_t launch_conv_implicit_narrow(const ImplicitArgs &a, hipStream_t s);
// pipelined row-block form (fp16/bf16, Cin % 32 == 0, stride 1, R * Wo <=
// 256, 1x1 or 3x3): `groups` persistent workgroups over tasks of R whole
// output rows x 64 output channels, 32-channel K chunks double-buffered in
// LDS by four loader waves while four waves contract; wst is w itself
hipError_t launch_conv_implicit_pipe(const ImplicitArgs &a, hipStream_t s);
// split-K row-block form (fp16/bf16, Cin % 128 == 0, stride 1 or 2, 3x3, 5x5
// or 1x1, images * R * Wo <= 208): one task of R whole output rows (or of
// `images` whole images) x 64 output channels per workgroup, the four waves
// splitting the input channels; wst is the filter in fragment order
// (launch_ksplit_stage)
hipError_t launch_conv_implicit_ksplit(const ImplicitArgs &a, hipStream_t s);
// w [Cout][Cin][taps] (fp16/bf16) -> wf in the split-K kernel's fragment
// order, ksplit_stage_bytes(Cout, Cin, taps) bytes (Cin % 32 == 0)
hipError_t launch_ksplit_stage(const void *w, void *wf, int Cout, int Cin, int taps, hipStream_t s);

}  // namespace im2win
