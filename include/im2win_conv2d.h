/*
 * im2win forward 2-D convolution for AMD Instinct MI355X (gfx950) -- C ABI.
 *
 * The operation (every entry point below serves it):
 *
 *   Ho = floor((H + 2*pad - KH) / stride) + 1,  Wo = floor((W + 2*pad - KW) / stride) + 1
 *   y[n][co][ho][wo] = sum_{ci, kh, kw} xp[n][ci][ho*stride + kh - pad][wo*stride + kw - pad]
 *                                       * w[co][ci][kh][kw]
 *
 * with xp = x zero-padded by `pad` on all four sides: a cross-correlation (no
 * kernel flip), one stride and one padding for both axes, no dilation or
 * groups. conv2d_fwd_ex adds the epilogue y = scale[co] * (conv + bias[co]).
 * Sources: "Enabling Memory-efficient Im2win Convolution with
 * Multi-precision Support on GPU CUDA and Tensor Cores", Sec. III-A Eq. (1)
 * (the sum), Sec. III-B Eq. (2) (the window tensor), Sec. III-C Eq. (3) and
 * Sec. III-D with Algorithm 1 (the window contraction as a GEMM with
 * M = Cout, N = N*Ho*Wo, K = Cin*KH*KW); the padded output extent of
 * "Unifying Convolutions and GEMM", Sec. 5.
 *
 * How it runs: conv2d_fwd takes, per layer, one of two forms of the same
 * method (conv2d_plan_t.algo names which):
 *   - the implicit form (every measured layer): one kernel builds the window
 *     rows of each output tile in LDS straight from x (the rows of Eq. (2))
 *     and contracts them against the filter on the matrix cores with fp32
 *     accumulation (fp32 inputs on the matrix cores' fp32 products); the
 *     workspace is at most a staged copy of the filter, often none;
 *   - the window form: the input is repacked, one chunk of window rows
 *     (n, ho) at a time, into the im2win window tensor held in the caller's
 *     workspace, the filter is restaged once per call into the window's K
 *     order, and a window-GEMM kernel contracts each chunk into y (fp32 on the
 *     vector ALUs, fp16/bf16 on the matrix cores). The chunk size keeps the
 *     workspace at most 1/KW of the im2col buffer whenever one window row fits
 *     in that budget.
 *
 * Layouts (conv2d_desc_t.layout): dense and contiguous,
 *   CONV2D_NCHW (default): x [N][Cin][H][W], w [Cout][Cin][KH][KW], y [N][Cout][Ho][Wo];
 *   CONV2D_NHWC          : x [N][H][W][Cin], w [Cout][KH][KW][Cin], y [N][Ho][Wo][Cout]
 *                          (fp16/bf16 inputs only; channels innermost, the input
 *                          layout of the tensor-core design of Sec. III-D).
 * x and w are of `dtype`; y of `y_dtype` (fp32 by default, whatever `dtype`).
 *
 * Pointers: x, w, y, ws and the pack/stage outputs are DEVICE pointers the
 * caller allocates and owns. The library allocates no device memory and
 * keeps no state between calls (apart from the optional profiling records
 * below). `stream` is a hipStream_t passed as void*; NULL means the default
 * stream. All GPU work is enqueued on `stream` and the calls return without
 * synchronising; results are valid once the stream's work completes.
 *
 * Errors: every entry point validates its arguments before enqueueing any
 * work; on an error nothing is launched and no output is touched. No entry
 * point aborts or exits. Every buffer must hold fewer than 2^31 elements.
 *
 * Thread safety: all entry points are reentrant; calls that share a
 * workspace must be ordered by the caller (same stream, or events). Plans
 * are cached per descriptor and per set of IM2WIN_* environment overrides
 * (a bounded cache behind a mutex), so repeated calls skip the planner.
 */
#ifndef IM2WIN_CONV2D_H
#define IM2WIN_CONV2D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of x and w (conv2d_desc_t.dtype) and of y (y_dtype). */
typedef enum {
    CONV2D_F32 = 0,   /* IEEE binary32; fp32 products on the matrix cores (row-
                         block and narrow kernels) or the vector ALUs           */
    CONV2D_F16 = 1,   /* IEEE binary16; matrix cores, fp32 accumulation        */
    CONV2D_BF16 = 2   /* bfloat16; matrix cores, fp32 accumulation             */
} conv2d_dtype_t;

/* Memory layout of x, w and y. */
typedef enum { CONV2D_NCHW = 0, CONV2D_NHWC = 1 } conv2d_layout_t;

/* The layer. All sizes in elements. A zero-initialised tail (y_dtype, layout,
 * reserved) is the plain convolution: fp32 NCHW output. */
typedef struct {
    int64_t N, Cin, H, W;     /* input batch, channels, height, width          */
    int64_t Cout, KH, KW;     /* filters, filter height, filter width          */
    int64_t stride, pad;      /* one stride and one zero padding for both axes */
    int32_t dtype;            /* a conv2d_dtype_t: storage type of x and w     */
    int32_t y_dtype;          /* a conv2d_dtype_t: storage type of y; the fp32
                                 result is rounded once, to nearest even       */
    int32_t layout;           /* a conv2d_layout_t (NHWC: fp16/bf16 only)      */
    int32_t reserved;         /* must be 0                                     */
} conv2d_desc_t;

typedef enum {
    CONV2D_OK = 0,
    CONV2D_ERR_INVALID_DESC = 1,  /* a size < 1 (pad < 0), no output, reserved != 0,
                                     or a buffer of 2^31 elements or more            */
    CONV2D_ERR_NULL_POINTER = 2,  /* a required pointer is NULL                     */
    CONV2D_ERR_MISALIGNED = 3,    /* x, w, y or an output not 16-byte aligned;
                                     ws not 256-byte aligned                        */
    CONV2D_ERR_UNSUPPORTED = 4,   /* unknown dtype, y_dtype or layout; NHWC with fp32
                                     inputs; a form that does not take the layer     */
    CONV2D_ERR_WORKSPACE = 5,     /* ws NULL although a workspace is needed         */
    CONV2D_ERR_HIP = 6,           /* the HIP runtime reported an error on launch    */
    CONV2D_ERR_RANGE = 7,         /* a row range outside [0, N*Ho)                  */
    CONV2D_ERR_SCRATCH = 8        /* conv2d_fwd_noalloc: the planned form needs more
                                     workspace than IM2WIN_NOALLOC_SCRATCH_BYTES    */
} conv2d_status_t;

/* Storage orders of the window tensor (Eq. (2) of the im2win paper, with r =
 * n*Ho + ho a window row, pos = w*KH + kh, w < W_win = (Wo-1)*stride + KW a
 * padded input column, and the value xp[n][ci][ho*stride + kh][w]):
 *   ROW : T[r][ci][pos]   channel outermost, the paper's order; the window of
 *         output column wo is the run pos in [wo*stride*KH, (wo*stride+KW)*KH)
 *         of each channel. Used by the fp32 path.
 *   CL  : T[r][pos][ci]   channels innermost; the window of column wo is ONE
 *         contiguous run of KW*KH*Cin_pad elements. Used by the fp16/bf16
 *         path. Cin is zero-padded to Cin_pad (see conv2d_plan_t). */
typedef enum { IM2WIN_LAYOUT_ROW = 0, IM2WIN_LAYOUT_CL = 1, IM2WIN_LAYOUT_FRAG = 2 } im2win_layout_t;
/* IM2WIN_LAYOUT_FRAG names no window tensor: it is the order of the staged
 * filter of the split-K implicit kernel (conv2d_implicit_plan_t.kernel 5),
 * for im2win_weight_stage only (see there). */

/* What conv2d_fwd will do for a descriptor (host-side only, no GPU needed). */
typedef struct {
    int64_t Ho, Wo, W_win;        /* output extent; padded columns per window row */
    int32_t path;                 /* 0: fp32 vector ALU, 1: fp16/bf16 matrix core  */
    int32_t layout;               /* an im2win_layout_t                           */
    int64_t Cin_pad;              /* channels stored per position (CL) or Cin     */
    int64_t pos_pad;              /* ROW: positions stored per channel: a multiple of 8,
                                     at least W_win*KH + 3 (spare, zero)          */
    int64_t row_elems;            /* elements of one window row in the workspace  */
    int64_t rows_total;           /* N*Ho                                         */
    int64_t rows_per_chunk;       /* window rows packed and contracted per chunk  */
    int64_t n_chunks;
    int64_t K;                    /* Cin*KH*KW                                    */
    int64_t K_stage;              /* staged filter row length (K order, padded)   */
    int64_t Cout_stage;           /* staged filter rows (Cout padded)             */
    int64_t wstage_bytes;         /* staged filter, at the start of ws            */
    int64_t win_offset_bytes;     /* where the window chunk starts in ws          */
    int64_t win_chunk_bytes;      /* window chunk buffer                          */
    int64_t ws_bytes;             /* workspace of conv2d_fwd = conv2d_workspace_size():
                                     staged filter + window chunk (algo 0), or what
                                     conv2d_implicit_workspace_size reports (algo 1) */
    int64_t im2col_bytes;         /* N*Ho*Wo*Cin*KH*KW*sizeof(dtype)              */
    int64_t ws_target_bytes;      /* im2col_bytes / KW                            */
    int32_t meets_ws_target;      /* ws_bytes <= ws_target_bytes                  */
    int32_t gemm_tile_m, gemm_tile_n;  /* output tile of one workgroup (M x N)     */
    int32_t gemm_kslice;          /* K per LDS stage per wave group (kernels 1, 3) */
    int32_t gemm_ksplit;          /* wave groups splitting K inside a workgroup    */
    int32_t gemm_kernel;          /* 0: vector ALU, 1: matrix core via LDS tiles,
                                     3: matrix core, tiles copied memory -> LDS
                                        directly (whole 64-element K stages);
                                     (2 is not used)                                */
    int32_t gemm_wave_m;          /* waves along M in a wave group (matrix path)   */
    int32_t algo;                 /* what conv2d_fwd runs: 0 the window tensor in ws
                                     (pack + window-GEMM per chunk), 1 the implicit
                                     form (conv2d_fwd_implicit)                     */
    int32_t gemm_ablate;          /* gemm_kernel 3 only, for measuring the page's
                                     optimisations one by one (0 as planned; set
                                     from IM2WIN_ABLATE): bit 0 no serpentine tile
                                     order, bit 1 no direct-to-LDS copies (through
                                     registers), bit 2 one stage buffer instead of
                                     three                                          */
    int32_t reserved2;            /* 0                                              */
    int64_t flops;                /* 2*N*Cout*Ho*Wo*Cin*KH*KW (padded taps included) */
} conv2d_plan_t;

/* Bytes of workspace conv2d_fwd needs for *d (0 if d is invalid). */
size_t conv2d_workspace_size(const conv2d_desc_t *d);

/* Fill *out with the plan for *d. Host only; never touches a GPU. */
conv2d_status_t conv2d_plan(const conv2d_desc_t *d, conv2d_plan_t *out);

/* y = conv2d(x, w) as defined at the top of this file, by the form the plan
 * names (conv2d_plan_t.algo): the window tensor in ws, or the implicit form
 * below where it measured faster for that layer class.
 * ws: device buffer of at least conv2d_workspace_size(d) bytes, 256-byte
 * aligned (NULL allowed only when that size is 0); its contents on return
 * are unspecified. The staged filter and the window chunk inside it start on
 * 256-byte boundaries of ws, so every window row and filter row the kernels
 * copy straight into LDS starts 16-byte aligned whatever the chunk's rows;
 * PyTorch's device allocations are 512-byte aligned. x, w, y: 16-byte
 * aligned device pointers. Errors: CONV2D_ERR_HIP when a launch fails (the
 * runtime refused it, or the kernel's own launch check did); launches of
 * earlier steps of the same call may then have been enqueued. */
conv2d_status_t conv2d_fwd(const conv2d_desc_t *d, const void *x, const void *w, void *y,
                           void *ws, void *stream);

/* y = scale[co] * (conv2d(x, w) + bias[co]), the same call with the
 * epilogue of a convolution layer: a per-output-channel bias (the bias
 * argument of the convolution of "Unifying Convolutions and GEMM", Sec. 5)
 * and a per-output-channel scale folded into the output pass (the scale
 * folding of "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
 * Reformulation": s * (X * W + b) = X * (s W) + s b, so the scale needs no
 * pass of its own). Both are applied to the fp32 accumulator in the kernel
 * that stores y, before the single rounding to y_dtype. scale, bias: fp32
 * [Cout] device arrays, 4-byte aligned, or NULL (scale 1, bias 0); owned by
 * the caller. Other arguments and errors as conv2d_fwd. */
conv2d_status_t conv2d_fwd_ex(const conv2d_desc_t *d, const void *x, const void *w, const float *scale,
                              const float *bias, void *y, void *ws, void *stream);

/* Row (a2) on its own: write window rows [row0, row0 + rows) of the window
 * tensor of x (Eq. (2) of the im2win paper, zero padding included) in the
 * given layout to `out`, with the row length, Cin_pad and pos_pad that
 * conv2d_plan reports for that layout. A pure copy: every value is bit-equal
 * to an element of x or zero. out must hold rows * row_elems elements of
 * dtype and be 16-byte aligned. x in the descriptor's layout (NHWC: the
 * channels-last window layout only). */
conv2d_status_t im2win_pack(const conv2d_desc_t *d, int32_t layout, const void *x, void *out,
                            int64_t row0, int64_t rows, void *stream);

/* Row (a3) on its own: restage w into the K order of the window of `layout`:
 *   ROW : out[cb][ci][kh][kw][j] = w[cb*16 + j][ci][kh][kw], j < 16, Cout padded
 *         to a multiple of 16 with zeros (fp32 path);
 *   CL  : out[co][(kw*KH + kh)*Cin_pad + ci] = w[co][ci][kh][kw], rows padded to
 *         Cout_stage and to K_stage with zeros (w[co][kh][kw][ci] for NHWC).
 *         out holds Cout_stage * K_stage elements of dtype;
 *   FRAG: the matrix-core fragment order of the split-K implicit kernel
 *         (fp16/bf16, NCHW, Cin % 32 == 0, 1x1, 3x3 or 5x5 filters): with
 *         taps t = kh*KW + kw, fragment (cb, blk, t, c4) is 64 lanes x 8
 *         elements, lane l holding w[cb*64 + c4*16 + (l % 16)][blk*32 +
 *         (l / 16)*8 + e][t], e < 8 (zero past Cout), fragments in the order
 *         ((cb*Cin/32 + blk)*taps + t)*4 + c4; out holds ceil(Cout/64)*64 *
 *         Cin * taps elements (conv2d_implicit_workspace_size(d) bytes when
 *         the plan's kernel is 5).
 * out is 16-byte aligned. CONV2D_ERR_UNSUPPORTED for a layout the layer does
 * not take. */
conv2d_status_t im2win_weight_stage(const conv2d_desc_t *d, int32_t layout, const void *w,
                                    void *out, void *stream);

/* Rows (a4, a5) on their own: the window-GEMM of window rows
 * [row0, row0 + rows), writing y[n][co][ho][wo] for those rows (r = n*Ho + ho)
 * and leaving the rest of y untouched. `win` holds exactly those rows in the
 * layout conv2d_plan reports for d (as im2win_pack writes them, row length
 * row_elems); `wst` holds the staged filter of that layout (as
 * im2win_weight_stage writes it; for a 1x1 filter whose plan has
 * wstage_bytes == 0, w itself). fp32 accumulation; y of the descriptor's
 * y_dtype and layout, no bias or scale.
 * ("Enabling Memory-efficient Im2win Convolution ...", Sec. III-C Eq. (3),
 * Sec. III-D Algorithm 1.) Device pointers, 16-byte aligned. */
conv2d_status_t im2win_window_gemm(const conv2d_desc_t *d, const void *win, const void *wst,
                                   void *y, int64_t row0, int64_t rows, void *stream);

const char *conv2d_status_string(conv2d_status_t s);

/* ---- allocation-free entry point ----------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * y = conv2d(x, w) as conv2d_fwd, with the workspace of the planned form taken
 * from a static device array of IM2WIN_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends (its address on a device is
 * looked up on the first call there, with that device current). Calls no
 * hipMalloc, hipFree or allocating library routine. x, w, y as conv2d_fwd.
 * Returns CONV2D_ERR_SCRATCH, and launches nothing, when the plan's
 * workspace (conv2d_workspace_size) exceeds the array. All calls on one GPU
 * share its array: calls that overlap on one GPU (several streams or host
 * threads) race on it and must be ordered by the caller. */
#define IM2WIN_NOALLOC_SCRATCH_BYTES (32u << 20)
conv2d_status_t conv2d_fwd_noalloc(const conv2d_desc_t *d, const void *x, const void *w, void *y,
                                   void *stream);

/* ---- implicit (fused) form ---------------------------------------------
 * The same y = conv2d(x, w), with the window rows built in LDS straight
 * from x instead of going through a window tensor in the workspace: each
 * output tile (tile_m output channels x cols_per_tile columns of
 * rows_per_tile window rows (n, ho) of one image) holds, per block of 64
 * input channels, the input rows its window rows interleave (Eq. (2) of the
 * im2win paper: window row ho = input rows ho*stride - pad .. + KH - 1) as a
 * channels-innermost patch, and contracts it against the staged filter in
 * the window's K order (Sec. III-C Eq. (3), Sec. III-D). Matrix cores with
 * fp32 accumulation, fp32 y: fp16/bf16 with Cin a multiple of 64 (or of 32
 * for 3x3 and 1x1 filters of stride 1 or 2), up to 8 input channels in any dtype,
 * fp32 on the row-block kernel's layers. The workspace holds only the staged
 * filter (none for a 1x1 filter or for the row-block kernels). */
typedef struct {
    int32_t tile_m, tile_n;       /* output channels x GEMM columns per workgroup  */
    int32_t wave_m;               /* waves along M                                 */
    int32_t rows_per_tile;        /* window rows (n, ho) of one image per tile      */
    int32_t cols_per_tile;        /* output columns wo per tile                     */
    int32_t patch_rows;           /* input rows held per tile: (rows-1)*stride + KH */
    int32_t patch_cols;           /* input columns held: (cols-1)*stride + KW       */
    int32_t kernel;               /* 0: the filter streamed through LDS per K stage,
                                     one workgroup per tile; (1 is not used);
                                     2 (default where it applies: Cin = 64,
                                     stride 1, W % 8 == 0, Wo <= 64, 3x3 or 1x1):
                                     row-block, rows_per_tile whole output rows
                                     of one image per workgroup with w as stored
                                     and the input rows resident in LDS, no
                                     staged filter (ws_bytes 0); 3: narrow-channel
                                     (Cin <= 8), the filter block gathered from w
                                     as stored into LDS when tiles <= 256
                                     (ws_bytes 0), else read from the staged
                                     filter; 4 (default for the other 3x3 and
                                     1x1 layers of stride 1 or 2 with Cin % 32 ==
                                     0 and Wo <= 256): pipelined row-block, tasks of
                                     rows_per_tile whole output rows (or of
                                     `images` whole images) x 64 output channels
                                     over 32-channel K chunks double-buffered in
                                     LDS, w as stored (ws_bytes 0); 5 (default
                                     for 5x5 filters and stride 2 with Cin %
                                     128 == 0, else by name): split-K
                                     row-block, tasks of rows_per_tile whole
                                     output rows (or of `images` whole images)
                                     x tile_m output channels, four K groups of
                                     two waves splitting the input channels
                                     (tile_m 64: the two waves split the task's
                                     outputs, at most 224; tile_m 128: they
                                     take 64 channels each, at most 112
                                     outputs), the filter staged in the
                                     workspace in fragment order
                                     (IM2WIN_LAYOUT_FRAG)                           */
    int32_t stages;               /* kernel 0: filter K stages in flight + 1 (LDS
                                     stage buffers); kernel 3: channels per window
                                     position; kernel 4: 2 = persistent workgroups
                                     (tiles of them) with loading and computing
                                     waves, 1 = one task per workgroup (tiles
                                     tasks), two workgroups per CU; kernel 5: LDS
                                     slots per K group (2, or 1 where two do not
                                     fit); 0 otherwise                              */
    int32_t images;               /* kernels 4, 5: whole images per task when > 1 (then
                                     rows_per_tile = Ho and patch_rows = images *
                                     (Ho + KH - 1)); 1 otherwise, 0 for the other
                                     kernels                                        */
    int64_t lds_bytes;            /* LDS per workgroup                              */
    int64_t tiles;                /* workgroups of the launch                       */
    int64_t Ho, Wo;
    int64_t K_stage;              /* staged filter row: KW*KH*Cin (kernel 3: the
                                     filter's LDS row, KW*KH*CP rounded up to the
                                     matrix-core K step)                            */
    int64_t ws_bytes;             /* the staged filter of kernel 0 (0 for a 1x1
                                     filter), of kernel 3 when tiles > 256 and of
                                     kernel 5 (fragment order); 0 for kernels 2
                                     and 4                                          */
    int64_t flops;                /* 2*N*Cout*Ho*Wo*Cin*KH*KW                        */
} conv2d_implicit_plan_t;

/* Fill *out for *d. CONV2D_ERR_UNSUPPORTED when the implicit form does not
 * take the layer (NHWC, fp32 outside the row-block and narrow kernels' layers,
 * Cin past 8 and not a multiple of 64 outside the pipelined row-block
 * kernel's layers, or no tile whose patch fits in LDS); other errors as
 * conv2d_plan. Host only. */
conv2d_status_t conv2d_implicit_plan(const conv2d_desc_t *d, conv2d_implicit_plan_t *out);

/* Bytes of workspace conv2d_fwd_implicit needs (0 if d is invalid or not
 * supported, for a 1x1 filter, for the row-block and pipelined kernels, and
 * for the narrow-channel kernel on launches of at most 256 workgroups). */
size_t conv2d_implicit_workspace_size(const conv2d_desc_t *d);

/* y = conv2d(x, w) by the implicit form. Arguments, alignment, ownership and
 * asynchrony as conv2d_fwd; ws of at least conv2d_implicit_workspace_size(d)
 * bytes (NULL allowed when that is 0). Returns CONV2D_ERR_UNSUPPORTED, and
 * launches nothing, for a layer conv2d_implicit_plan does not take. */
conv2d_status_t conv2d_fwd_implicit(const conv2d_desc_t *d, const void *x, const void *w,
                                    void *y, void *ws, void *stream);

/* Rows (a2, a4, a5) of the implicit form on their own: the implicit kernel
 * with a filter already staged in the window's K order (as
 * im2win_weight_stage writes it for IM2WIN_LAYOUT_CL; for IM2WIN_LAYOUT_FRAG
 * when the plan's kernel is 5, so that a caller whose filter does not change
 * stages it once), or w itself where the plan keeps no staged filter
 * (conv2d_implicit_workspace_size(d) == 0: a 1x1 filter outside kernel 5, or
 * the row-block, pipelined and small narrow-channel launches, which reorder w
 * in LDS on their own),
 * writing all of y (y_dtype of the descriptor, no bias or scale). Device
 * pointers, 16-byte aligned. */
conv2d_status_t im2win_implicit_gemm(const conv2d_desc_t *d, const void *x, const void *wst,
                                     void *y, void *stream);

/* ---- measurement hook --------------------------------------------------
 * While enabled, conv2d_fwd and conv2d_fwd_implicit record a HIP event pair
 * around every kernel they launch (on the call's stream). conv2d_profile_read
 * synchronises on the recorded events, returns per-kernel totals since the
 * last read, and clears them. Not for concurrent use from several threads. */
typedef enum {
    CONV2D_KERNEL_WEIGHT_STAGE = 0,
    CONV2D_KERNEL_PACK = 1,
    CONV2D_KERNEL_GEMM = 2,
    CONV2D_KERNEL_IMPLICIT = 3,   /* the implicit form's convolution kernel        */
    CONV2D_KERNEL_KINDS = 4
} conv2d_kernel_kind_t;

typedef struct {
    int64_t launches[CONV2D_KERNEL_KINDS];
    double total_ms[CONV2D_KERNEL_KINDS];
} conv2d_profile_t;

conv2d_status_t conv2d_profile_enable(int32_t on);
conv2d_status_t conv2d_profile_read(conv2d_profile_t *out);

#ifdef __cplusplus
}
#endif

#endif /* IM2WIN_CONV2D_H */
