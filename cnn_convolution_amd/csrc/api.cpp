// C ABI of the im2win forward convolution (declared in include/im2win_conv2d.h).
//
// conv2d_fwd: validate -> plan -> [stage filter] -> for each chunk of window
// rows { pack the chunk (Eq. (2) of the im2win paper) ; window-GEMM the chunk
// into y }. Everything is enqueued on the caller's stream; nothing is
// allocated and nothing synchronises (except conv2d_profile_read).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "im2win_conv2d.h"
#include "launch.hpp"
#include "plan.hpp"

using namespace im2win;

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- profiling hook: event pairs around each launch while enabled ----------
struct Rec {
    hipEvent_t a, b;
    int kind;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};  // read without the mutex by every launch
std::vector<Rec> g_recs;        // recorded since the last read
std::vector<hipEvent_t> g_pool;  // reusable events

hipEvent_t pool_get()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

struct ProfScope {
    hipStream_t s;
    int kind;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(hipStream_t s_, int kind_) : s(s_), kind(kind_)
    {
        if (!g_prof_on.load(std::memory_order_relaxed)) return;
        std::lock_guard<std::mutex> lk(g_prof_mu);
        a = pool_get();
        b = pool_get();
        if (a && b) (void)hipEventRecord(a, s);
    }
    ~ProfScope()
    {
        if (!a || !b) return;
        (void)hipEventRecord(b, s);
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_recs.push_back(Rec{a, b, kind});
    }
};

// y and its epilogue (scale and bias may be null) for the kernels
OutSpec make_out(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, void *y, const float *scale,
                 const float *bias)
{
    OutSpec o{};
    o.y = y;
    o.scale = scale;
    o.bias = bias;
    o.type = d.y_dtype;
    o.nhwc = d.layout == CONV2D_NHWC ? 1 : 0;
    o.plain = (o.type == CONV2D_F32 && !o.nhwc && !scale && !bias) ? 1 : 0;
    o.Cout = int(d.Cout);
    o.plane = Ho * Wo;
    return o;
}

PackArgs pack_args(const conv2d_desc_t &d, const conv2d_plan_t &p, int32_t layout,
                   const LayoutGeom &g, const void *x, void *out, int64_t row0, int64_t rows)
{
    PackArgs a{};
    a.x = x;
    a.out = out;
    a.N = int(d.N);
    a.Cin = int(d.Cin);
    a.H = int(d.H);
    a.W = int(d.W);
    a.KH = int(d.KH);
    a.stride = int(d.stride);
    a.pad = int(d.pad);
    a.Ho = int(p.Ho);
    a.Wwin = int(p.W_win);
    a.Cin_pad = int(g.Cin_pad);
    a.pos_pad = int(g.pos_pad);
    a.row_elems = int(g.row_elems);
    a.row0 = int(row0);
    a.rows = int(rows);
    a.esize = int(elem_size(d.dtype));
    a.nhwc = d.layout == CONV2D_NHWC ? 1 : 0;
    (void)layout;
    return a;
}

hipError_t launch_gemm(const conv2d_desc_t &d, const conv2d_plan_t &p, const LayoutGeom &g,
                       const void *win, const void *wst, const OutSpec &out, int64_t row0, int64_t rows,
                       hipStream_t s)
{
    if (p.path == 0) {
        ValuGemmArgs ga{};
        ga.win = static_cast<const float *>(win);
        ga.wst = static_cast<const float *>(wst);
        ga.out = out;
        ga.rows = int(rows);
        ga.row0 = int(row0);
        ga.Cin = int(d.Cin);
        ga.pos_pad = int(g.pos_pad);
        ga.row_elems = int(g.row_elems);
        ga.KH = int(d.KH);
        ga.KW = int(d.KW);
        ga.stride = int(d.stride);
        ga.Ho = int(p.Ho);
        ga.Wo = int(p.Wo);
        ga.Cout = int(d.Cout);
        ga.Cout_stage = int(p.Cout_stage);
        ga.ksplit = p.gemm_ksplit;
        return launch_gemm_valu_f32(ga, s);
    }
    MfmaGemmArgs ga{};
    ga.win = win;
    ga.wst = wst;
    ga.out = out;
    ga.rows = int(rows);
    ga.row0 = int(row0);
    ga.row_elems = int(g.row_elems);
    ga.col_step = int(d.stride * d.KH * g.Cin_pad);
    ga.krun = int(d.KW * d.KH * g.Cin_pad);
    ga.kstage = int(p.K_stage);
    ga.Ho = int(p.Ho);
    ga.Wo = int(p.Wo);
    ga.Cout = int(d.Cout);
    ga.tile_m = p.gemm_tile_m;
    ga.tile_n = p.gemm_tile_n;
    ga.kb = p.gemm_kslice;
    ga.ks = p.gemm_ksplit;
    ga.wm = p.gemm_wave_m;
    ga.bf16 = d.dtype == CONV2D_BF16 ? 1 : 0;
    ga.ablate = p.gemm_ablate;
    if (p.gemm_kernel == 3) return launch_gemm_mfma_dma(ga, s);
    return launch_gemm_mfma(ga, s);
}

ImplicitArgs implicit_args(const conv2d_desc_t &d, const conv2d_implicit_plan_t &p, const void *x,
                           const void *wst, const OutSpec &out)
{
    ImplicitArgs a{};
    a.x = x;
    a.wst = wst;
    a.out = out;
    a.N = int(d.N);
    a.Cin = int(d.Cin);
    a.H = int(d.H);
    a.W = int(d.W);
    a.Cout = int(d.Cout);
    a.KH = int(d.KH);
    a.KW = int(d.KW);
    a.stride = int(d.stride);
    a.pad = int(d.pad);
    a.Ho = int(p.Ho);
    a.Wo = int(p.Wo);
    a.kstage = int(p.K_stage);
    a.R = p.rows_per_tile;
    a.WB = p.cols_per_tile;
    a.IR = p.patch_rows;
    a.IW = p.patch_cols;
    a.tile_m = p.tile_m;
    a.tile_n = p.tile_n;
    a.wm = p.wave_m;
    a.stages = p.stages;
    a.bf16 = d.dtype == CONV2D_BF16 ? 1 : 0;
    a.f32 = d.dtype == CONV2D_F32 ? 1 : 0;
    a.narrow_cp = p.kernel == 3 ? p.stages : 0;
    // persistent forms: the pipelined row-block kernel's workgroups, the narrow
    // kernel's workgroups per 64-row filter block
    a.groups = p.kernel == 4 ? int(p.tiles) : int(p.tiles / ((d.Cout + 63) / 64));
    a.images = p.kernel == 4 || p.kernel == 5 ? p.images : 0;
    return a;
}

hipError_t launch_implicit(const conv2d_implicit_plan_t &p, const ImplicitArgs &a, hipStream_t s)
{
    if (p.kernel == 2) return launch_conv_implicit_rows(a, s);
    if (p.kernel == 3) return launch_conv_implicit_narrow(a, s);
    if (p.kernel == 4) return launch_conv_implicit_pipe(a, s);
    if (p.kernel == 5) return launch_conv_implicit_ksplit(a, s);
    if (p.kernel == 0) return launch_conv_implicit(a, s);
    return hipErrorInvalidValue;                     // no such kernel
}

// implicit form: (a3) the filter into the window's K order (kw, kh, ci) by a
// staging launch where the plan keeps a staged filter (the streamed kernel,
// and the narrow one on launches of more than one workgroup per CU; the
// others reorder w in LDS themselves), then (a2, a4, a5) in one kernel:
// window rows built in LDS, contracted, y written. Arguments checked by the
// caller.
conv2d_status_t run_implicit(const conv2d_desc_t &d, const conv2d_implicit_plan_t &p, const void *x,
                             const void *w, const OutSpec &out, void *ws, hipStream_t s)
{
    const void *wst = w;
    if (p.kernel == 5) {
        // the split-K kernel reads the filter in its fragment order
        ProfScope ps(s, CONV2D_KERNEL_WEIGHT_STAGE);
        if (launch_ksplit_stage(w, ws, int(d.Cout), int(d.Cin), int(d.KH * d.KW), s) != hipSuccess)
            return CONV2D_ERR_HIP;
        wst = ws;
    } else if (p.ws_bytes > 0) {
        const LayoutGeom g = layout_geom(d, IM2WIN_LAYOUT_CL);
        const StageGeom sg = stage_geom(d, IM2WIN_LAYOUT_CL, p.tile_m);
        StageArgs sa{};
        sa.w = w;
        sa.out = ws;
        sa.Cout = int(d.Cout);
        sa.Cin = int(d.Cin);
        sa.KH = int(d.KH);
        sa.KW = int(d.KW);
        // the narrow-channel kernel: CP channels per position, rows of Kp
        sa.Cin_pad = p.kernel == 3 ? p.stages : int(g.Cin_pad);
        sa.rows = int(sg.rows);
        sa.row_len = p.kernel == 3 ? int(p.K_stage) : int(sg.row_len);
        sa.esize = int(elem_size(d.dtype));
        ProfScope ps(s, CONV2D_KERNEL_WEIGHT_STAGE);
        if (launch_stage_cl(sa, s) != hipSuccess) return CONV2D_ERR_HIP;
        wst = ws;
    }
    ProfScope ps(s, CONV2D_KERNEL_IMPLICIT);
    return launch_implicit(p, implicit_args(d, p, x, wst, out), s) == hipSuccess ? CONV2D_OK
                                                                                 : CONV2D_ERR_HIP;
}

bool aligned_or_null(const void *p, uintptr_t a) { return !p || aligned(p, a); }

// conv2d_fwd and conv2d_fwd_ex: validate -> plan -> the planned form
conv2d_status_t fwd_impl(const conv2d_desc_t *d, const void *x, const void *w, const float *scale,
                         const float *bias, void *y, void *ws, void *stream);

}  // namespace

extern "C" {

size_t conv2d_workspace_size(const conv2d_desc_t *d)
{
    if (!d) return 0;
    conv2d_plan_t p;
    if (make_plan(*d, &p) != CONV2D_OK) return 0;
    return size_t(p.ws_bytes);
}

conv2d_status_t conv2d_plan(const conv2d_desc_t *d, conv2d_plan_t *out)
{
    if (!d || !out) return CONV2D_ERR_NULL_POINTER;
    return make_plan(*d, out);
}

const char *conv2d_status_string(conv2d_status_t s)
{
    switch (s) {
    case CONV2D_OK: return "ok";
    case CONV2D_ERR_INVALID_DESC: return "invalid descriptor";
    case CONV2D_ERR_NULL_POINTER: return "null pointer";
    case CONV2D_ERR_MISALIGNED: return "misaligned pointer";
    case CONV2D_ERR_UNSUPPORTED: return "unsupported dtype or layout";
    case CONV2D_ERR_WORKSPACE: return "workspace missing";
    case CONV2D_ERR_HIP: return "HIP runtime error";
    case CONV2D_ERR_RANGE: return "row range out of bounds";
    case CONV2D_ERR_SCRATCH: return "workspace exceeds the static scratch of conv2d_fwd_noalloc";
    }
    return "unknown status";
}

conv2d_status_t conv2d_fwd(const conv2d_desc_t *d, const void *x, const void *w, void *y,
                           void *ws, void *stream)
{
    return fwd_impl(d, x, w, nullptr, nullptr, y, ws, stream);
}

conv2d_status_t conv2d_fwd_ex(const conv2d_desc_t *d, const void *x, const void *w, const float *scale,
                              const float *bias, void *y, void *ws, void *stream)
{
    return fwd_impl(d, x, w, scale, bias, y, ws, stream);
}

}  // extern "C"

namespace {

conv2d_status_t fwd_impl(const conv2d_desc_t *d, const void *x, const void *w, const float *scale,
                         const float *bias, void *y, void *ws, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_plan_t p;
    const conv2d_status_t st = make_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (!x || !w || !y) return CONV2D_ERR_NULL_POINTER;
    if (p.ws_bytes > 0 && !ws) return CONV2D_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return CONV2D_ERR_MISALIGNED;
    if (ws && !aligned(ws, 256)) return CONV2D_ERR_MISALIGNED;
    if (!aligned_or_null(scale, 4) || !aligned_or_null(bias, 4)) return CONV2D_ERR_MISALIGNED;
    const OutSpec out = make_out(*d, p.Ho, p.Wo, y, scale, bias);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.algo == 1) {
        conv2d_implicit_plan_t ip;
        if (make_implicit_plan(*d, &ip) != CONV2D_OK) return CONV2D_ERR_UNSUPPORTED;
        return run_implicit(*d, ip, x, w, out, ws, s);
    }
    char *wsb = static_cast<char *>(ws);
    const LayoutGeom g = layout_geom(*d, p.layout);
    const StageGeom sg = stage_geom(*d, p.layout, p.gemm_tile_m);
    const int es = int(elem_size(d->dtype));
    hipError_t e = hipSuccess;

    // (a3) filter into the window's K order: carried by the first pack
    // launch when its form allows, else a launch of its own before the
    // first GEMM
    const void *wst = w;
    StageArgs sa{};
    if (sg.needed) {
        sa.w = w;
        sa.out = wsb;
        sa.Cout = int(d->Cout);
        sa.Cin = int(d->Cin);
        sa.KH = int(d->KH);
        sa.KW = int(d->KW);
        sa.Cin_pad = int(g.Cin_pad);
        sa.rows = int(sg.rows);
        sa.row_len = int(sg.row_len);
        sa.esize = es;
        sa.ohwi = d->layout == CONV2D_NHWC ? 1 : 0;
        wst = wsb;
    }
    void *win = wsb + p.win_offset_bytes;

    for (int64_t c = 0; c < p.n_chunks; ++c) {
        const int64_t row0 = c * p.rows_per_chunk;
        const int64_t rows = std::min<int64_t>(p.rows_per_chunk, p.rows_total - row0);
        // (a2) window rows of this chunk
        const PackArgs pa = pack_args(*d, p, p.layout, g, x, win, row0, rows);
        const StageArgs *fold = (c == 0 && sg.needed) ? &sa : nullptr;
        bool folded = false;
        {
            ProfScope ps(s, CONV2D_KERNEL_PACK);
            e = p.layout == IM2WIN_LAYOUT_ROW ? launch_pack_row(pa, s, fold, &folded)
                                              : launch_pack_cl(pa, s, fold, &folded);
        }
        if (e != hipSuccess) return CONV2D_ERR_HIP;
        if (fold && !folded) {
            ProfScope ps(s, CONV2D_KERNEL_WEIGHT_STAGE);
            e = p.layout == IM2WIN_LAYOUT_ROW ? launch_stage_row(sa, s) : launch_stage_cl(sa, s);
            if (e != hipSuccess) return CONV2D_ERR_HIP;
        }
        // (a4, a5) window-GEMM of the chunk, fp32 result written into y
        {
            ProfScope ps(s, CONV2D_KERNEL_GEMM);
            e = launch_gemm(*d, p, g, win, wst, out, row0, rows, s);
        }
        if (e != hipSuccess) return CONV2D_ERR_HIP;
    }
    return CONV2D_OK;
}

}  // namespace

extern "C" {

conv2d_status_t im2win_pack(const conv2d_desc_t *d, int32_t layout, const void *x, void *out,
                            int64_t row0, int64_t rows, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_plan_t p;
    const conv2d_status_t st = make_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (layout != IM2WIN_LAYOUT_ROW && layout != IM2WIN_LAYOUT_CL) return CONV2D_ERR_UNSUPPORTED;
    if (layout == IM2WIN_LAYOUT_CL && d->dtype == CONV2D_F32) return CONV2D_ERR_UNSUPPORTED;
    if (layout == IM2WIN_LAYOUT_ROW && d->layout == CONV2D_NHWC) return CONV2D_ERR_UNSUPPORTED;
    if (row0 < 0 || rows < 1 || row0 + rows > p.rows_total) return CONV2D_ERR_RANGE;
    if (!x || !out) return CONV2D_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(out, 16)) return CONV2D_ERR_MISALIGNED;
    const LayoutGeom g = layout_geom(*d, layout);
    if (rows * g.row_elems > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    const PackArgs pa = pack_args(*d, p, layout, g, x, out, row0, rows);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = layout == IM2WIN_LAYOUT_ROW ? launch_pack_row(pa, s) : launch_pack_cl(pa, s);
    return e == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

conv2d_status_t im2win_weight_stage(const conv2d_desc_t *d, int32_t layout, const void *w,
                                    void *out, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_plan_t p;
    const conv2d_status_t st = make_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (layout != IM2WIN_LAYOUT_ROW && layout != IM2WIN_LAYOUT_CL && layout != IM2WIN_LAYOUT_FRAG)
        return CONV2D_ERR_UNSUPPORTED;
    if (layout == IM2WIN_LAYOUT_ROW && d->layout == CONV2D_NHWC) return CONV2D_ERR_UNSUPPORTED;
    const int64_t taps = d->KH * d->KW;
    if (layout == IM2WIN_LAYOUT_FRAG &&
        (d->dtype == CONV2D_F32 || d->layout == CONV2D_NHWC || d->Cin % 32 != 0 ||
         !(taps == 1 || (d->KH == 3 && d->KW == 3) || (d->KH == 5 && d->KW == 5))))
        return CONV2D_ERR_UNSUPPORTED;
    if (!w || !out) return CONV2D_ERR_NULL_POINTER;
    if (!aligned(w, 16) || !aligned(out, 16)) return CONV2D_ERR_MISALIGNED;
    if (layout == IM2WIN_LAYOUT_FRAG)
        return launch_ksplit_stage(w, out, int(d->Cout), int(d->Cin), int(taps), static_cast<hipStream_t>(stream)) ==
                       hipSuccess
                   ? CONV2D_OK
                   : CONV2D_ERR_HIP;
    const LayoutGeom g = layout_geom(*d, layout);
    const StageGeom sg = stage_geom(*d, layout, p.gemm_tile_m);
    StageArgs sa{};
    sa.w = w;
    sa.out = out;
    sa.Cout = int(d->Cout);
    sa.Cin = int(d->Cin);
    sa.KH = int(d->KH);
    sa.KW = int(d->KW);
    sa.Cin_pad = int(g.Cin_pad);
    sa.rows = int(sg.rows);
    sa.row_len = int(sg.row_len);
    sa.esize = int(elem_size(d->dtype));
    sa.ohwi = d->layout == CONV2D_NHWC ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = layout == IM2WIN_LAYOUT_ROW ? launch_stage_row(sa, s) : launch_stage_cl(sa, s);
    return e == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

conv2d_status_t im2win_window_gemm(const conv2d_desc_t *d, const void *win, const void *wst,
                                   void *y, int64_t row0, int64_t rows, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_plan_t p;
    const conv2d_status_t st = make_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (row0 < 0 || rows < 1 || row0 + rows > p.rows_total) return CONV2D_ERR_RANGE;
    if (!win || !wst || !y) return CONV2D_ERR_NULL_POINTER;
    if (!aligned(win, 16) || !aligned(wst, 16) || !aligned(y, 16)) return CONV2D_ERR_MISALIGNED;
    const LayoutGeom g = layout_geom(*d, p.layout);
    if (rows * g.row_elems > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope ps(s, CONV2D_KERNEL_GEMM);
    const hipError_t e = launch_gemm(*d, p, g, win, wst, make_out(*d, p.Ho, p.Wo, y, nullptr, nullptr), row0,
                                     rows, s);
    return e == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

conv2d_status_t conv2d_implicit_plan(const conv2d_desc_t *d, conv2d_implicit_plan_t *out)
{
    if (!d || !out) return CONV2D_ERR_NULL_POINTER;
    return make_implicit_plan(*d, out);
}

size_t conv2d_implicit_workspace_size(const conv2d_desc_t *d)
{
    if (!d) return 0;
    conv2d_implicit_plan_t p;
    if (make_implicit_plan(*d, &p) != CONV2D_OK) return 0;
    return size_t(p.ws_bytes);
}

conv2d_status_t conv2d_fwd_implicit(const conv2d_desc_t *d, const void *x, const void *w,
                                    void *y, void *ws, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_implicit_plan_t p;
    const conv2d_status_t st = make_implicit_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (!x || !w || !y) return CONV2D_ERR_NULL_POINTER;
    if (p.ws_bytes > 0 && !ws) return CONV2D_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return CONV2D_ERR_MISALIGNED;
    if (ws && !aligned(ws, 256)) return CONV2D_ERR_MISALIGNED;
    return run_implicit(*d, p, x, w, make_out(*d, p.Ho, p.Wo, y, nullptr, nullptr), ws,
                        static_cast<hipStream_t>(stream));
}

conv2d_status_t im2win_implicit_gemm(const conv2d_desc_t *d, const void *x, const void *wst,
                                     void *y, void *stream)
{
    if (!d) return CONV2D_ERR_NULL_POINTER;
    conv2d_implicit_plan_t p;
    const conv2d_status_t st = make_implicit_plan(*d, &p);
    if (st != CONV2D_OK) return st;
    if (!x || !wst || !y) return CONV2D_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(wst, 16) || !aligned(y, 16)) return CONV2D_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope ps(s, CONV2D_KERNEL_IMPLICIT);
    return launch_implicit(p, implicit_args(*d, p, x, wst, make_out(*d, p.Ho, p.Wo, y, nullptr, nullptr)), s) ==
                   hipSuccess
               ? CONV2D_OK
               : CONV2D_ERR_HIP;
}

conv2d_status_t conv2d_profile_enable(int32_t on)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(on != 0, std::memory_order_relaxed);
    return CONV2D_OK;
}

conv2d_status_t conv2d_profile_read(conv2d_profile_t *out)
{
    if (!out) return CONV2D_ERR_NULL_POINTER;
    std::memset(out, 0, sizeof(*out));
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_recs);
    }
    conv2d_status_t st = CONV2D_OK;
    for (const Rec &r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            st = CONV2D_ERR_HIP;
        else if (r.kind >= 0 && r.kind < CONV2D_KERNEL_KINDS) {
            out->launches[r.kind] += 1;
            out->total_ms[r.kind] += ms;
        }
    }
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (const Rec &r : recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    return st;
}

}  // extern "C"
