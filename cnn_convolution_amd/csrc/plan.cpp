// Host planner: see plan.hpp.
#include "plan.hpp"

#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

namespace im2win {

conv2d_status_t check_desc(const conv2d_desc_t &d) {
    if (d.dtype != CONV2D_F32 && d.dtype != CONV2D_F16 && d.dtype != CONV2D_BF16)
        return CONV2D_ERR_UNSUPPORTED;
    if (d.y_dtype != CONV2D_F32 && d.y_dtype != CONV2D_F16 && d.y_dtype != CONV2D_BF16)
        return CONV2D_ERR_UNSUPPORTED;
    if (d.layout != CONV2D_NCHW && d.layout != CONV2D_NHWC) return CONV2D_ERR_UNSUPPORTED;
    // NHWC runs the channels-last window form only, which is half precision
    if (d.layout == CONV2D_NHWC && d.dtype == CONV2D_F32) return CONV2D_ERR_UNSUPPORTED;
    if (d.reserved != 0) return CONV2D_ERR_INVALID_DESC;
    if (d.N < 1 || d.Cin < 1 || d.H < 1 || d.W < 1 || d.Cout < 1 || d.KH < 1 || d.KW < 1 ||
        d.stride < 1 || d.pad < 0)
        return CONV2D_ERR_INVALID_DESC;
    // keep every product below well under int64 overflow before multiplying
    const int64_t lim = int64_t(1) << 20;
    if (d.N > lim || d.Cin > lim || d.H > lim || d.W > lim || d.Cout > lim || d.KH > lim ||
        d.KW > lim || d.stride > lim || d.pad > lim)
        return CONV2D_ERR_INVALID_DESC;
    const int64_t Ho = out_extent(d.H, d.KH, d.stride, d.pad);
    const int64_t Wo = out_extent(d.W, d.KW, d.stride, d.pad);
    if (Ho < 1 || Wo < 1) return CONV2D_ERR_INVALID_DESC;
    if (d.N * d.Cin * d.H * d.W > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    if (d.Cout * d.Cin * d.KH * d.KW > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    if (d.N * d.Cout * Ho * Wo > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    return CONV2D_OK;
}

LayoutGeom layout_geom(const conv2d_desc_t &d, int32_t layout) {
    const int64_t Wo = out_extent(d.W, d.KW, d.stride, d.pad);
    const int64_t Wwin = (Wo - 1) * d.stride + d.KW;
    LayoutGeom g{};
    if (layout == IM2WIN_LAYOUT_ROW) {
        // each channel's run of W_win*KH positions, padded to 8 elements so
        // every channel (and every row) starts 16-byte aligned, with at least
        // 3 spare elements: the fp32 kernel loads a lane's window run in whole
        // 16-byte vectors, and the last one may reach 3 elements past it
        g.Cin_pad = d.Cin;
        g.pos_pad = round_up(Wwin * d.KH + 3, 8);
        g.row_elems = d.Cin * g.pos_pad;
    } else {
        // channels innermost, padded so that every window start
        // (wo*stride*KH*Cin_pad) and every 8-element group is 16-byte aligned
        const bool four = d.Cin <= 4 && (d.stride * d.KH) % 2 == 0;
        g.Cin_pad = four ? 4 : round_up(d.Cin, 8);
        g.pos_pad = Wwin * d.KH;
        // a window whose length is 4 mod 8 ends in a half vector: the kernel
        // loads that vector whole, so the row keeps 4 spare elements after it
        const int64_t krun = d.KW * d.KH * g.Cin_pad;
        g.row_elems = round_up(Wwin * d.KH * g.Cin_pad + (krun % 8 ? 4 : 0), 8);
    }
    return g;
}

static int64_t mfma_kgran(int64_t krun);

StageGeom stage_geom(const conv2d_desc_t &d, int32_t layout, int tile_m) {
    (void)tile_m;
    StageGeom s{};
    if (layout == IM2WIN_LAYOUT_ROW) {
        s.rows = round_up(d.Cout, kValuMt);
        s.row_len = d.Cin * d.KH * d.KW;
        s.needed = true;
    } else {
        const LayoutGeom g = layout_geom(d, layout);
        const int64_t krun = d.KW * d.KH * g.Cin_pad;
        s.rows = d.Cout;
        s.row_len = round_up(krun, mfma_kgran(krun));
        // a 1x1 filter whose channel count needs no padding already is [Cout][K]
        s.needed = !(d.KH == 1 && d.KW == 1 && g.Cin_pad == d.Cin && s.row_len == d.Cin);
    }
    return s;
}

// Matrix-core tiles the kernel is compiled for: {MB, NB, KB, KS}.
static const int kMfmaTiles[][5] = {
    {64, 64, 64, 1, 2},   {64, 64, 32, 1, 2},   {64, 64, 32, 2, 2},   {64, 128, 64, 1, 2},
    {64, 128, 32, 1, 2},  {64, 128, 32, 2, 2},  {128, 64, 64, 1, 2},  {128, 64, 32, 1, 2},
    {128, 64, 32, 2, 2},  {128, 128, 64, 1, 2}, {128, 128, 32, 1, 2}, {128, 128, 32, 2, 2},
    {64, 128, 64, 1, 1},  {64, 256, 64, 1, 1},  {64, 256, 32, 1, 1},  {128, 256, 64, 1, 2},
    {128, 128, 64, 1, 1},
};

static bool mfma_tile_known(int m, int n, int kb, int ks, int wm) {
    for (const auto &t : kMfmaTiles)
        if (t[0] == m && t[1] == n && t[2] == kb && t[3] == ks && t[4] == wm) return true;
    return false;
}

// K granularity of the staged filter: 64 unless that pads more than 32 would.
static int64_t mfma_kgran(int64_t krun) { return round_up(krun, 64) == round_up(krun, 32) ? 64 : 32; }

// Tile for one chunk of `cols` output columns: enough workgroups to cover the
// 256 CUs a few times over, the largest tile that still does.
static void pick_mfma_tile(const conv2d_desc_t &d, int64_t cols, int64_t kgran, conv2d_plan_t *p) {
    // Measured on MI355X over the layer sweep (ResNet-style 3x3, 7x7 stem,
    // deep 3x3, 5x5, 3x3 stride 2, 512-channel 7x7, 1x1): the kernel is bound
    // by the latency of its LDS and memory round trips, so the choice is about
    // keeping enough independent waves per CU rather than about reuse.
    const int64_t t64 = ceil_div(d.Cout, 64) * ceil_div(cols, 64);   // 64x64 output tiles
    int m, n, kb, ks, wm;
    if (d.Cout <= 64) {
        // one M block; wide N tiles, all four waves along N
        if (kgran == 64) { m = 64; n = 128; kb = 64; ks = 1; wm = 1; }
        else             { m = 64; n = 64;  kb = 32; ks = 1; wm = 2; }
    } else if (t64 >= 4096) {
        m = 128; n = 128; kb = 64; ks = 1; wm = 2;    // plenty of tiles (large N*Ho*Wo)
    } else if (t64 >= 700) {
        m = 128; n = 128; kb = 64; ks = 1; wm = 1;
    } else if (d.Cout >= 512 || t64 < 200) {
        m = 64; n = 64; kb = 32; ks = 2; wm = 2;      // few tiles, deep K: split K in the workgroup
    } else {
        m = 128; n = 64; kb = 32; ks = 2; wm = 2;
    }
    // developer override for tile sweeps: IM2WIN_MFMA_TILE="MB,NB,KB,KS[,WM]"
    if (const char *e = std::getenv("IM2WIN_MFMA_TILE")) {
        int a = 0, b = 0, c = 0, k = 0, w = 2;
        const int got = std::sscanf(e, "%d,%d,%d,%d,%d", &a, &b, &c, &k, &w);
        if (got >= 4 && mfma_tile_known(a, b, c, k, w) && p->K_stage % (c * k) == 0) {
            p->gemm_tile_m = a; p->gemm_tile_n = b; p->gemm_kslice = c; p->gemm_ksplit = k;
            p->gemm_wave_m = w;
            return;
        }
    }
    if (!mfma_tile_known(m, n, kb, ks, wm) || p->K_stage % (kb * ks) != 0) {
        m = 64; n = 64; kb = 32; ks = 1; wm = 2;   // always compiled, K_stage is a multiple of 32
    }
    p->gemm_tile_m = m;
    p->gemm_tile_n = n;
    p->gemm_kslice = kb;
    p->gemm_ksplit = ks;
    p->gemm_wave_m = wm;
}

// Direct-to-LDS matrix-core form: whole 64-element K stages (the window
// length equals the staged filter row, a multiple of 64). Taken wherever it
// applies: it measured faster than the tiled kernel on the layers of the
// sweep. Tile rule from the same sweep: one 64-row block when Cout <= 64 (128
// columns, or 64 when that leaves fewer tiles than CUs); 64 x 64 for Cout >=
// 256 with a deep K; else 128 x 64. IM2WIN_MFMA_KERNEL=tiled turns it
// off; IM2WIN_MFMA_DMA_TILE="MB,NB,WM" overrides the tile for sweeps.
static const int kDmaTiles[][3] = {
    {64, 128, 1}, {64, 64, 2}, {128, 64, 2}, {128, 128, 2}, {128, 128, 1}, {64, 256, 1},
};

static bool dma_tile_known(int m, int n, int wm) {
    for (const auto &t : kDmaTiles)
        if (t[0] == m && t[1] == n && t[2] == wm) return true;
    return false;
}

// Which of the page's three optimisations the direct-to-LDS window-GEMM
// keeps for a launch, chosen per layer from measurements as the page's
// Table II does ("Enabling Memory-efficient Im2win Convolution ...", Sec.
// IV-B; the ablation of Sec. IV-E). On MI355X the direct-to-LDS copies and the
// serpentine tile order never lost (turning the order off gained at most
// 4.5%, within run-to-run spread), so both stay. Three stage buffers lose
// where their LDS (3 x (MB + NB) x 128 bytes per workgroup) is what makes the
// launch take more rounds of workgroups over the CUs than one buffer would,
// and K is either a single 64-element stage (nothing to overlap) or long (at
// least 16 stages, where the extra resident workgroups hide the loads
// instead): measured 1.22x on the 64 -> 256 1x1 layer and 1.13x on Table I's
// cv11, equal on cv10, and a loss of 13% on cv9 (9 stages), where they stay.
// Returns the ablation bits of the plan (bit 2: one stage buffer).
static int dma_variant(int m, int n, int64_t cols, int64_t stages, int64_t cout) {
    const int64_t tiles = ceil_div(cout, m) * ceil_div(cols, n);
    auto per_cu = [&](int64_t bufs) {
        const int64_t lds = bufs * (m + n) * 64 * 2;
        return std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / lds));
    };
    const int64_t rounds3 = ceil_div(tiles, 256 * per_cu(3));
    const int64_t rounds1 = ceil_div(tiles, 256 * per_cu(1));
    return (rounds1 < rounds3 && (stages == 1 || stages >= 16)) ? 4 : 0;
}

static void pick_mfma_dma(const conv2d_desc_t &d, int64_t krun, int64_t cols, conv2d_plan_t *p) {
    if (krun != p->K_stage || p->K_stage % 64 != 0) return;
    if (const char *k = std::getenv("IM2WIN_MFMA_KERNEL"))
        if (std::strcmp(k, "tiled") == 0) return;
    int m, n, wm;
    if (d.Cout <= 64) {
        m = 64; wm = 1; n = 128;
        if (ceil_div(cols, 128) < 256) { n = 64; wm = 2; }
    } else if (d.Cout >= 256 && p->K_stage >= 256) {
        m = 64; n = 64; wm = 2;
    } else {
        m = 128; n = 64; wm = 2;
    }
    if (const char *e = std::getenv("IM2WIN_MFMA_DMA_TILE")) {
        int a = 0, b = 0, w = 0;
        if (std::sscanf(e, "%d,%d,%d", &a, &b, &w) == 3 && dma_tile_known(a, b, w)) {
            m = a; n = b; wm = w;
        }
    }
    p->gemm_kernel = 3;
    p->gemm_tile_m = m;
    p->gemm_tile_n = n;
    p->gemm_kslice = 64;
    p->gemm_ksplit = 1;
    p->gemm_wave_m = wm;
    p->gemm_ablate = dma_variant(m, n, cols, p->K_stage / 64, d.Cout);
    // IM2WIN_ABLATE: a comma list of "serpentine", "dma", "buffers", each
    // turning one of the page's optimisations off in this kernel (the
    // ablation of "Enabling Memory-efficient Im2win Convolution ...",
    // Sec. IV-E, Fig. 4, of the optimisations of Sec. III-E); for
    // measurements only
    if (const char *e = std::getenv("IM2WIN_ABLATE")) {
        int bits = 0;
        if (std::strstr(e, "serpentine")) bits |= 1;
        if (std::strstr(e, "dma")) bits |= 2;
        if (std::strstr(e, "buffers")) bits |= 4;
        p->gemm_ablate = bits;
    }
}

// What conv2d_fwd runs for a matrix-core layer. The implicit form (window
// rows built in LDS, no window tensor) skips the window tensor's HBM round
// trip and measured faster on the stride-1 layers of the sweep (3x3, 5x5,
// 1x1, 512-channel 7x7, the Table I 3x3 layers) where its tiles fill at
// least 70 % of their GEMM columns; it lost where they do not (5x5 outputs),
// with stride 2 (a patch of 2R+1 input rows per R window rows) and for a 7x7
// filter (a patch that leaves one workgroup per CU).
// IM2WIN_ALGO=window|implicit overrides (implicit only where it applies).
static void pick_algo(const conv2d_desc_t &d, conv2d_plan_t *p) {
    conv2d_implicit_plan_t ip;
    const bool can = make_implicit_plan(d, &ip) == CONV2D_OK;
    const int64_t taps = d.KH * d.KW;
    bool use = false;
    if (can && ip.kernel >= 2) use = true;
    if (can && ip.kernel == 0 && d.stride == 1 && taps <= 25) {
        const double fill = double(p->Ho * p->Wo) /
            double(ceil_div(p->Ho, ip.rows_per_tile) * ceil_div(p->Wo, ip.cols_per_tile) * ip.tile_n);
        use = fill >= 0.7;
    }
    if (const char *e = std::getenv("IM2WIN_ALGO")) {
        if (std::strcmp(e, "window") == 0) use = false;
        if (std::strcmp(e, "implicit") == 0) use = can;
    }
    p->algo = use ? 1 : 0;
    if (use) {
        p->ws_bytes = ip.ws_bytes;
        p->meets_ws_target = p->ws_bytes <= p->ws_target_bytes ? 1 : 0;
    }
}

int valu_cols_per_lane(const conv2d_desc_t &d) {
    if (d.KH == 7 && d.KW == 7 && d.stride == 2) return 2;
    if (d.KH == 11 && d.KW == 11 && d.stride == 4) return 1;
    return 4;
}

// Channel split across the 4 waves of a vector-ALU workgroup: used when the
// output alone does not give every SIMD a couple of waves.
static int pick_valu_ksplit(const conv2d_desc_t &d, int64_t rows, int64_t Wo, int64_t Cout_stage) {
    if (const char *e = std::getenv("IM2WIN_VALU_KSPLIT")) {
        const int k = std::atoi(e);
        if (k == 1 || k == 2 || k == 4) return k;
    }
    const int64_t nt = valu_cols_per_lane(d);
    const int64_t waves = (Cout_stage / kValuMt) * ceil_div(rows * ceil_div(Wo, nt), 64);
    if (waves >= 2048) return 1;
    if (d.Cin >= 4) return 4;
    if (d.Cin >= 2) return 2;
    return 1;
}

static conv2d_status_t compute_plan(const conv2d_desc_t &d, conv2d_plan_t *p) {
    const conv2d_status_t st = check_desc(d);
    if (st != CONV2D_OK) return st;
    std::memset(p, 0, sizeof(*p));
    const int64_t es = elem_size(d.dtype);
    p->Ho = out_extent(d.H, d.KH, d.stride, d.pad);
    p->Wo = out_extent(d.W, d.KW, d.stride, d.pad);
    p->W_win = (p->Wo - 1) * d.stride + d.KW;
    p->path = d.dtype == CONV2D_F32 ? 0 : 1;
    p->layout = d.dtype == CONV2D_F32 ? IM2WIN_LAYOUT_ROW : IM2WIN_LAYOUT_CL;
    const LayoutGeom g = layout_geom(d, p->layout);
    p->Cin_pad = g.Cin_pad;
    p->pos_pad = g.pos_pad;
    p->row_elems = g.row_elems;
    p->rows_total = d.N * p->Ho;
    p->K = d.Cin * d.KH * d.KW;
    p->flops = 2 * d.N * d.Cout * p->Ho * p->Wo * p->K;

    const StageGeom sg = stage_geom(d, p->layout, p->gemm_tile_m);
    p->Cout_stage = sg.rows;
    p->K_stage = sg.row_len;
    if (sg.rows * sg.row_len > kMaxElems) return CONV2D_ERR_INVALID_DESC;
    p->wstage_bytes = sg.needed ? round_up(sg.rows * sg.row_len * es, 256) : 0;

    p->im2col_bytes = p->rows_total * p->Wo * p->K * es;
    p->ws_target_bytes = p->im2col_bytes / d.KW;
    const int64_t row_bytes = p->row_elems * es;
    int64_t rmax = (p->ws_target_bytes - p->wstage_bytes) / row_bytes;
    if (rmax < 1) rmax = 1;                       // the 1/KW target is out of reach
    if (rmax > p->rows_total) rmax = p->rows_total;
    // never exceed the 2^31-element limit inside one window chunk
    const int64_t rlim = kMaxElems / p->row_elems;
    if (rlim < 1) return CONV2D_ERR_INVALID_DESC;
    if (rmax > rlim) rmax = rlim;
    p->n_chunks = ceil_div(p->rows_total, rmax);
    p->rows_per_chunk = ceil_div(p->rows_total, p->n_chunks);
    p->win_offset_bytes = p->wstage_bytes;
    p->win_chunk_bytes = p->rows_per_chunk * row_bytes;
    p->ws_bytes = p->wstage_bytes + p->win_chunk_bytes;
    p->meets_ws_target = p->ws_bytes <= p->ws_target_bytes ? 1 : 0;
    if (p->path == 1) {
        pick_mfma_tile(d, p->rows_per_chunk * p->Wo, mfma_kgran(d.KW * d.KH * g.Cin_pad), p);
        p->gemm_kernel = 1;
        pick_mfma_dma(d, d.KW * d.KH * g.Cin_pad, p->rows_per_chunk * p->Wo, p);
        pick_algo(d, p);
    } else {
        p->gemm_kernel = 0;
        p->gemm_tile_m = 4 * kValuMt;
        p->gemm_tile_n = 64 * valu_cols_per_lane(d);
        p->gemm_kslice = 0;
        p->gemm_ksplit = pick_valu_ksplit(d, p->rows_per_chunk, p->Wo, p->Cout_stage);
        pick_algo(d, p);
    }
    return CONV2D_OK;
}

// Implicit form. A tile covers R window rows x WB output columns of one
// image (R*WB <= NB GEMM columns); its patch holds IR = (R-1)*s + KH input
// rows x IW = (WB-1)*s + KW input columns of one 64-channel block. Candidates
// are scored by the share of the tile that is real outputs, the tile size,
// the number of tiles per CU, and a penalty when the LDS of a workgroup
// leaves room for only one per CU.
// IM2WIN_IMPLICIT_TILE="MB,NB,WM,R,WB" overrides the choice (for sweeps).
static const int kImplicitTiles[][3] = {{64, 64, 1}, {64, 128, 1}, {128, 64, 2}, {128, 128, 2}};

// Row-block implicit kernel: stride 1, output rows of at most 64 columns, a
// 1x1 or 3x3 filter; fp16/bf16 with 64 input channels on rows of 8k elements,
// or any multiple of 64 channels where an image has at least 128 outputs;
// fp32 with a multiple of 32 channels on rows of 4k elements. A workgroup of eight waves takes RW whole output rows of one image
// (RW * Wo <= 512 outputs, 16-output blocks shared over the waves) and 64
// output channels, with the raw filter and the RW + KH - 1 input rows in LDS;
// no staged filter. RW minimises the rounds of workgroups over the CUs times
// the busiest SIMD's blocks plus a fixed set-up.
// Default where it applies; IM2WIN_IMPLICIT_KERNEL=streamed (or a
// tile in IM2WIN_IMPLICIT_TILE) selects the other kernels; IM2WIN_IMPLICIT_ROWS
// sets RW.
static void pick_implicit_rows(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p) {
    const int64_t taps = d.KH * d.KW;
    const bool f32 = d.dtype == CONV2D_F32;
    // fp16/bf16: one 64-channel block on rows of 8k elements (the one-block
    // kernel), or several blocks / any width (the channel-block loop) where an
    // image has at least 128 outputs (8 MFMA blocks: every wave busy); smaller
    // images stay on the streamed kernel
    const bool chans = f32 ? (d.Cin % 32 == 0 && (d.W % 4 == 0 || Ho * Wo >= 128))
                           : (d.Cin % 64 == 0 && ((d.Cin == 64 && d.W % 8 == 0) || Ho * Wo >= 128));
    if (!chans || d.stride != 1 || Wo > 64 || !((d.KH == 3 && d.KW == 3) || (d.KH == 1 && d.KW == 1)))
        return;
    if (d.Cin * d.H * d.W >= (int64_t(1) << 31)) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_KERNEL"))
        if (std::strcmp(e, "rows") != 0) return;
    if (std::getenv("IM2WIN_IMPLICIT_TILE")) return;   // a streamed-kernel tile was asked for
    const int64_t iw = d.W + 2 * d.pad;
    const int64_t co_blocks = ceil_div(d.Cout, 64);
    // the busiest SIMD's MFMA blocks: 16-output blocks shared over 8 waves in
    // contiguous ranges, waves w and w + 4 on one SIMD
    auto simd_blocks = [](int64_t outs) {
        const int64_t total = ceil_div(outs, 16);
        int64_t worst = 0;
        for (int64_t sm = 0; sm < 4; ++sm) {
            int64_t b = 0;
            for (int64_t w = sm; w < 8; w += 4) b += (w + 1) * total / 8 - w * total / 8;
            worst = std::max(worst, b);
        }
        return worst;
    };
    int64_t best_rw = 0;
    double best_cost = 0.0;
    for (int64_t rw = 1; rw <= Ho && rw * Wo <= 512; ++rw) {
        const int64_t lds = implicit_rows_lds_bytes(taps, rw + d.KH - 1, iw);
        if (lds > kImplicitMaxLdsBytes) break;
        const int64_t per_cu = std::min<int64_t>(2, kImplicitMaxLdsBytes / lds);
        const int64_t blocks = co_blocks * d.N * ceil_div(Ho, rw);
        // rounds of workgroups over the CUs, each costing its busiest SIMD's
        // blocks plus a fixed set-up (the block's loads and barrier) worth 12
        const int64_t nblk = f32 ? d.Cin / 32 : d.Cin / 64;
        const double cost = double(ceil_div(blocks, 256 * per_cu)) * double(simd_blocks(rw * Wo) * nblk + 12);
        if (best_rw == 0 || cost < best_cost) { best_rw = rw; best_cost = cost; }
    }
    if (best_rw == 0) return;
    // fp16/bf16 x, 3x3, fp32 y stored directly (Wo % 4 == 0): the kernel is
    // bound by HBM, and it writes the lines of y that it covers whole through
    // the L2 as it stores them (the others wait in L2 for the write-back at
    // the end of the kernel), so take the fewest rows whose plane segments
    // are whole 128-byte lines when that
    // costs at most 10 % more by the count above (measured on the ResNet 3x3
    // layer: 7 rows 14.2 us, 8 rows, every line written through, 12.2 us;
    // fp32 x stays on the count: 67 against 75 us there). The 1x1 form, whose
    // stores go through LDS, gains from whole-line segments too, in either
    // output type (the 64 -> 256 channel 56x56 layer, 7 -> 8 rows: fp32 y
    // 41.4 -> 39.6 us, fp16 y 41.9 -> 38.5 us), half-precision y of the 3x3
    // form does not (14.4 -> 14.8 us)
    const int64_t ysz = d.y_dtype == CONV2D_F32 ? 4 : 2;
    if (!f32 && Wo % 4 == 0 && (taps == 1 || d.y_dtype == CONV2D_F32) && (Ho * Wo * ysz) % 128 == 0) {
        for (int64_t rw = 1; rw <= Ho && rw * Wo <= 512; ++rw) {
            const int64_t lds = implicit_rows_lds_bytes(taps, rw + d.KH - 1, iw);
            if (lds > kImplicitMaxLdsBytes) break;
            if ((rw * Wo * ysz) % 128 != 0) continue;
            const int64_t per_cu = std::min<int64_t>(2, kImplicitMaxLdsBytes / lds);
            const int64_t blocks = co_blocks * d.N * ceil_div(Ho, rw);
            const double cost = double(ceil_div(blocks, 256 * per_cu)) * double(simd_blocks(rw * Wo) * (d.Cin / 64) + 12);
            if (cost <= 1.1 * best_cost) {
                best_rw = rw;
                break;
            }
        }
    }
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_ROWS")) {
        const int64_t v = std::min<int64_t>(std::atoi(e), Ho);
        if (v >= 1 && v * Wo <= 512 && implicit_rows_lds_bytes(taps, v + d.KH - 1, iw) <= kImplicitMaxLdsBytes)
            best_rw = v;
    }
    p->kernel = 2;
    p->tile_m = 64;
    p->tile_n = 64;
    p->wave_m = 1;
    p->rows_per_tile = int32_t(best_rw);
    p->cols_per_tile = int32_t(Wo);
    p->patch_rows = int32_t(best_rw + d.KH - 1);
    p->patch_cols = int32_t(iw);
    p->stages = 0;
    p->lds_bytes = implicit_rows_lds_bytes(taps, p->patch_rows, iw);
    p->tiles = co_blocks * d.N * ceil_div(Ho, best_rw);
    p->ws_bytes = 0;    // the kernel reads w as it is stored
}

// Whole images per task for the pipelined row-block kernels where images are
// small (fewer than 128 outputs, so a task of one image would leave waves
// idle): the most images (at most 256 outputs, the patches within the LDS
// limit) that still leave min_tasks tasks; 1 where even two do not.
// IM2WIN_IMPLICIT_IMAGES sets it.
static int64_t pick_images(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, int64_t min_tasks, bool pair) {
    const int64_t taps = d.KH * d.KW, iw = d.W + 2 * d.pad, sl = (Ho - 1) * d.stride + d.KH;
    const int64_t co_blocks = ceil_div(d.Cout, 64);
    auto fits = [&](int64_t img) {
        const int64_t lds = pair ? pair_lds_bytes(taps, img * sl, iw) : pipe_lds_bytes(taps, img * sl, iw);
        return img * Ho * Wo <= 256 && img <= d.N && lds <= (pair ? kImplicitPairLdsBytes : kImplicitMaxLdsBytes);
    };
    int64_t best = 1;
    if (Ho * Wo < 128)
        for (int64_t img = 2; fits(img); ++img)
            if (co_blocks * ceil_div(d.N, img) >= min_tasks) best = img;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_IMAGES")) {
        const int64_t v = std::atoi(e);
        if (v >= 1 && (v == 1 || fits(v))) best = v;
    }
    return best;
}

// Pipelined row-block implicit kernel: fp16/bf16, Cin % 32 == 0, stride 1,
// 3x3 or 1x1, Wo <= 256. Tasks of RW whole output rows x 64 output channels
// (RW * Wo <= 256: four computing waves of at most four 16-output blocks),
// walked by at most 256 persistent workgroups in 32-channel K chunks that
// four loader waves double-buffer in LDS. RW minimises an estimate of the
// busiest workgroup's cycles: per chunk the larger of the busiest computing
// wave's MFMA cycles and its LDS reads (128 bytes per clock per CU), against
// the chunk's loads and the task's stores at a CU's share of HBM bandwidth
// (13 bytes per clock). Taken when `dflt` (the caller's rule) or when
// IM2WIN_IMPLICIT_KERNEL=pipe; IM2WIN_IMPLICIT_ROWS sets RW.
static void pick_implicit_pipe(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p,
                               bool dflt) {
    if (d.dtype == CONV2D_F32 || d.Cin % 32 != 0 || d.stride > 2 || Wo > 256 || Wo < 1 || Ho < 1) return;
    if (!((d.KH == 3 && d.KW == 3) || (d.KH == 1 && d.KW == 1))) return;
    if (d.Cin * d.H * d.W >= (int64_t(1) << 31)) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_KERNEL")) {
        if (std::strcmp(e, "pipe") != 0) return;
    } else if (!dflt || std::getenv("IM2WIN_IMPLICIT_TILE")) {
        return;
    }
    const int64_t s = d.stride;
    const int64_t taps = d.KH * d.KW;
    const int64_t iw = d.W + 2 * d.pad;
    const int64_t co_blocks = ceil_div(d.Cout, 64);
    const int64_t nch = d.Cin / 32;
    constexpr double kHbmBytesPerClk = 13.0;
    int64_t best_rw = 0, best_groups = 0;
    double best_cost = 0.0;
    for (int64_t rw = 1; rw <= Ho && rw * Wo <= 256; ++rw) {
        const int64_t sl = (rw - 1) * s + d.KH;
        if (pipe_lds_bytes(taps, sl, iw) > kImplicitMaxLdsBytes) break;
        const int64_t tasks = co_blocks * d.N * ceil_div(Ho, rw);
        const int64_t groups = std::min<int64_t>(tasks, 256);
        const int64_t rounds = ceil_div(tasks, groups);
        const int64_t bw = ceil_div(ceil_div(rw * Wo, 16), 4);
        const double chunk = double(std::max(taps * bw * 64, taps * 32 * (bw + 4)));
        const double load = double(sl * d.W * 64 + taps * 4096) / kHbmBytesPerClk;
        const double store = double(rw * Wo * 64 * 4) / kHbmBytesPerClk;
        const double cost = double(rounds) * std::max(double(nch) * chunk, double(nch) * load + store);
        if (best_rw == 0 || cost < best_cost) { best_rw = rw; best_groups = groups; best_cost = cost; }
    }
    if (best_rw == 0) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_ROWS")) {
        const int64_t v = std::min<int64_t>(std::atoi(e), Ho);
        if (v >= 1 && v * Wo <= 256 && pipe_lds_bytes(taps, (v - 1) * s + d.KH, iw) <= kImplicitMaxLdsBytes) {
            best_rw = v;
            best_groups = std::min<int64_t>(co_blocks * d.N * ceil_div(Ho, v), 256);
        }
    }
    const int64_t img = pick_images(d, Ho, Wo, 256, false);
    if (img > 1) {
        best_rw = Ho;
        best_groups = std::min<int64_t>(co_blocks * ceil_div(d.N, img), 256);
    }
    p->kernel = 4;
    p->tile_m = 64;
    p->tile_n = 64;
    p->wave_m = 1;
    p->rows_per_tile = int32_t(best_rw);
    p->cols_per_tile = int32_t(Wo);
    p->patch_rows = int32_t(img * ((best_rw - 1) * s + d.KH));
    p->patch_cols = int32_t(iw);
    p->stages = 2;
    p->images = int32_t(img);
    p->lds_bytes = pipe_lds_bytes(taps, p->patch_rows, iw);
    p->tiles = best_groups;
    p->ws_bytes = 0;    // the kernel reads w as it is stored
}

// Paired row-block implicit kernel (the same kernel file, `stages` 1):
// fp16/bf16, Cin % 32 == 0, stride 1, 3x3 or 1x1, one task of RW whole
// output rows x 64 output channels per workgroup (RW * Wo <= 256), a single
// 32-channel chunk slot in LDS of at most 80 KB, so that two workgroups
// share a CU. Taken when `dflt` or when IM2WIN_IMPLICIT_KERNEL=pair;
// IM2WIN_IMPLICIT_ROWS sets RW.
static void pick_implicit_pair(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p,
                               bool dflt) {
    if (d.dtype == CONV2D_F32 || d.Cin % 32 != 0 || d.stride > 2 || Wo > 256 || Wo < 1 || Ho < 1) return;
    if (!((d.KH == 3 && d.KW == 3) || (d.KH == 1 && d.KW == 1))) return;
    if (d.Cin * d.H * d.W >= (int64_t(1) << 31)) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_KERNEL")) {
        if (std::strcmp(e, "pair") != 0) return;
    } else if (!dflt || std::getenv("IM2WIN_IMPLICIT_TILE")) {
        return;
    }
    const int64_t s = d.stride;
    const int64_t taps = d.KH * d.KW;
    const int64_t iw = d.W + 2 * d.pad;
    const int64_t co_blocks = ceil_div(d.Cout, 64);
    // the most rows per task (the most MFMA blocks per wave) that still leaves
    // 512 tasks, two per CU; the most rows that fit where none does
    int64_t best_rw = 0, fit_rw = 0;
    for (int64_t rw = 1; rw <= Ho && rw * Wo <= 256; ++rw) {
        if (pair_lds_bytes(taps, (rw - 1) * s + d.KH, iw) > kImplicitPairLdsBytes) break;
        fit_rw = rw;
        if (co_blocks * d.N * ceil_div(Ho, rw) >= 512) best_rw = rw;
    }
    if (best_rw == 0) best_rw = fit_rw;
    if (best_rw == 0) return;
    best_rw = ceil_div(Ho, ceil_div(Ho, best_rw));   // the same number of tasks, rows spread evenly
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_ROWS")) {
        const int64_t v = std::min<int64_t>(std::atoi(e), Ho);
        if (v >= 1 && v * Wo <= 256 && pair_lds_bytes(taps, (v - 1) * s + d.KH, iw) <= kImplicitMaxLdsBytes)
            best_rw = v;
    }
    const int64_t img = pick_images(d, Ho, Wo, 512, true);
    if (img > 1) best_rw = Ho;
    p->kernel = 4;
    p->tile_m = 64;
    p->tile_n = 64;
    p->wave_m = 1;
    p->rows_per_tile = int32_t(best_rw);
    p->cols_per_tile = int32_t(Wo);
    p->patch_rows = int32_t(img * ((best_rw - 1) * s + d.KH));
    p->patch_cols = int32_t(iw);
    p->stages = 1;
    p->images = int32_t(img);
    p->lds_bytes = pair_lds_bytes(taps, p->patch_rows, iw);
    p->tiles = img > 1 ? co_blocks * ceil_div(d.N, img) : co_blocks * d.N * ceil_div(Ho, best_rw);
    p->ws_bytes = 0;
}

// The pipelined row-block kernels where they apply by default: the paired
// form where its tasks number at least 512 (two per CU) and either hold at
// least 128 outputs (every one of its eight waves busy) or number at least
// 1024, else the persistent form
// (its four computing waves take up to four blocks each of a task of up to
// 256 outputs, small images several to a task). Measured against the
// row-block kernel over several channel blocks and the streamed kernel: paired
// 1.04-1.6x faster on cv6, cv8, cv10 and cv11, persistent 1.13x on the 14x14
// deep layer (paired tasks of 98 outputs), 1.36x on the 512-channel 7x7 layer
// and 1.9x on cv12 (several images per task); stride 2: paired 1.2x over the
// streamed kernel and the window form on the 28x28 -> 14x14 layer.
static void pick_implicit_pipelined(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p,
                                    bool dflt) {
    if (!dflt) {
        pick_implicit_pipe(d, Ho, Wo, p, false);
        pick_implicit_pair(d, Ho, Wo, p, false);
        return;
    }
    if (std::getenv("IM2WIN_IMPLICIT_KERNEL")) {   // a kernel asked for by name
        pick_implicit_pipe(d, Ho, Wo, p, false);
        pick_implicit_pair(d, Ho, Wo, p, false);
        return;
    }
    conv2d_implicit_plan_t pair = *p;
    pick_implicit_pair(d, Ho, Wo, &pair, true);
    if (pair.kernel == 4 && pair.tiles >= 512 &&
        (int64_t(pair.images) * pair.rows_per_tile * Wo >= 128 || pair.tiles >= 1024)) {
        *p = pair;
        return;
    }
    pick_implicit_pipe(d, Ho, Wo, p, true);
}

// Split-K row-block implicit kernel: fp16/bf16, Cin % 128 == 0, stride 1 or
// 2, 3x3, 5x5 or 1x1, one task per workgroup of RW whole output rows (or of
// several whole images), four K groups of two waves splitting the input
// channels. The two waves of a group either split the task's 16-output
// blocks (tasks of at most 224 outputs x 64 output channels) or, where
// patches are large (stride 2), split 128 output channels over tasks of at
// most 112 outputs (co_split 2, tile_m 128), so each wave keeps a tile of up
// to 7 blocks. The task shape, split and LDS slots per K group (two, or one
// where two do not fit) minimise the rounds of workgroups over the CUs times
// a wave's blocks plus a fixed cost per tap (3 blocks' worth), 15% more for
// one slot; ties go to the larger task (each filter fragment read by fewer
// workgroups), then to the split of the task's outputs. Default for 5x5
// filters (measured on the 28x28 5x5 layer: 46.7 us per kernel + 5.3 us
// filter staging against 59.3 us for the streamed kernel) and for stride 2
// (the 28x28 -> 14x14 layer, 512 output channels: 58.1 us + 3.3 us, tasks of
// 7 rows x 128 output channels with one slot, against 78.4 us for the paired
// pipelined kernel); on the stride-1 3x3 layers the staging launch cancels
// its gain over the pipelined kernels (deep 3x3: 22.6 + 3.1 against 25.3
// us), so there it is taken when IM2WIN_IMPLICIT_KERNEL=ksplit. IM2WIN_IMPLICIT_ROWS
// sets RW, IM2WIN_IMPLICIT_IMAGES the images per task, IM2WIN_KSPLIT_CO=1|2
// the split and IM2WIN_KSPLIT_SLOTS=1|2 the slots.
static void pick_implicit_ksplit(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p,
                                 bool dflt) {
    if (d.dtype == CONV2D_F32 || d.Cin % (32 * kKsplitGroups) != 0 || d.stride > 2 || Wo < 1 || Ho < 1) return;
    if (!((d.KH == 3 && d.KW == 3) || (d.KH == 1 && d.KW == 1) || (d.KH == 5 && d.KW == 5))) return;
    if (d.Cin * d.H * d.W >= (int64_t(1) << 31)) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_KERNEL")) {
        if (std::strcmp(e, "ksplit") != 0) return;
    } else if (!dflt || std::getenv("IM2WIN_IMPLICIT_TILE")) {
        return;
    }
    int64_t force_co = 0, force_slots = 0;
    if (const char *e = std::getenv("IM2WIN_KSPLIT_CO")) force_co = std::atoi(e);
    if (const char *e = std::getenv("IM2WIN_KSPLIT_SLOTS")) force_slots = std::atoi(e);
    const int64_t s = d.stride, iw = d.W + 2 * d.pad;
    // padded: the products a choice issues, in 16-output x 64-channel block
    // steps over all tasks (ties of the round count go to the fewest: the
    // 28x28 5x5 layer's 4-row x 128-channel tasks issue 6272, its 7-row x
    // 64-channel ones 6656 and measured 52.5 -> 47.7 us; the 14x14 deep
    // layer's whole images x 64 channels issue 3328 against 3584)
    struct Pick { int64_t rw, img, cos, slots; double cost; int64_t padded; };
    Pick best{0, 0, 0, 0, 0.0, 0};
    auto fits = [&](int64_t rw, int64_t img, int64_t cos, int64_t slots) {
        const int64_t outs = img * rw * Wo;
        if (outs > kKsplitMaxOuts / cos || (cos == 2 && d.Cout <= 64)) return false;
        const int64_t sl = img * ((rw - 1) * s + d.KH);
        return ksplit_lds_bytes(sl, iw, d.Cin, ksplit_nbw(outs, cos), slots) <= kImplicitMaxLdsBytes;
    };
    auto consider = [&](int64_t rw, int64_t img) {
        for (int64_t cos = 1; cos <= 2; ++cos) {
            if (force_co && cos != force_co) continue;
            for (int64_t slots = 2; slots >= 1; --slots) {
                if ((force_slots && slots != force_slots) || !fits(rw, img, cos, slots)) continue;
                const int64_t outs = img * rw * Wo;
                const int64_t nbt = ceil_div(outs, 16);
                const int64_t per_wave = cos == 2 ? nbt : ceil_div(nbt, 2);
                const int64_t co_blocks = ceil_div(d.Cout, 64 * cos);
                const int64_t tasks = img > 1 ? co_blocks * ceil_div(d.N, img) : co_blocks * d.N * ceil_div(Ho, rw);
                const double cost = double(ceil_div(tasks, 256)) * double(per_wave + 3) * (slots == 1 ? 1.15 : 1.0);
                const int64_t padded = tasks * nbt * cos;
                const int64_t bouts = best.img * best.rw * Wo;
                const bool tie = best.rw != 0 && cost == best.cost;
                if (best.rw == 0 || cost < best.cost ||
                    (tie && (padded < best.padded ||
                             (padded == best.padded && (cos < best.cos || (cos == best.cos && outs > bouts))))))
                    best = Pick{rw, img, cos, slots, cost, padded};
                break;                             // two slots where they fit
            }
        }
    };
    for (int64_t rw = 1; rw <= Ho; ++rw) consider(ceil_div(Ho, ceil_div(Ho, rw)), 1);
    for (int64_t img = 2; img <= d.N && img * Ho * Wo <= kKsplitMaxOuts; ++img) consider(Ho, img);
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_IMAGES")) {
        const int64_t v = std::atoi(e);
        if (v >= 2 && v <= d.N) {
            const Pick keep = best;
            best = Pick{0, 0, 0, 0, 0.0, 0};
            consider(Ho, v);
            if (best.rw == 0) best = keep;
        }
    }
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_ROWS")) {
        const int64_t v = std::min<int64_t>(std::atoi(e), Ho);
        if (v >= 1) {
            const Pick keep = best;
            best = Pick{0, 0, 0, 0, 0.0, 0};
            consider(v, 1);
            if (best.rw == 0) best = keep;
        }
    }
    if (best.rw == 0) return;
    const int64_t outs = best.img * best.rw * Wo;
    const int64_t co_blocks = ceil_div(d.Cout, 64 * best.cos);
    p->kernel = 5;
    p->tile_m = int32_t(64 * best.cos);
    p->tile_n = int32_t(ksplit_nbw(outs, best.cos) * 16);
    p->wave_m = int32_t(kKsplitGroups);
    p->rows_per_tile = int32_t(best.rw);
    p->cols_per_tile = int32_t(Wo);
    p->patch_rows = int32_t(best.img * ((best.rw - 1) * s + d.KH));
    p->patch_cols = int32_t(iw);
    p->stages = int32_t(best.slots);
    p->images = int32_t(best.img);
    p->lds_bytes = ksplit_lds_bytes(p->patch_rows, iw, d.Cin, ksplit_nbw(outs, best.cos), best.slots);
    p->tiles = best.img > 1 ? co_blocks * ceil_div(d.N, best.img) : co_blocks * d.N * ceil_div(Ho, best.rw);
    p->ws_bytes = round_up(ksplit_stage_bytes(d.Cout, d.Cin, d.KH * d.KW), 256);
}

// Narrow-channel implicit kernel: Cin <= 8 (the RGB stem and its kind), any
// filter and stride, Wo <= 512, fp16/bf16/fp32. A workgroup of eight waves
// takes R output rows of one image (R * Wo <= 512) and 64 output channels,
// with its R channels-last window rows (CP = 4 channels per position, or 8
// where 4 would leave a window start off a 16-byte boundary) and the filter in
// the window's K order in LDS, gathered from w as stored, or (launches of more
// than one workgroup per CU) read from the filter staged in the workspace.
// Default where it applies; IM2WIN_IMPLICIT_KERNEL names another kernel to
// leave it; IM2WIN_IMPLICIT_ROWS sets R. The plan's `stages` field carries CP
// and `K_stage` the filter's LDS row length Kp.
static void pick_implicit_narrow(const conv2d_desc_t &d, int64_t Ho, int64_t Wo, conv2d_implicit_plan_t *p) {
    if (d.Cin > 8 || Wo > 512 || Wo < 1 || Ho < 1) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_KERNEL"))
        if (std::strcmp(e, "narrow") != 0) return;
    if (d.Cin * d.H * d.W >= (int64_t(1) << 31) || d.Cout * d.Cin * d.KH * d.KW >= (int64_t(1) << 31)) return;
    const bool f32 = d.dtype == CONV2D_F32;
    const int64_t es = f32 ? 4 : 2;
    const int64_t cp = (d.Cin <= 4 && (d.stride * d.KH * 4 * es) % 16 == 0) ? 4 : 8;
    const int64_t K = d.KW * d.KH * cp;
    const int64_t kstep = f32 ? 16 : 32;
    const int64_t Kp = round_up(K, kstep);
    const int64_t L = ((Wo - 1) * d.stride + d.KW) * d.KH * cp;
    const int64_t Lp = round_up(L + Kp - K, f32 ? 4 : 8);
    const int64_t co_blocks = ceil_div(d.Cout, 64);
    // R: the largest that fits LDS and 512 outputs (measured best: the
    // block's set-up, its load round trip and barrier, is paid once per R
    // rows), made smaller only while the grid would leave CUs idle
    int64_t best_r = 0;
    for (int64_t r = 1; r <= Ho && r * Wo <= 512; ++r) {
        if (implicit_narrow_lds_bytes(es, Kp, Lp, r) > kImplicitMaxLdsBytes) break;
        best_r = r;
    }
    while (best_r > 1 && co_blocks * d.N * ceil_div(Ho, best_r) < 256) --best_r;
    if (best_r == 0) return;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_ROWS")) {
        const int64_t v = std::min<int64_t>(std::atoi(e), Ho);
        if (v >= 1 && v * Wo <= 512 && implicit_narrow_lds_bytes(es, Kp, Lp, v) <= kImplicitMaxLdsBytes)
            best_r = v;
    }
    p->kernel = 3;
    p->tile_m = 64;
    p->tile_n = int32_t(best_r * Wo);
    p->wave_m = 1;
    p->rows_per_tile = int32_t(best_r);
    p->cols_per_tile = int32_t(Wo);
    p->patch_rows = int32_t(best_r);               // window rows held
    p->patch_cols = int32_t(Lp);                   // elements per window row in LDS
    p->stages = int32_t(cp);
    p->lds_bytes = implicit_narrow_lds_bytes(es, Kp, Lp, best_r);
    // One row block per workgroup, or (fp32, and filter blocks over 48 KB)
    // persistent workgroups, one per CU, each walking a contiguous range of
    // the N * ceil(Ho / R) row blocks with its filter block staged once and
    // the next block's gathers in flight during the contraction: measured
    // faster there (stem fp32 159 -> 139 us, cv3 fp32 1164 -> 953 us, cv1
    // fp16 591 -> 528 us), slower for fp16 with small filters (stem 49 -> 61).
    const int64_t row_blocks = d.N * ceil_div(Ho, best_r);
    const bool persistent = f32 || 64 * Kp * es > 48 * 1024;
    const int64_t groups = persistent ? std::min(row_blocks, std::max<int64_t>(1, 256 / co_blocks)) : row_blocks;
    p->tiles = co_blocks * groups;
    // the filter block in LDS rows of Kp elements: gathered from w as stored
    // by launches of at most one workgroup per CU (no workspace), else read
    // from the filter staged into the workspace by the channels-last staging,
    // [Cout][Kp] with CP channels per position
    p->K_stage = Kp;
    p->ws_bytes = narrow_gathers_filter(p->tiles) ? 0 : round_up(d.Cout * Kp * es, 256);
}

static conv2d_status_t compute_implicit_plan(const conv2d_desc_t &d, conv2d_implicit_plan_t *p) {
    const conv2d_status_t st = check_desc(d);
    if (st != CONV2D_OK) return st;
    std::memset(p, 0, sizeof(*p));
    const int64_t Ho = out_extent(d.H, d.KH, d.stride, d.pad);
    const int64_t Wo = out_extent(d.W, d.KW, d.stride, d.pad);
    p->Ho = Ho;
    p->Wo = Wo;
    p->K_stage = d.KW * d.KH * d.Cin;
    p->flops = 2 * d.N * d.Cout * Ho * Wo * d.Cin * d.KH * d.KW;
    // the implicit kernels load NCHW planes; NHWC takes the window form
    if (d.layout == CONV2D_NHWC) return CONV2D_ERR_UNSUPPORTED;
    if (d.Cin <= 8) {
        // few input channels: the narrow-channel kernel, any dtype
        pick_implicit_narrow(d, Ho, Wo, p);
        return p->kernel == 3 ? CONV2D_OK : CONV2D_ERR_UNSUPPORTED;
    }
    if (d.dtype == CONV2D_F32) {
        // fp32: only the row-block kernel (fp32 matrix-core products)
        pick_implicit_rows(d, Ho, Wo, p);
        return p->kernel == 2 ? CONV2D_OK : CONV2D_ERR_UNSUPPORTED;
    }
    if (d.Cin % 64 != 0) {
        // 32-channel multiples: only the pipelined row-block kernel
        pick_implicit_pipelined(d, Ho, Wo, p, true);
        return p->kernel == 4 ? CONV2D_OK : CONV2D_ERR_UNSUPPORTED;
    }
    const StageGeom sg = stage_geom(d, IM2WIN_LAYOUT_CL, 64);
    if (sg.row_len != p->K_stage) return CONV2D_ERR_UNSUPPORTED;
    p->ws_bytes = sg.needed ? round_up(sg.rows * sg.row_len * elem_size(d.dtype), 256) : 0;

    struct Cand { int64_t mb, nb, wm, r, wb; double score; };
    Cand best{0, 0, 0, 0, 0, -1.0};
    auto consider = [&](int64_t mb, int64_t nb, int64_t wm, int64_t r, int64_t wb) {
        if (r < 1 || wb < 1 || r * wb > nb) return;
        const int64_t ir = (r - 1) * d.stride + d.KH, iw = (wb - 1) * d.stride + d.KW;
        const int64_t lds = implicit_lds_bytes(mb, ir, iw, 3);
        if (lds > kImplicitMaxLdsBytes) return;
        const double cols = double(Ho * Wo) / double(ceil_div(Ho, r) * ceil_div(Wo, wb) * nb);
        const double rowsm = double(d.Cout) / double(ceil_div(d.Cout, mb) * mb);
        const double tiles = double(ceil_div(d.Cout, mb) * d.N * ceil_div(Ho, r) * ceil_div(Wo, wb));
        // share of real outputs, a mild preference for larger tiles (less
        // per-tile set-up per output), and a penalty below ~1.5 tiles per CU;
        // fitted to a sweep of every tile on the measured layers
        double score = cols * rowsm * std::pow(double(mb * nb) / 8192.0, 0.2) *
                       std::sqrt(std::min(1.0, tiles / 384.0));
        if (lds > kImplicitPairLdsBytes) score *= 0.8;
        // ties go to the taller tile (each filter row read by fewer tiles)
        const bool tie = std::fabs(score - best.score) <= 1e-9 * best.score;
        if ((score > best.score && !tie) || (tie && mb > best.mb)) best = Cand{mb, nb, wm, r, wb, score};
    };
    for (const auto &t : kImplicitTiles) {
        const int64_t mb = t[0], nb = t[1], wm = t[2];
        if (mb == 128 && d.Cout <= 64) continue;
        if (Wo >= nb) {
            consider(mb, nb, wm, 1, nb);
        } else {
            // balanced rows: as many tiles as the widest R needs, rows spread evenly
            const int64_t rmax = std::min<int64_t>(Ho, nb / Wo);
            for (int64_t r = 1; r <= rmax; ++r) consider(mb, nb, wm, ceil_div(Ho, ceil_div(Ho, r)), Wo);
        }
        for (int64_t wb = std::min<int64_t>(Wo, nb); wb >= 8; wb /= 2) consider(mb, nb, wm, 1, wb);
    }
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_TILE")) {
        int m = 0, n = 0, w = 0, r = 0, b = 0;
        if (std::sscanf(e, "%d,%d,%d,%d,%d", &m, &n, &w, &r, &b) == 5) {
            bool known = false;
            for (const auto &t : kImplicitTiles) known = known || (t[0] == m && t[1] == n && t[2] == w);
            const int64_t ir = (r - 1) * d.stride + d.KH, iw = (int64_t(b) - 1) * d.stride + d.KW;
            if (known && r >= 1 && b >= 1 && int64_t(r) * b <= n &&
                implicit_lds_bytes(m, ir, iw, 3) <= kImplicitMaxLdsBytes)
                best = Cand{m, n, w, r, b, 1.0};
        }
    }
    if (best.score < 0) return CONV2D_ERR_UNSUPPORTED;
    p->kernel = 0;
    p->tile_m = int32_t(best.mb);
    p->tile_n = int32_t(best.nb);
    p->wave_m = int32_t(best.wm);
    p->rows_per_tile = int32_t(best.r);
    p->cols_per_tile = int32_t(best.wb);
    p->patch_rows = int32_t((best.r - 1) * d.stride + d.KH);
    p->patch_cols = int32_t((best.wb - 1) * d.stride + d.KW);
    // filter stage buffers: three (two stages in flight); four for 128-row
    // tiles when two workgroups still fit a CU (measured 2-3 % faster there,
    // no gain for 64-row tiles); IM2WIN_IMPLICIT_STAGES=3|4|5 overrides
    int ns = 3;
    if (best.mb == 128 && implicit_lds_bytes(best.mb, p->patch_rows, p->patch_cols, 4) <= kImplicitPairLdsBytes)
        ns = 4;
    if (const char *e = std::getenv("IM2WIN_IMPLICIT_STAGES")) {
        const int v = std::atoi(e);
        if (v >= 3 && v <= 5 && implicit_lds_bytes(best.mb, p->patch_rows, p->patch_cols, v) <= kImplicitMaxLdsBytes)
            ns = v;
    }
    p->stages = ns;
    p->lds_bytes = implicit_lds_bytes(best.mb, p->patch_rows, p->patch_cols, ns);
    p->tiles = ceil_div(d.Cout, best.mb) * d.N * ceil_div(Ho, best.r) * ceil_div(Wo, best.wb);
    if (p->tiles > 0x7fffffff) return CONV2D_ERR_INVALID_DESC;
    pick_implicit_rows(d, Ho, Wo, p);
    // the one-block row kernel stays where it applies (64 channels on rows of
    // 8k elements, measured faster than both pipelined forms); elsewhere the
    // pipelined forms take the 3x3 and 1x1 layers of stride 1 or 2
    const bool one_block = p->kernel == 2 && d.Cin == 64 && d.W % 8 == 0;
    pick_implicit_pipelined(d, Ho, Wo, p, !one_block);
    pick_implicit_ksplit(d, Ho, Wo, p, d.KH * d.KW >= 25 || d.stride == 2);
    return CONV2D_OK;
}

// Plans are cached per descriptor and per set of IM2WIN_* overrides in the
// environment (read on every call, so that a changed override takes effect):
// planning searches tiles and kernels for tens of microseconds, as long as a
// small layer's kernel. The cache is bounded and guarded by a mutex, so calls
// stay reentrant.
namespace {

std::string plan_key(const conv2d_desc_t &d) {
    std::string k(reinterpret_cast<const char *>(&d), sizeof(d));
    for (char **e = environ; e && *e; ++e)
        if (std::strncmp(*e, "IM2WIN_", 7) == 0) {
            k += '\n';
            k += *e;
        }
    return k;
}

struct CachedPlans {
    bool have_plan = false, have_implicit = false;
    conv2d_status_t plan_st = CONV2D_OK, implicit_st = CONV2D_OK;
    conv2d_plan_t plan{};
    conv2d_implicit_plan_t implicit{};
};

std::mutex g_plan_mutex;
std::unordered_map<std::string, CachedPlans> g_plans;
constexpr size_t kMaxCachedPlans = 1024;

CachedPlans &cached(const std::string &key) {
    if (g_plans.size() >= kMaxCachedPlans && g_plans.find(key) == g_plans.end()) g_plans.clear();
    return g_plans[key];
}

}  // namespace

conv2d_status_t make_plan(const conv2d_desc_t &d, conv2d_plan_t *p) {
    const std::string key = plan_key(d);
    {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        const CachedPlans &c = cached(key);
        if (c.have_plan) {
            *p = c.plan;
            return c.plan_st;
        }
    }
    conv2d_plan_t q;
    const conv2d_status_t st = compute_plan(d, &q);
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    CachedPlans &c = cached(key);
    c.have_plan = true;
    c.plan_st = st;
    c.plan = q;
    *p = q;
    return st;
}

conv2d_status_t make_implicit_plan(const conv2d_desc_t &d, conv2d_implicit_plan_t *p) {
    const std::string key = plan_key(d);
    {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        const CachedPlans &c = cached(key);
        if (c.have_implicit) {
            *p = c.implicit;
            return c.implicit_st;
        }
    }
    conv2d_implicit_plan_t q;
    const conv2d_status_t st = compute_implicit_plan(d, &q);
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    CachedPlans &c = cached(key);
    c.have_implicit = true;
    c.implicit_st = st;
    c.implicit = q;
    *p = q;
    return st;
}

}  // namespace im2win
