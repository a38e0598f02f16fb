"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Tolerances (relative L2 over the compared outputs, oracle in float64 fed the
same rounded inputs): fp32 <= 1e-5, fp16 <= 2e-3, bf16 <= 1e-2. Integer-valued
inputs must match bit for bit (every product and partial sum is exact in the
kernels' fp32 accumulators). The im2win pack and the filter staging are pure
copies and must be bit-identical to their definitions.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import cnn_convolution_amd as conv
from cnn_convolution_amd import _lib
import oracle
from oracle.im2win_model import im2win
import workloads
from parity import TOL, check, rel_l2

pytestmark = pytest.mark.gpu

CODE = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()   # the HIP library must load: no fallback


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_conv(x, w, s, p):
    y = conv.conv2d(x.to(DEV), w.to(DEV), stride=s, pad=p)
    torch.cuda.synchronize()
    return y.cpu()


# ----------------------------------------------------------------- pack (a2)

PACK_CASES = [
    # N, C, H, W, KH, KW, s, p
    (2, 3, 8, 9, 3, 3, 1, 1),
    (1, 16, 14, 14, 3, 3, 1, 1),
    (2, 8, 11, 13, 2, 3, 2, 1),
    (1, 3, 23, 21, 7, 7, 2, 3),
    (2, 72, 7, 7, 3, 3, 1, 1),       # two channel blocks, ragged
    (1, 5, 9, 70, 5, 4, 1, 2),       # wide rows: several column blocks
    (3, 64, 6, 6, 1, 1, 1, 0),
    (1, 8, 12, 12, 9, 9, 1, 4),      # KH > 8: two filter-row passes
    (1, 130, 3, 3, 3, 3, 1, 1),      # few rows: channels split over workgroups, ragged last block
    (1, 1, 2, 3, 1, 1, 1, 0),        # fewer than 8 input elements
    (1, 12, 3, 1100, 3, 3, 1, 1),    # long input rows: 8-channel blocks to fit LDS
    (1, 5, 3, 2400, 7, 3, 1, 3),     # rows too long to stage in LDS: tiled form
    (1, 3, 4, 4, 3, 3, 1, 5),        # padding wider than the filter: window rows all padding
    (2, 16, 3, 5, 2, 2, 3, 4),       # stride 3, pad 4: rows and columns all padding
]


@pytest.mark.parametrize("case", PACK_CASES)
@pytest.mark.parametrize("dt,layout", [("f32", conv.LAYOUT_ROW), ("f16", conv.LAYOUT_ROW),
                                        ("f16", conv.LAYOUT_CL), ("bf16", conv.LAYOUT_CL)])
def test_pack_bit_exact(case, dt, layout):
    N, C, H, W, KH, KW, s, p = case
    _say(f"pack {dt} layout={layout} {case}")
    x = workloads.make_tensor((N, C, H, W), "normal", seed=5, dtype=dt)
    xd = x.to(DEV)
    d = conv.describe(tuple(x.shape), (1, C, KH, KW), s, p, CODE[dt])
    total = conv.plan(d).rows_total
    ref, Ho, Wo, Wwin = im2win(x.view(torch.int16 if dt != "f32" else torch.int32).numpy(),
                               KH, KW, s, p, "row" if layout == conv.LAYOUT_ROW else "cl")
    for row0, rows in [(0, total), (total // 3, max(1, total // 2)), (total - 1, 1)]:
        out, geo = conv.pack(xd, KH, KW, s, p, layout, row0, rows)
        torch.cuda.synchronize()
        bits = out.cpu().view(torch.int16 if dt != "f32" else torch.int32).numpy()
        bits = bits.reshape(rows, geo["row_elems"])
        want = ref[row0:row0 + rows]
        if layout == conv.LAYOUT_ROW:
            body = bits[:, :C * geo["pos_pad"]].reshape(rows, C, geo["pos_pad"])
            assert np.array_equal(body[:, :, :Wwin * KH], want)
            assert np.all(body[:, :, Wwin * KH:] == 0)
        else:
            cp = geo["Cin_pad"]
            body = bits[:, :Wwin * KH * cp].reshape(rows, Wwin * KH, cp)
            assert np.array_equal(body[:, :, :C], want)
            assert np.all(body[:, :, C:] == 0)
            assert np.all(bits[:, Wwin * KH * cp:] == 0)


# ----------------------------------------------------------------- filter staging (a3)

@pytest.mark.parametrize("shape", [(16, 3, 3, 3), (20, 5, 2, 3), (64, 3, 7, 7), (40, 72, 3, 3),
                                   (256, 64, 1, 1)])
@pytest.mark.parametrize("dt,layout", [("f32", conv.LAYOUT_ROW), ("f16", conv.LAYOUT_CL),
                                        ("bf16", conv.LAYOUT_CL)])
def test_weight_stage_bit_exact(shape, dt, layout):
    Cout, Cin, KH, KW = shape
    _say(f"weight_stage {dt} layout={layout} {shape}")
    w = workloads.make_tensor(shape, "normal", seed=6, dtype=dt)
    out, geo = conv.weight_stage(w.to(DEV), 1, 1, (16, 16), layout)
    torch.cuda.synchronize()
    ity = torch.int32 if dt == "f32" else torch.int16
    got = out.cpu().view(ity).numpy()
    wb = w.view(ity).numpy()
    if layout == conv.LAYOUT_ROW:
        rows = geo["rows"]
        want = np.zeros((rows, Cin, KH, KW), wb.dtype)
        want[:Cout] = wb
        # [cb][ci][kh][kw][16]: 16 output channels innermost
        want = want.reshape(rows // 16, 16, Cin, KH, KW).transpose(0, 2, 3, 4, 1)
        assert np.array_equal(got, want.reshape(-1))
    else:
        d = conv.describe((1, Cin, 16, 16), shape, 1, 1, CODE[dt])
        cp = conv.plan(d).Cin_pad
        want = np.zeros((Cout, KW, KH, cp), wb.dtype)
        want[:, :, :, :Cin] = wb.transpose(0, 3, 2, 1)       # [co][kw][kh][ci]
        want = want.reshape(Cout, -1)
        full = np.zeros((Cout, geo["row_len"]), wb.dtype)
        full[:, :want.shape[1]] = want
        assert np.array_equal(got.reshape(Cout, -1), full)


# ----------------------------------------------------------------- the convolution

def _random_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        KH, KW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        s = int(rng.integers(1, 4))
        p = int(rng.integers(0, max(KH, KW)))
        H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        if H + 2 * p < KH or W + 2 * p < KW:
            continue
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 40)), H, W,
                    int(rng.integers(1, 150)), KH, KW, s, p))
    return out


FIXED = [
    # N, Cin, H, W, Cout, KH, KW, s, p   -- several tiles plus ragged tails
    (2, 3, 32, 32, 16, 3, 3, 1, 1),
    (3, 64, 17, 19, 70, 3, 3, 1, 1),
    (2, 24, 30, 29, 130, 3, 3, 2, 1),
    (2, 3, 45, 47, 64, 7, 7, 2, 3),
    (1, 40, 15, 15, 96, 5, 5, 1, 2),
    (2, 128, 9, 7, 200, 3, 3, 1, 1),
    (4, 64, 10, 10, 256, 1, 1, 1, 0),
    (1, 5, 13, 11, 9, 2, 4, 3, 2),
    (2, 6, 7, 9, 33, 7, 7, 1, 3),
    (1, 1, 1, 1, 1, 1, 1, 1, 0),
    (1, 2, 1, 1, 3, 3, 3, 1, 1),       # 1x1 image, 3x3 filter, pad 1: one output
    (2, 3, 5, 4, 6, 5, 4, 1, 0),       # dense-as-conv: 1x1 output
    (1, 4, 6, 6, 5, 3, 3, 4, 0),       # stride larger than the filter
    (1, 3, 4, 4, 2, 3, 3, 1, 5),       # padding wider than the filter: zero border
    (1, 5, 3, 2400, 8, 7, 3, 1, 3),    # input rows too long to stage: tiled pack, own staging launch
]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", FIXED + _random_cases(21, 16))
def test_window_form_matches_oracle(shape, dt, monkeypatch):
    """The window form (pack + window-GEMM) on every shape, also where the
    planner would take the implicit form."""
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    _say(f"conv-window {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape), dtype=dt,
                                 w_dist="normal")
    assert conv.plan(conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])).algo == 0
    y = run_conv(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(y, x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", FIXED + _random_cases(21, 16))
def test_conv_matches_oracle(shape, dt):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    _say(f"conv {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape), dtype=dt,
                                 w_dist="normal")
    y = run_conv(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert tuple(y.shape) == ref.shape
    check(y, x, w, s, p, dt, ref=ref)


# The tiled matrix-core GEMM form forced on every shape (the planner takes the
# direct-to-LDS form wherever the window is whole 64-element K stages).
MFMA_FORMS = [
    {"IM2WIN_MFMA_KERNEL": "tiled"},
    {"IM2WIN_MFMA_KERNEL": "tiled", "IM2WIN_MFMA_TILE": "128,64,32,2,2"},
    {"IM2WIN_MFMA_KERNEL": "tiled", "IM2WIN_MFMA_TILE": "64,256,32,1,1"},
]
FORM_SHAPES = [
    (2, 64, 17, 19, 70, 3, 3, 1, 1),    # Cout past one 64-row block, ragged columns
    (2, 3, 45, 47, 64, 7, 7, 2, 3),     # 4 channels per position, 4-value window tail
    (3, 64, 10, 10, 256, 1, 1, 1, 0),   # 1x1: the filter itself is the staged filter
    (1, 5, 13, 11, 9, 2, 4, 3, 2),      # KH != KW, stride 3
    (2, 32, 15, 14, 72, 3, 3, 2, 1),
    (1, 24, 9, 9, 40, 5, 5, 1, 2),      # filter rows of 608 halves
]


@pytest.mark.parametrize("form", MFMA_FORMS, ids=lambda f: "-".join(f.values()).replace(",", "."))
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", FORM_SHAPES)
def test_mfma_forms_match_oracle(shape, dt, form, monkeypatch):
    monkeypatch.setenv("IM2WIN_ALGO", "window")    # the window tensor path, not the implicit form
    for k, v in form.items():
        monkeypatch.setenv(k, v)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    d = conv.describe((N, Cin, H, W), (Cout, Cin, KH, KW), s, p, CODE[dt])
    pl = conv.plan(d)
    assert pl.gemm_kernel == 1
    if "IM2WIN_MFMA_TILE" in form:          # applies when K_stage is a multiple of its K stage
        tile = tuple(int(v) for v in form["IM2WIN_MFMA_TILE"].split(","))
        if pl.K_stage % (tile[2] * tile[3]) == 0:
            assert (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_kslice, pl.gemm_ksplit,
                    pl.gemm_wave_m) == tile
    _say(f"conv-form {form} {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape) + 7, dtype=dt,
                                 w_dist="normal")
    y = run_conv(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(y, x, w, s, p, dt, ref=ref)


# Direct-to-LDS form: windows of whole 64-element K stages. The K-stage counts
# 1, 2, 4, 9 and 18 leave the three-buffer loop after each of its three steps.
DMA_TILES = ["64,128,1", "64,64,2", "128,64,2", "128,128,2", "128,128,1", "64,256,1"]
DMA_SHAPES = [
    (2, 64, 17, 19, 70, 3, 3, 1, 1),    # 9 stages, Cout past one block, ragged columns
    (1, 5, 13, 11, 9, 2, 4, 3, 2),      # 8 padded channels x 8 taps: 1 stage
    (2, 128, 8, 9, 96, 1, 1, 1, 0),     # 1x1, filter used as staged: 2 stages
    (1, 256, 6, 7, 136, 1, 1, 1, 0),    # 4 stages
    (2, 128, 9, 10, 200, 3, 3, 1, 1),   # 18 stages
    (3, 64, 11, 12, 64, 3, 3, 2, 0),    # stride 2
]


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", DMA_SHAPES)
def test_dma_form_matches_oracle(shape, dt, tile, monkeypatch):
    monkeypatch.setenv("IM2WIN_ALGO", "window")    # the window tensor path, not the implicit form
    monkeypatch.setenv("IM2WIN_MFMA_DMA_TILE", tile)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    d = conv.describe((N, Cin, H, W), (Cout, Cin, KH, KW), s, p, CODE[dt])
    pl = conv.plan(d)
    assert pl.gemm_kernel == 3
    assert (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_wave_m) == tuple(int(v) for v in tile.split(","))
    _say(f"conv-dma {tile} {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape) + 11, dtype=dt,
                                 w_dist="normal")
    y = run_conv(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(y, x, w, s, p, dt, ref=ref)


ABLATE = ["serpentine", "dma", "buffers", "serpentine,dma", "dma,buffers", "serpentine,dma,buffers"]


@pytest.mark.parametrize("ablate", ABLATE)
@pytest.mark.parametrize("tile", ["64,128,1", "128,64,2"])
@pytest.mark.parametrize("shape", [DMA_SHAPES[0], DMA_SHAPES[2], DMA_SHAPES[4], DMA_SHAPES[5]])
def test_dma_form_ablations_match_oracle(shape, tile, ablate, monkeypatch):
    """The direct-to-LDS window-GEMM with the page's optimisations turned off
    (plain tile order, copies through registers, one stage buffer) computes
    the same sums in the same order: bit-equal to the planned kernel, and
    within tolerance of the oracle."""
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    monkeypatch.setenv("IM2WIN_MFMA_DMA_TILE", tile)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    d = conv.describe((N, Cin, H, W), (Cout, Cin, KH, KW), s, p, conv.F16)
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape) + 12, dtype="f16",
                                 w_dist="normal")
    assert conv.plan(d).gemm_kernel == 3 and conv.plan(d).gemm_ablate == 0
    base = run_conv(x, w, s, p)
    monkeypatch.setenv("IM2WIN_ABLATE", ablate)
    bits = sum(b for k, b in (("serpentine", 1), ("dma", 2), ("buffers", 4)) if k in ablate)
    assert conv.plan(d).gemm_ablate == bits
    _say(f"conv-dma-ablate {ablate} {tile} {shape}")
    y = run_conv(x, w, s, p)
    assert torch.equal(y, base)
    check(y, x, w, s, p, "f16")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 3, 32, 32, 16, 3, 3, 1, 1), (2, 32, 15, 14, 72, 3, 3, 2, 1),
                                   (1, 3, 30, 30, 64, 7, 7, 2, 3), (2, 64, 8, 8, 128, 1, 1, 1, 0),
                                   (1, 16, 12, 12, 40, 5, 5, 1, 2)])
def test_integer_inputs_bit_exact(shape, dt):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    _say(f"conv-int {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=3, dtype=dt,
                                 x_dist="int3", w_dist="int3")
    y = run_conv(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert np.array_equal(y.numpy().astype(np.float64), ref)


def test_outputs_in_padding_are_exactly_zero():
    x, w = workloads.make_inputs(1, 3, 4, 4, 2, 3, 3, seed=1, dtype="f16")
    y = run_conv(x, w, 1, 5)
    ref = oracle.conv2d(x, w, 1, 5)
    assert np.array_equal(y.numpy() == 0, ref == 0)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_guard_bands_untouched(dt):
    """y and the workspace sit inside larger buffers filled with a canary:
    nothing outside the requested ranges may change."""
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 10, 13, 11, 21, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=2, dtype=dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])
    pl = conv.plan(d)
    ny = N * Cout * pl.Ho * pl.Wo
    guard = 4096
    ybuf = torch.full((guard + ny + guard,), 12345.0, dtype=torch.float32, device=DEV)
    wsbuf = torch.full((guard + pl.ws_bytes + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    y = ybuf[guard:guard + ny]
    ws = wsbuf[guard:guard + pl.ws_bytes]
    assert ws.data_ptr() % 256 == 0
    xd, wd = x.to(DEV), w.to(DEV)
    st = _lib.fwd(d, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), ws.data_ptr(),
                  torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    yb = ybuf.cpu()
    assert torch.all(yb[:guard] == 12345.0) and torch.all(yb[guard + ny:] == 12345.0)
    wb = wsbuf.cpu()
    assert torch.all(wb[:guard] == 0xA5) and torch.all(wb[guard + pl.ws_bytes:] == 0xA5)
    ref = oracle.conv2d(x, w, s, p)
    check(y.reshape(ref.shape), x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_repeatable_bits(dt):
    x, w = workloads.make_inputs(4, 32, 20, 20, 48, 3, 3, seed=4, dtype=dt)
    a = run_conv(x, w, 1, 1)
    b = run_conv(x, w, 1, 1)
    assert torch.equal(a, b)


def test_profile_hook_counts_launches():
    x, w = workloads.make_inputs(2, 16, 12, 12, 32, 3, 3, seed=1, dtype="f16")
    xd, wd = x.to(DEV), w.to(DEV)
    d = conv.describe(tuple(x.shape), tuple(w.shape), 1, 1, conv.F16)
    pl = conv.plan(d)
    conv.profile_read()
    conv.profile_enable(True)
    try:
        conv.conv2d(xd, wd, 1, 1)
        conv.conv2d(xd, wd, 1, 1)
    finally:
        conv.profile_enable(False)
    prof = conv.profile_read()
    assert prof["pack"]["launches"] == 2 * pl.n_chunks
    assert prof["gemm"]["launches"] == 2 * pl.n_chunks
    # the filter staging rides in the first pack launch of each call
    assert prof["weight_stage"]["launches"] == 0
    assert all(v["total_ms"] >= 0 for v in prof.values())


# ----------------------------------------------------------------- full-size layers

def _sample_indices(N, Cout, Ho, Wo, rows_per_chunk, rng, count=3000):
    idx = set(rng.integers(0, N * Cout * Ho * Wo, count).tolist())
    rows = N * Ho
    edge_rows = {0, rows - 1}
    r = rows_per_chunk
    while r < rows:
        edge_rows.update({r - 1, r})
        r += rows_per_chunk
    cos = sorted({0, Cout - 1, Cout // 2} | set(rng.integers(0, Cout, 3).tolist()))
    for rr in edge_rows:
        n, ho = divmod(rr, Ho)
        for co in cos:
            for wo in {0, 1, Wo // 2, Wo - 2, Wo - 1}:
                if 0 <= wo < Wo:
                    idx.add(((n * Cout + co) * Ho + ho) * Wo + wo)
    return np.array(sorted(idx), dtype=np.int64)


FULL = [(name, dt) for name, cfg in sorted(workloads.CONFIGS.items()) for dt in cfg.dtypes]


@pytest.mark.parametrize("name,dt", FULL)
def test_full_size_layers_sampled(name, dt, monkeypatch):
    """At the measured sizes, through the window tensor path (the implicit form
    has its own full-size test): sampled outputs (random, plus borders and
    chunk boundaries) against the oracle computed point by point."""
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    cfg = workloads.get_config(name)
    _say(f"full-size {name} {dt} {cfg.desc()}")
    x, w = workloads.make_config_inputs(cfg, dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad, CODE[dt])
    pl = conv.plan(d)
    assert pl.meets_ws_target == 1 and pl.algo == 0
    y = run_conv(x, w, cfg.stride, cfg.pad)
    ho, wo = cfg.out_hw()
    assert tuple(y.shape) == (cfg.N, cfg.Cout, ho, wo)
    yf = y.numpy().reshape(-1)
    assert np.isfinite(yf).all()
    rng = np.random.default_rng(cfg.seed)
    idx = _sample_indices(cfg.N, cfg.Cout, ho, wo, pl.rows_per_chunk, rng)
    check(yf[idx], x, w, cfg.stride, cfg.pad, dt, idx=idx, what=f"{name} {dt}")


# ----------------------------------------------------------------- Table I layers of the im2win paper

@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("name", list(workloads.TABLE1))
def test_table1_layers_small_batch(name, dt):
    """Every Table I layer (its shape, stride and no padding) at N=2, element by
    element against the oracle."""
    cfg = workloads.TABLE1[name]
    _say(f"table1 {name} {dt} N=2")
    x, w = workloads.make_inputs(2, cfg.Cin, cfg.H, cfg.W, cfg.Cout, cfg.KH, cfg.KW,
                                 seed=cfg.seed, dtype=dt, x_dist=cfg.x_dist, w_dist=cfg.w_dist)
    y = run_conv(x, w, cfg.stride, cfg.pad)
    ref = oracle.conv2d(x, w, cfg.stride, cfg.pad)
    assert tuple(y.shape) == ref.shape
    check(y, x, w, cfg.stride, cfg.pad, dt, ref=ref)


@pytest.mark.parametrize("name,dt", [("cv4", "f16"), ("cv1", "f32")])
def test_table1_full_batch_sampled(name, dt):
    """Table I layers at the paper's batch (N=256): a multi-GB window tensor in
    several chunks (cv4), and stride 4 with an 11x11 filter in five chunks
    (cv1); sampled outputs, chunk boundaries included, against the oracle."""
    cfg = workloads.TABLE1[name]
    _say(f"table1 full batch {name} {dt} {cfg.desc()}")
    x, w = workloads.make_config_inputs(cfg, dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad, CODE[dt])
    pl = conv.plan(d)
    assert pl.meets_ws_target == 1 and pl.n_chunks >= 3
    y = run_conv(x, w, cfg.stride, cfg.pad)
    ho, wo = cfg.out_hw()
    assert tuple(y.shape) == (cfg.N, cfg.Cout, ho, wo)
    yf = y.numpy().reshape(-1)
    rng = np.random.default_rng(cfg.seed)
    idx = _sample_indices(cfg.N, cfg.Cout, ho, wo, pl.rows_per_chunk, rng)
    assert np.isfinite(yf[idx]).all()
    check(yf[idx], x, w, cfg.stride, cfg.pad, dt, idx=idx, what=f"{name} {dt}")


# ----------------------------------------------------------------- window-GEMM alone (a4, a5)

def _host_window_rows(x, d, pl, row0, rows):
    """The window rows in the plan's padded layout, built on the host from the
    oracle's model of the transform (values copied as raw bits)."""
    ity = torch.int32 if x.dtype == torch.float32 else torch.int16
    bits = x.view(ity).numpy()
    layout = "row" if pl.layout == conv.LAYOUT_ROW else "cl"
    t, Ho, Wo, Wwin = im2win(bits, d.KH, d.KW, d.stride, d.pad, layout)
    t = t[row0:row0 + rows]
    out = np.zeros((rows, pl.row_elems), dtype=bits.dtype)
    if layout == "row":
        body = out[:, :d.Cin * pl.pos_pad].reshape(rows, d.Cin, pl.pos_pad)
        body[:, :, :Wwin * d.KH] = t
    else:
        body = out[:, :Wwin * d.KH * pl.Cin_pad].reshape(rows, Wwin * d.KH, pl.Cin_pad)
        body[:, :, :d.Cin] = t
    return torch.from_numpy(out.reshape(-1)).view(x.dtype)


def _host_staged_filter(w, d, pl):
    ity = torch.int32 if w.dtype == torch.float32 else torch.int16
    wb = w.view(ity).numpy()
    Cout, Cin, KH, KW = wb.shape
    if pl.layout == conv.LAYOUT_ROW:
        rows = pl.Cout_stage
        full = np.zeros((rows, Cin, KH, KW), wb.dtype)
        full[:Cout] = wb
        out = full.reshape(rows // 16, 16, Cin, KH, KW).transpose(0, 2, 3, 4, 1).reshape(-1)
    else:
        cw = np.zeros((Cout, KW, KH, pl.Cin_pad), wb.dtype)
        cw[:, :, :, :Cin] = wb.transpose(0, 3, 2, 1)
        out = np.zeros((Cout, pl.K_stage), wb.dtype)
        out[:, :KW * KH * pl.Cin_pad] = cw.reshape(Cout, -1)
        out = out.reshape(-1)
    return torch.from_numpy(np.ascontiguousarray(out)).view(w.dtype)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 16, 12, 13, 40, 3, 3, 1, 1), (1, 3, 23, 21, 64, 7, 7, 2, 3),
                                   (2, 64, 9, 9, 130, 3, 3, 2, 1), (1, 24, 10, 10, 20, 5, 3, 1, 2)])
def test_window_gemm_alone(shape, dt):
    """The GEMM entry point on a window tensor packed on the host by the
    oracle's model: the rows it is given are written, the others are not."""
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    _say(f"window_gemm {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=7, dtype=dt, w_dist="normal")
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])
    pl = conv.plan(d)
    ref = oracle.conv2d(x, w, s, p)
    total = pl.rows_total
    row0, rows = total // 3, max(1, total // 2)
    win = _host_window_rows(x, d, pl, row0, rows).to(DEV)
    wst = (_host_staged_filter(w, d, pl) if pl.wstage_bytes else w.reshape(-1)).to(DEV)
    y = torch.full((N, Cout, pl.Ho, pl.Wo), 777.0, dtype=torch.float32, device=DEV)
    conv.window_gemm(win, wst, y, d, row0, rows)
    torch.cuda.synchronize()
    got = y.cpu().numpy().transpose(0, 2, 1, 3).reshape(total, Cout, pl.Wo)
    sel = slice(row0, row0 + rows)
    # the rows given, as flat output indices of y, against the oracle point by point
    flat = np.arange(N * Cout * pl.Ho * pl.Wo, dtype=np.int64).reshape(N, Cout, pl.Ho, pl.Wo)
    idx = flat.transpose(0, 2, 1, 3).reshape(total, Cout, pl.Wo)[sel].reshape(-1)
    check(got[sel].reshape(-1), x, w, s, p, dt, idx=idx)
    outside = np.ones(total, bool)
    outside[sel] = False
    assert np.all(got[outside] == 777.0)
