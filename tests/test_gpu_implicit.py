"""GPU parity of the implicit form (conv2d_fwd_implicit: window rows built in
LDS straight from x, no window tensor) against the CPU oracle, through the C
ABI. Same tolerances as the two-kernel path: relative L2 over the compared
outputs <= 2e-3 (fp16) and <= 1e-2 (bf16), oracle in float64 on the same
rounded inputs; integer-valued inputs bit for bit."""
import sys

import numpy as np
import pytest
import torch

import cnn_convolution_amd as conv
from cnn_convolution_amd import _lib
import oracle
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


def run_implicit(x, w, s, p):
    y = conv.conv2d_implicit(x.to(DEV), w.to(DEV), stride=s, pad=p)
    torch.cuda.synchronize()
    return y.cpu()


# N, Cin, H, W, Cout, KH, KW, s, p: several tiles, ragged rows/columns/channels
SHAPES = [
    (2, 64, 9, 10, 70, 3, 3, 1, 1),      # Cout past one 64-row block
    (1, 128, 6, 7, 40, 1, 1, 1, 0),      # 1x1: the filter is used as staged; two channel blocks
    (2, 64, 11, 12, 130, 3, 3, 2, 0),    # stride 2, three M blocks
    (1, 64, 9, 9, 20, 5, 5, 1, 2),       # 5x5
    (1, 64, 5, 40, 8, 3, 3, 1, 1),       # one image row of tiles
    (1, 64, 3, 3, 3, 3, 3, 1, 5),        # padding wider than the filter: zero border
    (2, 192, 8, 8, 96, 3, 3, 1, 1),      # three channel blocks: the patch is rebuilt twice
    (1, 64, 12, 140, 16, 3, 3, 1, 1),    # output rows wider than one tile: column tiles
    (1, 64, 16, 16, 64, 7, 7, 2, 3),     # 7x7 stride 2
    (1, 64, 8, 11, 24, 2, 4, 3, 2),      # KH != KW, stride 3
]
TILES = [None, "64,64,1,1,16", "128,128,2,3,8", "128,64,2,2,5", "64,128,1,4,9"]


@pytest.mark.parametrize("tile", TILES, ids=lambda t: "planned" if t is None else t.replace(",", "."))
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_implicit_matches_oracle(shape, dt, tile, monkeypatch):
    if tile is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_TILE", tile)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    d = conv.describe((N, Cin, H, W), (Cout, Cin, KH, KW), s, p, CODE[dt])
    pl = conv.implicit_plan(d)
    if tile is not None:
        want = tuple(int(v) for v in tile.split(","))
        got = (pl.tile_m, pl.tile_n, pl.wave_m, pl.rows_per_tile, pl.cols_per_tile)
        assert got == want
    _say(f"implicit {tile} {dt} {shape} tiles={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape) + 5, dtype=dt,
                                 w_dist="normal")
    y = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert tuple(y.shape) == ref.shape
    check(y, x, w, s, p, dt, ref=ref)


# the streamed implicit kernel forced on short-K and many-tile shapes
FS_SHAPES = [
    (2, 64, 9, 10, 70, 3, 3, 1, 1),      # two 64-row filter blocks
    (4, 64, 66, 20, 256, 3, 3, 1, 1),    # more tiles than workgroups: several tiles per workgroup
    (8, 64, 56, 56, 64, 3, 3, 1, 1),     # the ResNet layer's shape at N=8
    (3, 256, 20, 9, 130, 1, 1, 1, 0),    # 1x1, four channel blocks, ragged Cout
    (2, 128, 5, 9, 20, 1, 1, 1, 0),      # 1x1, two channel blocks
    (3, 64, 4, 4, 200, 1, 1, 2, 1),      # 1x1 with stride and padding: zero border outputs
    (1, 64, 5, 70, 8, 3, 3, 1, 1),       # column tiles along wo
    (2, 64, 11, 12, 30, 3, 3, 2, 0),     # stride 2
    (1, 64, 3, 3, 3, 3, 3, 1, 5),        # padding wider than the filter
    # input rows a multiple of 8 long: the patch loaded as 16-byte row chunks
    (2, 64, 9, 16, 70, 3, 3, 1, 1),
    (1, 64, 5, 72, 8, 3, 3, 1, 1),       # column tiles along wo
    (1, 64, 3, 8, 3, 3, 3, 1, 5),        # padding wider than the image: zero columns on both sides
    (3, 64, 4, 8, 200, 1, 1, 2, 1),
    (1, 256, 4, 16, 65, 1, 1, 1, 0),
    (2, 64, 40, 24, 256, 3, 3, 1, 1),
]


@pytest.mark.parametrize("kernel", ["streamed"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", FS_SHAPES)
def test_streamed_kernel_forced_matches_oracle(shape, dt, kernel, monkeypatch):
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", kernel)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    d = conv.describe((N, Cin, H, W), (Cout, Cin, KH, KW), s, p, CODE[dt])
    pl = conv.implicit_plan(d)
    assert pl.kernel == 0
    _say(f"implicit-{kernel} {dt} {shape} workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=sum(shape) + 13, dtype=dt,
                                 w_dist="normal")
    y = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(y, x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 64, 9, 10, 70, 3, 3, 1, 1), (2, 128, 7, 6, 33, 3, 3, 2, 1),
                                   (1, 64, 12, 12, 64, 1, 1, 1, 0), (4, 64, 66, 20, 256, 3, 3, 1, 1)])
def test_implicit_integer_inputs_bit_exact(shape, dt):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    _say(f"implicit-int {dt} {shape}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=4, dtype=dt,
                                 x_dist="int3", w_dist="int3")
    y = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert np.array_equal(y.numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_implicit_agrees_with_two_kernel_path(dt, monkeypatch):
    """Same inputs through both forms: each against the oracle, and close to each other."""
    shape = (2, 128, 10, 9, 80, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=9, dtype=dt, w_dist="normal")
    xd, wd = x.to(DEV), w.to(DEV)
    a = conv.conv2d_implicit(xd, wd, s, p)
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    assert conv.plan(conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])).algo == 0
    b = conv.conv2d(xd, wd, s, p)
    torch.cuda.synchronize()
    ref = oracle.conv2d(x, w, s, p)
    check(a, x, w, s, p, dt, ref=ref)
    check(b, x, w, s, p, dt, ref=ref)
    assert rel_l2(a.cpu().numpy(), b.cpu().numpy()) <= TOL[dt]


def test_implicit_leaves_memory_past_y_untouched():
    """The kernel stores exactly the N*Cout*Ho*Wo outputs: a guard band after y
    keeps its sentinel."""
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 64, 9, 10, 70, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=2, dtype="f16")
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.F16)
    pl = conv.implicit_plan(d)
    n_out = N * Cout * pl.Ho * pl.Wo
    buf = torch.full((n_out + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(pl.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    conv.conv2d_implicit_into(x.to(DEV), w.to(DEV), buf, ws, s, p)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[n_out:] == 12345.0).all()
    ref = oracle.conv2d(x, w, s, p).reshape(-1)
    check(host[:n_out], x, w, s, p, "f16", ref=ref)


def test_implicit_profile_hook_counts_launches():
    x, w = workloads.make_inputs(2, 64, 8, 8, 32, 3, 3, seed=1, dtype="f16")
    xd, wd = x.to(DEV), w.to(DEV)
    conv.conv2d_implicit(xd, wd, 1, 1)
    torch.cuda.synchronize()
    conv.profile_read()
    conv.profile_enable(True)
    try:
        conv.conv2d_implicit(xd, wd, 1, 1)
        conv.conv2d_implicit(xd, wd, 1, 1)
    finally:
        conv.profile_enable(False)
    prof = conv.profile_read()
    assert prof["implicit"]["launches"] == 2
    # the filter staging runs only where the plan keeps a staged filter in ws
    staged = conv.implicit_plan(conv.describe(tuple(x.shape), tuple(w.shape), 1, 1, conv.F16)).ws_bytes > 0
    assert prof["weight_stage"]["launches"] == (2 if staged else 0)
    assert prof["pack"]["launches"] == 0 and prof["gemm"]["launches"] == 0


def _sample_indices(N, Cout, Ho, Wo, rng, count=3000):
    idx = set(rng.integers(0, N * Cout * Ho * Wo, count).tolist())
    cos = sorted({0, Cout - 1, Cout // 2} | set(rng.integers(0, Cout, 3).tolist()))
    for n in {0, N - 1}:
        for ho in {0, 1, Ho // 2, Ho - 1}:
            for co in cos:
                for wo in {0, 1, Wo // 2, Wo - 2, Wo - 1}:
                    if 0 <= wo < Wo and 0 <= ho < Ho:
                        idx.add(((n * Cout + co) * Ho + ho) * Wo + wo)
    return np.array(sorted(idx), dtype=np.int64)


def _eligible_configs():
    out = []
    for name, cfg in sorted(workloads.CONFIGS.items()):
        for dt in cfg.dtypes:
            if (dt != "f32" and cfg.Cin % 64 == 0) or (name, dt) == ("resnet3x3", "f32"):
                out.append((name, dt))
    for name in ("cv4", "cv6", "cv8", "cv10", "cv11", "cv12"):
        out.append((name, "f16"))
    return out


def test_conv2d_fwd_runs_the_planned_form(monkeypatch):
    """conv2d_fwd follows the plan's algo: the implicit form's kernel for a layer
    it is planned for, pack + window-GEMM when the window form is forced."""
    x, w = workloads.make_inputs(2, 64, 10, 10, 32, 3, 3, seed=6, dtype="f16")
    xd, wd = x.to(DEV), w.to(DEV)
    d = conv.describe(tuple(x.shape), tuple(w.shape), 1, 1, conv.F16)
    ref = oracle.conv2d(x, w, 1, 1)
    for algo, kind in (("implicit", "implicit"), ("window", "gemm")):
        monkeypatch.setenv("IM2WIN_ALGO", algo)
        pl = conv.plan(d)
        assert pl.algo == (1 if algo == "implicit" else 0)
        conv.conv2d(xd, wd, 1, 1)
        torch.cuda.synchronize()
        conv.profile_read()
        conv.profile_enable(True)
        try:
            y = conv.conv2d(xd, wd, 1, 1)
        finally:
            conv.profile_enable(False)
        prof = conv.profile_read()
        assert prof[kind]["launches"] >= 1
        other = "gemm" if kind == "implicit" else "implicit"
        assert prof[other]["launches"] == 0
        check(y, x, w, 1, 1, "f16", ref=ref)


def test_implicit_kernel_alone_with_staged_filter(monkeypatch):
    """im2win_implicit_gemm on a filter staged by im2win_weight_stage (the
    streamed kernel, whose plan keeps a staged filter)."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "streamed")
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 128, 9, 8, 40, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=8, dtype="bf16")
    xd, wd = x.to(DEV), w.to(DEV)
    wst, _ = conv.weight_stage(wd, s, p, (H, W), conv.LAYOUT_CL)
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.BF16)
    pl = conv.implicit_plan(d)
    assert pl.kernel == 0 and conv.implicit_workspace_size(d) > 0
    y = torch.empty((N, Cout, pl.Ho, pl.Wo), dtype=torch.float32, device=DEV)
    conv.implicit_gemm(xd, wst, y, d)
    torch.cuda.synchronize()
    ref = oracle.conv2d(x, w, s, p)
    check(y, x, w, s, p, "bf16", ref=ref)


@pytest.mark.parametrize("name,dt", _eligible_configs())
def test_implicit_full_size_sampled(name, dt):
    """At the measured sizes, with the launch configuration the benchmark times:
    sampled outputs (random, borders, first and last image) against the oracle
    point by point."""
    cfg = workloads.get_config(name)
    _say(f"implicit full-size {name} {dt} {cfg.desc()}")
    x, w = workloads.make_config_inputs(cfg, dt)
    y = run_implicit(x, w, cfg.stride, cfg.pad)
    ho, wo = cfg.out_hw()
    assert tuple(y.shape) == (cfg.N, cfg.Cout, ho, wo)
    yf = y.numpy().reshape(-1)
    rng = np.random.default_rng(cfg.seed + 1)
    idx = _sample_indices(cfg.N, cfg.Cout, ho, wo, rng)
    assert np.isfinite(yf[idx]).all()
    check(yf[idx], x, w, cfg.stride, cfg.pad, dt, idx=idx, what=f"{name} {dt}")


# row-block kernel (64 input channels, stride 1, W % 8 == 0, Wo <= 64, 3x3 or
# 1x1): whole output rows per workgroup, raw filter and input rows in LDS
ROWS_SHAPES = [
    (2, 64, 10, 16, 40, 3, 3, 1, 1),     # Cout inside one 64-channel block
    (3, 64, 13, 24, 130, 3, 3, 1, 1),    # three channel blocks, the last ragged
    (1, 64, 9, 64, 16, 3, 3, 1, 1),      # 64 output columns: every column of a wave real
    (2, 64, 11, 16, 24, 3, 3, 1, 0),     # no padding: Wo = 14, columns not a multiple of 4
    (1, 64, 6, 8, 8, 3, 3, 1, 2),        # padding 2: zero rows and columns around a small image
    (1, 64, 5, 56, 72, 3, 3, 1, 3),      # padding wider than the filter: zero border rows
    (2, 64, 7, 8, 200, 1, 1, 1, 0),      # 1x1
    (1, 64, 9, 24, 64, 1, 1, 1, 1),      # 1x1 with padding: zero border outputs
]


# fp32 (channel blocks of 32, W % 4 == 0): more channel blocks, rows of 4k columns
ROWS_SHAPES_F32 = [
    (2, 32, 9, 12, 40, 3, 3, 1, 1),      # one 32-channel block, W = 12
    (1, 96, 7, 20, 70, 3, 3, 1, 0),      # three blocks, Wo = 18
    (2, 128, 6, 28, 64, 1, 1, 1, 0),     # 1x1, four blocks
    (1, 64, 5, 4, 16, 3, 3, 1, 2),       # W = 4: one chunk per row, padding 2
    # rows of any width (gathered 4 channels of one position at a time)
    (2, 64, 14, 14, 72, 3, 3, 1, 1),     # the deep layer's 14x14 image
    (1, 96, 13, 15, 40, 3, 3, 1, 0),     # 11x13 outputs
    (2, 32, 18, 18, 16, 1, 1, 1, 0),     # 1x1
    (1, 32, 17, 9, 24, 3, 3, 1, 2),      # padding 2: rows outside the image, 19x11 outputs
]


# half precision over several 64-channel blocks, and rows of any width (the
# deep 3x3 layers); images of at least 128 outputs
ROWS_SHAPES_MULTI = [
    (2, 256, 14, 14, 72, 3, 3, 1, 1),    # the deep layer's image: 4 channel blocks, 14-wide rows (gathered)
    (1, 128, 16, 14, 130, 3, 3, 1, 0),   # two blocks, 14x12 outputs, three channel blocks of Cout
    (2, 192, 12, 16, 64, 3, 3, 1, 1),    # three blocks, 16-wide rows (16-byte chunks)
    (1, 128, 14, 18, 40, 1, 1, 1, 0),    # 1x1 over two blocks, 18-wide rows
    (2, 64, 12, 12, 16, 3, 3, 1, 1),     # one block, 12-wide rows: the gathering loader
]

ROWS_CASES = [(s, dt) for dt in ("f32", "f16", "bf16") for s in ROWS_SHAPES] + \
             [(s, "f32") for s in ROWS_SHAPES_F32] + \
             [(s, dt) for dt in ("f16", "bf16") for s in ROWS_SHAPES_MULTI]


@pytest.mark.parametrize("shape,dt", ROWS_CASES, ids=[f"{dt}-{s}" for s, dt in ROWS_CASES])
@pytest.mark.parametrize("rw", [None, 1, 3, 8])
def test_row_block_kernel_matches_oracle(shape, dt, rw, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    if rw is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rw))
    d = conv.make_desc(*shape, CODE[dt])
    pl = conv.implicit_plan(d)
    assert pl.kernel == 2 and pl.ws_bytes == 0
    if rw is not None:
        assert pl.rows_per_tile == min(rw, pl.Ho)
    _say(f"implicit-rows {dt} {shape} rows/block={pl.rows_per_tile} workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=21, dtype=dt)
    got = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(got, x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("shape", ROWS_SHAPES[:4] + ROWS_SHAPES[6:7], ids=[str(s) for s in ROWS_SHAPES[:4] + ROWS_SHAPES[6:7]])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_row_block_kernel_integer_inputs_exact(shape, dt, monkeypatch):
    """Integer-valued inputs: every product and partial sum is exact in fp32,
    so the row-block kernel matches the oracle bit for bit."""
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=22, dtype=dt,
                                 x_dist="int3", w_dist="int3")
    assert conv.implicit_plan(conv.make_desc(*shape, CODE[dt])).kernel == 2
    got = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_row_block_kernel_leaves_memory_past_y_untouched(dt, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 64, 9, 16, 70, 3, 3, 1, 0
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=23, dtype=dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])
    pl = conv.implicit_plan(d)
    assert pl.kernel == 2
    n_out = N * Cout * pl.Ho * pl.Wo
    buf = torch.full((n_out + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    conv.conv2d_implicit_into(x.to(DEV), w.to(DEV), buf, None, s, p)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[n_out:] == 12345.0).all()
    check(host[:n_out], x, w, s, p, dt)


def test_row_block_kernel_agrees_with_streamed_kernel(monkeypatch):
    """The ResNet-style layer at full size, both implicit kernels, element by
    element (each is checked against the oracle on sampled outputs elsewhere)."""
    x, w = workloads.make_config_inputs(workloads.get_config("resnet3x3"), "f16")
    xd, wd = x.to(DEV), w.to(DEV)
    a = conv.conv2d_implicit(xd, wd, 1, 1)
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "streamed")
    b = conv.conv2d_implicit(xd, wd, 1, 1)
    torch.cuda.synchronize()
    assert rel_l2(a.cpu().numpy(), b.cpu().numpy()) <= 1e-6


# narrow-channel kernel (Cin <= 8, any filter and stride): window rows built in
# LDS channels-last, CP = 4 (or 8) channels per position
NARROW_SHAPES = [
    (2, 3, 30, 30, 64, 7, 7, 2, 3),      # the stem's geometry, small image
    (1, 3, 35, 35, 96, 11, 11, 4, 0),    # 11x11 stride 4, two channel blocks of Cout (ragged)
    (2, 3, 20, 22, 16, 3, 3, 1, 1),      # stride 1, KH odd: CP = 8 in half precision
    (1, 1, 9, 13, 8, 5, 3, 2, 2),        # one channel, KH != KW
    (2, 8, 11, 10, 70, 3, 3, 1, 1),      # eight channels: CP = 8
    (1, 5, 7, 9, 20, 2, 4, 3, 1),        # five channels, stride 3
    (1, 3, 4, 4, 2, 3, 3, 1, 5),         # padding wider than the filter: zero border
    (2, 2, 5, 4, 6, 5, 4, 1, 0),         # dense-as-conv: one output per image
    (1, 3, 6, 600, 12, 3, 3, 2, 1),      # 300 outputs per row: one row per workgroup
    (9, 3, 130, 128, 40, 3, 3, 1, 1),    # more than 256 one-block workgroups in half precision: staged filter
]


@pytest.mark.parametrize("shape", NARROW_SHAPES, ids=[str(s) for s in NARROW_SHAPES])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows", [None, 1, 3])
def test_narrow_kernel_matches_oracle(shape, dt, rows, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    if rows is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rows))
    d = conv.make_desc(*shape, CODE[dt])
    pl = conv.implicit_plan(d)
    # the filter gathered from w by launches of at most 256 workgroups, else staged
    assert pl.kernel == 3 and (pl.ws_bytes == 0) == (pl.tiles <= 256) and conv.plan(d).algo == 1
    _say(f"implicit-narrow {dt} {shape} rows/block={pl.rows_per_tile} cp={pl.stages} workgroups={pl.tiles}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=31, dtype=dt, w_dist="normal")
    got = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    assert tuple(got.shape) == ref.shape
    check(got, x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("shape", NARROW_SHAPES[:5], ids=[str(s) for s in NARROW_SHAPES[:5]])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_narrow_kernel_integer_inputs_exact(shape, dt):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=32, dtype=dt,
                                 x_dist="int3", w_dist="int3")
    got = run_implicit(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(x, w, s, p))


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_narrow_kernel_leaves_memory_past_y_untouched(dt):
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 3, 17, 19, 70, 7, 7, 2, 3
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=33, dtype=dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[dt])
    pl = conv.implicit_plan(d)
    assert pl.kernel == 3
    n_out = N * Cout * pl.Ho * pl.Wo
    buf = torch.full((n_out + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(pl.ws_bytes, dtype=torch.uint8, device=DEV) if pl.ws_bytes else None
    conv.conv2d_implicit_into(x.to(DEV), w.to(DEV), buf, ws, s, p)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[n_out:] == 12345.0).all()
    check(host[:n_out], x, w, s, p, dt)


# 4 channels per position on rows of 4k elements: window rows written from
# whole input rows (each input row into every window row that interleaves
# it), padding columns zeroed apart; in fp32 also in the persistent form
NARROW_ROWVEC = [
    (2, 3, 28, 32, 64, 7, 7, 2, 3),      # the stem's geometry: 3 zero columns left, 2 right
    (1, 4, 12, 16, 24, 5, 5, 2, 0),      # four real channels; input column 15 in no window
    (2, 2, 9, 8, 16, 3, 3, 2, 2),        # two channels, rows above and below the image
    (3, 1, 10, 12, 8, 1, 1, 2, 0),       # 1x1 stride 2: every other input row unused
    (1, 3, 9, 1000, 8, 9, 9, 2, 0),      # 9 x 250 row units: three rounds per thread
    (20, 3, 64, 64, 64, 7, 7, 2, 3),     # more than 256 workgroups: the staged filter (half), persistent (fp32)
    (1, 3, 600, 600, 8, 7, 7, 2, 0),     # 297 row blocks of two unit rounds each: persistent in fp32
]


# (the 9x9 filter's 999-column window rows do not fit LDS in fp32)
ROWVEC_CASES = [(s, dt) for s in NARROW_ROWVEC for dt in ("f16", "bf16", "f32")
                if not (dt == "f32" and s[3] == 1000)]


@pytest.mark.parametrize("shape,dt", ROWVEC_CASES, ids=[f"{d}-{s}" for s, d in ROWVEC_CASES])
@pytest.mark.parametrize("rows", [None, 2, 3])
def test_narrow_kernel_from_whole_input_rows(shape, dt, rows, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    if rows is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rows))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 3 and pl.stages == 4 and W % 4 == 0
    _say(f"implicit-narrow rows {dt} {shape} rows/block={pl.rows_per_tile} workgroups={pl.tiles}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=35, dtype=dt, w_dist="normal")
    got = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(got, x, w, s, p, dt, ref=ref)
    xi, wi = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=36, dtype=dt, x_dist="int3", w_dist="int3")
    assert np.array_equal(run_implicit(xi, wi, s, p).numpy().astype(np.float64), oracle.conv2d(xi, wi, s, p))


# the narrow kernel's two launch forms and its multi-round window loads:
# persistent workgroups (fp32, or filter blocks over 48 KB) walking several
# row blocks with the next block's gathers prefetched, and window rows whose
# gathers take more than one round per thread
NARROW_PERSISTENT = [
    ((64, 3, 16, 16, 16, 3, 3, 1, 1), "f32", 1),       # 1024 row blocks, one per output row
    ((32, 3, 47, 47, 96, 11, 11, 4, 0), "f16", 1),     # 11x11: a 64 KB filter block, two channel blocks
    ((32, 3, 47, 47, 96, 11, 11, 4, 0), "bf16", 2),
    ((1, 3, 9, 1000, 8, 9, 9, 2, 0), "f16", None),     # 9 x 999 window positions: two gather rounds
    ((1, 6, 9, 600, 8, 7, 7, 3, 1), "bf16", None),     # 8 channels per position: two rounds of 8 units
]


@pytest.mark.parametrize("shape,dt,rows", NARROW_PERSISTENT, ids=[f"{d}-{s}-r{r}" for s, d, r in NARROW_PERSISTENT])
def test_narrow_kernel_persistent_and_multiround(shape, dt, rows, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    if rows is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rows))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 3
    row_blocks = N * -(-pl.Ho // pl.rows_per_tile)
    _say(f"implicit-narrow {dt} {shape} workgroups={pl.tiles} row blocks={row_blocks}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=34, dtype=dt, w_dist="normal")
    got = run_implicit(x, w, s, p)
    ref = oracle.conv2d(x, w, s, p)
    check(got, x, w, s, p, dt, ref=ref)


@pytest.mark.parametrize("shape", ROWS_SHAPES_MULTI, ids=[str(s) for s in ROWS_SHAPES_MULTI])
def test_row_block_multi_integer_inputs_exact(shape, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    assert conv.implicit_plan(conv.make_desc(*shape, conv.F16)).kernel == 2
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=24, dtype="f16",
                                 x_dist="int3", w_dist="int3")
    got = run_implicit(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(x, w, s, p))


# pipelined row-block kernels (fp16/bf16, Cin % 32 == 0, stride 1, 3x3 or 1x1,
# Wo <= 256) over 32-channel K chunks: "pipe", persistent workgroups whose
# four loader waves fill one of two LDS slots while four waves contract the
# other; "pair", one task and one slot per workgroup, two workgroups per CU
PIPE_SHAPES = [
    (2, 32, 10, 16, 40, 3, 3, 1, 1),     # one chunk; planes of 8k positions (16-byte loads)
    (2, 64, 14, 14, 72, 3, 3, 1, 1),     # planes of 4k positions (8-byte loads), Cout past one block
    (1, 96, 9, 13, 64, 3, 3, 1, 0),      # odd planes (2-byte loads), three chunks, Wo = 11
    (3, 128, 12, 20, 130, 1, 1, 1, 0),   # 1x1, three blocks of Cout
    (1, 64, 6, 8, 8, 3, 3, 1, 2),        # padding 2: zero rows and columns
    (1, 64, 5, 56, 72, 3, 3, 1, 3),      # padding wider than the filter: tasks with no input row
    (2, 256, 14, 14, 256, 3, 3, 1, 1),   # the deep 3x3 layer's image, eight chunks
    (1, 32, 5, 160, 16, 3, 3, 1, 1),     # 160-column output rows (10 blocks per row)
    (1, 64, 9, 24, 64, 1, 1, 1, 1),      # 1x1 with padding: zero border outputs
    (8, 64, 8, 4, 64, 1, 1, 1, 2),       # 1x1 pad 2: the last row tasks lie below the image
    (2, 64, 6, 6, 72, 3, 3, 1, 4),       # 3x3 pad 4: row tasks above and below the image
]
PIPE_CASES = [(s, dt, k) for k in ("pipe", "pair") for dt in ("f16", "bf16") for s in PIPE_SHAPES]


@pytest.mark.parametrize("shape,dt,form", PIPE_CASES, ids=[f"{k}-{dt}-{s}" for s, dt, k in PIPE_CASES])
@pytest.mark.parametrize("rw", [None, 1, 3])
def test_pipelined_kernel_matches_oracle(shape, dt, form, rw, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    if rw is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rw))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 4 and pl.ws_bytes == 0 and pl.stages == (2 if form == "pipe" else 1)
    if rw is not None and rw * pl.Wo <= 256:     # else the override is ignored
        assert pl.rows_per_tile == min(rw, pl.Ho)
    _say(f"implicit-{form} {dt} {shape} rows/task={pl.rows_per_tile} workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=25, dtype=dt)
    got = run_implicit(x, w, s, p)
    check(got, x, w, s, p, dt)


@pytest.mark.parametrize("form", ["pipe", "pair"])
@pytest.mark.parametrize("shape", PIPE_SHAPES[:6], ids=[str(s) for s in PIPE_SHAPES[:6]])
def test_pipelined_kernel_integer_inputs_exact(shape, form, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    assert conv.implicit_plan(conv.make_desc(*shape, conv.F16)).kernel == 4
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=26, dtype="f16",
                                 x_dist="int3", w_dist="int3")
    got = run_implicit(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(x, w, s, p))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_pipelined_kernel_several_tasks_per_workgroup(dt, monkeypatch):
    """More tasks than workgroups (one output row per task): each persistent
    workgroup carries its chunk pipeline across task boundaries."""
    shape = (4, 64, 30, 30, 256, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "pipe")
    monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", "1")
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    tasks = 4 * N * pl.Ho
    assert pl.kernel == 4 and pl.tiles == 256 and tasks > pl.tiles
    _say(f"implicit-pipe {dt} {shape} tasks={tasks} workgroups={pl.tiles}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=27, dtype=dt)
    got = run_implicit(x, w, s, p)
    check(got, x, w, s, p, dt)


@pytest.mark.parametrize("form", ["pipe", "pair"])
def test_pipelined_kernel_leaves_memory_past_y_untouched(form, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 64, 9, 13, 70, 3, 3, 1, 0
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=28, dtype="f16")
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.F16)
    pl = conv.implicit_plan(d)
    assert pl.kernel == 4
    n_out = N * Cout * pl.Ho * pl.Wo
    buf = torch.full((n_out + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    conv.conv2d_implicit_into(x.to(DEV), w.to(DEV), buf, None, s, p)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[n_out:] == 12345.0).all()
    check(host[:n_out], x, w, s, p, "f16")


# tasks of several whole images (small images: fewer than 128 outputs each),
# their patches stacked in LDS; the last task of a layer may hold fewer images
PIPE_IMAGE_SHAPES = [
    (6, 64, 7, 7, 72, 3, 3, 1, 1),       # 49 outputs per image, Cout past one block
    (9, 96, 5, 6, 40, 3, 3, 1, 0),       # 3x4 outputs, odd planes (2-byte loads), Wo = 4
    (5, 32, 4, 4, 130, 1, 1, 1, 0),      # 1x1, 16 outputs, three blocks of Cout
    (4, 64, 12, 12, 64, 3, 3, 1, 0),     # 10x10 outputs
    (7, 128, 7, 7, 512, 3, 3, 1, 1),     # the 512-channel 7x7 layer's shape with 128 channels
]
PIPE_IMAGE_CASES = [(s, dt, k, im) for k in ("pipe", "pair") for dt in ("f16", "bf16")
                    for s in PIPE_IMAGE_SHAPES for im in (2, 3, 5)]


@pytest.mark.parametrize("shape,dt,form,images", PIPE_IMAGE_CASES,
                         ids=[f"{k}-{dt}-{s}-i{im}" for s, dt, k, im in PIPE_IMAGE_CASES])
def test_pipelined_kernel_whole_image_tasks(shape, dt, form, images, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    monkeypatch.setenv("IM2WIN_IMPLICIT_IMAGES", str(images))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 4
    if images * pl.Ho * pl.Wo <= 256 and images <= N:
        assert pl.images == images and pl.rows_per_tile == pl.Ho
        assert pl.patch_rows == images * (pl.Ho + KH - 1)
    else:
        assert pl.images == 1
    _say(f"implicit-{form} {dt} {shape} images/task={pl.images} workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=29, dtype=dt)
    got = run_implicit(x, w, s, p)
    check(got, x, w, s, p, dt)


@pytest.mark.parametrize("form", ["pipe", "pair"])
def test_pipelined_kernel_whole_image_tasks_exact(form, monkeypatch):
    shape = (5, 64, 7, 7, 72, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    monkeypatch.setenv("IM2WIN_IMPLICIT_IMAGES", "3")
    assert conv.implicit_plan(conv.make_desc(*shape, conv.F16)).images == 3
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=30, dtype="f16",
                                 x_dist="int3", w_dist="int3")
    got = run_implicit(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(x, w, s, p))


# stride 2 (asked for by name): patches of (R - 1) * 2 + KH input rows, the
# windows of consecutive outputs two positions apart
PIPE_STRIDE_SHAPES = [
    (2, 64, 14, 14, 72, 3, 3, 2, 1),     # 7x7 outputs, Cout past one block
    (1, 96, 17, 23, 64, 3, 3, 2, 0),     # odd planes, 8x11 outputs
    (3, 128, 12, 16, 130, 1, 1, 2, 0),   # 1x1 stride 2 (a downsampling shortcut)
    (2, 32, 28, 28, 40, 3, 3, 2, 1),     # 14x14 outputs
]
PIPE_STRIDE_CASES = [(s, dt, k, im) for k in ("pipe", "pair") for dt in ("f16", "bf16")
                     for s in PIPE_STRIDE_SHAPES for im in (None, 1, 2)]


@pytest.mark.parametrize("shape,dt,form,images", PIPE_STRIDE_CASES,
                         ids=[f"{k}-{dt}-{s}-i{im}" for s, dt, k, im in PIPE_STRIDE_CASES])
def test_pipelined_kernel_stride_two(shape, dt, form, images, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    if images is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_IMAGES", str(images))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 4
    assert pl.patch_rows == pl.images * ((pl.rows_per_tile - 1) * s + KH)
    _say(f"implicit-{form} {dt} {shape} rows/task={pl.rows_per_tile} images={pl.images}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=31, dtype=dt)
    got = run_implicit(x, w, s, p)
    check(got, x, w, s, p, dt)
    if dt == "f16" and images is None:
        xi, wi = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=32, dtype="f16",
                                       x_dist="int3", w_dist="int3")
        got = run_implicit(xi, wi, s, p)
        assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(xi, wi, s, p))


# the write-through stores of the row-block and narrow kernels: repeated
# launches give the same bits as the first and match the oracle (a store
# form that skipped the wait rule around its data registers wrote another
# instruction's values for a few outputs, different ones each run)
REPEAT_CASES = [
    ((9, 3, 130, 128, 40, 3, 3, 1, 1), "f32", None),   # persistent narrow kernel, fp32
    ((2, 3, 66, 64, 64, 7, 7, 2, 3), "f16", None),      # narrow kernel, whole input rows
    ((4, 64, 32, 56, 64, 3, 3, 1, 1), "f16", 8),        # row-block kernel, 8 rows: every line whole
    ((2, 64, 16, 32, 96, 3, 3, 1, 1), "f32", 4),        # fp32 row-block kernel
]


@pytest.mark.parametrize("shape,dt,rows", REPEAT_CASES, ids=[f"{d}-{s}" for s, d, _ in REPEAT_CASES])
def test_write_through_stores_repeat_exactly(shape, dt, rows, monkeypatch):
    if rows is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rows))
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=37, dtype=dt, w_dist="normal")
    xd, wd = x.to(DEV), w.to(DEV)
    runs = []
    for _ in range(5):
        runs.append(conv.conv2d_implicit(xd, wd, stride=s, pad=p))
    torch.cuda.synchronize()
    for y in runs[1:]:
        assert torch.equal(y, runs[0])
    check(runs[0].cpu(), x, w, s, p, dt, ref=oracle.conv2d(x, w, s, p))
