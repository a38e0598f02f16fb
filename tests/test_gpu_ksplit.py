"""GPU parity of the split-K row-block implicit kernel (fp16/bf16, Cin a
multiple of 128: the four waves of a workgroup each contract a quarter of the
input channels over the whole task, then exchange partial sums in LDS)
against the CPU oracle, through the C ABI. Per-output bound and relative L2
as every float parity test (``parity.check``); integer-valued inputs bit for
bit."""
import sys

import numpy as np
import pytest
import torch

import cnn_convolution_amd as conv
from cnn_convolution_amd import _lib
import oracle
import workloads
from parity import check

pytestmark = pytest.mark.gpu

CODE = {"f16": conv.F16, "bf16": conv.BF16}
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
    y = conv.conv2d_implicit(x.to(DEV), w.to(DEV), stride=s, pad=p)
    torch.cuda.synchronize()
    return y.cpu()


# N, Cin, H, W, Cout, KH, KW, s, p
KS_SHAPES = [
    (2, 128, 10, 16, 40, 3, 3, 1, 1),    # one chunk per wave, planes of 8k positions, Cout < 64
    (2, 256, 14, 14, 72, 3, 3, 1, 1),    # the deep layer's image: two chunks per wave, Cout past one block
    (1, 128, 9, 13, 64, 3, 3, 1, 0),     # odd planes (2-byte loads), Wo = 11
    (3, 128, 12, 20, 130, 1, 1, 1, 0),   # 1x1, three blocks of Cout
    (1, 128, 6, 8, 8, 3, 3, 1, 2),       # padding 2: zero rows and columns
    (1, 128, 5, 30, 72, 3, 3, 1, 3),     # padding wider than the filter: tasks with no input row
    (2, 128, 12, 12, 64, 5, 5, 1, 2),    # 5x5
    (2, 256, 14, 14, 72, 3, 3, 2, 1),    # stride 2
    (2, 128, 17, 23, 40, 3, 3, 2, 0),    # stride 2, odd planes
    (1, 384, 6, 9, 64, 3, 3, 1, 1),      # three chunks per wave: slots alternate an odd number of times
    (1, 128, 9, 24, 64, 1, 1, 1, 1),     # 1x1 with padding: zero border outputs
]
KS_CASES = [(s, dt) for dt in ("f16", "bf16") for s in KS_SHAPES]


@pytest.mark.parametrize("shape,dt", KS_CASES, ids=[f"{dt}-{s}" for s, dt in KS_CASES])
@pytest.mark.parametrize("rw", [None, 1, 3])
def test_ksplit_kernel_matches_oracle(shape, dt, rw, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    if rw is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rw))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 5 and pl.ws_bytes >= 2 * Cin * KH * KW * 64 * ((Cout + 63) // 64)
    if rw is not None:
        assert pl.rows_per_tile == min(rw, pl.Ho) and pl.images == 1
    _say(f"implicit-ksplit {dt} {shape} rows/task={pl.rows_per_tile} images={pl.images} "
         f"workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=41, dtype=dt)
    got = run_conv(x, w, s, p)
    check(got, x, w, s, p, dt)


# the two waves of a K group on 64 output channels each (tasks of 128 output
# channels, at most 112 outputs), and one LDS slot per K group (the chunk
# written after every wave has read the previous one)
KS_MODE_SHAPES = [
    (2, 256, 14, 14, 200, 3, 3, 1, 1),   # Cout past one 128-block: the last half lies past Cout
    (2, 256, 28, 28, 130, 3, 3, 2, 1),   # stride 2 (the planned split there), Cout ragged
    (1, 384, 9, 13, 72, 3, 3, 1, 0),     # three chunks per K group, odd planes
    (3, 128, 12, 20, 256, 1, 1, 2, 0),   # 1x1 stride 2
    (2, 128, 12, 12, 192, 5, 5, 1, 2),   # 5x5
]
KS_MODE_CASES = [(s, dt, co, sl) for dt in ("f16", "bf16") for s in KS_MODE_SHAPES
                 for co, sl in ((2, None), (2, 1), (1, 1))]


@pytest.mark.parametrize("shape,dt,co,slots", KS_MODE_CASES,
                         ids=[f"{dt}-{s}-co{co}-s{sl}" for s, dt, co, sl in KS_MODE_CASES])
@pytest.mark.parametrize("rw", [None, 2])
def test_ksplit_kernel_channel_split_and_one_slot(shape, dt, co, slots, rw, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    monkeypatch.setenv("IM2WIN_KSPLIT_CO", str(co))
    if slots is not None:
        monkeypatch.setenv("IM2WIN_KSPLIT_SLOTS", str(slots))
    if rw is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rw))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 5 and pl.tile_m == 64 * co
    if slots is not None:
        assert pl.stages == slots
    _say(f"implicit-ksplit {dt} {shape} co_split={co} slots={pl.stages} rows/task={pl.rows_per_tile} "
         f"workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=48, dtype=dt)
    got = run_conv(x, w, s, p)
    check(got, x, w, s, p, dt)
    if dt == "f16" and rw is None:
        xi, wi = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=49, dtype="f16",
                                       x_dist="int3", w_dist="int3")
        got = run_conv(xi, wi, s, p)
        assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(xi, wi, s, p))


@pytest.mark.parametrize("shape", KS_SHAPES[:8], ids=[str(s) for s in KS_SHAPES[:8]])
def test_ksplit_kernel_integer_inputs_exact(shape, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    assert conv.implicit_plan(conv.make_desc(*shape, conv.F16)).kernel == 5
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=42, dtype="f16",
                                 x_dist="int3", w_dist="int3")
    got = run_conv(x, w, s, p)
    assert np.array_equal(got.numpy().astype(np.float64), oracle.conv2d(x, w, s, p))


# tasks of several whole images (the last task of a layer may hold fewer)
KS_IMAGE_SHAPES = [
    (6, 128, 7, 7, 72, 3, 3, 1, 1),      # 49 outputs per image (odd planes), Cout past one block
    (9, 128, 5, 6, 40, 3, 3, 1, 0),      # 3x4 outputs
    (5, 256, 4, 4, 130, 1, 1, 1, 0),     # 1x1, 16 outputs per image
    (7, 512, 7, 7, 96, 3, 3, 1, 1),      # the 512-channel 7x7 layer's shape
]
KS_IMAGE_CASES = [(s, dt, im) for dt in ("f16", "bf16") for s in KS_IMAGE_SHAPES for im in (2, 3, 4)]


@pytest.mark.parametrize("shape,dt,images", KS_IMAGE_CASES,
                         ids=[f"{dt}-{s}-i{im}" for s, dt, im in KS_IMAGE_CASES])
def test_ksplit_kernel_whole_image_tasks(shape, dt, images, monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    monkeypatch.setenv("IM2WIN_IMPLICIT_IMAGES", str(images))
    pl = conv.implicit_plan(conv.make_desc(*shape, CODE[dt]))
    assert pl.kernel == 5
    sl = images * ((pl.Ho - 1) * s + KH)
    nbw = 4 if images * pl.Ho * pl.Wo <= 128 else 7
    plane = ((sl * (W + 2 * p) + 6) // 8) * 8 + 1          # positions per granule plane, 1 mod 8
    fits = max(4 * plane * 64, 12 * nbw * 1024) <= 160 * 1024    # one LDS slot per K group at least
    if images * pl.Ho * pl.Wo <= 208 and images <= N and fits:
        assert pl.images == images and pl.rows_per_tile == pl.Ho and pl.patch_rows == sl
    else:
        assert pl.images != images
    _say(f"implicit-ksplit {dt} {shape} images/task={pl.images} workgroups={pl.tiles} lds={pl.lds_bytes}")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=43, dtype=dt)
    got = run_conv(x, w, s, p)
    check(got, x, w, s, p, dt)


def test_ksplit_kernel_leaves_memory_past_y_untouched(monkeypatch):
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 128, 9, 13, 70, 3, 3, 1, 0
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=44, dtype="f16")
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.F16)
    pl = conv.implicit_plan(d)
    assert pl.kernel == 5
    n_out = N * Cout * pl.Ho * pl.Wo
    buf = torch.full((n_out + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(conv.implicit_workspace_size(d), dtype=torch.uint8, device=DEV)
    conv.conv2d_implicit_into(x.to(DEV), w.to(DEV), buf, ws, s, p)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[n_out:] == 12345.0).all()
    check(host[:n_out], x, w, s, p, "f16")


@pytest.mark.parametrize("out_dt", ["f16", "bf16"])
def test_ksplit_kernel_epilogue(out_dt, monkeypatch):
    """Half-precision y with a per-channel scale and bias: y = s * (conv + b),
    rounded once to the output type."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 256, 14, 14, 72, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=45, dtype="f16")
    g = torch.Generator().manual_seed(46)
    bias = torch.randn(Cout, generator=g, dtype=torch.float32)
    scale = torch.rand(Cout, generator=g, dtype=torch.float32) + 0.5
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[out_dt]
    y = conv.conv2d(x.to(DEV), w.to(DEV), s, p, bias=bias.to(DEV), scale=scale.to(DEV), out_dtype=tdt)
    torch.cuda.synchronize()
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.F16)
    assert conv.implicit_plan(d).kernel == 5
    check(y, x, w, s, p, "f16", out_dt=out_dt, bias=bias, scale=scale)


def _sample_indices(N, Cout, Ho, Wo, rng, count=3000):
    idx = set(rng.integers(0, N * Cout * Ho * Wo, count).tolist())
    cos = sorted({0, 15, 16, 63, 64, Cout - 1, Cout // 2} | set(rng.integers(0, Cout, 3).tolist()))
    for n in {0, 1, N - 1}:
        for ho in {0, 1, Ho // 2, Ho - 1}:
            for co in cos:
                for wo in {0, 1, Wo // 2, Wo - 2, Wo - 1}:
                    if 0 <= wo < Wo and 0 <= ho < Ho and 0 <= co < Cout:
                        idx.add(((n * Cout + co) * Ho + ho) * Wo + wo)
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("name", ["deep3x3", "mix512", "mix3x3s2", "mix5x5"])
def test_ksplit_full_size_sampled(name, monkeypatch):
    """The measured layers at full size on this kernel: sampled outputs
    (random, borders, first and last images, every 16-channel block edge)
    against the oracle point by point."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    cfg = workloads.get_config(name)
    dt = cfg.dtypes[-1]
    pl = conv.implicit_plan(conv.make_desc(*cfg.desc().values(), CODE[dt]))
    assert pl.kernel == 5
    _say(f"implicit-ksplit full-size {name} {dt} rows/task={pl.rows_per_tile} images={pl.images} "
         f"workgroups={pl.tiles}")
    x, w = workloads.make_config_inputs(cfg, dt)
    y = run_conv(x, w, cfg.stride, cfg.pad)
    ho, wo = cfg.out_hw()
    yf = y.numpy().reshape(-1)
    rng = np.random.default_rng(cfg.seed + 7)
    idx = _sample_indices(cfg.N, cfg.Cout, ho, wo, rng)
    assert np.isfinite(yf[idx]).all()
    check(yf[idx], x, w, cfg.stride, cfg.pad, dt, idx=idx, what=f"{name} {dt}")


def test_ksplit_kernel_alone_with_filter_staged_once(monkeypatch):
    """A filter staged once in fragment order (im2win_weight_stage,
    IM2WIN_LAYOUT_FRAG) serves two calls of the kernel alone
    (im2win_implicit_gemm), equal bit for bit to conv2d_fwd's output."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 256, 14, 14, 72, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=47, dtype="bf16")
    xd, wd = x.to(DEV), w.to(DEV)
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, conv.BF16)
    pl = conv.implicit_plan(d)
    assert pl.kernel == 5
    wst, geo = conv.weight_stage(wd, s, p, (H, W), conv.LAYOUT_FRAG)
    assert wst.numel() * 2 == conv.implicit_workspace_size(d) == geo["rows"] * geo["row_len"] * 2
    ys = []
    for _ in range(2):
        y = torch.empty((N, Cout, pl.Ho, pl.Wo), dtype=torch.float32, device=DEV)
        conv.implicit_gemm(xd, wst, y, d)
        ys.append(y)
    ref = conv.conv2d_implicit(xd, wd, stride=s, pad=p)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ref) and torch.equal(ys[1], ref)
    check(ys[0], x, w, s, p, "bf16")


FRAG_SHAPES = [
    # Cout, Cin, taps: rows past Cout, one and several chunks and blocks
    (72, 64, 9),
    (40, 128, 25),
    (130, 96, 1),
    (512, 512, 9),
]


@pytest.mark.parametrize("shape", FRAG_SHAPES, ids=[str(s) for s in FRAG_SHAPES])
def test_fragment_order_staging_layout(shape):
    """The staged filter holds, for fragment (cb, blk, t, c4) and lane l, the
    8 halves w[cb*64 + c4*16 + l % 16][blk*32 + (l // 16)*8 + e][t], e = 0..7,
    and zeros for output channels past Cout: byte for byte against the same
    layout built with numpy indexing."""
    Cout, Cin, taps = shape
    k = {1: 1, 9: 3, 25: 5}[taps]
    g = torch.Generator().manual_seed(Cout * 1000 + Cin + taps)
    w = torch.randint(-30000, 30000, (Cout, Cin, k, k), generator=g, dtype=torch.int16).view(torch.float16)
    wst, geo = conv.weight_stage(w.to(DEV), 1, k // 2, (8, 8), conv.LAYOUT_FRAG)
    torch.cuda.synchronize()
    got = wst.cpu().view(torch.int16).numpy().reshape(-1)
    cbs, nch = (Cout + 63) // 64, Cin // 32
    wn = np.zeros((cbs * 64, Cin, taps), np.int16)
    wn[:Cout] = w.view(torch.int16).numpy().reshape(Cout, Cin, taps)
    # [cb][c4][col][blk][grp][e][t] -> [cb][blk][t][c4][grp][col][e]
    exp = wn.reshape(cbs, 4, 16, nch, 4, 8, taps).transpose(0, 3, 6, 1, 4, 2, 5).reshape(-1)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp)
