"""GPU parity of the layer epilogue and the output/layout variants, through
the C ABI (conv2d_fwd_ex): y = scale[co] * (conv + bias[co]) rounded once to
fp32, fp16 or bf16 y, for every kernel family (each forced where it is not
the planned one), and the NHWC layout (x [N][H][W][Cin], w [Cout][KH][KW][Cin],
y [N][Ho][Wo][Cout]) through the channels-last window form. Reference: the
oracle's float64 conv2d_ex on the same rounded inputs; the per-output bound
includes the rounding of y to its storage type (tests/parity.py)."""
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

CODE = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _epi(kind, Cout, seed):
    rng = np.random.default_rng(seed)
    b = torch.from_numpy(rng.standard_normal(Cout).astype(np.float32))
    s = torch.from_numpy((rng.uniform(0.25, 2.0, Cout) * rng.choice([-1.0, 1.0], Cout)).astype(np.float32))
    return {"none": (None, None), "bias": (b, None), "scale_bias": (b, s), "scale": (None, s)}[kind]


def _run(x, w, s, p, ydt, bias, scale, layout="nchw", guard=0):
    """conv2d_fwd_ex into a y buffer followed by `guard` sentinel elements."""
    d = conv.describe(tuple(x.shape), tuple(w.shape), s, p, CODE[_dt(x)], CODE[ydt], layout)
    pl = conv.plan(d)
    shape = conv.out_shape(d, pl)
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), 77.0, dtype=TDT[ydt], device=DEV)
    ws = torch.empty(max(pl.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    xd, wd = x.to(DEV), w.to(DEV)
    bd = bias.to(DEV) if bias is not None else None
    sd = scale.to(DEV) if scale is not None else None
    st = _lib.fwd_ex(d, xd.data_ptr(), wd.data_ptr(), sd.data_ptr() if sd is not None else None,
                     bd.data_ptr() if bd is not None else None, buf.data_ptr(),
                     ws.data_ptr() if pl.ws_bytes else None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, conv.status_string(st)
    torch.cuda.synchronize()
    host = buf.cpu()
    if guard:
        assert bool((host[n:] == 77.0).all()), "stores past the end of y"
    return host[:n].reshape(shape), pl


def _dt(t):
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


# (shape, dtype, forced environment, what it exercises)
KERNEL_CASES = [
    ((2, 64, 10, 16, 40, 3, 3, 1, 1), "f16", {}, "row-block, 16-byte stores"),
    ((2, 64, 11, 16, 24, 3, 3, 1, 0), "bf16", {}, "row-block, LDS-staged stores (Wo = 14)"),
    ((2, 256, 14, 14, 72, 3, 3, 1, 1), "f16", {"IM2WIN_IMPLICIT_KERNEL": "rows"}, "row-block, channel blocks"),
    ((2, 32, 9, 12, 40, 3, 3, 1, 1), "f32", {}, "fp32 row-block"),
    ((1, 96, 13, 15, 40, 3, 3, 1, 0), "f32", {}, "fp32 row-block, gathered rows"),
    ((2, 64, 14, 14, 72, 3, 3, 1, 1), "bf16", {"IM2WIN_IMPLICIT_KERNEL": "pipe"}, "pipelined, persistent"),
    ((2, 64, 14, 14, 72, 3, 3, 2, 1), "f16", {"IM2WIN_IMPLICIT_KERNEL": "pair"}, "pipelined, paired, stride 2"),
    ((6, 64, 7, 7, 72, 3, 3, 1, 1), "f16", {"IM2WIN_IMPLICIT_KERNEL": "pipe", "IM2WIN_IMPLICIT_IMAGES": "2"},
     "pipelined, whole-image tasks"),
    ((2, 3, 30, 30, 64, 7, 7, 2, 3), "f16", {}, "narrow-channel"),
    ((2, 3, 30, 30, 40, 7, 7, 2, 3), "f32", {}, "narrow-channel fp32"),
    ((2, 128, 12, 12, 96, 5, 5, 1, 2), "bf16", {"IM2WIN_IMPLICIT_KERNEL": "streamed"}, "streamed implicit"),
    ((2, 64, 17, 19, 70, 3, 3, 1, 1), "f16", {"IM2WIN_ALGO": "window"}, "window form, direct-to-LDS GEMM"),
    ((2, 3, 45, 47, 64, 7, 7, 2, 3), "bf16", {"IM2WIN_ALGO": "window"}, "window form, tiled GEMM"),
    ((2, 16, 12, 13, 40, 3, 3, 1, 1), "f32", {"IM2WIN_ALGO": "window"}, "window form, vector-ALU GEMM"),
]
EPIS = ["none", "bias", "scale_bias"]
YDTS = ["f32", "f16", "bf16"]


@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("ydt", YDTS)
@pytest.mark.parametrize("case", KERNEL_CASES, ids=[c[3].replace(" ", "_") for c in KERNEL_CASES])
def test_epilogue_every_kernel(case, ydt, epi, monkeypatch):
    shape, dt, env, what = case
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=61, dtype=dt)
    bias, scale = _epi(epi, Cout, 62)
    _say(f"epilogue {what}: {dt} -> {ydt} {epi} {shape}")
    y, pl = _run(x, w, s, p, ydt, bias, scale, guard=512)
    check(y, x, w, s, p, dt, out_dt=ydt, bias=bias, scale=scale, what=f"{what} {ydt} {epi}")


def test_epilogue_integer_inputs_exact():
    """Integer inputs and bias, power-of-two scales, fp32 y: bit-equal."""
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 64, 12, 16, 40, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=63, dtype="f16", x_dist="int3", w_dist="int3")
    bias = torch.arange(Cout, dtype=torch.float32) - 20
    scale = torch.tensor([0.5, 2.0, -1.0, 4.0] * 10, dtype=torch.float32)
    y, _ = _run(x, w, s, p, "f32", bias, scale)
    assert np.array_equal(y.numpy().astype(np.float64), oracle.conv2d_ex(x, w, s, p, bias=bias, scale=scale))


# NHWC through the channels-last window form (fp16/bf16)
NHWC_SHAPES = [
    (2, 64, 17, 19, 68, 3, 3, 1, 1),     # Cin % 8 == 0: 16-byte pack loads; Cout % 4 == 0: vector stores
    (2, 64, 9, 9, 70, 3, 3, 2, 1),       # Cout % 4 != 0: per-channel stores
    (2, 3, 45, 47, 64, 7, 7, 2, 3),      # 3 channels (padded to 4 or 8): gathered pack
    (1, 5, 13, 11, 9, 2, 4, 3, 2),       # KH != KW, stride 3
    (3, 64, 10, 10, 256, 1, 1, 1, 0),    # 1x1: the filter is its own staged form
    (1, 24, 4, 4, 8, 3, 3, 1, 5),        # padding wider than the filter
    (2, 128, 8, 9, 96, 3, 3, 1, 1),      # deeper K
]


@pytest.mark.parametrize("epi", ["none", "scale_bias"])
@pytest.mark.parametrize("ydt", YDTS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", NHWC_SHAPES, ids=[str(s) for s in NHWC_SHAPES])
def test_nhwc_layout(shape, dt, ydt, epi):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=64, dtype=dt)
    xh, wh = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
    bias, scale = _epi(epi, Cout, 65)
    _say(f"nhwc {dt} -> {ydt} {epi} {shape}")
    y, pl = _run(xh, wh, s, p, ydt, bias, scale, layout="nhwc", guard=512)
    assert pl.algo == 0 and pl.layout == conv.LAYOUT_CL
    check(y, xh, wh, s, p, dt, out_dt=ydt, bias=bias, scale=scale, layout="nhwc", what=f"nhwc {shape}")


def test_nhwc_integer_inputs_match_nchw_bits():
    """The same integer-valued layer in both layouts: bit-equal outputs."""
    N, Cin, H, W, Cout, KH, KW, s, p = 2, 64, 11, 12, 72, 3, 3, 1, 1
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=66, dtype="f16", x_dist="int3", w_dist="int3")
    a, _ = _run(x, w, s, p, "f32", None, None)
    b, _ = _run(x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous(), s, p, "f32", None, None,
                layout="nhwc")
    assert torch.equal(a.permute(0, 2, 3, 1), b)


def test_nhwc_rejected_for_fp32():
    d = conv.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, conv.F32, conv.F32, conv.NHWC)
    with pytest.raises(conv.Conv2dError):
        conv.plan(d)


# the measured layers with half-precision y (and NHWC for the ResNet layer),
# full size, sampled outputs
FULL = [("resnet3x3", "f16", "f16", "nchw"), ("stem7x7", "f16", "f16", "nchw"), ("mix1x1", "f16", "f16", "nchw"),
        ("deep3x3", "bf16", "bf16", "nchw"), ("resnet3x3", "f16", "f16", "nhwc")]


@pytest.mark.parametrize("name,dt,ydt,layout", FULL, ids=[f"{n}-{d}-y{y}-{l}" for n, d, y, l in FULL])
def test_full_size_half_output(name, dt, ydt, layout):
    cfg = workloads.get_config(name)
    x, w = workloads.make_config_inputs(cfg, dt)
    if layout == "nhwc":
        x, w = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
    bias, scale = _epi("scale_bias", cfg.Cout, 67)
    _say(f"full-size {name} {dt} -> {ydt} {layout}")
    y, pl = _run(x, w, cfg.stride, cfg.pad, ydt, bias, scale, layout=layout, guard=1024)
    rng = np.random.default_rng(cfg.seed + 11)
    idx = np.unique(np.concatenate([rng.integers(0, y.numel(), 4000), [0, y.numel() - 1]]))
    check(y.reshape(-1)[torch.from_numpy(idx)], x, w, cfg.stride, cfg.pad, dt, idx=idx, out_dt=ydt, bias=bias,
          scale=scale, layout=layout, what=f"{name} {ydt} {layout}")
