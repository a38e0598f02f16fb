"""Pins of the parity helper (tests/parity.py) on the CPU: results of a
library convolution in fp32 pass both bounds; a single wrong output, or one
wrong border row, fails the per-output bound even where the global relative
L2 stays under its tolerance."""
import numpy as np
import pytest
import torch

import workloads
from parity import TOL, check, rel_l2


def _lib_conv32(x, w, s, p):
    # torch's CPU convolution in fp32 on the same (rounded) inputs: an fp32
    # summation in some order, as a GPU kernel's
    return torch.nn.functional.conv2d(x.float(), w.float(), stride=s, padding=p)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 64, 12, 12, 32, 3, 3, 1, 1), (1, 3, 31, 29, 16, 7, 7, 2, 3),
                                   (1, 256, 6, 6, 40, 3, 3, 1, 0)])
def test_fp32_library_result_passes(shape, dt):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=3, dtype=dt)
    rel, ratio = check(_lib_conv32(x, w, s, p), x, w, s, p, dt)
    assert rel < TOL[dt] and ratio < 1.0


def test_one_wrong_output_is_caught():
    shape = (4, 64, 28, 28, 64, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=4, dtype="f16")
    y = _lib_conv32(x, w, s, p).clone()
    y[3, 17, 27, 0] += 0.05 * float(y.abs().max())
    # the global norm does not see it ...
    import oracle
    assert rel_l2(y.double().numpy(), oracle.conv2d(x, w, s, p)) < TOL["f16"]
    # ... the per-output bound does
    with pytest.raises(AssertionError, match="beyond the per-output bound"):
        check(y, x, w, s, p, "f16")


def test_wrong_border_row_is_caught():
    shape = (2, 32, 20, 20, 16, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=5, dtype="bf16")
    y = _lib_conv32(x, w, s, p).clone()
    # the top output row computed as if there were no padding row above it:
    # the taps kh = 0 (which meet padding) replaced by row 1's taps
    y[:, :, 0, :] = _lib_conv32(x[:, :, :3, :], w, 1, (0, 1))[:, :, 0, :]
    with pytest.raises(AssertionError, match="beyond the per-output bound"):
        check(y, x, w, s, p, "bf16")


def test_sampled_outputs_and_fp16_output_rounding():
    shape = (2, 16, 10, 10, 24, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=6, dtype="f16")
    y = _lib_conv32(x, w, s, p)
    idx = np.array([0, 5, 99, 1000, y.numel() - 1], dtype=np.int64)
    check(y.reshape(-1)[idx], x, w, s, p, "f16", idx=idx)
    # y stored in fp16: the output rounding is inside the bound
    check(y.half(), x, w, s, p, "f16", out_dt="f16")
    with pytest.raises(AssertionError):
        check(y.half(), x, w, s, p, "f16")          # but not inside the fp32-output bound


def test_epilogue_and_nhwc_bounds():
    """A library convolution with bias, scaled, in NHWC and rounded to bf16
    passes with those arguments; the result without the bias does not."""
    shape = (2, 16, 10, 10, 24, 3, 3, 1, 1)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=7, dtype="bf16")
    b = torch.linspace(-1, 1, Cout)
    sc = torch.linspace(0.5, 2, Cout)
    y = torch.nn.functional.conv2d(x.float(), w.float(), b, stride=s, padding=p) * sc[None, :, None, None]
    xh, wh = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
    yh = y.permute(0, 2, 3, 1).contiguous().bfloat16()
    check(yh, xh, wh, s, p, "bf16", out_dt="bf16", bias=b, scale=sc, layout="nhwc")
    idx = np.array([0, 3, 100, yh.numel() - 1], dtype=np.int64)
    check(yh.reshape(-1)[idx], xh, wh, s, p, "bf16", idx=idx, out_dt="bf16", bias=b, scale=sc,
          layout="nhwc")
    y0 = (torch.nn.functional.conv2d(x.float(), w.float(), stride=s, padding=p) * sc[None, :, None, None])
    with pytest.raises(AssertionError):
        check(y0.permute(0, 2, 3, 1).contiguous(), xh, wh, s, p, "bf16", bias=b, scale=sc, layout="nhwc")
