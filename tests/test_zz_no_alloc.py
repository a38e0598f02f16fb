"""conv2d_fwd_noalloc (the allocation-free entry point, workspace in the
library's static device array) against conv2d_fwd with a caller-allocated
workspace, through the C ABI: the same kernels on the same inputs, so the
outputs must be bit-equal, and both within the parity bounds of the oracle.
Each case makes two calls in a row, the second on a smaller input, so the
second runs on what the first left in the array. A plan whose workspace
exceeds the array is refused before any launch."""
import sys

import numpy as np
import pytest
import torch

import cnn_convolution_amd as conv
from cnn_convolution_amd import _lib
import workloads
from parity import check

pytestmark = pytest.mark.gpu

CODE = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _both(shape, dt, seed):
    """(y from conv2d_fwd_noalloc, y from conv2d_fwd, x, w, plan)"""
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=seed, dtype=dt)
    d = conv.make_desc(*shape, CODE[dt])
    pl = conv.plan(d)
    assert 0 < pl.ws_bytes <= _lib.NOALLOC_SCRATCH_BYTES or pl.ws_bytes == 0
    xd, wd = x.to(DEV), w.to(DEV)
    y1 = torch.full((N, Cout, pl.Ho, pl.Wo), 777.0, dtype=torch.float32, device=DEV)
    y2 = torch.full_like(y1, 555.0)
    st = _lib.fwd_noalloc(d, xd.data_ptr(), wd.data_ptr(), y1.data_ptr(), _stream())
    assert st == 0, conv.status_string(st)
    ws = torch.empty(max(pl.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    st = _lib.fwd(d, xd.data_ptr(), wd.data_ptr(), y2.data_ptr(), ws.data_ptr() if pl.ws_bytes else None,
                  _stream())
    assert st == 0, conv.status_string(st)
    torch.cuda.synchronize()
    return y1.cpu(), y2.cpu(), x, w, pl


# (first call, second call on a smaller input, dtype, forced form)
CASES = [
    ((4, 3, 64, 64, 64, 7, 7, 2, 3), (2, 3, 40, 36, 64, 7, 7, 2, 3), "f16", None),      # narrow kernel: no workspace
    ((4, 3, 48, 48, 40, 7, 7, 2, 3), (1, 3, 21, 19, 24, 7, 7, 2, 3), "f32", None),      # narrow kernel, fp32: no workspace
    ((8, 64, 28, 28, 64, 3, 3, 1, 1), (2, 64, 14, 14, 64, 3, 3, 1, 1), "f16", "window"),  # window tensor + staged filter
    ((4, 32, 20, 20, 48, 3, 3, 1, 1), (1, 16, 9, 11, 40, 3, 3, 2, 1), "f32", "window"),  # row-interleaved window tensor
    ((2, 128, 12, 12, 96, 5, 5, 1, 2), (1, 64, 9, 9, 40, 5, 5, 1, 2), "bf16", None),    # streamed implicit kernel
    ((4, 64, 16, 16, 64, 3, 3, 1, 1), (2, 64, 8, 8, 32, 3, 3, 1, 1), "f16", None),      # row-block kernel: no workspace
]


@pytest.mark.parametrize("first,second,dt,algo", CASES,
                         ids=[f"{dt}-{a or 'planned'}-{f}" for f, _, dt, a in CASES])
def test_noalloc_matches_conv2d_fwd(first, second, dt, algo, monkeypatch):
    if algo:
        monkeypatch.setenv("IM2WIN_ALGO", algo)
    for k, shape in enumerate((first, second)):
        _say(f"noalloc call {k + 1}: {dt} {algo or 'planned'} {shape}")
        y1, y2, x, w, pl = _both(shape, dt, seed=40 + k)
        if algo == "window":
            assert pl.algo == 0 and pl.ws_bytes > 0
        assert torch.equal(y1, y2)
        check(y1, x, w, shape[7], shape[8], dt, what=f"noalloc {shape}")


def test_noalloc_refuses_a_workspace_past_the_array(monkeypatch):
    """The ResNet layer's fp32 window form needs about 42 MB of workspace: refused,
    nothing launched, y untouched."""
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    d = conv.make_desc(32, 64, 56, 56, 64, 3, 3, 1, 1, conv.F32)
    pl = conv.plan(d)
    assert pl.algo == 0 and pl.ws_bytes > _lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((32, 64, 56, 56), dtype=torch.float32, device=DEV)
    w = torch.zeros((64, 64, 3, 3), dtype=torch.float32, device=DEV)
    y = torch.full((32, 64, 56, 56), 9.0, dtype=torch.float32, device=DEV)
    st = _lib.fwd_noalloc(d, x.data_ptr(), w.data_ptr(), y.data_ptr(), _stream())
    assert st == 8 and conv.status_string(st).startswith("workspace exceeds")
    torch.cuda.synchronize()
    assert bool((y == 9.0).all())


WS_CASES = CASES[2:5]                                  # the forms that use a workspace


@pytest.mark.parametrize("shape,dt,algo", [(c[0], c[2], c[3]) for c in WS_CASES],
                         ids=[f"{c[2]}-{c[3] or 'planned'}" for c in WS_CASES])
def test_workspace_contents_are_never_read_before_written(shape, dt, algo, monkeypatch):
    """conv2d_fwd with a workspace full of NaN bytes gives the same bits as with
    a zeroed one: no kernel reads a workspace element the call has not written
    (which is what lets the allocation-free entry point skip clearing its
    array between calls)."""
    if algo:
        monkeypatch.setenv("IM2WIN_ALGO", algo)
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    x, w = workloads.make_inputs(N, Cin, H, W, Cout, KH, KW, seed=44, dtype=dt)
    d = conv.make_desc(*shape, CODE[dt])
    pl = conv.plan(d)
    assert pl.ws_bytes > 0
    xd, wd = x.to(DEV), w.to(DEV)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((pl.ws_bytes,), fill, dtype=torch.uint8, device=DEV)
        y = torch.empty((N, Cout, pl.Ho, pl.Wo), dtype=torch.float32, device=DEV)
        assert _lib.fwd(d, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), ws.data_ptr(), _stream()) == 0
        torch.cuda.synchronize()
        outs.append(y.cpu())
    assert torch.equal(outs[0], outs[1])
    assert np.isfinite(outs[1].numpy()).all()
