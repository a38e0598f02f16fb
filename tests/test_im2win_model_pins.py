"""Pins for the oracle's numpy model of the im2win transform.

* the window of every output position, read from the window tensor, holds the
  same values as that position's im2col patch (lowering written here);
* the convolution read off the window tensor equals a library convolution,
  for both storage orders and for non-square filters (this fixes the reading
  of the window index in the im2win convolution equation);
* sizes: the element count, the saving against im2col, and the sizes that
  follow from the shapes of the paper's Fig. 1.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.im2win_model import im2win, im2win_width, window_conv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

CASES = [
    # N, C, H, W, Cout, KH, KW, s, p
    (1, 3, 3, 3, 2, 2, 2, 1, 0),      # the shapes of Fig. 1
    (2, 3, 8, 9, 4, 3, 3, 1, 1),
    (1, 2, 9, 7, 3, 2, 3, 1, 0),      # KH != KW
    (2, 4, 10, 11, 3, 3, 2, 2, 1),    # KH != KW, stride 2
    (1, 3, 13, 12, 2, 7, 7, 2, 3),    # stem-like
    (1, 2, 8, 8, 2, 5, 5, 1, 2),
    (2, 5, 6, 7, 3, 1, 1, 1, 0),      # 1x1
    (1, 2, 7, 9, 2, 3, 4, 3, 2),      # stride 3, ragged
    (1, 1, 5, 5, 1, 5, 5, 1, 0),      # one window
]


def _im2col_rows(x, KH, KW, s, p):
    """[N][Ho][Wo][C][KH][KW] patches by direct slicing of the padded input."""
    N, C, H, W = x.shape
    xp = np.pad(x, ((0, 0), (0, 0), (p, p), (p, p)))
    Ho = (H + 2 * p - KH) // s + 1
    Wo = (W + 2 * p - KW) // s + 1
    out = np.empty((N, Ho, Wo, C, KH, KW), x.dtype)
    for ho in range(Ho):
        for wo in range(Wo):
            out[:, ho, wo] = xp[:, :, ho * s:ho * s + KH, wo * s:wo * s + KW]
    return out


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("layout", ["row", "cl"])
def test_windows_are_im2col_patches(case, layout):
    N, C, H, W, Co, KH, KW, s, p = case
    x = np.random.default_rng(1).standard_normal((N, C, H, W))
    t, Ho, Wo, Wwin = im2win(x, KH, KW, s, p, layout)
    if layout == "cl":
        t = t.transpose(0, 2, 1)
    patches = _im2col_rows(x, KH, KW, s, p)
    for n in range(N):
        for ho in range(Ho):
            r = n * Ho + ho
            for wo in range(Wo):
                # the window of column wo: KW*KH contiguous positions from wo*s*KH,
                # filter column outer, filter row inner
                win = t[r, :, wo * s * KH:(wo * s + KW) * KH].reshape(C, KW, KH)
                assert np.array_equal(win.transpose(0, 2, 1), patches[n, ho, wo])


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("layout", ["row", "cl"])
def test_window_convolution_matches_library(case, layout):
    N, C, H, W, Co, KH, KW, s, p = case
    rng = np.random.default_rng(2)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, KH, KW))
    t, Ho, Wo, _ = im2win(x, KH, KW, s, p, layout)
    y = window_conv(t, w, N, Ho, Wo, s, layout)
    ref = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=s, padding=p).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, oracle.conv2d(x, w, s, p), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("KH,KW,square", [(2, 3, False), (3, 3, True), (2, 2, True)])
def test_printed_window_index_only_holds_for_square_filters(KH, KW, square):
    """The printed index (n*s)*W_f + v*W_f + u of the im2win convolution
    equation lands on the same cell as (n*s + v)*H_f + u only when H_f = W_f."""
    N, C, H, W, Co, s, p = 1, 2, 9, 7, 3, 1, 0
    rng = np.random.default_rng(3)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, KH, KW))
    t, Ho, Wo, _ = im2win(x, KH, KW, s, p, "row")
    wo = np.arange(Wo)
    y = np.zeros((N * Ho, Co, Wo))
    for kh in range(KH):
        for kw in range(KW):
            pos = (wo * s) * KW + kw * KW + kh
            ok = pos < t.shape[2]
            y[:, :, ok] += np.einsum("rcw,oc->row", t[:, :, pos[ok]], w[:, :, kh, kw])
    ref = oracle.conv2d(x, w, s, p).transpose(0, 2, 1, 3).reshape(N * Ho, Co, Wo)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12) == square


@pytest.mark.parametrize("case", CASES)
def test_sizes(case):
    N, C, H, W, Co, KH, KW, s, p = case
    x = np.zeros((N, C, H, W))
    t, Ho, Wo, Wwin = im2win(x, KH, KW, s, p, "row")
    assert Wwin == im2win_width(W, KW, s, p) == (Wo - 1) * s + KW
    assert t.size == N * C * Ho * Wwin * KH
    im2col = N * Ho * Wo * C * KH * KW
    if s <= KW:
        # the saving against im2col: N*C*Ho*KH*(Wo-1)*(KW-s)
        assert im2col - t.size == N * C * Ho * KH * (Wo - 1) * (KW - s)
    if s == KW:
        assert t.size == im2col                    # no overlap, nothing saved


def test_fig1_sizes():
    g = {}
    with open(os.path.join(GOLDEN, "page_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                g[k.strip()] = [int(a) for a in v.split()]
    n, c, h, w = g["fig1_input"]
    co, _, fh, fw = g["fig1_filter"]
    x = np.zeros((n, c, h, w))
    t, Ho, Wo, _ = im2win(x, fh, fw, 1, 0)
    assert t.size == g["fig1_im2win_elements"][0]
    assert n * Ho * Wo * c * fh * fw == g["fig1_im2col_elements"][0]


def test_layouts_hold_the_same_values():
    x = np.random.default_rng(4).standard_normal((2, 5, 7, 6))
    tr, *_ = im2win(x, 3, 2, 2, 1, "row")
    tc, *_ = im2win(x, 3, 2, 2, 1, "cl")
    assert np.array_equal(tr, tc.transpose(0, 2, 1))


def test_padding_cells_are_zero_and_copies_are_exact():
    x = np.arange(1, 1 + 2 * 3 * 4 * 5, dtype=np.float32).reshape(2, 3, 4, 5)
    t, Ho, Wo, Wwin = im2win(x, 3, 3, 1, 1, "row")
    assert t.dtype == np.float32
    # first output row, filter row 0 reads padded row -1: all zeros
    assert np.all(t[0, :, 0::3] == 0)
    # window column 0 is the left padding column for every filter row
    assert np.all(t[:, :, 0:3] == 0)
    # every nonzero value is a copy of an input value
    vals = set(x.reshape(-1).tolist())
    assert set(t[t != 0].tolist()) <= vals
