"""numpy model of the im2win transform -- TEST INFRASTRUCTURE ONLY.

Source: "Enabling Memory-efficient Im2win Convolution with Multi-precision
Support on GPU CUDA and Tensor Cores", Sec. III-B, Eq. (2) (the transform) and
Sec. III-C, Eq. (3) (the convolution read off the window tensor).

Eq. (2) places, for every output row m of image i and channel r, the H_f input
rows m*s .. m*s+H_f-1 side by side column by column: element (column k, filter
row u) of the window row sits at position k*H_f + u. Readings taken here:

* zero padding: the input is first padded by p zeros on every side (the page's
  equation has no padding; the layers measured here do pad);
* the channel range of Eq. (2) runs over the *input* channels (the page prints
  C_o there);
* only the W_win = (Wo-1)*s + KW padded columns that some window touches are
  stored (the page stores all W_i columns; the extra columns are never read);
* in Eq. (3) the window of output column n starts at position n*s*H_f, and the
  filter tap (u, v) sits at offset v*H_f + u inside it, i.e. position
  (n*s + v)*H_f + u, the same cell Eq. (2) gives for input column n*s + v (the
  printed (n*s)*W_f + v*W_f + u agrees with this only when H_f = W_f).

Two storage orders of the same values are modelled:
  layout "row": T[r][ci][w*KH + kh]      (the page's order, channel outermost)
  layout "cl" : T[r][w*KH + kh][ci]      (channels innermost)
with r = n*Ho + ho, and T[..] = Xp[n][ci][ho*s + kh][w] for w < W_win.
"""
from __future__ import annotations

import numpy as np


def _extent(n, k, s, p):
    return (n + 2 * p - k) // s + 1


def im2win_width(W: int, KW: int, stride: int, pad: int) -> int:
    """W_win: number of padded input columns that windows of one output row touch."""
    Wo = _extent(W, KW, stride, pad)
    return (Wo - 1) * stride + KW


def im2win(x: np.ndarray, KH: int, KW: int, stride: int, pad: int, layout: str = "row"):
    """Window tensor of Eq. (2) for x [N][C][H][W]; returns (T, Ho, Wo, W_win).

    The values are copied, not computed: T has x's dtype."""
    x = np.asarray(x)
    N, C, H, W = x.shape
    Ho, Wo = _extent(H, KH, stride, pad), _extent(W, KW, stride, pad)
    Wwin = (Wo - 1) * stride + KW
    xp = np.zeros((N, C, H + 2 * pad, W + 2 * pad), dtype=x.dtype)
    xp[:, :, pad:pad + H, pad:pad + W] = x
    # rows[ho, kh] = ho*s + kh  (padded coordinates)
    rows = np.arange(Ho)[:, None] * stride + np.arange(KH)[None, :]
    g = xp[:, :, rows, :Wwin]                      # [N][C][Ho][KH][Wwin]
    if layout == "row":
        t = g.transpose(0, 2, 1, 4, 3)             # [N][Ho][C][Wwin][KH]
        t = t.reshape(N * Ho, C, Wwin * KH)
    elif layout == "cl":
        t = g.transpose(0, 2, 4, 3, 1)             # [N][Ho][Wwin][KH][C]
        t = t.reshape(N * Ho, Wwin * KH, C)
    else:
        raise ValueError(layout)
    return np.ascontiguousarray(t), Ho, Wo, Wwin


def window_conv(t: np.ndarray, w: np.ndarray, N: int, Ho: int, Wo: int, stride: int,
                layout: str = "row") -> np.ndarray:
    """Eq. (3): the convolution summed straight off the window tensor, in float64.

    Y[n][co][ho][wo] = sum_{ci,kh,kw} T(r=n*Ho+ho, ci, pos=(wo*s + kw)*KH + kh) * w[co][ci][kh][kw]
    """
    w = np.asarray(w, dtype=np.float64)
    Cout, Cin, KH, KW = w.shape
    t = np.asarray(t, dtype=np.float64)
    if layout == "cl":
        t = t.transpose(0, 2, 1)                   # -> [R][C][pos]
    y = np.zeros((N * Ho, Cout, Wo), dtype=np.float64)
    wo = np.arange(Wo)
    for kh in range(KH):
        for kw in range(KW):
            pos = (wo * stride + kw) * KH + kh     # [Wo]
            win = t[:, :, pos]                     # [R][Cin][Wo]
            y += np.einsum("rcw,oc->row", win, w[:, :, kh, kw])
    return y.reshape(N, Ho, Cout, Wo).transpose(0, 2, 1, 3).copy()
