"""CPU oracle for the forward 2-D convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package. The product library never does, and
this package imports nothing from it.

* ``conv2d`` / ``conv2d_points``: the direct sum in float64 (plain C, OpenMP),
  see ``conv2d_oracle.c`` for the definition and its sources.
* ``conv2d_ex`` / ``conv2d_points_ex``: the same sum with the layer epilogue
  y = scale[co] * (sum + bias[co]) and the NHWC layout, in float64.
* ``im2win`` / ``window_conv``: a numpy model of the im2win transform and of
  the convolution read off the window tensor (``im2win_model.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .im2win_model import im2win, window_conv, im2win_width  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "conv2d_oracle.c")
LIBPATH = os.path.join(_HERE, "liboracle_conv2d.so")

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(source: str = SOURCE, out: str = LIBPATH) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP). Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Werror",
           "-o", out + ".tmp", source]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes view of one build of the C oracle (the default build, or a test's own)."""

    def __init__(self, libpath: str = LIBPATH):
        self.lib = ctypes.CDLL(libpath)
        self.lib.oracle_out_extent.restype = _i64
        self.lib.oracle_out_extent.argtypes = [_i64] * 4
        self.lib.oracle_conv2d_f64.restype = ctypes.c_int
        self.lib.oracle_conv2d_f64.argtypes = [_i64] * 9 + [_dp, _dp, _dp, ctypes.c_int]
        self.lib.oracle_conv2d_f64_points.restype = ctypes.c_int
        self.lib.oracle_conv2d_f64_points.argtypes = ([_i64] * 9 + [_dp, _dp, _lp, _i64, _dp,
                                                                    ctypes.c_int])

    def out_extent(self, n: int, k: int, s: int, p: int) -> int:
        return int(self.lib.oracle_out_extent(n, k, s, p))

    @staticmethod
    def _f64(a) -> np.ndarray:
        if hasattr(a, "detach"):  # torch tensor: exact widening to float64
            a = a.detach().cpu().double().numpy()
        return np.ascontiguousarray(a, dtype=np.float64)

    def conv2d(self, x, w, stride: int = 1, pad: int = 0, nthreads: int = 0) -> np.ndarray:
        x = self._f64(x)
        w = self._f64(w)
        N, Cin, H, W = x.shape
        Cout, Cin2, KH, KW = w.shape
        if Cin2 != Cin:
            raise ValueError("channel mismatch")
        Ho, Wo = self.out_extent(H, KH, stride, pad), self.out_extent(W, KW, stride, pad)
        y = np.empty((N, Cout, Ho, Wo), dtype=np.float64)
        rc = self.lib.oracle_conv2d_f64(N, Cin, H, W, Cout, KH, KW, stride, pad,
                                        x.ctypes.data_as(_dp), w.ctypes.data_as(_dp),
                                        y.ctypes.data_as(_dp), nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the shape (rc={rc})")
        return y

    def conv2d_points(self, x, w, stride: int, pad: int, idx, nthreads: int = 0) -> np.ndarray:
        x = self._f64(x)
        w = self._f64(w)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        N, Cin, H, W = x.shape
        Cout, _, KH, KW = w.shape
        out = np.empty(idx.shape[0], dtype=np.float64)
        rc = self.lib.oracle_conv2d_f64_points(N, Cin, H, W, Cout, KH, KW, stride, pad,
                                               x.ctypes.data_as(_dp), w.ctypes.data_as(_dp),
                                               idx.ctypes.data_as(_lp), idx.shape[0],
                                               out.ctypes.data_as(_dp), nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the request (rc={rc})")
        return out


_default = None
_lock = threading.Lock()


def default() -> Oracle:
    """The oracle built from this directory (compiled on first use if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIBPATH) or os.path.getmtime(LIBPATH) < os.path.getmtime(SOURCE):
                build()
            _default = Oracle(LIBPATH)
    return _default


def out_extent(n, k, s, p):
    return default().out_extent(n, k, s, p)


def conv2d(x, w, stride=1, pad=0, nthreads=0):
    return default().conv2d(x, w, stride, pad, nthreads)


def conv2d_points(x, w, stride, pad, idx, nthreads=0):
    return default().conv2d_points(x, w, stride, pad, idx, nthreads)


def _vec64(v, n):
    if v is None:
        return None
    v = np.asarray(v.detach().cpu().double().numpy() if hasattr(v, "detach") else v, np.float64)
    if v.shape != (n,):
        raise ValueError(f"expected {n} per-channel values, got shape {v.shape}")
    return v


def _nchw(x, w, layout):
    """x, w of `layout` as NCHW / OIHW float64 arrays (a transpose, no arithmetic)."""
    x = Oracle._f64(x)
    w = Oracle._f64(w)
    if layout == "nhwc":                 # x [N][H][W][C], w [Cout][KH][KW][Cin]
        x = np.ascontiguousarray(x.transpose(0, 3, 1, 2))
        w = np.ascontiguousarray(w.transpose(0, 3, 1, 2))
    elif layout != "nchw":
        raise ValueError(f"unknown layout {layout!r}")
    return x, w


def conv2d_ex(x, w, stride=1, pad=0, bias=None, scale=None, layout="nchw", nthreads=0):
    """y = scale[co] * (conv2d(x, w) + bias[co]) in float64, x, w and y in
    `layout` ("nchw", or "nhwc": x [N][H][W][Cin], w [Cout][KH][KW][Cin],
    y [N][Ho][Wo][Cout]).

    The bias is the per-output-channel bias of the convolution call of
    "Unifying Convolutions and GEMM" (Sec. 5); the scale is the learned
    per-channel scale of "Fast and Memory-Efficient Wavelet Convolutions via
    I/O-Aware Reformulation" (scale folding), which multiplies the
    convolution and its bias alike (s * (X * W + b) = X * (s W) + s b).
    The NHWC layout is the input layout of the tensor-core design of
    "Enabling Memory-efficient Im2win Convolution ...", Sec. III-D. Either
    factor may be None."""
    x, w = _nchw(x, w, layout)
    y = conv2d(x, w, stride, pad, nthreads)
    b = _vec64(bias, w.shape[0])
    s = _vec64(scale, w.shape[0])
    if b is not None:
        y = y + b[None, :, None, None]
    if s is not None:
        y = y * s[None, :, None, None]
    return np.ascontiguousarray(y.transpose(0, 2, 3, 1)) if layout == "nhwc" else y


def conv2d_points_ex(x, w, stride, pad, idx, bias=None, scale=None, layout="nchw", nthreads=0):
    """conv2d_ex at the flat output indices idx of y in `layout` only."""
    x, w = _nchw(x, w, layout)
    N, _, H, W = x.shape
    Cout, _, KH, KW = w.shape
    Ho, Wo = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    idx = np.asarray(idx, np.int64)
    if layout == "nhwc":                 # flat NHWC index -> flat NCHW index of the same output
        n, ho, wo, co = np.unravel_index(idx, (N, Ho, Wo, Cout))
    else:
        n, co, ho, wo = np.unravel_index(idx, (N, Cout, Ho, Wo))
    y = conv2d_points(x, w, stride, pad, np.ravel_multi_index((n, co, ho, wo), (N, Cout, Ho, Wo)),
                      nthreads)
    b = _vec64(bias, Cout)
    s = _vec64(scale, Cout)
    if b is not None:
        y = y + b[co]
    if s is not None:
        y = y * s[co]
    return y
