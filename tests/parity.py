"""Comparison of GPU outputs with the CPU oracle (test helper, no arithmetic of
the method: the reference values all come from ``oracle``).

Every floating-point comparison applies two bounds:

* over the compared outputs, relative L2 error <= TOL[dtype]
  (fp32 1e-5, fp16 2e-3, bf16 1e-2), the oracle in float64 on the same
  rounded inputs;
* per output, |y - ref| <= 2 * (K + 1) * u32 * sum_k |x_k * w_k|
  (+ u_out * |ref| when y is stored in a 16-bit type), where K = Cin*KH*KW,
  u32 = 2^-24 and the magnitude sum is the oracle's convolution of |x| with
  |w|. Whatever order the K products are added in, a sum in fp32 of terms
  that are exact (fp16/bf16 products) or rounded once (fp32 products) is
  within gamma_{K+1} * sum|terms| of the exact sum, gamma_n = n*u/(1 - n*u)
  (the a-priori bound of floating-point summation, Higham, "Accuracy and
  Stability of Numerical Algorithms", ch. 4); the factor 2 covers a matrix
  core that truncates instead of rounding. A single wrong output (a dropped
  block, a wrong border row or channel) breaks it even where the global
  relative L2 would still pass.

With the layer epilogue y = s * (sum + b) the magnitude is |s| (sum|x w| +
|b|) and K + 1 becomes K + 3 (the bias add and the scale multiply each round
once more in fp32).
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
U32 = 2.0 ** -24
U_OUT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def _abs(t):
    return t.abs() if hasattr(t, "abs") else np.abs(t)


def _host(y):
    if hasattr(y, "detach"):
        y = y.detach().cpu()
        if y.dtype.is_floating_point:
            y = y.double()
        return y.numpy()
    return np.asarray(y, np.float64)


def check(got, x, w, stride, pad, dt, *, ref=None, idx=None, out_dt="f32", what="",
          bias=None, scale=None, layout="nchw"):
    """Assert both bounds for y = scale * (conv2d(x, w) + bias) in `layout`
    (all outputs, or the flat output indices ``idx``). ``got`` holds the
    compared outputs: the whole y, or y flattened and already indexed by
    ``idx``. Returns (rel_l2, max ratio of error to the per-output bound)."""
    g = _host(got).reshape(-1)
    epi = bias is not None or scale is not None or layout != "nchw"
    ab = None if bias is None else _abs(bias)
    asc = None if scale is None else _abs(scale)
    if not epi and idx is None:
        r = oracle.conv2d(x, w, stride, pad) if ref is None else ref
        mag = oracle.conv2d(_abs(x), _abs(w), stride, pad)
    elif not epi:
        r = oracle.conv2d_points(x, w, stride, pad, idx) if ref is None else ref
        mag = oracle.conv2d_points(_abs(x), _abs(w), stride, pad, idx)
    elif idx is None:
        r = oracle.conv2d_ex(x, w, stride, pad, bias, scale, layout) if ref is None else ref
        mag = oracle.conv2d_ex(_abs(x), _abs(w), stride, pad, ab, asc, layout)
    else:
        r = oracle.conv2d_points_ex(x, w, stride, pad, idx, bias, scale, layout) if ref is None else ref
        mag = oracle.conv2d_points_ex(_abs(x), _abs(w), stride, pad, idx, ab, asc, layout)
    r = np.asarray(r, np.float64).reshape(-1)
    mag = np.asarray(mag, np.float64).reshape(-1)
    assert g.shape == r.shape, f"{what}: {g.shape} outputs compared with {r.shape}"
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    K = int(np.prod(w.shape[1:]))
    bound = 2.0 * (K + (3 if epi else 1)) * U32 * mag + U_OUT[out_dt] * np.abs(r)
    err = np.abs(g - r)
    bad = np.flatnonzero(err > bound)
    ratio = float(np.max(err / np.where(bound > 0, bound, 1.0))) if err.size else 0.0
    assert bad.size == 0, (
        f"{what}: {bad.size} of {g.size} outputs beyond the per-output bound; first at "
        f"{int(bad[0]) if idx is None else int(np.asarray(idx)[bad[0]])}: got {g[bad[0]]!r}, "
        f"oracle {r[bad[0]]!r}, bound {bound[bad[0]]:.3e}")
    rel = rel_l2(g, r)
    tol = max(TOL[dt], TOL[out_dt])
    assert rel <= tol, f"{what}: rel L2 {rel:.3e} > {tol}"
    return rel, ratio
