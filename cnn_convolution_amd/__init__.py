"""im2win forward 2-D convolution for MI355X (gfx950).

    y = cnn_convolution_amd.conv2d(x, w, stride=1, pad=0,
                                   bias=None, scale=None, out_dtype=None, layout="nchw")

x [N][Cin][H][W] and w [Cout][Cin][KH][KW] (layout "nhwc": x [N][H][W][Cin],
w [Cout][KH][KW][Cin], half precision only) are contiguous CUDA (HIP)
tensors of float32, float16 or bfloat16 (the same dtype); y is float32 unless
out_dtype says otherwise, y = scale[co] * (conv + bias[co]) when the fp32
[Cout] tensors scale / bias are given. PyTorch provides the device memory and
the current stream; the convolution itself runs in libim2win_conv2d.so (see
include/im2win_conv2d.h).
"""
from __future__ import annotations

from . import _lib
from ._lib import (Conv2dError, Desc, Plan, ImplicitPlan, LAYOUT_CL, LAYOUT_FRAG, LAYOUT_ROW,  # noqa: F401
                   F16, F32, BF16, NCHW, NHWC, make_desc, workspace_size, plan, implicit_plan,
                   implicit_workspace_size, profile_enable, profile_read, status_string)

__all__ = ["conv2d", "conv2d_into", "conv2d_implicit", "conv2d_implicit_into", "pack",
           "weight_stage", "window_gemm", "describe", "plan", "implicit_plan", "workspace_size",
           "implicit_workspace_size", "implicit_gemm",
           "Conv2dError", "profile_enable", "profile_read"]


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


_LAYOUTS = {"nchw": NCHW, "nhwc": NHWC}


def _layout_code(layout) -> int:
    if layout in (NCHW, NHWC):
        return layout
    if layout not in _LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    return _LAYOUTS[layout]


def describe(x_shape, w_shape, stride=1, pad=0, dtype=F32, y_dtype=F32, layout=NCHW) -> Desc:
    """The descriptor of a layer from the shapes of x and w in `layout`."""
    lay = _layout_code(layout)
    if lay == NHWC:
        N, H, W, Cin = x_shape
        Cout, KH, KW, Cin2 = w_shape
    else:
        N, Cin, H, W = x_shape
        Cout, Cin2, KH, KW = w_shape
    if Cin2 != Cin:
        raise ValueError(f"channel mismatch: x has {Cin}, w has {Cin2}")
    return make_desc(N, Cin, H, W, Cout, KH, KW, stride, pad, dtype, y_dtype, lay)


def out_shape(d: Desc, p) -> tuple:
    """Shape of y for descriptor d and its plan p."""
    return (d.N, p.Ho, p.Wo, d.Cout) if d.layout == NHWC else (d.N, d.Cout, p.Ho, p.Wo)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def conv2d_into(x, w, y, ws, stride=1, pad=0, *, bias=None, scale=None, layout="nchw") -> None:
    """Enqueue y = conv2d(x, w) on the current stream using caller buffers
    (y's dtype is the output type; scale / bias: fp32 [Cout] device tensors)."""
    d = describe(tuple(x.shape), tuple(w.shape), stride, pad, _dtype_code(x), _dtype_code(y), layout)
    if w.dtype != x.dtype:
        raise TypeError("x and w must share a dtype")
    for t, name in ((scale, "scale"), (bias, "bias")):
        if t is not None and (t.dtype.itemsize != 4 or not t.is_floating_point() or t.numel() != d.Cout):
            raise ValueError(f"{name} must be an fp32 tensor of Cout elements")
    ws_ptr = ws.data_ptr() if ws is not None and ws.numel() else None
    if bias is None and scale is None:
        st = _lib.fwd(d, x.data_ptr(), w.data_ptr(), y.data_ptr(), ws_ptr, _stream())
    else:
        st = _lib.fwd_ex(d, x.data_ptr(), w.data_ptr(), scale.data_ptr() if scale is not None else None,
                         bias.data_ptr() if bias is not None else None, y.data_ptr(), ws_ptr, _stream())
    if st != 0:
        raise Conv2dError(st, "conv2d_fwd")


def conv2d(x, w, stride: int = 1, pad: int = 0, *, bias=None, scale=None, out_dtype=None,
           layout="nchw"):
    import torch
    _check(x, "x")
    _check(w, "w")
    odt = torch.float32 if out_dtype is None else out_dtype
    d = describe(tuple(x.shape), tuple(w.shape), stride, pad, _dtype_code(x),
                 _dtype_code(torch.empty(0, dtype=odt)), layout)
    p = plan(d)
    y = torch.empty(out_shape(d, p), dtype=odt, device=x.device)
    ws = torch.empty(max(p.ws_bytes, 1), dtype=torch.uint8, device=x.device)
    conv2d_into(x, w, y, ws if p.ws_bytes else None, stride, pad, bias=bias, scale=scale, layout=layout)
    return y


def conv2d_implicit_into(x, w, y, ws, stride=1, pad=0) -> None:
    """Enqueue y = conv2d(x, w) by the implicit form (window rows built in LDS,
    no window tensor) on the current stream, using caller buffers."""
    d = describe(tuple(x.shape), tuple(w.shape), stride, pad, _dtype_code(x))
    if w.dtype != x.dtype:
        raise TypeError("x and w must share a dtype")
    st = _lib.fwd_implicit(d, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                           ws.data_ptr() if ws is not None and ws.numel() else None, _stream())
    if st != 0:
        raise Conv2dError(st, "conv2d_fwd_implicit")


def conv2d_implicit(x, w, stride: int = 1, pad: int = 0):
    """y = conv2d(x, w) by the implicit form (fp16/bf16, Cin a multiple of 64)."""
    import torch
    _check(x, "x")
    _check(w, "w")
    d = describe(tuple(x.shape), tuple(w.shape), stride, pad, _dtype_code(x))
    p = implicit_plan(d)
    y = torch.empty((d.N, d.Cout, p.Ho, p.Wo), dtype=torch.float32, device=x.device)
    ws = torch.empty(max(p.ws_bytes, 1), dtype=torch.uint8, device=x.device)
    conv2d_implicit_into(x, w, y, ws if p.ws_bytes else None, stride, pad)
    return y


def implicit_gemm(x, wst, y, desc: Desc) -> None:
    """Enqueue the implicit kernel alone: y from x and a filter already staged
    in the channels-last K order (w itself for a 1x1 filter)."""
    st = _lib.implicit_gemm(desc, x.data_ptr(), wst.data_ptr(), y.data_ptr(), _stream())
    if st != 0:
        raise Conv2dError(st, "im2win_implicit_gemm")


def pack(x, KH: int, KW: int, stride: int, pad: int, layout: int, row0: int = 0, rows=None):
    """Rows [row0, row0+rows) of the im2win window tensor of x, as a flat tensor."""
    import torch
    _check(x, "x")
    code = _dtype_code(x)
    d = describe(tuple(x.shape), (1, x.shape[1], KH, KW), stride, pad, code)
    p = plan(d)
    if rows is None:
        rows = p.rows_total - row0
    geo = layout_geometry(d, layout)
    out = torch.empty(max(rows, 0) * geo["row_elems"], dtype=x.dtype, device=x.device)
    st = _lib.pack(d, layout, x.data_ptr(), out.data_ptr(), row0, rows, _stream())
    if st != 0:
        raise Conv2dError(st, "im2win_pack")
    return out, geo


def layout_geometry(d: Desc, layout: int) -> dict:
    """Cin_pad, pos_pad and row_elems of a layout (as the planner computes them)."""
    p = plan(d)
    if layout == p.layout:
        return {"Cin_pad": p.Cin_pad, "pos_pad": p.pos_pad, "row_elems": p.row_elems}
    # the other layout: ask the planner for the dtype that uses it
    other = make_desc(d.N, d.Cin, d.H, d.W, d.Cout, d.KH, d.KW, d.stride, d.pad,
                      F16 if layout == LAYOUT_CL else F32)
    q = plan(other)
    return {"Cin_pad": q.Cin_pad, "pos_pad": q.pos_pad, "row_elems": q.row_elems}


def weight_stage(w, stride: int, pad: int, x_hw, layout: int):
    """The staged filter of w for `layout`, as a flat tensor (with its geometry)."""
    import torch
    _check(w, "w")
    Cout, Cin, KH, KW = w.shape
    code = _dtype_code(w)
    d = describe((1, Cin, x_hw[0], x_hw[1]), tuple(w.shape), stride, pad, code)
    p = plan(d)
    if layout == LAYOUT_ROW:
        rows, row_len = -(-Cout // 16) * 16, Cin * KH * KW
    elif layout == LAYOUT_FRAG:
        rows, row_len = -(-Cout // 64) * 64, Cin * KH * KW
    else:
        rows, row_len = Cout, p.K_stage if p.layout == LAYOUT_CL else None
        if row_len is None:
            raise ValueError("channels-last staging is for fp16/bf16 filters")
    out = torch.empty(rows * row_len, dtype=w.dtype, device=w.device)
    st = _lib.weight_stage(d, layout, w.data_ptr(), out.data_ptr(), _stream())
    if st != 0:
        raise Conv2dError(st, "im2win_weight_stage")
    return out, {"rows": rows, "row_len": row_len}


def window_gemm(win, wst, y, desc: Desc, row0: int, rows: int) -> None:
    """Enqueue the window-GEMM of window rows [row0, row0+rows) into y.

    win: those rows of the window tensor in the plan's layout (flat device
    tensor), wst: the staged filter of that layout, y: the full fp32 output."""
    st = _lib.window_gemm(desc, win.data_ptr(), wst.data_ptr(), y.data_ptr(), row0, rows,
                          _stream())
    if st != 0:
        raise Conv2dError(st, "im2win_window_gemm")
