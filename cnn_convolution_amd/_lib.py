"""ctypes view of libim2win_conv2d.so (declarations in include/im2win_conv2d.h).

Argument marshalling only: every step of the convolution runs in the HIP
library. Loading fails loudly when the library has not been built; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(PKG, "lib", "libim2win_conv2d.so")

F32, F16, BF16 = 0, 1, 2
NCHW, NHWC = 0, 1                    # conv2d_layout_t: memory layout of x, w and y
LAYOUT_ROW, LAYOUT_CL = 0, 1         # im2win_layout_t: storage order of the window tensor
LAYOUT_FRAG = 2                      # im2win_layout_t: the split-K kernel's staged filter order
KERNEL_WEIGHT_STAGE, KERNEL_PACK, KERNEL_GEMM, KERNEL_IMPLICIT, KERNEL_KINDS = 0, 1, 2, 3, 4

STATUS = {
    0: "CONV2D_OK", 1: "CONV2D_ERR_INVALID_DESC", 2: "CONV2D_ERR_NULL_POINTER",
    3: "CONV2D_ERR_MISALIGNED", 4: "CONV2D_ERR_UNSUPPORTED", 5: "CONV2D_ERR_WORKSPACE",
    6: "CONV2D_ERR_HIP", 7: "CONV2D_ERR_RANGE", 8: "CONV2D_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 << 20     # IM2WIN_NOALLOC_SCRATCH_BYTES

# every symbol the header declares
EXPORTS = [
    "conv2d_workspace_size", "conv2d_plan", "conv2d_fwd", "im2win_pack", "im2win_weight_stage",
    "im2win_window_gemm", "conv2d_status_string", "conv2d_profile_enable", "conv2d_profile_read",
    "conv2d_implicit_plan", "conv2d_implicit_workspace_size", "conv2d_fwd_implicit",
    "im2win_implicit_gemm", "conv2d_fwd_noalloc", "conv2d_fwd_ex",
]


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("N", "Cin", "H", "W", "Cout", "KH", "KW", "stride", "pad")] + \
               [("dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_PLAN_FIELDS = [
    ("Ho", ctypes.c_int64), ("Wo", ctypes.c_int64), ("W_win", ctypes.c_int64),
    ("path", ctypes.c_int32), ("layout", ctypes.c_int32),
    ("Cin_pad", ctypes.c_int64), ("pos_pad", ctypes.c_int64), ("row_elems", ctypes.c_int64),
    ("rows_total", ctypes.c_int64), ("rows_per_chunk", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
    ("K", ctypes.c_int64), ("K_stage", ctypes.c_int64), ("Cout_stage", ctypes.c_int64),
    ("wstage_bytes", ctypes.c_int64), ("win_offset_bytes", ctypes.c_int64),
    ("win_chunk_bytes", ctypes.c_int64), ("ws_bytes", ctypes.c_int64),
    ("im2col_bytes", ctypes.c_int64), ("ws_target_bytes", ctypes.c_int64),
    ("meets_ws_target", ctypes.c_int32), ("gemm_tile_m", ctypes.c_int32),
    ("gemm_tile_n", ctypes.c_int32), ("gemm_kslice", ctypes.c_int32),
    ("gemm_ksplit", ctypes.c_int32), ("gemm_kernel", ctypes.c_int32),
    ("gemm_wave_m", ctypes.c_int32), ("algo", ctypes.c_int32),
    ("gemm_ablate", ctypes.c_int32), ("reserved2", ctypes.c_int32),
    ("flops", ctypes.c_int64),
]


class Plan(ctypes.Structure):
    _fields_ = _PLAN_FIELDS

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in _PLAN_FIELDS}


_IMPLICIT_PLAN_FIELDS = [
    ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("wave_m", ctypes.c_int32),
    ("rows_per_tile", ctypes.c_int32), ("cols_per_tile", ctypes.c_int32),
    ("patch_rows", ctypes.c_int32), ("patch_cols", ctypes.c_int32), ("kernel", ctypes.c_int32),
    ("stages", ctypes.c_int32), ("images", ctypes.c_int32),
    ("lds_bytes", ctypes.c_int64), ("tiles", ctypes.c_int64), ("Ho", ctypes.c_int64),
    ("Wo", ctypes.c_int64), ("K_stage", ctypes.c_int64), ("ws_bytes", ctypes.c_int64),
    ("flops", ctypes.c_int64),
]


class ImplicitPlan(ctypes.Structure):
    _fields_ = _IMPLICIT_PLAN_FIELDS

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in _IMPLICIT_PLAN_FIELDS}


class Profile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * KERNEL_KINDS),
                ("total_ms", ctypes.c_double * KERNEL_KINDS)]


class Conv2dError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise RuntimeError(
                f"the HIP library {LIBPATH} is not built; run __graft_entry__.build() "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIBPATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        dp = ctypes.POINTER(Desc)
        L.conv2d_workspace_size.restype = ctypes.c_size_t
        L.conv2d_workspace_size.argtypes = [dp]
        L.conv2d_plan.restype = ctypes.c_int
        L.conv2d_plan.argtypes = [dp, ctypes.POINTER(Plan)]
        L.conv2d_fwd.restype = ctypes.c_int
        L.conv2d_fwd.argtypes = [dp, vp, vp, vp, vp, vp]
        L.conv2d_fwd_ex.restype = ctypes.c_int
        L.conv2d_fwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp]
        L.im2win_pack.restype = ctypes.c_int
        L.im2win_pack.argtypes = [dp, i32, vp, vp, i64, i64, vp]
        L.im2win_weight_stage.restype = ctypes.c_int
        L.im2win_weight_stage.argtypes = [dp, i32, vp, vp, vp]
        L.im2win_window_gemm.restype = ctypes.c_int
        L.im2win_window_gemm.argtypes = [dp, vp, vp, vp, i64, i64, vp]
        L.conv2d_status_string.restype = ctypes.c_char_p
        L.conv2d_status_string.argtypes = [ctypes.c_int]
        L.conv2d_implicit_plan.restype = ctypes.c_int
        L.conv2d_implicit_plan.argtypes = [dp, ctypes.POINTER(ImplicitPlan)]
        L.conv2d_implicit_workspace_size.restype = ctypes.c_size_t
        L.conv2d_implicit_workspace_size.argtypes = [dp]
        L.conv2d_fwd_implicit.restype = ctypes.c_int
        L.conv2d_fwd_implicit.argtypes = [dp, vp, vp, vp, vp, vp]
        L.im2win_implicit_gemm.restype = ctypes.c_int
        L.im2win_implicit_gemm.argtypes = [dp, vp, vp, vp, vp]
        L.conv2d_fwd_noalloc.restype = ctypes.c_int
        L.conv2d_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp]
        L.conv2d_profile_enable.restype = ctypes.c_int
        L.conv2d_profile_enable.argtypes = [i32]
        L.conv2d_profile_read.restype = ctypes.c_int
        L.conv2d_profile_read.argtypes = [ctypes.POINTER(Profile)]
        _lib = L
    return _lib


def make_desc(N, Cin, H, W, Cout, KH, KW, stride, pad, dtype, y_dtype=F32, layout=NCHW) -> Desc:
    return Desc(N, Cin, H, W, Cout, KH, KW, stride, pad, dtype, y_dtype, layout, 0)


def workspace_size(d: Desc) -> int:
    return int(lib().conv2d_workspace_size(ctypes.byref(d)))


def plan(d: Desc) -> Plan:
    p = Plan()
    st = lib().conv2d_plan(ctypes.byref(d), ctypes.byref(p))
    if st != 0:
        raise Conv2dError(st, "conv2d_plan")
    return p


def fwd(d: Desc, x: int, w: int, y: int, ws: int, stream: int) -> int:
    return lib().conv2d_fwd(ctypes.byref(d), x, w, y, ws, stream)


def fwd_ex(d: Desc, x: int, w: int, scale: int, bias: int, y: int, ws: int, stream: int) -> int:
    return lib().conv2d_fwd_ex(ctypes.byref(d), x, w, scale, bias, y, ws, stream)


def fwd_noalloc(d: Desc, x: int, w: int, y: int, stream: int) -> int:
    return lib().conv2d_fwd_noalloc(ctypes.byref(d), x, w, y, stream)


def implicit_plan(d: Desc) -> ImplicitPlan:
    p = ImplicitPlan()
    st = lib().conv2d_implicit_plan(ctypes.byref(d), ctypes.byref(p))
    if st != 0:
        raise Conv2dError(st, "conv2d_implicit_plan")
    return p


def implicit_plan_status(d: Desc) -> int:
    p = ImplicitPlan()
    return int(lib().conv2d_implicit_plan(ctypes.byref(d), ctypes.byref(p)))


def implicit_workspace_size(d: Desc) -> int:
    return int(lib().conv2d_implicit_workspace_size(ctypes.byref(d)))


def fwd_implicit(d: Desc, x: int, w: int, y: int, ws: int, stream: int) -> int:
    return lib().conv2d_fwd_implicit(ctypes.byref(d), x, w, y, ws, stream)


def implicit_gemm(d: Desc, x: int, wst: int, y: int, stream: int) -> int:
    return lib().im2win_implicit_gemm(ctypes.byref(d), x, wst, y, stream)


def pack(d: Desc, layout: int, x: int, out: int, row0: int, rows: int, stream: int) -> int:
    return lib().im2win_pack(ctypes.byref(d), layout, x, out, row0, rows, stream)


def weight_stage(d: Desc, layout: int, w: int, out: int, stream: int) -> int:
    return lib().im2win_weight_stage(ctypes.byref(d), layout, w, out, stream)


def window_gemm(d: Desc, win: int, wst: int, y: int, row0: int, rows: int, stream: int) -> int:
    return lib().im2win_window_gemm(ctypes.byref(d), win, wst, y, row0, rows, stream)


def status_string(st: int) -> str:
    return lib().conv2d_status_string(st).decode()


def profile_enable(on: bool) -> None:
    lib().conv2d_profile_enable(1 if on else 0)


def profile_read() -> dict:
    p = Profile()
    st = lib().conv2d_profile_read(ctypes.byref(p))
    if st != 0:
        raise Conv2dError(st, "conv2d_profile_read")
    names = ("weight_stage", "pack", "gemm", "implicit")
    return {names[k]: {"launches": int(p.launches[k]), "total_ms": float(p.total_ms[k])}
            for k in range(KERNEL_KINDS)}
