"""Host-side checks of the HIP library (no GPU needed): the shared library
loads, exports every entry point the header declares, plans every layer,
honours the workspace target, and rejects bad arguments before touching
the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import cnn_convolution_amd as conv
from cnn_convolution_amd import _lib
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "im2win_conv2d.h")


# LDS of the row-block and narrow kernels is at least their per-wave store
# scratch (8 waves x 16 x 68 floats)
STORE_SCRATCH = 8 * 16 * 68 * 4

def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z0-9_]+)\s*\([^;{]*\)\s*;", text)))


def test_header_declarations_match_binding():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_symbol():
    L = _lib.lib()
    for name in _lib.EXPORTS:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBPATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _lib.EXPORTS:
        assert name in exported, name


def test_device_code_is_gfx950_only():
    data = open(_lib.LIBPATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}


def test_status_strings():
    for code in range(9):
        s = conv.status_string(code)
        assert s and s != "unknown status"
    assert conv.status_string(99) == "unknown status"


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_plans_of_the_measured_layers(name):
    cfg = workloads.get_config(name)
    for dt in cfg.dtypes:
        code = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}[dt]
        d = conv.make_desc(*cfg.desc().values(), code)
        p = conv.plan(d)
        ho, wo = cfg.out_hw()
        assert (p.Ho, p.Wo) == (ho, wo)
        assert p.W_win == (wo - 1) * cfg.stride + cfg.KW
        assert p.rows_total == cfg.N * ho
        assert p.n_chunks * p.rows_per_chunk >= p.rows_total
        assert (p.n_chunks - 1) * p.rows_per_chunk < p.rows_total
        esz = 4 if dt == "f32" else 2
        assert p.im2col_bytes == cfg.N * ho * wo * cfg.Cin * cfg.KH * cfg.KW * esz
        assert p.ws_target_bytes == p.im2col_bytes // cfg.KW
        # the workspace target: at most 1/KW of the im2col buffer
        assert p.meets_ws_target == 1 and p.ws_bytes <= p.ws_target_bytes, (name, dt)
        assert conv.workspace_size(d) == p.ws_bytes
        assert p.flops == workloads.nominal_flops(**cfg.desc())
        assert p.path == (0 if dt == "f32" else 1)
        assert p.layout == (conv.LAYOUT_ROW if dt == "f32" else conv.LAYOUT_CL)
        # window rows and chunk buffer stay 16-byte aligned
        assert (p.row_elems * esz) % 16 == 0
        assert p.win_offset_bytes % 256 == 0


def test_plan_layout_geometry():
    d = conv.make_desc(32, 3, 224, 224, 64, 7, 7, 2, 3, conv.F16)
    p = conv.plan(d)
    assert p.Cin_pad == 4               # 3 channels, stride*KH even: padded to 4
    assert p.K_stage % 32 == 0 and p.K_stage >= 7 * 7 * 4
    d = conv.make_desc(1, 3, 32, 32, 16, 3, 3, 1, 1, conv.F16)
    assert conv.plan(d).Cin_pad == 8    # stride*KH odd: padded to 8
    d = conv.make_desc(1, 3, 32, 32, 16, 3, 3, 1, 1, conv.F32)
    p = conv.plan(d)
    assert p.Cin_pad == 3 and p.pos_pad % 8 == 0 and p.pos_pad >= 34 * 3
    d = conv.make_desc(64, 64, 56, 56, 256, 1, 1, 1, 0, conv.F16)
    p = conv.plan(d)
    assert p.wstage_bytes == 0          # 1x1 filter already in K order


def test_unreachable_target_is_reported(monkeypatch):
    # dense-as-conv: one window row alone exceeds 1/KW of im2col (window form)
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    d = conv.make_desc(2, 3, 5, 4, 6, 5, 4, 1, 0, conv.F32)
    p = conv.plan(d)
    assert p.Ho == 1 and p.Wo == 1 and p.meets_ws_target == 0
    assert p.rows_per_chunk == 1 and p.n_chunks == 2


@pytest.mark.parametrize("bad", [
    dict(N=0), dict(Cin=0), dict(H=0), dict(W=-1), dict(Cout=0), dict(KH=0), dict(KW=0),
    dict(stride=0), dict(pad=-1), dict(H=2, KH=5), dict(reserved=1),
    dict(N=1 << 21), dict(N=4096, Cin=4096, H=64, W=64),
])
def test_invalid_descriptors_rejected(bad):
    f = dict(N=1, Cin=3, H=8, W=8, Cout=4, KH=3, KW=3, stride=1, pad=1, dtype=conv.F32,
             reserved=0)
    f.update(bad)
    d = _lib.Desc(**f)
    assert conv.workspace_size(d) == 0
    p = _lib.Plan()
    assert _lib.lib().conv2d_plan(ctypes.byref(d), ctypes.byref(p)) == 1
    # conv2d_fwd validates before touching any pointer or the GPU
    assert _lib.fwd(d, 16, 16, 16, 256, None) == 1


def test_unknown_dtype_rejected():
    d = _lib.Desc(1, 3, 8, 8, 4, 3, 3, 1, 1, 7, 0)
    assert _lib.fwd(d, 16, 16, 16, 256, None) == 4


def test_pointer_checks_before_launch(monkeypatch):
    monkeypatch.setenv("IM2WIN_ALGO", "window")     # a form with a workspace
    d = conv.make_desc(1, 3, 8, 8, 4, 3, 3, 1, 1, conv.F32)
    ws = conv.workspace_size(d)
    assert ws > 0
    assert _lib.fwd(d, None, 16, 16, 256, None) == 2
    assert _lib.fwd(d, 16, None, 16, 256, None) == 2
    assert _lib.fwd(d, 16, 16, None, 256, None) == 2
    assert _lib.fwd(d, 16, 16, 16, None, None) == 5
    assert _lib.fwd(d, 8, 16, 16, 256, None) == 3
    assert _lib.fwd(d, 16, 16, 20, 256, None) == 3
    assert _lib.fwd(d, 16, 16, 16, 16, None) == 3          # ws must be 256-byte aligned
    assert _lib.pack(d, 0, 16, 16, 0, 0, None) == 7         # empty row range
    assert _lib.pack(d, 0, 16, 16, 5, 4, None) == 7         # past N*Ho
    assert _lib.pack(d, 1, 16, 16, 0, 1, None) == 4         # channels-last is half precision
    assert _lib.pack(d, 2, 16, 16, 0, 1, None) == 4
    assert _lib.weight_stage(d, 3, 16, 16, None) == 4
    assert _lib.weight_stage(d, conv.LAYOUT_FRAG, 16, 16, None) == 4   # fragment order: fp16/bf16 only
    assert _lib.pack(d, 0, None, 16, 0, 1, None) == 2
    for shape in [(1, 48, 8, 8, 16, 3, 3, 1, 1), (1, 64, 8, 8, 16, 7, 7, 1, 3)]:   # Cin % 32, filter
        assert _lib.weight_stage(conv.make_desc(*shape, conv.F16), conv.LAYOUT_FRAG, 16, 16, None) == 4


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0      # counts devices without initialising one


@pytest.mark.parametrize("algo", ["implicit", "window"])
@pytest.mark.parametrize("dt", [conv.F32, conv.F16])
def test_launch_failure_reports_hip_status(algo, dt, monkeypatch):
    """A valid call whose launch the HIP runtime refuses returns
    CONV2D_ERR_HIP (6) and does not abort: with no GPU in this process every
    launch fails after validation has passed. The pointers are aligned
    dummies, so the test never runs where a GPU is visible."""
    if _gpu_visible():
        pytest.skip("a GPU is visible: dummy pointers must never reach a real launch")
    monkeypatch.setenv("IM2WIN_ALGO", algo)
    X, W_, Y, WS = 1 << 20, 2 << 20, 3 << 20, 4 << 20      # aligned, never dereferenced
    for shape in [(2, 64, 12, 12, 64, 3, 3, 1, 1), (1, 3, 30, 30, 64, 7, 7, 2, 3),
                  (2, 128, 9, 9, 96, 3, 3, 2, 1)]:
        d = conv.make_desc(*shape, dt)
        st = _lib.fwd(d, X, W_, Y, WS, None)
        assert st == 6, (shape, st)
        assert conv.status_string(st) == "HIP runtime error"
    d = conv.make_desc(2, 64, 12, 12, 64, 3, 3, 1, 1, conv.F16)
    assert _lib.fwd_implicit(d, X, W_, Y, WS, None) == 6
    assert _lib.implicit_gemm(d, X, W_, Y, None) == 6
    assert _lib.pack(d, conv.LAYOUT_CL, X, WS, 0, 3, None) == 6
    assert _lib.weight_stage(d, conv.LAYOUT_CL, W_, WS, None) == 6
    assert _lib.window_gemm(d, WS, W_, Y, 0, 3, None) == 6
    d = conv.make_desc(2, 128, 12, 12, 64, 5, 5, 1, 2, conv.F16)     # the split-K kernel: staging, then the kernel
    assert conv.implicit_plan(d).kernel == 5
    assert _lib.fwd_implicit(d, X, W_, Y, WS, None) == 6
    assert _lib.weight_stage(d, conv.LAYOUT_FRAG, W_, WS, None) == 6


def _compiled_mfma_tiles():
    """The (MB, NB, KB, KS, WM) tiles the tiled matrix-core kernel is instantiated for,
    read from its dispatch list."""
    import re
    with open(os.path.join(ROOT, "cnn_convolution_amd", "csrc", "kernels", "gemm_mfma.hip")) as f:
        src = f.read()
    return {tuple(int(v) for v in m.groups())
            for m in re.finditer(r"^\s*IM2WIN_TILE\((\d+), (\d+), (\d+), (\d+), (\d+)\)",
                                 src, re.M)}


def test_planned_tiles_are_compiled():
    """Every tile the planner can pick is one the matrix-core kernels are built for."""
    import numpy as np
    compiled = _compiled_mfma_tiles()
    assert len(compiled) >= 15
    rng = np.random.default_rng(0)
    for _ in range(400):
        KH, KW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        s, p = int(rng.integers(1, 4)), int(rng.integers(0, 4))
        H, W = int(rng.integers(KH, 80)), int(rng.integers(KW, 80))
        d = conv.make_desc(int(rng.integers(1, 65)), int(rng.integers(1, 300)), H, W,
                           int(rng.integers(1, 600)), KH, KW, s, p,
                           [conv.F16, conv.BF16][int(rng.integers(0, 2))])
        pl = conv.plan(d)
        t = (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_kslice, pl.gemm_ksplit, pl.gemm_wave_m)
        assert pl.gemm_kernel in (1, 3)
        if pl.gemm_kernel == 3:
            assert (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_wave_m) in _compiled_dma_tiles()
            assert pl.K_stage % 64 == 0 and pl.gemm_kslice == 64 and pl.gemm_ksplit == 1
            continue
        assert t in compiled, t
        assert pl.K_stage % (pl.gemm_kslice * pl.gemm_ksplit) == 0


def test_tile_override_accepts_only_compiled_tiles(monkeypatch):
    """IM2WIN_MFMA_TILE selects a compiled tile and is ignored for anything else."""
    d = conv.make_desc(2, 64, 20, 20, 128, 3, 3, 1, 1, conv.F16)
    monkeypatch.setenv("IM2WIN_MFMA_KERNEL", "tiled")
    for t in sorted(_compiled_mfma_tiles()):
        monkeypatch.setenv("IM2WIN_MFMA_TILE", ",".join(str(v) for v in t))
        pl = conv.plan(d)
        got = (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_kslice, pl.gemm_ksplit, pl.gemm_wave_m)
        assert got == t
    monkeypatch.setenv("IM2WIN_MFMA_TILE", "96,96,64,1,2")
    pl = conv.plan(d)
    got = (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_kslice, pl.gemm_ksplit, pl.gemm_wave_m)
    assert got in _compiled_mfma_tiles()


def _compiled_dma_tiles():
    path = os.path.join(ROOT, "cnn_convolution_amd", "csrc", "kernels", "gemm_mfma_dma.hip")
    with open(path) as f:
        src = f.read()
    return {tuple(int(v) for v in m.groups())
            for m in re.finditer(r"launch_dma_tile<(\d+), (\d+), (\d+)>\(a, s\)", src)}


def test_dma_form_only_for_whole_k_stages(monkeypatch):
    """The direct-to-LDS form is planned wherever the window is a whole number of
    64-element K stages, and only there, with a tile it is built for."""
    import numpy as np
    compiled = _compiled_dma_tiles()
    assert len(compiled) == 6
    rng = np.random.default_rng(3)
    seen = 0
    for _ in range(300):
        KH, KW = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        Cin = int(rng.choice([3, 5, 8, 16, 24, 64, 96, 128, 256]))
        s, p = int(rng.integers(1, 3)), int(rng.integers(0, 3))
        H, W = int(rng.integers(KH, 40)), int(rng.integers(KW, 40))
        d = conv.make_desc(int(rng.integers(1, 9)), Cin, H, W, int(rng.integers(1, 300)),
                           KH, KW, s, p, conv.F16)
        monkeypatch.setenv("IM2WIN_MFMA_DMA_TILE", ",".join(map(str, sorted(compiled)[seen % 6])))
        pl = conv.plan(d)
        whole = pl.K_stage == KH * KW * pl.Cin_pad and pl.K_stage % 64 == 0
        assert (pl.gemm_kernel == 3) == whole
        if whole:
            seen += 1
            assert (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_wave_m) in compiled
            assert pl.gemm_kslice == 64 and pl.gemm_ksplit == 1
    assert seen > 20
    d = conv.make_desc(2, 64, 20, 20, 128, 3, 3, 1, 1, conv.F16)
    monkeypatch.delenv("IM2WIN_MFMA_DMA_TILE")
    default = conv.plan(d)
    monkeypatch.setenv("IM2WIN_MFMA_DMA_TILE", "96,96,2")     # not built: the planned tile
    pl = conv.plan(d)
    assert pl.gemm_kernel == 3
    assert (pl.gemm_tile_m, pl.gemm_tile_n, pl.gemm_wave_m) == \
        (default.gemm_tile_m, default.gemm_tile_n, default.gemm_wave_m)
    monkeypatch.setenv("IM2WIN_MFMA_KERNEL", "tiled")            # the other form, forced
    assert conv.plan(d).gemm_kernel == 1


def test_row_layout_keeps_slack_after_every_run():
    """The fp32 GEMM reads a lane's window run in whole 16-byte vectors (up to 3
    elements past it), so every channel run of the row-interleaved layout keeps at
    least 3 spare elements and the last read of a chunk stays inside it."""
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(300):
        KH, KW = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        s, p = int(rng.integers(1, 5)), int(rng.integers(0, 4))
        H, W = int(rng.integers(KH, 90)), int(rng.integers(KW, 90))
        d = conv.make_desc(int(rng.integers(1, 5)), int(rng.integers(1, 70)), H, W, 16, KH, KW,
                           s, p, conv.F32)
        pl = conv.plan(d)
        assert pl.pos_pad % 8 == 0 and pl.pos_pad >= pl.W_win * KH + 3
        assert pl.row_elems == d.Cin * pl.pos_pad


def test_implicit_plan_takes_only_its_layers():
    """The implicit form takes fp16/bf16 layers with Cin a multiple of 64 (and
    3x3 / 1x1 ones of stride 1 or 2 with Cin a multiple of 32) and reports UNSUPPORTED
    (status 4) for the rest, before touching any pointer."""
    assert conv._lib.implicit_plan_status(conv.make_desc(2, 64, 9, 9, 8, 3, 3, 1, 1, conv.F32)) == 4
    assert conv._lib.implicit_plan_status(conv.make_desc(2, 80, 9, 9, 8, 3, 3, 1, 1, conv.F16)) == 4
    assert conv._lib.implicit_plan_status(conv.make_desc(2, 96, 9, 9, 8, 3, 3, 3, 1, conv.F16)) == 4
    assert conv._lib.implicit_plan_status(conv.make_desc(2, 96, 9, 9, 8, 5, 5, 1, 1, conv.F16)) == 4
    assert conv.implicit_plan(conv.make_desc(2, 96, 9, 9, 8, 3, 3, 1, 1, conv.F16)).kernel == 4
    assert conv._lib.implicit_plan_status(conv.make_desc(2, 12, 9, 9, 8, 3, 3, 1, 1, conv.BF16)) == 4
    # up to 8 input channels: the narrow-channel kernel, any dtype
    for dt in (conv.F32, conv.F16, conv.BF16):
        assert conv.implicit_plan(conv.make_desc(2, 3, 9, 9, 8, 3, 3, 1, 1, dt)).kernel == 3
    assert conv._lib.implicit_plan_status(conv.make_desc(0, 64, 9, 9, 8, 3, 3, 1, 1, conv.F16)) == 1
    d = conv.make_desc(2, 80, 9, 9, 8, 3, 3, 1, 1, conv.F16)
    assert conv.implicit_workspace_size(d) == 0
    assert _lib.fwd_implicit(d, 16, 16, 16, 256, None) == 4
    d = conv.make_desc(2, 64, 9, 9, 8, 5, 5, 1, 2, conv.F16)     # the streamed kernel: a staged filter
    assert conv.implicit_workspace_size(d) > 0
    assert _lib.fwd_implicit(d, None, 16, 16, 256, None) == 2
    assert _lib.fwd_implicit(d, 16, 16, 16, None, None) == 5
    assert _lib.fwd_implicit(d, 8, 16, 16, 256, None) == 3
    assert _lib.fwd_implicit(d, 16, 16, 16, 16, None) == 3


def test_implicit_plan_geometry(monkeypatch):
    """Every implicit plan: the patch holds the tile's windows, the tile's columns
    fit its GEMM columns, LDS fits one CU, and the grid covers every output once."""
    import numpy as np
    rng = np.random.default_rng(11)
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "streamed")
    for _ in range(400):
        KH, KW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        s, p = int(rng.integers(1, 4)), int(rng.integers(0, 4))
        H, W = int(rng.integers(KH, 120)), int(rng.integers(KW, 240))
        Cin = 64 * int(rng.integers(1, 6))
        if rng.integers(0, 3) == 0:       # short K
            KH, KW = [(3, 3), (1, 1), (1, 1)][int(rng.integers(0, 3))]
            Cin = 64 if KH == 3 else int(rng.choice([64, 128, 256]))
            H, W = max(H, KH), max(W, KW)
        N, Cout = int(rng.integers(1, 9)), int(rng.integers(1, 600))
        d = conv.make_desc(N, Cin, H, W, Cout, KH, KW, s, p, [conv.F16, conv.BF16][int(rng.integers(0, 2))])
        pl = conv.implicit_plan(d)
        assert pl.rows_per_tile * pl.cols_per_tile <= pl.tile_n
        assert pl.patch_rows == (pl.rows_per_tile - 1) * s + KH
        assert pl.patch_cols == (pl.cols_per_tile - 1) * s + KW
        col_tiles = N * (-(-pl.Ho // pl.rows_per_tile)) * (-(-pl.Wo // pl.cols_per_tile))
        K = KH * KW * Cin
        assert pl.kernel == 0
        assert (pl.tile_m, pl.tile_n, pl.wave_m) in {(64, 64, 1), (64, 128, 1), (128, 64, 2), (128, 128, 2)}
        assert 3 <= pl.stages <= 5
        assert pl.lds_bytes == (pl.stages * pl.tile_m + pl.patch_rows * pl.patch_cols) * 128 <= 160 * 1024
        if pl.stages > 3:
            assert pl.lds_bytes <= 80 * 1024
        assert pl.tiles == (-(-Cout // pl.tile_m)) * col_tiles
        assert pl.K_stage == KW * KH * Cin
        staged = not (KH == 1 and KW == 1)
        assert (pl.ws_bytes > 0) == staged
        if staged:
            assert pl.ws_bytes >= Cout * pl.K_stage * 2


def test_conv2d_plan_names_the_form_conv2d_fwd_runs(monkeypatch):
    """algo 1 (implicit) only where the implicit form applies; its workspace is
    then the implicit one; IM2WIN_ALGO forces either form where it applies."""
    d = conv.make_desc(32, 64, 56, 56, 64, 3, 3, 1, 1, conv.F16)
    p = conv.plan(d)
    assert p.algo == 1
    assert p.ws_bytes == conv.implicit_workspace_size(d) == conv.workspace_size(d)
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    q = conv.plan(d)
    assert q.algo == 0 and q.ws_bytes == q.wstage_bytes + q.win_chunk_bytes
    monkeypatch.setenv("IM2WIN_ALGO", "implicit")
    for args in [(2, 16, 20, 20, 16, 3, 3, 1, 1, conv.F16), (2, 48, 20, 20, 16, 3, 3, 1, 1, conv.F32),
                 (2, 80, 20, 20, 16, 3, 3, 1, 1, conv.BF16)]:
        assert conv.plan(conv.make_desc(*args)).algo == 0     # not applicable: stays on the window form
    assert conv.plan(conv.make_desc(2, 256, 14, 14, 16, 3, 3, 1, 1, conv.BF16)).algo == 1


def test_row_block_plan_geometry(monkeypatch):
    """The row-block implicit kernel (asked for by name) is planned exactly for
    its layers (fp16/bf16, stride 1, Wo <= 64, a 3x3 or 1x1 filter; 64 input
    channels on rows of 8k elements, or any multiple of 64 channels where an
    image has at least 128 outputs): whole output rows per workgroup, the
    block's input rows and the filter in LDS, no workspace, one workgroup per
    (64-channel block, row block, image)."""
    import numpy as np
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    rng = np.random.default_rng(12)
    taken = 0
    for _ in range(600):
        KH, KW = [(3, 3), (1, 1), (5, 5), (3, 1)][int(rng.integers(0, 4))]
        s = int(rng.choice([1, 1, 1, 2]))
        p = int(rng.integers(0, 4))
        Cin = int(rng.choice([64, 64, 64, 128, 256]))
        W = int(rng.choice([8, 12, 14, 16, 24, 56, 60, 64, 72]))
        H = int(rng.integers(max(KH, 1), 40))
        N, Cout = int(rng.integers(1, 9)), int(rng.integers(1, 300))
        dt = [conv.F16, conv.BF16][int(rng.integers(0, 2))]
        d = conv.make_desc(N, Cin, H, W, Cout, KH, KW, s, p, dt)
        if conv._lib.implicit_plan_status(d) != 0:
            continue
        pl = conv.implicit_plan(d)
        eligible = (s == 1 and pl.Wo <= 64 and (KH, KW) in ((3, 3), (1, 1)) and
                    ((Cin == 64 and W % 8 == 0) or pl.Ho * pl.Wo >= 128))
        assert (pl.kernel == 2) == eligible, (N, Cin, H, W, Cout, KH, KW, s, p)
        if not eligible:
            continue
        taken += 1
        R = pl.rows_per_tile
        assert 1 <= R <= pl.Ho and R * pl.Wo <= 512
        assert pl.patch_rows == R + KH - 1 and pl.patch_cols == W + 2 * p
        assert pl.cols_per_tile == pl.Wo and pl.tile_m == 64 and pl.tile_n == 64
        assert pl.lds_bytes == max(KH * KW * 8192 + pl.patch_rows * pl.patch_cols * 128, STORE_SCRATCH) <= 160 * 1024
        assert pl.tiles == -(-Cout // 64) * N * -(-pl.Ho // R)
        assert pl.ws_bytes == 0 == conv.implicit_workspace_size(d)
        assert conv.plan(d).algo == 1 and conv.workspace_size(d) == 0
    assert taken > 50
    # the other kernels stay reachable
    monkeypatch.delenv("IM2WIN_IMPLICIT_KERNEL")
    d = conv.make_desc(32, 64, 56, 56, 64, 3, 3, 1, 1, conv.F16)
    # 8 rows: 8 * 56 fp32 outputs are whole 128-byte lines, written through (7 rows by the count alone)
    assert conv.implicit_plan(d).kernel == 2 and conv.implicit_plan(d).rows_per_tile == 8
    d32 = conv.make_desc(32, 64, 56, 56, 64, 3, 3, 1, 1, conv.F32)
    assert conv.implicit_plan(d32).rows_per_tile == 7
    d16 = conv.make_desc(32, 64, 56, 56, 64, 3, 3, 1, 1, conv.F16, conv.F16)
    assert conv.implicit_plan(d16).rows_per_tile == 7          # half y: the LDS-staged stores
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "streamed")
    assert conv.implicit_plan(d).kernel == 0 and conv.implicit_plan(d).ws_bytes > 0
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", "3")
    assert conv.implicit_plan(d).kernel == 2 and conv.implicit_plan(d).rows_per_tile == 3


def test_pipelined_plan_geometry(monkeypatch):
    """By default the one-block row kernel keeps its layers (64 channels on rows
    of 8k elements, Wo <= 64) and the pipelined row-block kernels take the other
    3x3 and 1x1 fp16/bf16 layers of stride 1 or 2 with Cin a multiple of 32 and
    Wo <= 256: tasks of R whole output rows x 64 output channels, or of several whole
    small images, at most 256 outputs, 32-channel chunks in LDS (two slots and
    persistent workgroups, or one slot of at most 80 KB, one task per
    workgroup), no workspace."""
    import numpy as np
    seen = {1: 0, 2: 0, "images": 0}
    for form, images in ((None, None), ("pair", None), ("pipe", "3"), ("pair", "2")):
        if form:
            monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
        if images:
            monkeypatch.setenv("IM2WIN_IMPLICIT_IMAGES", images)
        rng = np.random.default_rng(14)
        for _ in range(800):
            KH, KW = [(3, 3), (1, 1), (5, 5)][int(rng.integers(0, 3))]
            s = int(rng.choice([1, 1, 1, 2]))
            p = int(rng.integers(0, 3))
            Cin = int(rng.choice([32, 64, 96, 128, 256]))
            W = int(rng.choice([4, 7, 8, 12, 14, 16, 28, 56, 60, 112, 150]))
            H = int(rng.integers(max(KH, 1), 40))
            N, Cout = int(rng.integers(1, 9)), int(rng.integers(1, 300))
            d = conv.make_desc(N, Cin, H, W, Cout, KH, KW, s, p, [conv.F16, conv.BF16][int(rng.integers(0, 2))])
            if conv._lib.implicit_plan_status(d) != 0:
                continue
            pl = conv.implicit_plan(d)
            pipelined = s <= 2 and (KH, KW) in ((3, 3), (1, 1)) and Cin % 32 == 0 and pl.Wo <= 256
            one_block = Cin == 64 and W % 8 == 0 and s == 1 and pl.Wo <= 64 and (KH, KW) in ((3, 3), (1, 1))
            if form is None and one_block:
                assert pl.kernel == 2, (N, Cin, H, W, Cout, KH, KW, s, p)
                continue
            if pl.kernel != 4:
                # only where a pipelined form does not apply, or its LDS does not
                # fit, or (by default) the split-K kernel takes the layer: stride
                # 2 with Cin a multiple of 128
                splitk = form is None and s == 2 and Cin % 128 == 0 and pl.kernel == 5
                assert not pipelined or pl.lds_bytes == 0 or form or splitk, (N, Cin, H, W, Cout, KH, KW, s, p)
                continue
            assert pipelined
            seen[pl.stages] += 1
            R, img = pl.rows_per_tile, pl.images
            assert img >= 1 and 1 <= R <= pl.Ho and img * R * pl.Wo <= 256
            if img > 1:
                seen["images"] += 1
                assert R == pl.Ho and img <= N and (images or pl.Ho * pl.Wo < 128)
            assert pl.patch_rows == img * ((R - 1) * s + KH) and pl.patch_cols == W + 2 * p
            assert pl.cols_per_tile == pl.Wo
            cob = -(-Cout // 64)
            tasks = cob * -(-N // img) if img > 1 else cob * N * -(-pl.Ho // R)
            taps = KH * KW
            if pl.stages == 2:
                assert pl.lds_bytes == 2 * (taps * 4096 + pl.patch_rows * pl.patch_cols * 64) + 4 * 16 * 68 * 4
                assert pl.tiles == min(tasks, 256)
            else:
                assert pl.lds_bytes == max(taps * 4096 + pl.patch_rows * pl.patch_cols * 64, STORE_SCRATCH)
                assert pl.lds_bytes <= 80 * 1024 and pl.tiles == tasks
                if form is None:
                    assert tasks >= 512 and (img * R * pl.Wo >= 128 or tasks >= 1024)
            assert pl.lds_bytes <= 160 * 1024
            assert pl.ws_bytes == 0 == conv.implicit_workspace_size(d)
            assert conv.plan(d).algo == 1
    assert seen[1] > 20 and seen[2] > 20 and seen["images"] > 10, seen
    # the layers measured: the persistent form for the deep 14x14 layer and the
    # small-image 512-channel layers, the paired one for the Table I 28x28,
    # 14x14, 12x12 and 112x112 3x3 layers
    monkeypatch.delenv("IM2WIN_IMPLICIT_KERNEL")
    monkeypatch.delenv("IM2WIN_IMPLICIT_IMAGES")
    for name, stages, img in [("deep3x3", 2, 1), ("mix512", 2, 2), ("cv12", 2, 8), ("cv6", 1, 2),
                              ("cv8", 1, 1), ("cv10", 1, 1), ("cv11", 1, 1)]:
        cfg = workloads.get_config(name)
        dt = conv.BF16 if name == "deep3x3" else conv.F16
        pl = conv.implicit_plan(conv.make_desc(*cfg.desc().values(), dt))
        assert (pl.kernel, pl.stages, pl.images) == (4, stages, img), name


def test_row_block_plan_fp32():
    """fp32 layers go to the implicit form only through the row-block kernel
    (fp32 matrix-core products): Cin a multiple of 32, stride 1, W % 4 == 0
    (or any width where an image has at least 128 outputs),
    Wo <= 64, a 3x3 or 1x1 filter; every other fp32 layer stays on the
    vector-ALU window form."""
    import numpy as np
    rng = np.random.default_rng(13)
    seen = {True: 0, False: 0}
    for _ in range(500):
        KH, KW = [(3, 3), (1, 1), (5, 5), (1, 3)][int(rng.integers(0, 4))]
        s = int(rng.choice([1, 1, 2]))
        p = int(rng.integers(0, 3))
        Cin = int(rng.choice([3, 32, 48, 64, 96, 128]))
        W = int(rng.choice([6, 8, 12, 14, 28, 56, 60, 64, 70]))
        H = int(rng.integers(KH, 30))
        N, Cout = int(rng.integers(1, 5)), int(rng.integers(1, 200))
        d = conv.make_desc(N, Cin, H, W, Cout, KH, KW, s, p, conv.F32)
        Wo = (W + 2 * p - KW) // s + 1
        Ho = (H + 2 * p - KH) // s + 1
        if Wo < 1 or Ho < 1:
            continue
        eligible = (Cin % 32 == 0 and s == 1 and (W % 4 == 0 or Ho * Wo >= 128) and Wo <= 64 and
                    (KH, KW) in ((3, 3), (1, 1)))
        narrow = Cin <= 8 and Wo <= 512
        seen[eligible] += 1
        st = conv._lib.implicit_plan_status(d)
        assert (st == 0) == (eligible or narrow), (N, Cin, H, W, Cout, KH, KW, s, p)
        pl = conv.plan(d)
        assert pl.algo == (1 if eligible or narrow else 0)
        if eligible or narrow:
            ip = conv.implicit_plan(d)
            assert ip.kernel == (2 if eligible else 3) and pl.ws_bytes == ip.ws_bytes
            # w read as stored, except by narrow launches of more than 256 workgroups
            assert (ip.ws_bytes == 0) == (eligible or ip.tiles <= 256)
            if eligible:
                assert ip.lds_bytes == max(KH * KW * 8192 + ip.patch_rows * ip.patch_cols * 128, STORE_SCRATCH) <= 160 * 1024
        else:
            assert pl.ws_bytes == pl.wstage_bytes + pl.win_chunk_bytes
    assert seen[True] > 30 and seen[False] > 30


def test_narrow_plan_geometry():
    """Layers with up to 8 input channels take the narrow-channel implicit kernel
    in every dtype: CP = 4 channels per window position (8 where a window start
    would leave a 16-byte boundary, or for 5..8 channels), R * Wo <= 512 outputs
    per workgroup, the filter block and R window rows (with slack for the padded
    K of the last window) in LDS, no workspace."""
    import numpy as np
    rng = np.random.default_rng(14)
    taken = 0
    for _ in range(600):
        KH, KW = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        s, p = int(rng.integers(1, 5)), int(rng.integers(0, 4))
        Cin = int(rng.integers(1, 9))
        H, W = int(rng.integers(KH, 240)), int(rng.integers(KW, 240))
        N, Cout = int(rng.integers(1, 9)), int(rng.integers(1, 200))
        dt = [conv.F32, conv.F16, conv.BF16][int(rng.integers(0, 3))]
        d = conv.make_desc(N, Cin, H, W, Cout, KH, KW, s, p, dt)
        es = 4 if dt == conv.F32 else 2
        if conv._lib.implicit_plan_status(d) != 0:
            # not taken: output rows too long, or the filter block and one
            # window row do not fit LDS
            Wo = (W + 2 * p - KW) // s + 1
            cp = 4 if (Cin <= 4 and (s * KH * 4 * es) % 16 == 0) else 8
            K = KW * KH * cp
            Kp = -(-K // (16 if dt == conv.F32 else 32)) * (16 if dt == conv.F32 else 32)
            L = ((Wo - 1) * s + KW) * KH * cp
            Lp = -(-(L + Kp - K) // (16 // es)) * (16 // es)
            assert Wo > 512 or 64 * (Kp + 16 // es) * es + max(Lp * es, STORE_SCRATCH) > 160 * 1024
            continue
        pl = conv.implicit_plan(d)
        assert pl.kernel == 3
        taken += 1
        cp = pl.stages
        assert cp in (4, 8) and Cin <= cp
        assert (s * KH * cp * es) % 16 == 0
        if cp == 8 and Cin <= 4:
            assert (s * KH * 4 * es) % 16 != 0
        K = KW * KH * cp
        kstep = 16 if dt == conv.F32 else 32
        Kp = -(-K // kstep) * kstep
        L = ((pl.Wo - 1) * s + KW) * KH * cp
        vec = 16 // es
        Lp = -(-(L + Kp - K) // vec) * vec
        R = pl.rows_per_tile
        assert pl.patch_cols == Lp and pl.patch_rows == R and 1 <= R <= pl.Ho and R * pl.Wo <= 512
        assert pl.lds_bytes == 64 * (Kp + 16 // es) * es + max(R * Lp * es, STORE_SCRATCH) <= 160 * 1024
        # one row block per workgroup, or (fp32, filter blocks over 48 KB)
        # persistent workgroups, one per CU
        cob = -(-Cout // 64)
        rb = N * -(-pl.Ho // R)
        persistent = dt == conv.F32 or 64 * Kp * es > 48 * 1024
        assert pl.tiles == cob * (min(rb, max(1, 256 // cob)) if persistent else rb)
        # the filter gathered from w as stored into LDS rows of Kp by launches
        # of at most 256 workgroups (no workspace), else staged [Cout][Kp]
        staged = -(-(Cout * Kp * es) // 256) * 256
        assert pl.K_stage == Kp and pl.ws_bytes == (0 if pl.tiles <= 256 else staged)
        assert conv.implicit_workspace_size(d) == pl.ws_bytes
    assert taken > 300


def test_plans_are_cached_per_descriptor_and_override(monkeypatch):
    """Repeated plans of one descriptor are the same; an IM2WIN_* override in
    the environment is part of the cache key, so changing it changes the plan,
    and removing it brings the first plan back."""
    for k in [k for k in os.environ if k.startswith("IM2WIN_")]:
        monkeypatch.delenv(k)
    d = conv.make_desc(2, 128, 14, 14, 72, 3, 3, 1, 1, conv.F16)
    first = conv.implicit_plan(d).as_dict()
    assert conv.implicit_plan(d).as_dict() == first and first["kernel"] == 4
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "streamed")
    assert conv.implicit_plan(d).kernel == 0
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "rows")
    assert conv.implicit_plan(d).kernel == 2
    monkeypatch.delenv("IM2WIN_IMPLICIT_KERNEL")
    assert conv.implicit_plan(d).as_dict() == first
    # the window-form plan follows the same rule
    p0 = conv.plan(d).as_dict()
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    assert conv.plan(d).algo == 0 and p0["algo"] == 1
    monkeypatch.delenv("IM2WIN_ALGO")
    assert conv.plan(d).as_dict() == p0
    # more descriptors than the cache holds: plans stay right
    for n in range(1, 1200):
        q = conv.plan(conv.make_desc(n, 16, 8, 8, 8, 3, 3, 1, 1, conv.F32))
        assert q.rows_total == n * 8
    assert conv.implicit_plan(d).as_dict() == first


# the variant of the direct-to-LDS window-GEMM the planner keeps per layer
# (as Table II of the im2win paper picks per layer), against the fastest
# measured variant of the ablation on MI355X: one stage buffer (bit 2) for the
# 1x1 layer and Table I's cv10 / cv11, all three optimisations elsewhere
_ABLATION_CHOICE = {"resnet3x3": 0, "deep3x3": 0, "mix5x5": 0, "mix512": 0, "mix3x3s2": 0, "mix1x1": 4,
                    "cv9": 0, "cv10": 4, "cv11": 4, "cv12": 0}


@pytest.mark.parametrize("name", sorted(_ABLATION_CHOICE))
def test_planner_picks_the_measured_ablation_variant(name, monkeypatch):
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    cfg = workloads.get_config(name)
    dt = conv.BF16 if name == "deep3x3" else conv.F16
    p = conv.plan(conv.make_desc(*cfg.desc().values(), dt))
    assert p.gemm_kernel == 3 and p.gemm_ablate == _ABLATION_CHOICE[name]
    monkeypatch.setenv("IM2WIN_ABLATE", "serpentine")          # the override still wins
    assert conv.plan(conv.make_desc(*cfg.desc().values(), dt)).gemm_ablate == 1


def test_ksplit_plan_geometry(monkeypatch):
    """The split-K kernel (5): planned by default for 5x5 filters with Cin a
    multiple of 128, by name elsewhere; tasks of at most 224 outputs, whole
    images stacked for small images, the fragment-ordered filter as workspace
    and LDS within one CU."""
    from cnn_convolution_amd import _lib as L
    # 5x5: 4-row tasks of 128 output channels (the rounds tie with 7-row tasks
    # of 64 channels; the 4-row ones issue fewer padded products)
    five = conv.implicit_plan(conv.make_desc(64, 128, 28, 28, 128, 5, 5, 1, 2, conv.F16))
    assert five.kernel == 5 and five.rows_per_tile == 4 and five.images == 1
    assert (five.tile_m, five.stages) == (128, 2)
    assert five.tiles == 1 * 64 * 7 and five.ws_bytes == 128 * 128 * 25 * 2
    assert five.lds_bytes <= 160 * 1024 and five.wave_m == 4
    assert conv.plan(conv.make_desc(64, 128, 28, 28, 128, 5, 5, 1, 2, conv.F16)).ws_bytes == five.ws_bytes
    for shape in [(64, 256, 14, 14, 256, 3, 3, 1, 1), (64, 512, 7, 7, 512, 3, 3, 1, 1),
                  (2, 64, 28, 28, 64, 5, 5, 1, 2)]:          # stride-1 3x3 layers, and Cin % 128 != 0
        assert conv.implicit_plan(conv.make_desc(*shape, conv.F16)).kernel != 5, shape
    # stride 2: 7-row tasks of 128 output channels (the two waves of a K group
    # on 64 channels each), one LDS slot per K group (two do not fit)
    s2 = conv.implicit_plan(conv.make_desc(64, 256, 28, 28, 512, 3, 3, 2, 1, conv.F16))
    assert (s2.kernel, s2.tile_m, s2.stages, s2.rows_per_tile, s2.images) == (5, 128, 1, 7, 1)
    assert s2.tiles == 4 * 64 * 2 and s2.lds_bytes <= 160 * 1024
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    deep = conv.implicit_plan(conv.make_desc(64, 256, 14, 14, 256, 3, 3, 1, 1, conv.BF16))
    assert (deep.kernel, deep.rows_per_tile, deep.images, deep.tiles) == (5, 14, 1, 256)
    assert (deep.tile_m, deep.stages) == (64, 2)
    assert deep.ws_bytes == 256 * 256 * 9 * 2 and deep.patch_rows == 16 and deep.patch_cols == 16
    m512 = conv.implicit_plan(conv.make_desc(64, 512, 7, 7, 512, 3, 3, 1, 1, conv.F16))
    assert (m512.kernel, m512.images, m512.rows_per_tile, m512.tiles) == (5, 2, 7, 8 * 32)
    assert m512.patch_rows == 2 * 9 and m512.lds_bytes <= 160 * 1024
    odd = conv.implicit_plan(conv.make_desc(3, 128, 9, 9, 70, 3, 3, 1, 1, conv.F16))
    assert odd.kernel == 5 and odd.ws_bytes == 128 * 128 * 9 * 2       # Cout padded to 128
    for p in (five, deep, m512, odd):
        assert p.images * p.rows_per_tile * p.Wo <= 224
    assert conv.implicit_plan(conv.make_desc(2, 64, 9, 9, 64, 3, 3, 1, 1, conv.F16)).kernel != 5
    assert L.LAYOUT_FRAG == 2
