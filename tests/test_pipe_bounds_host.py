"""Host model of the input reads of the pipelined row-block kernels
(conv_implicit_pipe.hip: task decomposition, chunk_geom and load_patch_unit),
checked on the CPU: every 16-, 8- or 2-byte load of every task and channel
chunk stays inside its own channel plane of x. The shapes include padding
wider than the filter, where the last row tasks lie wholly in the padding
below the image, planes that are not a multiple of 8 positions, and stride 2.
No GPU is used; the plans come from the library's planner."""
import pytest

import cnn_convolution_amd as conv

SHAPES = [
    # N, Cin, H, W, Cout, KH, KW, stride, pad
    (8, 64, 8, 4, 64, 1, 1, 1, 2),       # 1x1 pad 2: the last row task lies below the image
    (2, 64, 6, 6, 72, 3, 3, 1, 4),       # 3x3 pad 4
    (1, 32, 5, 7, 40, 3, 3, 1, 4),       # odd planes (2-byte loads)
    (3, 64, 7, 6, 64, 1, 1, 2, 3),       # stride 2, 1x1 pad 3
    (2, 96, 9, 10, 64, 3, 3, 2, 4),      # stride 2, planes of 2 mod 4
    (4, 64, 12, 12, 64, 3, 3, 1, 1),     # the usual case
    (6, 64, 7, 7, 72, 3, 3, 1, 1),       # whole-image tasks
]


def _vec(hw):
    return 8 if hw % 8 == 0 else 4 if hw % 4 == 0 else 1


def _reads(shape, pl, clamp=True):
    """Yield (plane index, first position, V) of every load the kernel issues."""
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    Ho, R, img = pl.Ho, pl.rows_per_tile, max(pl.images, 1)
    co_blocks = -(-Cout // 64)
    row_groups = -(-Ho // R)
    ntasks = co_blocks * (-(-N // img) if img > 1 else N * row_groups)
    V = _vec(H * W)
    for t in range(ntasks):
        r = t // co_blocks
        if img > 1:
            n, nimg, ho0, rw = r * img, min(img, N - r * img), 0, Ho
        else:
            n, nimg, ho0 = r // row_groups, 1, (r % row_groups) * R
            rw = min(R, Ho - ho0)
        ih0 = ho0 * s - p
        SL = (rw - 1) * s + KH
        if clamp:
            r_lo = min(max(ih0, 0), H)
            r_hi = max(min(ih0 + SL, H), r_lo)
            p_lo, p_hi = r_lo * W, r_hi * W
        else:                                   # the form before the clamp
            r_lo, r_hi = max(ih0, 0), min(ih0 + SL, H)
            p_lo, p_hi = r_lo * W, max(r_hi, r_lo) * W
        j_lo = p_lo // V
        units1 = 4 * (-(-p_hi // V) - j_lo)
        for u in range(units1 * nimg):
            im, u1 = divmod(u, units1)
            g, j = u1 & 3, j_lo + (u1 >> 2)
            for blk in range(Cin // 32):
                for e in range(8):
                    yield (n + im) * Cin + blk * 32 + g * 8 + e, j * V, V


@pytest.mark.parametrize("form", ["pipe", "pair"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_pipelined_kernel_reads_stay_in_their_planes(shape, form, monkeypatch):
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", form)
    pl = conv.implicit_plan(conv.make_desc(*shape, conv.F16))
    assert pl.kernel == 4 and pl.stages == (2 if form == "pipe" else 1)
    N, Cin, H, W = shape[:4]
    n = 0
    for plane, pos, V in _reads(shape, pl):
        assert 0 <= plane < N * Cin and 0 <= pos and pos + V <= H * W, (plane, pos, V)
        n += 1
    assert n > 0


def test_unclamped_row_range_read_past_the_plane(monkeypatch):
    """The model catches what the clamp fixed: with pad > KH the last row task's
    rows start below the image, and the unclamped range loaded a unit past the
    end of the plane (past the end of x for the last image)."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "pipe")
    shape = SHAPES[0]
    pl = conv.implicit_plan(conv.make_desc(*shape, conv.F16))
    N, Cin, H, W = shape[:4]
    bad = [(pl_, pos, V) for pl_, pos, V in _reads(shape, pl, clamp=False) if pos + V > H * W]
    assert bad and max(pl_ for pl_, _, _ in bad) == N * Cin - 1


KS_SHAPES = [
    # N, Cin, H, W, Cout, KH, KW, stride, pad (Cin a multiple of 128)
    (8, 128, 8, 4, 64, 1, 1, 1, 2),      # 1x1 pad 2: row tasks below the image
    (2, 128, 6, 6, 72, 3, 3, 1, 4),      # 3x3 pad 4
    (1, 256, 5, 7, 40, 3, 3, 1, 4),      # odd planes
    (3, 128, 7, 6, 64, 1, 1, 2, 3),      # stride 2
    (2, 384, 9, 10, 64, 3, 3, 2, 4),     # stride 2, three chunks per K group
    (64, 256, 14, 14, 256, 3, 3, 1, 1),  # the deep 3x3 layer
    (64, 512, 7, 7, 512, 3, 3, 1, 1),    # the 512-channel 7x7 layer (two images per task)
    (4, 128, 28, 28, 128, 5, 5, 1, 2),   # the 5x5 layer's images
]


@pytest.mark.parametrize("rows", [None, 1, 2])
@pytest.mark.parametrize("shape", KS_SHAPES, ids=[str(s) for s in KS_SHAPES])
def test_ksplit_kernel_reads_and_patch_writes_stay_in_bounds(shape, rows, monkeypatch):
    """The split-K kernel loads its patches with the same task and chunk
    geometry: every read stays inside its own plane of x, and every position
    the loads write (row0 + r) * IW + pad + col lies inside the task's patch
    of images * SL rows of IW positions."""
    monkeypatch.setenv("IM2WIN_IMPLICIT_KERNEL", "ksplit")
    if rows is not None:
        monkeypatch.setenv("IM2WIN_IMPLICIT_ROWS", str(rows))
    pl = conv.implicit_plan(conv.make_desc(*shape, conv.F16))
    assert pl.kernel == 5
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    n = 0
    for plane, pos, V in _reads(shape, pl):
        assert 0 <= plane < N * Cin and 0 <= pos and pos + V <= H * W, (plane, pos, V)
        n += 1
    assert n > 0
    # patch positions written: rows of the image inside the task, shifted by the task's first row
    Ho, R, img = pl.Ho, pl.rows_per_tile, max(pl.images, 1)
    IW = W + 2 * p
    for ho0 in range(0, Ho, R):
        rw = min(R, Ho - ho0)
        ih0, SL = ho0 * s - p, (rw - 1) * s + KH
        assert img * SL <= pl.patch_rows and pl.patch_cols == IW
        for ih in range(max(ih0, 0), min(ih0 + SL, H)):
            for col in range(W):
                q = (ih - ih0) * IW + p + col
                assert 0 <= q < SL * IW
