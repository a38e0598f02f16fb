"""Pins for the CPU oracle: what the pages and the mathematics fix, independent
of the oracle's own code (no retyping of its formula).

* output extents against Table I and the pages' worked examples;
* the whole sum against a library convolution (torch, CPU, float64) and against
  an im2col + matmul lowering written here;
* bit-exact agreement on integer-valued inputs;
* closed forms: delta filters, all-ones input, 1x1 = GEMM, dense = GEMV,
  linearity, and the 1-D worked example of the Winograd section.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=")
            out[k.strip()] = [int(t) for t in v.split()]
    return out


def _torch_conv(x, w, s, p):
    return F.conv2d(torch.from_numpy(np.asarray(x, np.float64)),
                    torch.from_numpy(np.asarray(w, np.float64)), stride=s, padding=p).numpy()


def _im2col(x, KH, KW, s, p):
    """Lowering as one gather: entry ((c, kh, kw), (ho, wo)) of image n is
    x[n, c, ho*s + kh - p, wo*s + kw - p], or zero where that index leaves the
    image (zero padding). Returns [N][Cin*KH*KW][Ho*Wo]."""
    N, C, H, W = x.shape
    Ho = (H + 2 * p - KH) // s + 1
    Wo = (W + 2 * p - KW) // s + 1
    kh, kw, ho, wo = np.meshgrid(np.arange(KH), np.arange(KW), np.arange(Ho), np.arange(Wo),
                                 indexing="ij")
    ih = ho * s + kh - p                          # [KH][KW][Ho][Wo] input row of each entry
    iw = wo * s + kw - p
    inside = (ih >= 0) & (ih < H) & (iw >= 0) & (iw < W)
    g = x[:, :, np.clip(ih, 0, H - 1), np.clip(iw, 0, W - 1)]   # [N][C][KH][KW][Ho][Wo]
    g = np.where(inside, g, np.zeros((), x.dtype))
    return g.reshape(N, C * KH * KW, Ho * Wo), Ho, Wo


def _im2col_conv(x, w, s, p):
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cols, Ho, Wo = _im2col(x, w.shape[2], w.shape[3], s, p)
    y = np.einsum("ok,nkl->nol", w.reshape(w.shape[0], -1), cols)
    return y.reshape(x.shape[0], w.shape[0], Ho, Wo)


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < count:
        N = int(rng.integers(1, 3))
        Cin = int(rng.integers(1, 6))
        Cout = int(rng.integers(1, 6))
        KH = int(rng.integers(1, 5))
        KW = int(rng.integers(1, 5))
        s = int(rng.integers(1, 4))
        p = int(rng.integers(0, max(KH, KW) + 1))
        H = int(rng.integers(1, 10))
        W = int(rng.integers(1, 10))
        if H + 2 * p < KH or W + 2 * p < KW:
            continue
        shapes.append((N, Cin, H, W, Cout, KH, KW, s, p))
    return shapes


# ---------------------------------------------------------------- shapes

def test_table1_output_extents(orc):
    rows = []
    with open(os.path.join(GOLDEN, "table1_shapes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                rows.append(line)
    assert len(rows) == 12
    for r in rows:
        ci, hi, wi, co, hf, wf, s, oco, oho, owo = map(int, r[1:])
        assert co == oco
        assert orc.out_extent(hi, hf, s, 0) == oho, r[0]
        assert orc.out_extent(wi, wf, s, 0) == owo, r[0]


def test_page_shape_examples(orc):
    g = _read_golden_kv("page_examples.txt")
    C, H, W = g["p5_im2col_input"]
    kh, kw, s, p = g["p5_im2col_kernel"]
    rows, cols = g["p5_im2col_shape"]
    assert C * kh * kw == rows
    assert orc.out_extent(H, kh, s, p) * orc.out_extent(W, kw, s, p) == cols
    # the same shape from the test's own lowering
    c, Ho, Wo = _im2col(np.zeros((1, C, H, W)), kh, kw, s, p)
    assert c.shape[1:] == (rows, cols)

    cin, h, w, k, s, p = g["p5_buffer_layer"]
    elems = cin * k * k * orc.out_extent(h, k, s, p) * orc.out_extent(w, k, s, p)
    assert elems == g["p5_buffer_elements"][0]
    assert round(elems * 4 / 1e6) == g["p5_buffer_mb_approx"][0]

    n, c, h, w = g["fig1_input"]
    co, ci, fh, fw = g["fig1_filter"]
    assert ci == c
    ho, wo = orc.out_extent(h, fh, 1, 0), orc.out_extent(w, fw, 1, 0)
    assert [n, co, ho, wo] == g["fig1_output"]

    N, Cin, H, W, Cout, KH, KW, s, p = g["p4_layer"]
    assert [N, Cout, orc.out_extent(H, KH, s, p), orc.out_extent(W, KW, s, p)] == g["p4_output"]


def test_bad_shapes_rejected(orc):
    assert orc.out_extent(3, 5, 1, 0) == 0
    assert orc.out_extent(3, 5, 1, 1) == 1
    assert orc.out_extent(10, 3, 0, 1) == 0
    with pytest.raises(ValueError):
        orc.conv2d(np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 3, 3)), 1, 0)


# ---------------------------------------------------------------- the sum

@pytest.mark.parametrize("shape", _random_shapes(7, 40))
def test_matches_library_conv(orc, shape):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    rng = np.random.default_rng(hash(shape) % (2 ** 32))
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin, KH, KW))
    y = orc.conv2d(x, w, s, p)
    ref = _torch_conv(x, w, s, p)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", _random_shapes(8, 25))
def test_matches_im2col_lowering(orc, shape):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    rng = np.random.default_rng(1 + hash(shape) % (2 ** 32))
    x = rng.uniform(-1, 1, (N, Cin, H, W))
    w = rng.uniform(-1, 1, (Cout, Cin, KH, KW))
    np.testing.assert_allclose(orc.conv2d(x, w, s, p), _im2col_conv(x, w, s, p),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", _random_shapes(9, 20) + [(2, 3, 32, 32, 16, 3, 3, 1, 1),
                                                           (1, 3, 23, 23, 4, 7, 7, 2, 3)])
def test_integer_inputs_bit_exact(orc, shape):
    N, Cin, H, W, Cout, KH, KW, s, p = shape
    rng = np.random.default_rng(11)
    x = rng.integers(-3, 4, (N, Cin, H, W)).astype(np.float64)
    w = rng.integers(-3, 4, (Cout, Cin, KH, KW)).astype(np.float64)
    y = orc.conv2d(x, w, s, p)
    assert np.array_equal(y, _torch_conv(x, w, s, p))
    assert np.array_equal(y, _im2col_conv(x, w, s, p))
    assert np.array_equal(y, np.round(y))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K,s,a,b,p", [(3, 1, 1, 1, 1), (3, 1, 0, 2, 1), (5, 1, 2, 2, 2),
                                       (3, 2, 1, 1, 1), (4, 1, 3, 0, 0), (3, 3, 2, 0, 2)])
def test_delta_filter(orc, K, s, a, b, p):
    rng = np.random.default_rng(3)
    N, C, H, W = 2, 3, 9, 11
    x = rng.standard_normal((N, C, H, W))
    w = np.zeros((C, C, K, K))
    for c in range(C):
        w[c, c, a, b] = 1.0
    y = orc.conv2d(x, w, s, p)
    xp = np.pad(x, ((0, 0), (0, 0), (p, p), (p, p)))
    Ho, Wo = y.shape[2:]
    # Y[n,c,ho,wo] = Xp[n,c, ho*s + a, wo*s + b]   (padded coordinates)
    expect = xp[:, :, a:a + s * (Ho - 1) + 1:s, b:b + s * (Wo - 1) + 1:s]
    assert np.array_equal(y, expect)
    if s == 1 and a == b == p and 2 * p + 1 == K:
        assert np.array_equal(y, x)                # identity


def test_all_ones_input(orc):
    rng = np.random.default_rng(5)
    N, C, H, W, Co, K, s, p = 1, 4, 8, 9, 3, 3, 1, 1
    w = rng.standard_normal((Co, C, K, K))
    y = orc.conv2d(np.ones((N, C, H, W)), w, s, p)
    # interior: the full filter sum per output channel
    np.testing.assert_allclose(y[0, :, 1:-1, 1:-1],
                               np.broadcast_to(w.sum(axis=(1, 2, 3))[:, None, None],
                                               (Co, H - 2, W - 2)), rtol=1e-13)
    # top-left corner: taps kh=0 and kw=0 fall in the padding
    np.testing.assert_allclose(y[0, :, 0, 0], w[:, :, 1:, 1:].sum(axis=(1, 2, 3)), rtol=1e-13)
    # top edge, interior column: row kh=0 is padding
    np.testing.assert_allclose(y[0, :, 0, 4], w[:, :, 1:, :].sum(axis=(1, 2, 3)), rtol=1e-13)
    # bottom-right corner: kh=2 and kw=2 fall in the padding
    np.testing.assert_allclose(y[0, :, -1, -1], w[:, :, :2, :2].sum(axis=(1, 2, 3)), rtol=1e-13)


def test_1x1_is_gemm(orc):
    rng = np.random.default_rng(6)
    N, C, H, W, Co = 3, 7, 5, 6, 4
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, 1, 1))
    y = orc.conv2d(x, w, 1, 0)
    for n in range(N):
        np.testing.assert_allclose(y[n].reshape(Co, -1), w[:, :, 0, 0] @ x[n].reshape(C, -1),
                                   rtol=1e-12, atol=1e-13)


def test_dense_as_conv_is_gemv(orc):
    rng = np.random.default_rng(7)
    N, C, H, W, Co = 2, 3, 5, 4, 6
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, H, W))
    y = orc.conv2d(x, w, 1, 0)
    assert y.shape == (N, Co, 1, 1)
    for n in range(N):
        np.testing.assert_allclose(y[n, :, 0, 0], w.reshape(Co, -1) @ x[n].reshape(-1),
                                   rtol=1e-12, atol=1e-13)


def test_linearity(orc):
    rng = np.random.default_rng(8)
    x1 = rng.standard_normal((2, 3, 7, 8))
    x2 = rng.standard_normal((2, 3, 7, 8))
    w = rng.standard_normal((4, 3, 3, 2))
    a, b = 0.75, -2.5
    np.testing.assert_allclose(orc.conv2d(a * x1 + b * x2, w, 2, 1),
                               a * orc.conv2d(x1, w, 2, 1) + b * orc.conv2d(x2, w, 2, 1),
                               rtol=1e-12, atol=1e-12)


def test_winograd_section_worked_example(orc):
    g = _read_golden_kv("page_examples.txt")
    d = np.array(g["p5_f23_d"], np.float64)
    f = np.array(g["p5_f23_g"], np.float64)
    y = orc.conv2d(d.reshape(1, 1, 1, 4), f.reshape(1, 1, 1, 3), 1, 0)
    assert y.reshape(-1).tolist() == [float(v) for v in g["p5_f23_direct"]]
    # the same two outputs by F(2,3) minimal filtering with the page's transform matrices
    G = np.array([[1, 0, 0], [0.5, 0.5, 0.5], [0.5, -0.5, 0.5], [0, 0, 1]])
    Bt = np.array([[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]])
    At = np.array([[1, 1, 1, 0], [0, 1, -1, -1]])
    np.testing.assert_allclose(y.reshape(-1), At @ ((Bt @ d) * (G @ f)), atol=1e-15)


def test_points_match_full(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 5, 9, 7))
    w = rng.standard_normal((6, 5, 3, 2))
    y = orc.conv2d(x, w, 2, 1)
    idx = rng.integers(0, y.size, 300)
    assert np.array_equal(orc.conv2d_points(x, w, 2, 1, idx), y.reshape(-1)[idx])
    with pytest.raises(ValueError):
        orc.conv2d_points(x, w, 2, 1, np.array([y.size]))


def test_half_precision_inputs_widen_exactly(orc):
    """The oracle reads fp16/bf16 bits exactly (conversion to float64 is exact)."""
    import workloads
    x, w = workloads.make_inputs(1, 4, 6, 6, 3, 3, 3, seed=3, dtype="bf16")
    y = orc.conv2d(x, w, 1, 1)
    ref = _torch_conv(x.double().numpy(), w.double().numpy(), 1, 1)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- layer epilogue and NHWC

def _epi_case(seed, N=2, Cin=5, H=9, W=8, Cout=6, KH=3, KW=2, s=2, p=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin, KH, KW))
    b = rng.standard_normal(Cout)
    sc = rng.uniform(0.25, 4.0, Cout) * rng.choice([-1.0, 1.0], Cout)
    return x, w, b, sc, s, p


@pytest.mark.parametrize("seed", range(6))
def test_bias_matches_library_conv(seed):
    """The bias of the convolution call of "Unifying Convolutions and GEMM"
    (Sec. 5): a library convolution with its bias argument, in float64."""
    x, w, b, _, s, p = _epi_case(seed)
    got = oracle.conv2d_ex(x, w, s, p, bias=b)
    want = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b), stride=s, padding=p).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_scale_folding_identity(seed):
    """The scale folding of "Fast and Memory-Efficient Wavelet Convolutions via
    I/O-Aware Reformulation": s * (X * W + b) equals X * (s W) + s b, the
    convolution with the scale folded into the filter and the bias."""
    x, w, b, sc, s, p = _epi_case(seed)
    got = oracle.conv2d_ex(x, w, s, p, bias=b, scale=sc)
    folded = oracle.conv2d(x, w * sc[:, None, None, None], s, p) + (sc * b)[None, :, None, None]
    np.testing.assert_allclose(got, folded, rtol=1e-12, atol=1e-12)
    # the other reading (scale the sum, then add the unscaled bias) is a
    # different operator and must not pass
    wrong = oracle.conv2d(x, w, s, p) * sc[None, :, None, None] + b[None, :, None, None]
    assert np.max(np.abs(wrong - got)) > 1e-3


def test_epilogue_exact_on_integers():
    """Integer inputs and bias, power-of-two scales: every step is exact."""
    rng = np.random.default_rng(9)
    x = rng.integers(-3, 4, (2, 4, 7, 6)).astype(np.float64)
    w = rng.integers(-3, 4, (5, 4, 3, 3)).astype(np.float64)
    b = rng.integers(-9, 10, 5).astype(np.float64)
    sc = np.array([0.5, 2.0, -1.0, 4.0, 0.25])
    got = oracle.conv2d_ex(x, w, 1, 1, bias=b, scale=sc)
    want = (F.conv2d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b), padding=1).numpy()
            * sc[None, :, None, None])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_nhwc_layout_matches_library_conv(seed):
    """x [N][H][W][Cin], w [Cout][KH][KW][Cin], y [N][Ho][Wo][Cout]: a library
    convolution on the channels-first views, and the NCHW oracle transposed
    (the same sum, so bit-equal)."""
    x, w, b, sc, s, p = _epi_case(seed + 20)
    xh = np.ascontiguousarray(x.transpose(0, 2, 3, 1))
    wh = np.ascontiguousarray(w.transpose(0, 2, 3, 1))
    got = oracle.conv2d_ex(xh, wh, s, p, bias=b, scale=sc, layout="nhwc")
    lib = F.conv2d(torch.from_numpy(xh).permute(0, 3, 1, 2), torch.from_numpy(wh).permute(0, 3, 1, 2),
                   torch.from_numpy(b), stride=s, padding=p).permute(0, 2, 3, 1).numpy() * sc
    np.testing.assert_allclose(got, lib, rtol=1e-12, atol=1e-12)
    assert np.array_equal(got, oracle.conv2d_ex(x, w, s, p, bias=b, scale=sc).transpose(0, 2, 3, 1))


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_points_ex_index_the_whole_output(layout):
    x, w, b, sc, s, p = _epi_case(31)
    if layout == "nhwc":
        x = np.ascontiguousarray(x.transpose(0, 2, 3, 1))
        w = np.ascontiguousarray(w.transpose(0, 2, 3, 1))
    full = oracle.conv2d_ex(x, w, s, p, bias=b, scale=sc, layout=layout).reshape(-1)
    idx = np.array([0, 1, 7, full.size // 2, full.size - 2, full.size - 1], np.int64)
    got = oracle.conv2d_points_ex(x, w, s, p, idx, bias=b, scale=sc, layout=layout)
    np.testing.assert_allclose(got, full[idx], rtol=1e-13, atol=1e-13)
