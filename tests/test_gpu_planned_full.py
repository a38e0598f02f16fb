"""Every measured layer at its full size through conv2d_fwd exactly as planned
(the form, kernel and launch configuration the benchmark times), against the
oracle on sampled outputs: random outputs plus every border row and column,
the first and last images, the first and last output channels, and the
outputs on both sides of every boundary between the plan's row blocks,
column tiles, channel blocks and window-row chunks. Each compared output is
held to the per-output error bound and the set to the relative L2 tolerance
(tests/parity.py).

The five layer configurations of the benchmark, and the twelve layers of
Table I of "Enabling Memory-efficient Im2win Convolution with Multi-precision
Support on GPU CUDA and Tensor Cores" (Sec. IV-B) at the batch the paper
measures them with (N = 256, no padding), in fp16 and fp32."""
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
    _lib.lib()   # the HIP library must load: no fallback


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _edges(extent, step, cap=24):
    """0, 1, the middle, the last two, and both sides of each multiple of step."""
    out = {0, 1, extent // 2, extent - 2, extent - 1}
    if step and 0 < step < extent:
        ks = list(range(step, extent, step))
        if len(ks) > cap:                      # keep the first, last and an even spread
            pick = np.linspace(0, len(ks) - 1, cap).round().astype(int)
            ks = [ks[i] for i in sorted(set(pick.tolist()))]
        for k in ks:
            out.update({k - 1, k})
    return sorted(v for v in out if 0 <= v < extent)


def sample_indices(N, Cout, Ho, Wo, rng, *, row_step=0, col_step=0, co_step=64, flat_row_step=0,
                   count=3000):
    """Flat indices into y [N][Cout][Ho][Wo]: random outputs and the edges of
    every block the plan cuts the layer into."""
    idx = set(rng.integers(0, N * Cout * Ho * Wo, count).tolist())
    ns = sorted({0, 1, N // 2, N - 1} & set(range(N)))
    hos = _edges(Ho, row_step)
    wos = _edges(Wo, col_step)
    cos = sorted(set(_edges(Cout, co_step, cap=8)) | set(rng.integers(0, Cout, 3).tolist()))
    for n in ns:
        for ho in hos:
            for co in cos:
                for wo in wos:
                    idx.add(((n * Cout + co) * Ho + ho) * Wo + wo)
    if flat_row_step:                           # window-row chunks: rows r = n*Ho + ho
        for r in _edges(N * Ho, flat_row_step, cap=16):
            n, ho = divmod(r, Ho)
            for co in cos:
                for wo in wos:
                    idx.add(((n * Cout + co) * Ho + ho) * Wo + wo)
    return np.array(sorted(idx), dtype=np.int64)


def _planned_blocks(d):
    """The block edges of the planned form: (row_step, col_step, flat_row_step)."""
    pl = conv.plan(d)
    if pl.algo == 0:
        return pl, None, (0, 0, pl.rows_per_chunk)
    ip = conv.implicit_plan(d)
    if ip.kernel == 4 and ip.images > 1:       # tasks of whole images: image edges are covered
        return pl, ip, (0, 0, 0)
    return pl, ip, (ip.rows_per_tile, ip.cols_per_tile if ip.kernel == 0 else 0, 0)


def _run_planned_sampled(cfg, dt):
    x, w = workloads.make_config_inputs(cfg, dt)
    d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad, CODE[dt])
    pl, ip, (rs, cs, fs) = _planned_blocks(d)
    form = "window" if pl.algo == 0 else f"implicit kernel {ip.kernel}"
    _say(f"planned full-size {cfg.name} {dt} {cfg.desc()} form={form} row_step={rs} col_step={cs} "
         f"chunk_rows={fs}")
    assert pl.meets_ws_target == 1
    ho, wo = cfg.out_hw()
    y = conv.conv2d(x.to(DEV), w.to(DEV), stride=cfg.stride, pad=cfg.pad)
    assert tuple(y.shape) == (cfg.N, cfg.Cout, ho, wo)
    rng = np.random.default_rng(cfg.seed + 7)
    idx = sample_indices(cfg.N, cfg.Cout, ho, wo, rng, row_step=rs, col_step=cs, flat_row_step=fs)
    got = y.reshape(-1)[torch.from_numpy(idx).to(DEV)].cpu()
    torch.cuda.synchronize()
    del y
    rel, ratio = check(got, x, w, cfg.stride, cfg.pad, dt, idx=idx, what=f"{cfg.name} {dt}")
    _say(f"  {idx.size} outputs: rel L2 {rel:.3e}, worst error / bound {ratio:.3f}")
    return pl, ip


CONFIG_CASES = [(name, dt) for name, cfg in sorted(workloads.CONFIGS.items()) for dt in cfg.dtypes]


@pytest.mark.parametrize("name,dt", CONFIG_CASES, ids=[f"{n}-{d}" for n, d in CONFIG_CASES])
def test_measured_layers_planned_full_size(name, dt):
    pl, ip = _run_planned_sampled(workloads.get_config(name), dt)
    if name == "stem7x7":                       # the RGB stem runs on the narrow-channel kernel
        assert pl.algo == 1 and ip.kernel == 3


TABLE1_CASES = [(name, dt) for name in workloads.TABLE1 for dt in ("f16", "f32")]


@pytest.mark.parametrize("name,dt", TABLE1_CASES, ids=[f"{n}-{d}" for n, d in TABLE1_CASES])
def test_table1_layers_planned_full_batch(name, dt):
    _run_planned_sampled(workloads.TABLE1[name], dt)
    torch.cuda.empty_cache()


def test_sampler_covers_block_edges():
    """Host check of the sampler itself: both sides of every row-block edge."""
    idx = sample_indices(2, 70, 20, 9, np.random.default_rng(0), row_step=6, count=0)
    ho = (idx // 9) % 20
    assert {0, 1, 5, 6, 11, 12, 17, 18, 19} <= set(ho.tolist())
    co = (idx // (9 * 20)) % 70
    assert {0, 63, 64, 69} <= set(co.tolist())
