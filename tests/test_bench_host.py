"""bench.py host-side logic (no GPU): the --gpus contract and the traffic record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import cnn_convolution_amd as conv  # noqa: E402
import workloads  # noqa: E402


CODES = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}


def _plan(name, dt, ydt="f32"):
    cfg = workloads.get_config(name)
    d = conv.describe(cfg.x_shape, cfg.w_shape, cfg.stride, cfg.pad, CODES[dt], CODES[ydt])
    return d, conv.plan(d)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and line["value"] is None and "one GPU" in line["error"]


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_traffic_records_are_consistent(dt):
    """The committed counter summary holds one well-formed record whose measured bytes are
    close to the algorithmic bytes of the same launch (whether or not it still applies to
    the current kernel: that is what the sha, tile and rows keys decide)."""
    path = os.path.join(ROOT, "profiles", f"resnet3x3_{dt}_gemm_counters.md")
    with open(path) as f:
        recs = [dict(kv.split("=", 1) for kv in line.split()[1:])
                for line in f if line.startswith("traffic-record:")]
    assert len(recs) == 1
    rec = recs[0]
    assert set(rec) >= {"kernel", "sha", "tile", "rows", "bytes_per_launch", "alg_bytes"}
    ratio = float(rec["bytes_per_launch"]) / float(rec["alg_bytes"])
    assert 0.9 < ratio < 1.5


def test_traffic_is_null_once_the_kernel_changes(monkeypatch):
    d, p = _plan("resnet3x3", "f16")
    monkeypatch.setattr(bench, "gemm_source_sha", lambda kernel: "0" * 16)
    assert bench.recorded_traffic("resnet3x3", "f16", d, p) is None


def test_traffic_is_null_for_another_form_or_tile(monkeypatch):
    d, p = _plan("resnet3x3", "f16")
    base = bench.dominant_key(d, p)
    monkeypatch.setenv("IM2WIN_ALGO", "window" if p.algo == 1 else "implicit")
    d2, q = _plan("resnet3x3", "f16")
    assert bench.dominant_key(d2, q) != base
    if bench.recorded_traffic("resnet3x3", "f16", d, p) is not None:
        assert bench.recorded_traffic("resnet3x3", "f16", d2, q) is None
    monkeypatch.delenv("IM2WIN_ALGO")
    monkeypatch.setenv("IM2WIN_IMPLICIT_TILE", "64,64,1,1,56")
    monkeypatch.setenv("IM2WIN_MFMA_DMA_TILE", "128,128,1")
    d3, r = _plan("resnet3x3", "f16")
    assert bench.dominant_key(d3, r) != base
    assert bench.recorded_traffic("resnet3x3", "f16", d3, r) is None


def test_dominant_kernel_follows_the_plan(monkeypatch):
    d, p = _plan("resnet3x3", "f16")
    kid, tile, rows = bench.dominant_key(d, p)
    if p.algo == 1:
        assert kid in (4, 5, 6, 7, 8) and rows == p.rows_total and tile.startswith("i")
    monkeypatch.setenv("IM2WIN_ALGO", "window")
    d, p = _plan("resnet3x3", "f16")
    kid, tile, rows = bench.dominant_key(d, p)
    assert p.algo == 0 and kid == p.gemm_kernel
    assert rows == p.rows_total - (p.n_chunks - 1) * p.rows_per_chunk


def test_traffic_is_null_without_a_summary():
    # no counter summary is committed for the 512-channel layer in bf16
    d, p = _plan("mix512", "bf16")
    assert not os.path.exists(os.path.join(bench.ROOT, "profiles", "mix512_bf16_gemm_counters.md"))
    assert bench.recorded_traffic("mix512", "bf16", d, p) is None


def test_every_measured_layer_has_a_traffic_record():
    """Each layer of the default bench line, in its measured input/output
    types, has a committed counter summary with one well-formed record for its
    planned tile and launch size (whether the record still applies to the
    current kernel sources is what its sha key decides at run time)."""
    for name, dt, ydt in [("resnet3x3", "f16", "f32"), ("resnet3x3", "f32", "f32"), ("deep3x3", "bf16", "f32"),
                          ("stem7x7", "f16", "f32"), ("stem7x7", "f32", "f32"), ("mix5x5", "f16", "f32"),
                          ("mix512", "f16", "f32"), ("mix3x3s2", "f16", "f32"), ("mix1x1", "f16", "f32"),
                          ("resnet3x3", "f16", "f16"), ("stem7x7", "f16", "f16"), ("mix1x1", "f16", "f16")]:
        d, p = _plan(name, dt, ydt)
        ysuf = "" if ydt == "f32" else f"_y{ydt}"
        path = os.path.join(ROOT, "profiles", f"{name}_{dt}{ysuf}_gemm_counters.md")
        with open(path) as f:
            recs = [dict(kv.split("=", 1) for kv in line.split()[1:])
                    for line in f if line.startswith("traffic-record:")]
        assert len(recs) == 1, path
        kid, tile, rows = bench.dominant_key(d, p)
        assert recs[0]["kernel"] == bench.GEMM_KERNEL_NAMES[kid] and recs[0]["tile"] == tile, path
        assert recs[0]["rows"] == str(rows), path
        assert 0.9 < float(recs[0]["bytes_per_launch"]) / float(recs[0]["alg_bytes"]) < 6.0, path
