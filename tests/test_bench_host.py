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


def _plan(name, dt):
    cfg = workloads.get_config(name)
    code = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}[dt]
    d = conv.describe(cfg.x_shape, cfg.w_shape, cfg.stride, cfg.pad, code)
    p = conv.plan(d)
    return p, p.rows_total - (p.n_chunks - 1) * p.rows_per_chunk


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and line["value"] is None and "one GPU" in line["error"]


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_traffic_record_matches_the_current_kernel(dt):
    """The committed counter summary applies to the GEMM that runs now."""
    p, rows = _plan("resnet3x3", dt)
    t = bench.recorded_traffic("resnet3x3", dt, p, rows)
    assert t is not None and t > 0


def test_traffic_is_null_once_the_kernel_changes(monkeypatch):
    p, rows = _plan("resnet3x3", "f16")
    monkeypatch.setattr(bench, "gemm_source_sha", lambda kind: "0" * 16)
    assert bench.recorded_traffic("resnet3x3", "f16", p, rows) is None


def test_traffic_is_null_for_another_launch_size_or_tile(monkeypatch):
    p, rows = _plan("resnet3x3", "f16")
    assert bench.recorded_traffic("resnet3x3", "f16", p, rows - 1) is None
    monkeypatch.setenv("IM2WIN_MFMA_TILE", "64,64,32,1,2")
    q, rows_q = _plan("resnet3x3", "f16")
    assert bench.recorded_traffic("resnet3x3", "f16", q, rows_q) is None


def test_traffic_is_null_without_a_summary():
    p, rows = _plan("mix512", "f16")
    assert bench.recorded_traffic("mix512", "f16", p, rows) is None
