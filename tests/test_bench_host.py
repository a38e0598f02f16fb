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
    d, p = _plan("mix512", "f16")
    assert bench.recorded_traffic("mix512", "f16", d, p) is None


def test_bench_functions_reference_only_defined_names():
    """Every free name a function of bench.py reads is a module-level name or a
    builtin (catches a variable used outside the function that defines it,
    which only a GPU run would otherwise reach)."""
    import builtins
    import os
    import symtable
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py")
    top = symtable.symtable(open(path).read(), path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    bad = []

    def walk(t):
        for ch in t.get_children():
            if ch.get_type() == "function":
                for s in ch.get_symbols():
                    if (s.is_global() and s.is_referenced() and s.get_name() not in module_names
                            and not hasattr(builtins, s.get_name())):
                        bad.append((ch.get_name(), s.get_name()))
            walk(ch)
    walk(top)
    assert not bad, bad
