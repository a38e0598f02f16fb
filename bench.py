#!/usr/bin/env python3
"""Forward-convolution benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 20]
    python bench.py --config NAME [--dtype DT]     # one layer, its own line

A step is one conv2d_fwd call in the form the library plans for the layer:
either the window tensor (filter staging, then for every chunk of window rows
the im2win pack and the window-GEMM) or the implicit form (one kernel that
builds the window rows in LDS and contracts them, after a small filter
staging launch where the plan keeps a staged filter), each writing the fp32
output. Inputs are seeded synthetic tensors already resident in device
memory. The timed region is `steps` back-to-back calls on one stream,
bracketed by device syncs and HIP events; warm-up calls run first and caches
stay warm (50 timed calls after 20 warm-up ones, the protocol of the
fused-WTConv measurements). The warm-up also lasts at least 50 ms of
back-to-back calls per layer: from idle the GPU's clocks take 15-20 ms of
continuous work to ramp up (measured), and a layer timed before that reads
up to 20 % slow. Each layer reports the warm-up calls it made.

The default run prints ONE JSON line. Its headline is the ResNet-style 3x3
layer in fp16 (TFLOPS = 2 * multiply-adds / time, padded taps included, and
the fraction of the MI355X peak); "layers" holds every layer configuration
and dtype (tiny, resnet3x3 f32/f16, deep3x3 bf16, stem7x7 f32/f16, mix5x5,
mix512, mix3x3s2, mix1x1 f16), each with the roofline of its dominant kernel
(back-to-back launches of that kernel alone between HIP events), the HBM
traffic from committed counter summaries, workspace bytes against the im2col
buffer, and a parity check of its timed output against the CPU oracle on
sampled points. The CPU-baseline leg -- the only part that uses the oracle,
run after all GPU timing -- times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv2d fwd TFLOPS and % of MFMA/fp32 peak per layer on 1 MI355X"
# the untimed warmup of every layer: at least --warmup calls and at least this
# many seconds of back-to-back calls (the clocks' ramp from idle)
WARMUP_MIN_S = 0.05
# MI355X published peaks
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}   # dense MFMA / vector fp32
HBM_GBPS = 8000.0
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


# sources that decide what the dominant kernel of a call does, per kernel id
# (0: fp32 vector-ALU window-GEMM, 1: tiled matrix-core window-GEMM,
# 3: direct-to-LDS matrix-core window-GEMM, 4: implicit convolution, window
# rows built in LDS, filter streamed, 6: the row-block implicit kernel, filter
# and input rows resident in LDS, 7: the narrow-channel implicit kernel, 8: the
# pipelined row-block kernel, 32-channel K chunks double-buffered by loader
# waves, 9: the split-K row-block kernel, input channels split over the waves)
GEMM_SOURCES = {
    0: ["cnn_convolution_amd/csrc/kernels/gemm_valu.hip",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    1: ["cnn_convolution_amd/csrc/kernels/gemm_mfma.hip",
        "cnn_convolution_amd/csrc/kernels/tile_map.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    3: ["cnn_convolution_amd/csrc/kernels/gemm_mfma_dma.hip",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/tile_map.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    4: ["cnn_convolution_amd/csrc/kernels/conv_implicit.hip",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/tile_map.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    6: ["cnn_convolution_amd/csrc/kernels/conv_implicit_rows.hip",
        "cnn_convolution_amd/csrc/kernels/out_blocks.hpp",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/tile_map.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    7: ["cnn_convolution_amd/csrc/kernels/conv_implicit_narrow.hip",
        "cnn_convolution_amd/csrc/kernels/out_blocks.hpp",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/tile_map.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    8: ["cnn_convolution_amd/csrc/kernels/conv_implicit_pipe.hip",
        "cnn_convolution_amd/csrc/kernels/pipe_patch.hpp",
        "cnn_convolution_amd/csrc/kernels/out_blocks.hpp",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
    9: ["cnn_convolution_amd/csrc/kernels/conv_implicit_ksplit.hip",
        "cnn_convolution_amd/csrc/kernels/pipe_patch.hpp",
        "cnn_convolution_amd/csrc/kernels/lds_dma.hpp",
        "cnn_convolution_amd/csrc/kernels/epilogue.hpp"],
}
GEMM_KERNEL_NAMES = {0: "gemm_valu_f32", 1: "gemm_mfma",
                     3: "gemm_mfma_dma", 4: "conv_implicit",
                     6: "conv_implicit_rows", 7: "conv_implicit_narrow", 8: "conv_implicit_pipe",
                     9: "conv_implicit_ksplit"}
COPY_BYTES = 256 << 20     # calibration copy for the HBM byte counters


def gemm_source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES[kernel] + ["cnn_convolution_amd/csrc/launch.hpp"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dominant_key(d, plan):
    """(kernel id, tile key, rows per launch) of the dominant kernel of a call:
    the implicit kernel (all N*Ho window rows in one launch) or the window-GEMM
    (timed on the last chunk of window rows)."""
    import cnn_convolution_amd as conv
    if plan.algo == 1:
        ip = conv.implicit_plan(d)
        kid = {0: 4, 2: 6, 3: 7, 4: 8, 5: 9}[ip.kernel]
        # the pipelined row-block kernel: stages 2 = persistent, 1 = paired form
        form = f"/s{ip.stages}" if ip.kernel == 4 else ""
        return (kid, f"i{ip.kernel}:{ip.tile_m}x{ip.tile_n}/{ip.wave_m}/r{ip.rows_per_tile}/"
                f"c{ip.cols_per_tile}/g{ip.tiles}{form}", plan.rows_total)
    rows = plan.rows_total - (plan.n_chunks - 1) * plan.rows_per_chunk
    return (plan.gemm_kernel, f"k{plan.gemm_kernel}:{plan.gemm_tile_m}x{plan.gemm_tile_n}/"
            f"{plan.gemm_kslice}/{plan.gemm_ksplit}/{plan.gemm_wave_m}", rows)


def recorded_traffic(name, dt, d, plan, ydt="f32"):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/<layer>_<dtype>[_y<output type>]_gemm_counters.md), or
    None when there is none or the kernel sources, tile or launch size differ
    from what the counters measured."""
    ysuf = "" if ydt == "f32" else f"_y{ydt}"
    path = os.path.join(ROOT, "profiles", f"{name}_{dt}{ysuf}_gemm_counters.md")
    if not os.path.exists(path):
        return None
    kid, tile, rows = dominant_key(d, plan)
    want = {"kernel": GEMM_KERNEL_NAMES[kid], "sha": gemm_source_sha(kid), "tile": tile,
            "rows": str(rows)}
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                rec = dict(kv.split("=", 1) for kv in line.split()[1:])
                if all(rec.get(k) == v for k, v in want.items()):
                    return float(rec["bytes_per_launch"])
    return None


def algorithmic_bytes(cfg, dt, plan, ydt="f32"):
    """Per-kernel algorithmic HBM bytes of one call (each tensor moved once).

    pack     : reads x, writes the window tensor (N*Ho rows of Cin*W_win*KH)
    gemm     : reads the window tensor and the staged filter, writes y (fp32)
    stage    : reads w, writes the staged filter
    implicit : reads x and the staged filter, writes y (no window tensor)
    """
    es = 4 if dt == "f32" else 2
    ho, wo = plan.Ho, plan.Wo
    x = cfg.N * cfg.Cin * cfg.H * cfg.W * es
    w = cfg.Cout * cfg.Cin * cfg.KH * cfg.KW * es
    win = cfg.N * ho * cfg.Cin * plan.W_win * cfg.KH * es
    y = cfg.N * cfg.Cout * ho * wo * (4 if ydt == "f32" else 2)
    # a staging launch runs only where the plan keeps a staged filter (the
    # window form's, or the implicit form's workspace)
    staged = plan.wstage_bytes > 0 if plan.algo == 0 else plan.ws_bytes > 0
    return {"pack": x + win, "gemm": win + w * plan.n_chunks + y,
            "weight_stage": 2 * w if staged else 0,
            "implicit": x + w + y}


_INPUTS = {}


def layer_inputs(cfg, dt):
    """Seeded inputs of a layer in dtype dt. The half-precision tensors are the
    float32 draws rounded once to nearest-even, so one draw serves every dtype
    (the same bits the generator gives for each dtype on its own)."""
    import torch

    import workloads
    if cfg.name not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[cfg.name] = workloads.make_config_inputs(cfg, "f32")
    x32, w32 = _INPUTS[cfg.name]
    if dt == "f32":
        return x32, w32
    t = workloads.TORCH_DTYPES[dt]
    return x32.to(t).contiguous(), w32.to(t).contiguous()


def time_variant(cfg, dt, steps, warmup, dev, algo=None, ydt="f32"):
    """Time conv2d_fwd on one layer and dtype, in the form the planner picks
    (or the one `algo` forces: "window" or "implicit"), and its dominant kernel
    alone; check the timed output against the oracle on sampled points."""
    import torch

    import cnn_convolution_amd as conv

    saved = os.environ.get("IM2WIN_ALGO")
    if algo:
        os.environ["IM2WIN_ALGO"] = algo
    else:
        os.environ.pop("IM2WIN_ALGO", None)
    try:
        return _time_variant(cfg, dt, steps, warmup, dev, ydt)
    finally:
        if saved is None:
            os.environ.pop("IM2WIN_ALGO", None)
        else:
            os.environ["IM2WIN_ALGO"] = saved


def _time_variant(cfg, dt, steps, warmup, dev, ydt="f32"):
    import torch

    import cnn_convolution_amd as conv
    import workloads
    from cnn_convolution_amd import _lib

    x, w = layer_inputs(cfg, dt)
    xd, wd = x.to(dev), w.to(dev)
    codes = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}
    d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad, codes[dt], codes[ydt])
    plan = conv.plan(d)
    y = torch.empty((cfg.N, cfg.Cout, plan.Ho, plan.Wo), dtype=workloads.TORCH_DTYPES[ydt], device=dev)
    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
    wsarg = ws if plan.ws_bytes else None

    # untimed warmup: at least `warmup` calls and at least WARMUP_MIN_S of
    # back-to-back calls, so that the GPU's clocks have ramped up from idle
    # (measured: 15-20 ms of continuous work before calls reach their
    # steady time; the layer's input set-up on the host idles the GPU)
    n_warm = 0
    tw = time.perf_counter()
    while n_warm < warmup or time.perf_counter() - tw < WARMUP_MIN_S:
        for _ in range(max(1, min(warmup, 20))):
            conv.conv2d_into(xd, wd, y, wsarg, cfg.stride, cfg.pad)
        n_warm += max(1, min(warmup, 20))
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        conv.conv2d_into(xd, wd, y, wsarg, cfg.stride, cfg.pad)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps

    # each call on its own between two events: median and best call
    per_call = []
    for _ in range(steps):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        conv.conv2d_into(xd, wd, y, wsarg, cfg.stride, cfg.pad)
        c1.record()
        per_call.append((c0, c1))
    torch.cuda.synchronize()
    call_ms = sorted(a.elapsed_time(b) for a, b in per_call)

    # second timed pass: HIP events around every kernel launch (same stream);
    # the event pairs add a few microseconds to each short kernel, so this pass
    # gives the split between kernels, not the roofline figure
    conv.profile_read()
    conv.profile_enable(True)
    try:
        for _ in range(steps):
            conv.conv2d_into(xd, wd, y, wsarg, cfg.stride, cfg.pad)
    finally:
        conv.profile_enable(False)
    prof = conv.profile_read()

    # dominant kernel alone, back to back between two events on the same
    # stream: after a call the workspace holds the staged filter (and, for the
    # window form, the last chunk of window rows)
    es = 4 if dt == "f32" else 2
    kid, tile, rows = dominant_key(d, plan)
    sptr = torch.cuda.current_stream().cuda_stream
    pack_us = None
    if plan.algo == 1:
        ip = conv.implicit_plan(d)
        wst = ws if ip.ws_bytes else wd
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps):
            conv.implicit_gemm(xd, wst, y, d)
        g1.record()
        torch.cuda.synchronize()
        kern_us = g0.elapsed_time(g1) / steps * 1e3
        dom_flops = plan.flops
        dom_bytes = algorithmic_bytes(cfg, dt, plan, ydt)["implicit"]
        n_chunks = 1
    else:
        row0 = (plan.n_chunks - 1) * plan.rows_per_chunk
        # the back-to-back launches below read (GEMM) and rewrite (pack) the
        # window chunk inside ws: check on the host that it is all there
        if plan.ws_bytes < plan.win_offset_bytes + rows * plan.row_elems * es:
            raise RuntimeError(f"{cfg.name} {dt}: workspace holds no whole window chunk")
        win = ws[plan.win_offset_bytes:plan.win_offset_bytes + rows * plan.row_elems * es]
        wst = ws if plan.wstage_bytes else wd
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps):
            conv.window_gemm(win, wst, y, d, row0, rows)
        g1.record()
        torch.cuda.synchronize()
        kern_us = g0.elapsed_time(g1) / steps * 1e3
        # the pack of the same chunk, back to back as well (rewrites the same rows)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for _ in range(steps):
            _lib.pack(d, plan.layout, xd.data_ptr(), win.data_ptr(), row0, rows, sptr)
        p1.record()
        torch.cuda.synchronize()
        pack_us = p0.elapsed_time(p1) / steps * 1e3
        dom_flops = 2 * rows * plan.Wo * cfg.Cout * cfg.Cin * cfg.KH * cfg.KW
        dom_bytes = (rows * cfg.Cin * plan.W_win * cfg.KH * es
                     + cfg.Cout * cfg.Cin * cfg.KH * cfg.KW * es
                     + rows * plan.Wo * cfg.Cout * (4 if ydt == "f32" else 2))
        n_chunks = plan.n_chunks
    conv.conv2d_into(xd, wd, y, wsarg, cfg.stride, cfg.pad)   # y whole again for the parity check
    torch.cuda.synchronize()

    # the sampled outputs of the timed call, for the parity check that the
    # CPU-baseline leg runs (the only place the oracle is used)
    rng = np.random.default_rng(cfg.seed)
    idx = sample_points(cfg, plan, rng)
    got = y.reshape(-1)[torch.from_numpy(idx).to(dev)].double().cpu().numpy()

    flops = plan.flops
    tflops = flops / (ms * 1e-3) / 1e12
    ab = algorithmic_bytes(cfg, dt, plan, ydt)
    kern = {}
    for k in ("weight_stage", "pack", "gemm", "implicit"):
        n = prof[k]["launches"]
        if n:
            avg = prof[k]["total_ms"] / n
            kern[k] = {"launches_per_step": n / steps, "avg_launch_us": avg * 1e3,
                       "ms_per_step": prof[k]["total_ms"] / steps,
                       "alg_bytes_per_launch": ab[k] / (n / steps)}
    # roofline of the dominant kernel: algorithmic work of one launch (each
    # tensor moved once) over its back-to-back launch time
    kern_s = kern_us * 1e-6
    ai = dom_flops / dom_bytes
    peak = PEAK_TFLOPS[dt]
    ridge = peak * 1e12 / (HBM_GBPS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": dom_bytes / kern_s / 1e9, "peak": HBM_GBPS,
                "unit": "GB/s"}
    else:
        # fp32 runs on the matrix cores in the implicit form, on the vector ALUs otherwise
        roof = {"bound": "mfma" if (dt != "f32" or plan.algo == 1) else "alu",
                "achieved": dom_flops / kern_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch from FETCH_SIZE + WRITE_SIZE counters scaled by a copy
    # of known size (committed summary); null once the kernel has changed
    roof["traffic"] = recorded_traffic(cfg.name, dt, d, plan, ydt)
    roof["kernel"] = GEMM_KERNEL_NAMES[kid]
    roof["tile"] = tile
    roof["alg_bytes_per_launch"] = dom_bytes
    roof["flops_per_launch"] = dom_flops
    roof["avg_launch_us"] = kern_us
    roof["rows_per_launch"] = rows
    roof["tflops_in_kernel"] = dom_flops / kern_s / 1e12
    return {
        "dtype": dt, "form": "implicit" if plan.algo == 1 else "window",
        "value": tflops, "ms_per_step": ms, "wall_s": wall, "warmup_calls": n_warm,
        "ms_per_call_median": call_ms[len(call_ms) // 2], "ms_per_call_best": call_ms[0],
        "chunk_pack_us": pack_us, "chunk_gemm_us": kern_us if plan.algo == 0 else None,
        "kernel_us": kern_us, "chunk_rows": rows,
        "pct_of_peak": 100.0 * tflops / peak, "peak_tflops": peak,
        "sample_idx": idx, "sample_got": got, "y_dtype": ydt,
        "ws_bytes": plan.ws_bytes, "im2col_bytes": plan.im2col_bytes,
        "ws_over_im2col": plan.ws_bytes / plan.im2col_bytes, "ws_target": 1.0 / cfg.KW,
        "n_chunks": n_chunks, "kernels": kern, "roofline": roof,
    }


def sample_points(cfg, plan, rng, count=2000):
    """Flat output indices checked against the oracle: random outputs plus the
    first and last output of every (first/last image, first/last channel)
    plane's border rows."""
    ho, wo = plan.Ho, plan.Wo
    idx = set(rng.integers(0, cfg.N * cfg.Cout * ho * wo, count).tolist())
    for n in {0, cfg.N - 1}:
        for co in {0, cfg.Cout - 1}:
            for h in {0, ho - 1}:
                for c in {0, wo - 1}:
                    idx.add(((n * cfg.Cout + co) * ho + h) * wo + c)
    return np.array(sorted(idx), dtype=np.int64)


def host_cpu():
    """Threads the oracle runs with (OMP_NUM_THREADS, else every core this
    process may run on), the host's core count and CPU model."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or avail
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, {"host_nproc": os.cpu_count(), "host_affinity": avail, "cpu_model": model,
                     "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_leg(cfg, dt, res, min_seconds):
    """The CPU-baseline leg, the only part of the benchmark that uses the
    oracle (after every GPU timing is done):
    * the fp64 oracle's throughput on the host cores over a bounded sample of
      the layer (whole images of the same batch, repeated until about
      min_seconds), reported as a baseline only;
    * the parity of the timed call: its sampled outputs against the oracle
      point by point, relative L2 over the sample and the per-output bound
      |y - ref| <= 2 (K + 1) 2^-24 sum|x w| of any fp32 summation order.
    Returns (cpu_baseline, parity)."""
    import oracle
    threads, host = host_cpu()
    x, w = layer_inputs(cfg, dt)
    idx, got = res["sample_idx"], res["sample_got"]
    ref = oracle.conv2d_points(x, w, cfg.stride, cfg.pad, idx, nthreads=threads)
    mag = oracle.conv2d_points(x.abs(), w.abs(), cfg.stride, cfg.pad, idx, nthreads=threads)
    K = cfg.Cin * cfg.KH * cfg.KW
    u_out = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[res.get("y_dtype", "f32")]
    bound = 2.0 * (K + 1) * 2.0 ** -24 * mag + u_out * np.abs(ref)
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    ratio = float(np.max(err / np.where(bound > 0, bound, 1.0)))
    tol = max(TOL[dt], TOL[res.get("y_dtype", "f32")])
    parity = {"rel_l2_sampled": rel, "max_err_over_bound": ratio, "points": int(idx.size),
              "parity_ok": bool(rel <= tol and np.all(err <= bound))}
    ho, wo = cfg.out_hw()
    per_img = 2 * cfg.Cout * ho * wo * cfg.Cin * cfg.KH * cfg.KW
    # size the sample from a one-image probe
    t = time.perf_counter()
    oracle.conv2d(x[:1], w, cfg.stride, cfg.pad, nthreads=threads)
    probe = max(time.perf_counter() - t, 1e-4)
    imgs = int(max(1, min(cfg.N, min_seconds / probe)))
    reps = int(max(1, min(400, min_seconds / (probe * imgs))))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.conv2d(x[:imgs], w, cfg.stride, cfg.pad, nthreads=threads)
    el = time.perf_counter() - t
    base = {"value": per_img * imgs * reps / el / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "seconds": el,
            "sample": f"{imgs} of {cfg.N} images of the {cfg.name} layer, {reps} pass(es), "
                      f"fp64 direct sum, {dt} inputs", **host}
    return base, parity


def layer_entry(cfg, dt, r):
    """The per-layer record of the benchmark line."""
    ho, wo = cfg.out_hw()
    out = {"workload": f"{cfg.name}: N={cfg.N} Cin={cfg.Cin} H=W={cfg.H} Cout={cfg.Cout} "
                       f"{cfg.KH}x{cfg.KW} s{cfg.stride} p{cfg.pad}",
           "dtype": dt, "y_dtype": r.get("y_dtype", "f32"),
           "value": r["value"], "unit": "TFLOPS", "pct_of_peak": r["pct_of_peak"],
           "peak_tflops": r["peak_tflops"], "ms_per_step": r["ms_per_step"],
           "warmup_calls": r["warmup_calls"],
           "ms_per_call_median": r["ms_per_call_median"], "form": r["form"],
           "flops_per_call": 2 * cfg.N * cfg.Cout * ho * wo * cfg.Cin * cfg.KH * cfg.KW,
           "roofline": r["roofline"], "kernels": r["kernels"],
           "ws_bytes": r["ws_bytes"], "im2col_bytes": r["im2col_bytes"],
           "ws_over_im2col": r["ws_over_im2col"], "ws_target": r["ws_target"]}
    for k in ("rel_l2_sampled", "max_err_over_bound", "parity_ok", "cpu_oracle_tflops"):
        if k in r:
            out[k] = r[k]
    return out


def implicit_applies(cfg, dt):
    import cnn_convolution_amd as conv
    from cnn_convolution_amd import _lib
    d = conv.make_desc(cfg.N, cfg.Cin, cfg.H, cfg.W, cfg.Cout, cfg.KH, cfg.KW, cfg.stride,
                       cfg.pad, {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}[dt])
    return _lib.implicit_plan_status(d) == 0


def probe(args, dev):
    """Kernel launches for the counter passes, nothing else timed or printed on
    stdout: warm-up calls of the layer (at least WARMUP_MIN_S), then `steps`
    launches of its dominant kernel alone."""
    import torch

    import cnn_convolution_amd as conv
    import workloads
    if args.probe == "copy":
        a = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        _say(f"probe copy: {args.steps} copies of {COPY_BYTES} bytes")
        return
    cfg = workloads.get_config(args.config or HEADLINE[0])
    dt = args.dtype or next((d for d in cfg.dtypes if d != "f32"), cfg.dtypes[0])
    ydt = args.ydtype
    x, w = workloads.make_config_inputs(cfg, dt)
    xd, wd = x.to(dev), w.to(dev)
    codes = {"f32": conv.F32, "f16": conv.F16, "bf16": conv.BF16}
    d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad, codes[dt], codes[ydt])
    plan = conv.plan(d)
    y = torch.empty((cfg.N, cfg.Cout, plan.Ho, plan.Wo), dtype=workloads.TORCH_DTYPES[ydt], device=dev)
    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
    # warm-up calls as in the timed runs (the clocks' ramp from idle); a
    # profile of the probe keeps only the last `steps` launches of the kernel
    n_warm = 0
    tw = time.perf_counter()
    while time.perf_counter() - tw < WARMUP_MIN_S:
        for _ in range(10):
            conv.conv2d_into(xd, wd, y, ws if plan.ws_bytes else None, cfg.stride, cfg.pad)
        n_warm += 10
        torch.cuda.synchronize()
    kid, tile, rows = dominant_key(d, plan)
    if plan.algo == 1:
        ip = conv.implicit_plan(d)
        wst = ws if ip.ws_bytes else wd
        for _ in range(args.steps):
            conv.implicit_gemm(xd, wst, y, d)
    else:
        row0 = (plan.n_chunks - 1) * plan.rows_per_chunk
        es = 4 if dt == "f32" else 2
        if plan.ws_bytes < plan.win_offset_bytes + rows * plan.row_elems * es:
            raise RuntimeError(f"{cfg.name} {dt}: workspace holds no whole window chunk")
        win = ws[plan.win_offset_bytes:plan.win_offset_bytes + rows * plan.row_elems * es]
        wst = ws if plan.wstage_bytes else wd
        for _ in range(args.steps):
            conv.window_gemm(win, wst, y, d, row0, rows)
    torch.cuda.synchronize()
    _say(f"probe gemm: {cfg.name} {dt} rows={rows} tile={tile} "
         f"kernel={GEMM_KERNEL_NAMES[kid]} sha={gemm_source_sha(kid)} launches={args.steps} "
         f"after {n_warm} warm-up calls")


ABLATIONS = [("none", ""), ("serpentine", "serpentine"), ("dma", "dma"), ("buffers", "buffers"),
             ("all", "serpentine,dma,buffers")]
ABLATION_LAYERS = [("resnet3x3", "f16"), ("deep3x3", "bf16"), ("mix5x5", "f16"), ("mix512", "f16"),
                   ("mix3x3s2", "f16"), ("mix1x1", "f16"), ("cv9", "f16"), ("cv10", "f16"),
                   ("cv11", "f16"), ("cv12", "f16")]


def ablation(args, dev):
    """The page's optimisations turned off one at a time in the direct-to-LDS
    window-GEMM (IM2WIN_ABLATE): the window form is forced, the window rows of
    the last chunk are packed once, and the GEMM alone on them is timed with
    events over back-to-back launches for each variant, whose output is also
    checked against the planned kernel's. One JSON line per layer."""
    import torch

    import cnn_convolution_amd as conv
    import workloads
    os.environ["IM2WIN_ALGO"] = "window"
    for name, dt in ABLATION_LAYERS:
        cfg = workloads.get_config(name)
        x, w = layer_inputs(cfg, dt)
        xd, wd = x.to(dev), w.to(dev)
        d = conv.describe(tuple(x.shape), tuple(w.shape), cfg.stride, cfg.pad,
                          {"f16": conv.F16, "bf16": conv.BF16}[dt])
        plan = conv.plan(d)
        if plan.gemm_kernel != 3:
            _say(f"ablation: {name} {dt}: the window-GEMM is not the direct-to-LDS kernel, skipped")
            continue
        y = torch.zeros((cfg.N, cfg.Cout, plan.Ho, plan.Wo), dtype=torch.float32, device=dev)
        ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
        conv.conv2d_into(xd, wd, y, ws, cfg.stride, cfg.pad)
        row0 = (plan.n_chunks - 1) * plan.rows_per_chunk
        rows = plan.rows_total - row0
        win = ws[plan.win_offset_bytes:plan.win_offset_bytes + rows * plan.row_elems * 2]
        wst = ws if plan.wstage_bytes else wd
        flops = 2 * cfg.Cout * rows * plan.Wo * cfg.Cin * cfg.KH * cfg.KW
        ref = None
        out = {}
        for label, env in ABLATIONS:
            if env:
                os.environ["IM2WIN_ABLATE"] = env
            else:
                os.environ.pop("IM2WIN_ABLATE", None)
            assert conv.plan(d).gemm_ablate == sum(b for k, b in (("serpentine", 1), ("dma", 2), ("buffers", 4))
                                                   if k in env)
            y.zero_()
            for _ in range(args.warmup):
                conv.window_gemm(win, wst, y, d, row0, rows)
            torch.cuda.synchronize()
            got = y.clone()
            if ref is None:
                ref = got
            same = bool(torch.equal(got, ref))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                conv.window_gemm(win, wst, y, d, row0, rows)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / args.steps * 1e3
            out[label] = {"us": round(us, 2), "tflops": round(flops / us / 1e6, 1), "same_output": same}
            _say(f"ablation: {name} {dt} {label}: {us:.2f} us")
        os.environ.pop("IM2WIN_ABLATE", None)
        print(json.dumps({"workload": name, "dtype": dt, "kernel": "gemm_mfma_dma",
                          "tile": f"{plan.gemm_tile_m}x{plan.gemm_tile_n}/{plan.gemm_wave_m}",
                          "rows_per_launch": rows, "variants": out}), flush=True)
    os.environ.pop("IM2WIN_ALGO", None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None, help="one layer only (its own line)")
    ap.add_argument("--dtype", default=None, help="headline dtype (default: the layer's "
                    "half-precision variant if it has one)")
    ap.add_argument("--ydtype", default="f32", choices=["f32", "f16", "bf16"],
                    help="with --probe: the storage type of y")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="with --all-configs: time the oracle on every layer, not only the first")
    ap.add_argument("--single", action="store_true", help="time the headline dtype only")
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per layer and dtype (profiling / results table)")
    ap.add_argument("--table1", action="store_true",
                    help="one JSON line per layer of the im2win paper's Table I (N=256, "
                         "no padding), fp16 headline with the fp32 variant")
    ap.add_argument("--ablation", action="store_true",
                    help="the window-GEMM with each of the page's optimisations turned off, "
                         "one JSON line per layer (not the benchmark line)")
    ap.add_argument("--probe", choices=["gemm", "copy"], default=None,
                    help="for hardware counters: launch only the dominant kernel of the "
                         "layer (last chunk, --steps times) or a device copy of a known size")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"metric": METRIC, "value": None, "n_gpus": args.gpus,
                          "error": "this benchmark runs on one GPU only; a per-GPU share of a "
                                   "sharded layer is the same kernel at N/G images"}))
        _say("bench.py: only --gpus 1 is supported (one GPU per process, no collectives)")
        sys.exit(2)

    import torch
    import workloads
    import cnn_convolution_amd  # noqa: F401  (fails loudly without the HIP library)

    if not torch.cuda.is_available():
        _say("bench.py: no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.probe:
        probe(args, dev)
        return
    if args.ablation:
        ablation(args, dev)
        return
    if args.table1 or args.all_configs or args.config:
        per_layer_lines(args, dev)
        return
    default_line(args, dev)


DEFAULT_LAYERS = ("tiny", "resnet3x3", "deep3x3", "stem7x7", "mix5x5", "mix512", "mix3x3s2", "mix1x1")
HEADLINE = ("resnet3x3", "f16")
# the layers whose fp32 output is most of their HBM traffic, also with the
# fp16 output epilogue (y rounded once to fp16 in the kernel that stores it)
HALF_OUTPUT_LAYERS = (("resnet3x3", "f16", "f16"), ("stem7x7", "f16", "f16"), ("mix1x1", "f16", "f16"))


def other_form(cfg, dt, res, args, dev):
    """The layer's other form (window <-> implicit) where it has both, or None."""
    if not implicit_applies(cfg, dt):
        return None
    alt = "window" if res["form"] == "implicit" else "implicit"
    _say(f"bench: {cfg.name} {dt} other form ({alt})")
    return time_variant(cfg, dt, args.steps, args.warmup, dev, algo=alt)


def finish(cfg, dt, res, seconds, args):
    """CPU leg of one timed variant: parity fields into res, the baseline returned."""
    if args.no_cpu_baseline:
        return None
    base, par = cpu_leg(cfg, dt, res, seconds)
    res.update(par)
    res["cpu_oracle_tflops"] = base["value"]
    return base


def clean(res):
    return {k: v for k, v in res.items() if k not in ("sample_idx", "sample_got")}


def head_fields(cfg, dt, h):
    return {
        "metric": METRIC, "value": h["value"], "unit": "TFLOPS", "n_gpus": 1,
        "ms_per_step": h["ms_per_step"], "warmup_calls": h["warmup_calls"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: N={cfg.N} Cin={cfg.Cin} H=W={cfg.H} "
                               f"Cout={cfg.Cout} {cfg.KH}x{cfg.KW} s{cfg.stride} p{cfg.pad}",
                   "N": cfg.N, "Cin": cfg.Cin, "H": cfg.H, "W": cfg.W, "Cout": cfg.Cout,
                   "KH": cfg.KH, "KW": cfg.KW, "stride": cfg.stride, "pad": cfg.pad,
                   "output": "fp32", "parallelism": "single GPU"},
        "pct_of_peak": h["pct_of_peak"], "peak_tflops": h["peak_tflops"],
        "roofline": h["roofline"], "kernels": h["kernels"],
        "ws_bytes": h["ws_bytes"], "im2col_bytes": h["im2col_bytes"],
        "ws_over_im2col": h["ws_over_im2col"], "ws_target": h["ws_target"],
        "rel_l2_sampled": h.get("rel_l2_sampled"), "max_err_over_bound": h.get("max_err_over_bound"),
        "parity_ok": h.get("parity_ok"),
        "ms_per_call_median": h["ms_per_call_median"], "ms_per_call_best": h["ms_per_call_best"],
        "form": h["form"], "kernel_us": h["kernel_us"],
        "chunk_pack_us": h["chunk_pack_us"], "chunk_gemm_us": h["chunk_gemm_us"],
        "chunk_rows": h["chunk_rows"], "n_chunks": h["n_chunks"],
    }


def default_line(args, dev):
    """One JSON line: the headline layer (the ResNet-style 3x3 layer in fp16)
    plus every layer configuration and dtype under "layers", each with its
    TFLOPS, roofline of the dominant kernel, HBM traffic where counters were
    taken, workspace, parity and the oracle's own throughput."""
    import workloads
    todo = [(n, dt, "f32") for n in DEFAULT_LAYERS for dt in workloads.CONFIGS[n].dtypes]
    todo += list(HALF_OUTPUT_LAYERS)
    res = {}
    for name, dt, ydt in todo:
        _say(f"bench: {name} {dt} -> y {ydt} warmup={args.warmup} steps={args.steps}")
        res[(name, dt, ydt)] = time_variant(workloads.CONFIGS[name], dt, args.steps, args.warmup, dev,
                                            ydt=ydt)
    head = HEADLINE + ("f32",)
    hcfg = workloads.CONFIGS[HEADLINE[0]]
    other = other_form(hcfg, HEADLINE[1], res[head], args, dev)
    # every GPU timing is done: the CPU leg (oracle baseline + parity of the samples)
    base = None
    for name, dt, ydt in todo:
        _say(f"bench: cpu leg {name} {dt} -> y {ydt}")
        b = finish(workloads.CONFIGS[name], dt, res[(name, dt, ydt)],
                   10.0 if (name, dt, ydt) == head else (1.5 if ydt == "f32" else 0.0), args)
        if (name, dt, ydt) == head:
            base = b
    if other is not None:
        finish(hcfg, HEADLINE[1], other, 0.0, args)
    h = res[head]
    line = head_fields(hcfg, HEADLINE[1], h)
    line.update({"steps": args.steps, "warmup": args.warmup})
    line["other_form"] = clean(other) if other is not None else None
    line["layers"] = [layer_entry(workloads.CONFIGS[n], dt, res[(n, dt, y)]) for n, dt, y in todo]
    line["all_parity_ok"] = (None if args.no_cpu_baseline
                             else all(res[k].get("parity_ok") for k in todo))
    if base is not None:
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)


def per_layer_lines(args, dev):
    """One JSON line per layer (--config, --all-configs or --table1): the
    layer's half-precision variant as the headline, its other dtypes under
    "variants", the other form of each dtype under "other_form"."""
    import workloads
    names = (list(workloads.TABLE1) if args.table1 else
             sorted(workloads.CONFIGS) if args.all_configs else [args.config])
    for name in names:
        cfg = workloads.get_config(name)
        dts = list(cfg.dtypes)
        head = args.dtype if args.dtype and args.dtype in dts else \
            next((d for d in dts if d != "f32"), dts[0])
        order = [head] + ([] if args.single else [d for d in dts if d != head])
        results = {}
        for dt in order:
            _say(f"bench: {name} {dt} warmup={args.warmup} steps={args.steps}")
            results[dt] = time_variant(cfg, dt, args.steps, args.warmup, dev)
        others = {dt: other_form(cfg, dt, results[dt], args, dev) for dt in order}
        base = None
        first = name == names[0] or args.cpu_baseline_all
        for dt in order:
            b = finish(cfg, dt, results[dt], 10.0 if (first and dt == head) else 0.0, args)
            if dt == head:
                base = b
            if others[dt] is not None:
                finish(cfg, dt, others[dt], 0.0, args)
        line = head_fields(cfg, head, results[head])
        line.update({"steps": args.steps, "warmup": args.warmup})
        for dt in order[1:]:
            if others[dt] is not None:
                results[dt]["other_form"] = clean(others[dt])
        line["variants"] = [clean(results[d]) for d in order[1:]]
        line["other_form"] = clean(others[head]) if others[head] is not None else None
        if base is not None and first:
            line["cpu_baseline"] = base
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
