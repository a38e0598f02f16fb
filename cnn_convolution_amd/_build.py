"""Build the HIP library for gfx950 in-tree: cnn_convolution_amd/lib/libim2win_conv2d.so.

Every HIP source is compiled with hipcc for gfx950 only; packed fp32 vector
instructions are switched off for all device code. The build always
recompiles (it is the "does it build" check as well as the build).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libim2win_conv2d.so"
LIBPATH = os.path.join(LIBDIR, LIBNAME)
BUILDDIR = os.path.join(PKG, "_build")

SOURCES = [
    os.path.join(CSRC, "plan.cpp"),
    os.path.join(CSRC, "api.cpp"),
    os.path.join(CSRC, "noalloc.hip"),
    os.path.join(CSRC, "kernels", "pack.hip"),
    os.path.join(CSRC, "kernels", "weight_stage.hip"),
    os.path.join(CSRC, "kernels", "gemm_valu.hip"),
    os.path.join(CSRC, "kernels", "gemm_mfma.hip"),
    os.path.join(CSRC, "kernels", "gemm_mfma_dma.hip"),
    os.path.join(CSRC, "kernels", "conv_implicit.hip"),
    os.path.join(CSRC, "kernels", "conv_implicit_rows.hip"),
    os.path.join(CSRC, "kernels", "conv_implicit_narrow.hip"),
    os.path.join(CSRC, "kernels", "conv_implicit_pipe.hip"),
    os.path.join(CSRC, "kernels", "conv_implicit_ksplit.hip"),
]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(src: str, obj: str, extra=()) -> None:
    if src.endswith(".hip"):
        cmd = [hipcc(), *COMMON, *DEVICE, *extra, "-c", src, "-o", obj]
    else:
        # host-only C++: HIP runtime API headers, no device code
        cmd = [hipcc(), *COMMON, "-x", "c++", f"-I{rocm()}/include", "-D__HIP_PLATFORM_AMD__",
               *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag: drop that note
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = True, jobs: int = 8) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(BUILDDIR, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        futs = []
        for src in SOURCES:
            obj = os.path.join(BUILDDIR, os.path.basename(src) + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, src, obj))
        for f in futs:
            f.result()
    tmp = LIBPATH + ".tmp"
    cmd = [hipcc(), *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIBPATH)
    if verbose:
        print(f"built {LIBPATH}")
    return LIBPATH


if __name__ == "__main__":
    build()
