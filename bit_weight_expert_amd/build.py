"""Build libmoe_w4a16.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage:  python -m bit_weight_expert_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_w4a16.so")
SOURCES = ["api.hip", "route_align.hip", "gemm.hip", "act_order.hip", "mxfp8.hip", "nvfp4_chunk.hip"]
# gemm_inst.hip is built once per (weight format, epilogue) pair: formats
# NVFP4 / MXFP4 / GPTQ = 0 / 1 / 2, epilogues swigluoai / ReLU^2 / none /
# down projection = 0 / 1 / 2 / 3.
INSTANCES = [(f, e) for f in range(3) for e in range(4)]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic is kept off for every device function
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = [(s, os.path.join(objdir, s.replace(".hip", ".o")), ()) for s in SOURCES]
    jobs += [("gemm_inst.hip", os.path.join(objdir, f"gemm_inst_{f}_{e}.o"),
              (f"-DMOE_FMT={f}", f"-DMOE_EPI={e}")) for f, e in INSTANCES]
    objs = [j[1] for j in jobs]
    # the instantiation units first: they take the longest
    jobs.sort(key=lambda j: j[0] != "gemm_inst.hip")
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
