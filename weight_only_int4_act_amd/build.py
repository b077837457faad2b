"""Build libawq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m weight_only_int4_act_amd.build

Objects go to weight_only_int4_act_amd/_build/, the library to
weight_only_int4_act_amd/libawq.so.  A second library, libawq_ldspoison.so, is the same sources
compiled with AWQ_LDS_POISON (pipelined LDS buffers filled with NaN between their last reader and
their next writer): a debug build for the race test, never loaded by the product path.  Every call
recompiles both.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq.so")
LIB_POISON = os.path.join(PKG, "libawq_ldspoison.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled: the compiler never emits v_pk_{add,mul,fma}_f32.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
SOURCES = ["awq_api.hip", "awq_stats.hip", "awq_search.hip", "awq_pack.hip", "awq_gemm.hip", "awq_greedy.hip"]


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _compile(job) -> str:
    src, extra, tag = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = [(src, [], "") for src in SOURCES] + [(src, ["-DAWQ_LDS_POISON"], "_poison") for src in SOURCES]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(jobs_list)))) as ex:
        objs = list(ex.map(_compile, jobs_list))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], LIB_POISON)
    if verbose:
        print(f"built {LIB} and {LIB_POISON}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
