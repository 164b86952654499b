"""Build libprofk.so (HIP kernels for gfx950 + host controller + C ABI) in-tree.

Every translation unit is compiled with hipcc for --offload-arch=gfx950 into
_build/, then linked into sampling_threshold_filtering_amd/libprofk.so.
"""
from __future__ import annotations

import os
import resource
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libprofk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "k_sample.hip", "k_select.hip", "k_filter.hip", "k_refine.hip", "k_sort.hip", "k_batched.hip", "k_merge.hip", "k_probe.hip",
           "solver.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _raise_stack_limit() -> None:
    """The compiler's interprocedural value analysis recurses once per link of a long
    select chain (the unrolled register sorting networks); with the usual 8 MB stack
    it overflows on k_refine.hip.  Child processes inherit the raised soft limit."""
    soft, hard = resource.getrlimit(resource.RLIMIT_STACK)
    want = hard if hard == resource.RLIM_INFINITY else max(soft, hard)
    if soft != resource.RLIM_INFINITY and (want == resource.RLIM_INFINITY or want > soft):
        resource.setrlimit(resource.RLIMIT_STACK, (want, hard))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _raise_stack_limit()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
