"""Build libfp4.so (gfx950) in-tree with hipcc.

Each translation unit under csrc/ is compiled to an object in parallel, then
linked into block_scaled_fp4_mx_amd/libfp4.so.  The peak-rate microbenchmarks
(probes/peak.hip, not part of the library) build into probes/libfp4_peak.so.
Every build recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfp4.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "moe.hip"]
PROBES = os.path.join(HERE, "probes")
PROBE_OUT = os.path.join(PROBES, "libfp4_peak.so")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off (scalar fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def _build_probes() -> None:
    tmp = PROBE_OUT + ".tmp"
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-shared", os.path.join(PROBES, "peak.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probes/peak.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_OUT)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        probes = ex.submit(_build_probes)
        objs = list(ex.map(_compile, SOURCES))
        probes.result()
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build()
