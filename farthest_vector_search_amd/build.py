"""Build libvs.so (the HIP library) in-tree for gfx950 with hipcc.

Usage: python -m farthest_vector_search_amd.build   (or build() from Python)
Objects go to farthest_vector_search_amd/_build/, the library next to this
file.  Every HIP source is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvs.so")
ROOF_LIB = os.path.join(HERE, "libvs_roofs.so")  # measurement kernels, not the search ABI
ARCH = os.environ.get("VS_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "prep.hip", "bmu_mfma.hip", "bmu_qreg.hip", "bmu_q16.hip", "bmu_small.hip", "bmu_csr.hip", "finalize.hip",
           "div_gram.hip", "div_ref.hip", "som.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out):
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + ["roofs.hip"]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], ROOF_LIB)
    if verbose:
        print(f"built {LIB} and {ROOF_LIB}")
    return LIB


if __name__ == "__main__":
    build()
