"""Build ``libpq2.so`` (the C-ABI library of include/pq2.h) and
``libpq2_probe.so`` (the measurement probes of include/pq2_probe.h) for gfx950
with hipcc.

Run ``python gemm_pq2_w2a8_amd/build.py`` (or call :func:`build`); as a script it
does not import the package, which needs a built library. Objects go to
``gemm_pq2_w2a8_amd/_build/``; the libraries are written next to this file.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpq2.so")
PROBE_LIB = os.path.join(HERE, "libpq2_probe.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["pq2_abi.cpp", "quantize.hip", "gemv_dot4.hip", "small_mfma.hip", "small_panel.hip",
           "prefill_mfma.hip"]
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the quantiser needs IEEE division and float32 denormals
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # MFMA sources and results in ordinary VGPRs: the kernels' epilogues read
    # every MFMA result with VALU instructions, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", INCLUDE,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
