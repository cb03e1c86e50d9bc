"""CPU check of the compiled gfx950 kernels: no kernel may use scratch memory.

A register array that the compiler cannot keep in registers is demoted to
per-lane scratch (global memory), which turned into ~5x slower kernels when
it happened; hipcc's resource remarks expose it at build time.
"""

import os
import re
import shutil
import subprocess

import importlib.util

import pytest

# the build script, loaded by path (importing the package needs a built library)
_spec = importlib.util.spec_from_file_location(
    "pq2_hip_build", os.path.join(os.path.dirname(__file__), "..", "gemm_pq2_w2a8_amd", "build.py"))
hip_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(hip_build)

SOURCES = [s for s in hip_build.SOURCES + hip_build.PROBE_SOURCES if s.endswith(".hip")]


@pytest.mark.skipif(shutil.which(hip_build.HIPCC) is None and not os.path.exists(hip_build.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(src):
    flags = [f for f in hip_build.CFLAGS if f != "-fPIC"]
    cmd = [hip_build.HIPCC, *flags, "--cuda-device-only", "-c",
           os.path.join(hip_build.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", out.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
    assert names and len(names) == len(scratch)
    bad = [(n, s) for n, s in zip(names, scratch) if s != 0]
    assert not bad, f"kernels using scratch: {bad}"
