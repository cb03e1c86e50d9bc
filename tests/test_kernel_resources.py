"""CPU check of the compiled gfx950 kernels: no kernel may use scratch memory.

A register array that the compiler cannot keep in registers is demoted to
per-lane scratch (global memory), which turned into ~5x slower kernels when
it happened; hipcc's resource remarks expose it at build time.
"""

import os
import re
import shutil
import subprocess

import pytest

from gemm_pq2_w2a8_amd import build as hip_build

SOURCES = [s for s in hip_build.SOURCES if s.endswith(".hip")]


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
