"""CPU check of the compiled gfx950 kernels: no kernel may use scratch memory.

A register array that the compiler cannot keep in registers is demoted to
per-lane scratch (global memory), which turned into ~5x slower kernels when
it happened. Every kernel's private segment size is recorded in the code
object's metadata note; this test reads it from the objects the build wrote
(the device code bundled in each object's .hip_fatbin section), so it checks
exactly what was built without compiling anything again.
"""

import importlib.util
import os
import re
import subprocess
import tempfile

import pytest

# the build script, loaded by path (importing the package needs a built library)
_spec = importlib.util.spec_from_file_location(
    "pq2_hip_build", os.path.join(os.path.dirname(__file__), "..", "gemm_pq2_w2a8_amd", "build.py"))
hip_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(hip_build)

LLVM = "/opt/rocm/llvm/bin"
SOURCES = [s for s in hip_build.SOURCES + hip_build.PROBE_SOURCES if s.endswith(".hip")]


def kernel_scratch(obj: str):
    """{kernel name: private segment bytes} of the gfx950 code object in obj."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        co = os.path.join(d, "dev.co")
        subprocess.run([f"{LLVM}/llvm-objcopy", "--dump-section", f".hip_fatbin={fat}", obj,
                        os.devnull], check=True, capture_output=True)
        targets = subprocess.run([f"{LLVM}/clang-offload-bundler", "--list", "--type=o",
                                  f"--input={fat}"], check=True, capture_output=True,
                                 text=True).stdout.split()
        target = [t for t in targets if t.endswith(hip_build.ARCH)]
        assert len(target) == 1, targets
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                        f"--input={fat}", f"--targets={target[0]}", f"--output={co}"],
                       check=True, capture_output=True)
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True,
                               capture_output=True, text=True).stdout
    names = re.findall(r"^\s+\.name:\s+(\S+)", notes, re.M)
    sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    assert names and len(names) == len(sizes), (len(names), len(sizes))
    return dict(zip(names, sizes))


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/clang-offload-bundler"),
                    reason="ROCm LLVM tools not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(src):
    obj = os.path.join(hip_build.BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        pytest.skip(f"{obj} not built (run gemm_pq2_w2a8_amd/build.py)")
    scratch = kernel_scratch(obj)
    bad = {n: s for n, s in scratch.items() if s != 0}
    assert not bad, f"kernels using scratch: {bad}"
