"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pq2.h")

pq2 = pytest.importorskip("gemm_pq2_w2a8_amd")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_HIP, ERR_ARG = 0, 1, 2, 3, 4, 5
P = 0x100000  # a fake, 256-byte-aligned non-null address; never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pq2_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(pq2.ABI_SYMBOLS)
    for name in names:
        assert hasattr(pq2.lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define\s+PQ2_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert pq2.abi_version() == int(m.group(1))


def test_status_strings():
    for st in range(7):
        s = pq2.lib.pq2_status_str(st)
        assert s and s.startswith(b"PQ2_")
    assert pq2.lib.pq2_status_str(99)


def test_quantize_validation():
    f = pq2.lib.pq2_quantize_act
    assert f(None, P, P, P, 1, 128, None) == ERR_NULL
    assert f(P, P, P, None, 1, 128, None) == ERR_NULL
    assert f(P, P, P, P, 0, 128, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, 64, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, 200, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, -128, None) == ERR_SHAPE
    assert f(P, P, P, P, (1 << 30) + 1, 128, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, (1 << 24) + 128, None) == ERR_SHAPE   # K above PQ2_MAX_K
    assert f(P + 4, P, P, P, 1, 128, None) == ERR_ALIGN     # x needs 16 B
    assert f(P, P + 8, P, P, 1, 128, None) == ERR_ALIGN     # q needs 16 B
    assert f(P, P, P + 2, P, 1, 128, None) == ERR_ALIGN     # s needs 4 B
    assert f(P, P, P, P + 1, 1, 128, None) == ERR_ALIGN     # t needs 4 B


def test_gemm_validation():
    f = pq2.lib.pq2_gemm
    assert f(None, P, P, P, P, P, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, None, P, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, None, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, P, 1, 0, 128, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 0, 8, 128, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 1, 8, 129, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 1, 8, (1 << 24) + 128, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 1, (1 << 30) + 1, 128, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 1 << 30, 1 << 30, 128, None, 0, None) == ERR_SHAPE        # M*N > 2^40
    assert f(P, P, P, P, P, P, 1 << 20, 8, 1 << 21, None, 0, None) == ERR_SHAPE         # M*K > 2^40
    assert f(P, P, P, P, P, P, 1, 1 << 30, 1 << 14, None, 0, None) == ERR_SHAPE         # N*K/4 > 2^40
    assert f(P, P, P, P + 8, P, P, 1, 8, 128, None, 0, None) == ERR_ALIGN   # codes needs 16 B
    assert f(P, P, P, P, P + 1, P, 1, 8, 128, None, 0, None) == ERR_ALIGN   # wscale needs 2 B
    assert f(P, P, P, P, P, P + 2, 1, 8, 128, None, 0, None) == ERR_ALIGN   # y needs 4 B
    assert f(P, P, P, P, P, P, 1, 8, 128, P + 4, 64, None) == ERR_ALIGN     # workspace 16 B


def test_gemm_bf16_validation():
    f = pq2.lib.pq2_gemm_bf16
    assert f(None, P, P, P, P, P, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, None, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, P, 1, 8, 129, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P + 8, P, P, 1, 8, 128, None, 0, None) == ERR_ALIGN   # codes needs 16 B
    assert f(P, P, P, P, P, P + 1, 1, 8, 128, None, 0, None) == ERR_ALIGN   # y needs 2 B


def test_quantize_16bit_validation():
    f = pq2.lib.pq2_quantize_act_16
    BF, F16 = pq2.ACT_BF16, pq2.ACT_F16
    assert f(None, BF, P, P, P, 1, 128, None) == ERR_NULL
    assert f(P, F16, P, None, P, 1, 128, None) == ERR_NULL
    assert f(P, BF, P, P, P, 0, 128, None) == ERR_SHAPE
    assert f(P, BF, P, P, P, 1, 200, None) == ERR_SHAPE
    assert f(P + 4, BF, P, P, P, 1, 128, None) == ERR_ALIGN      # x needs 8 B
    assert f(P, F16, P + 8, P, P, 1, 128, None) == ERR_ALIGN     # q needs 16 B
    assert f(P, 0, P, P, P, 1, 128, None) == ERR_ARG              # float32 goes to pq2_quantize_act
    assert f(P, 3, P, P, P, 1, 128, None) == ERR_ARG


def test_linear_validation():
    f = pq2.lib.pq2_linear
    assert f(None, P, P, P, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, None, P, 1, 8, 128, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, 0, 8, 128, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, 1, 8, 200, None, 0, None) == ERR_SHAPE
    assert f(P + 4, P, P, P, 1, 8, 128, None, 0, None) == ERR_ALIGN     # x needs 16 B
    assert f(P, P + 8, P, P, 1, 8, 128, None, 0, None) == ERR_ALIGN     # codes needs 16 B
    assert f(P, P, P, P, 1, 8, 128, P + 4, 64, None) == ERR_ALIGN       # workspace 16 B
    assert f(P, P, P, P, 17, 8, 2048, None, 0, None) == ERR_ARG         # M above PQ2_LINEAR_MAX_M
    assert f(P, P, P, P, 5, 8, 640, None, 0, None) == ERR_ARG           # 5..16 rows: K % 1024 == 0


def test_linear_queries():
    """Pure host queries: no fused kernel above PQ2_LINEAR_MAX_M or for bad
    shapes; the dot4 GEMV for one or two rows, which needs no workspace."""
    assert pq2.LINEAR_MAX_M == 16
    assert pq2.linear_kernel_path(17, 8, 2048, 0) == -1
    assert pq2.linear_kernel_path(1, 8, 200, 0) == -1
    assert pq2.linear_workspace_bytes(17, 5120, 17408) == 0
    assert pq2.linear_workspace_bytes(0, 5120, 17408) == 0
    for M, N, K in ((1, 5120, 6144), (2, 5120, 17408), (1, 34816, 5120)):
        assert pq2.linear_kernel_path(M, N, K, 0) == pq2.PATH_GEMV
        assert pq2.linear_workspace_bytes(M, N, K) == 0
    assert pq2.linear_kernel_path(5, 8, 640, 1 << 20) == -1   # 5..16 rows need a ring plan


def test_group_dots_validation():
    f = pq2.lib.pq2_gemm_group_dots
    assert f(P, P, P, None, 1, 8, 128, 0, None) == ERR_NULL
    assert f(P, P, P, P, 1, 8, 100, 0, None) == ERR_SHAPE
    assert f(P, P, P, P, 5, 8, 128, pq2.PATH_GEMV, None) == ERR_ARG   # GEMV: M <= 4
    assert f(P, P, P, P, 17, 8, 128, pq2.PATH_SMALL, None) == ERR_ARG
    assert f(P, P, P, P, 16, 8, 32768 + 128, pq2.PATH_SMALL, None) == ERR_ARG
    assert f(P, P, P, P, 8, 8, 1920, pq2.PATH_PANEL, None) == ERR_ARG
    assert f(P, P, P, P, 1, 8, 128, 7, None) == ERR_ARG
    assert f(P, P, P, P, 1, 8, 128, -1, None) == ERR_ARG
    assert f(P, P, P + 8, P, 1, 8, 128, 0, None) == ERR_ALIGN   # codes needs 16 B
    assert f(P + 8, P, P, P, 1, 8, 128, 0, None) == ERR_ALIGN   # q needs 16 B


def test_gemm_path_validation():
    f = pq2.lib.pq2_gemm_path
    assert f(None, P, P, P, P, P, 1, 8, 128, 0, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, None, 1, 8, 128, 0, None, 0, None) == ERR_NULL
    assert f(P, P, P, P, P, P, 1, 8, 200, 0, None, 0, None) == ERR_SHAPE
    assert f(P, P, P, P + 8, P, P, 1, 8, 128, 1, None, 0, None) == ERR_ALIGN
    assert f(P, P, P, P, P, P, 5, 8, 128, pq2.PATH_GEMV, None, 0, None) == ERR_ARG
    assert f(P, P, P, P, P, P, 17, 8, 1024, pq2.PATH_SMALL, None, 0, None) == ERR_ARG
    assert f(P, P, P, P, P, P, 65, 8, 2048, pq2.PATH_PANEL, None, 0, None) == ERR_ARG   # M <= 64
    assert f(P, P, P, P, P, P, 8, 8, 1920, pq2.PATH_PANEL, None, 0, None) == ERR_ARG    # K >= 2048
    assert f(P, P, P, P, P, P, 8, 8, 18560, pq2.PATH_PANEL, None, 0, None) == ERR_ARG   # K <= 18432
    assert f(P, P, P, P, P, P, 1, 8, 128, 5, None, 0, None) == ERR_ARG


def test_kernel_path_query():
    f = pq2.lib.pq2_gemm_kernel_path
    big = 1 << 40
    assert f(1, 8, 100, big) == -1 and f(0, 8, 128, big) == -1
    assert f(1, 5120, 6144, 0) == pq2.PATH_GEMV
    assert f(2, 17408, 5120, big) == pq2.PATH_GEMV
    assert f(17, 8, 128, big) == pq2.PATH_PREFILL
    assert f(16, 8, 32768 + 128, big) == pq2.PATH_PREFILL
    # 17..64 rows where the tiled GEMM fills two blocks per CU: the tiled GEMM
    assert f(32, 17408, 5120, big) == pq2.PATH_PREFILL
    # without a GPU the panel kernel never fits: the 16-token kernel is chosen
    assert f(8, 5120, 17408, big) == pq2.PATH_SMALL
    assert f(8, 5120, 17408, 0) == pq2.PATH_SMALL


def test_workspace_query():
    f = pq2.lib.pq2_gemm_workspace_bytes
    assert f(1, 8, 100) == 0 and f(0, 8, 128) == 0     # invalid shapes
    assert f(1, 5120, 6144) == 0                        # the GEMV never splits K
    # The wide prefill tile splits the K range of the tiles left over after
    # whole rounds of two blocks per CU (256 CUs assumed where no GPU is
    # visible): 4096 x 17408 is 2176 tiles of 128 x 256, 128 left over, split
    # into 4 chunks of 128 x 256 float32 partial sums each.
    assert f(4096, 17408, 5120) == 128 * 4 * 128 * 256 * 4
    assert f(4096, 4096, 5120) == 0                     # 512 tiles: whole rounds only
    # 512 x 17408: the 256 x 64 tile, 544 tiles, 32 left over in 4 chunks
    assert f(512, 17408, 5120) == 32 * 4 * 64 * 256 * 4
    assert f(512, 5120, 5120) == 0                      # the 64 x 64 tile: no split
    assert f(4096, 17408, 5248) == 0                    # 41 groups, not a multiple of 8: not the wide tile


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 128)
    with pytest.raises(ValueError):
        pq2.quantize_act(x)


PROBE_HEADER = os.path.join(ROOT, "include", "pq2_probe.h")
PROBE_LIB = os.path.join(ROOT, "gemm_pq2_w2a8_amd", "libpq2_probe.so")


def probe_lib():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libpq2_probe.so not built")
    lib = ctypes.CDLL(PROBE_LIB)
    Pv, SZ = ctypes.c_void_p, ctypes.c_size_t
    lib.pq2_probe_stream_read.argtypes = [Pv, SZ, Pv, ctypes.c_int, Pv]
    lib.pq2_probe_mfma_i8.argtypes = [Pv, ctypes.c_int, ctypes.c_int, Pv]
    lib.pq2_probe_epilogue_mix.argtypes = [Pv, ctypes.c_int, ctypes.c_int, Pv]
    lib.pq2_probe_clock.argtypes = [Pv, ctypes.c_uint64, Pv]
    return lib


def test_probe_header_symbols_exported():
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pq2_[a-z0-9_]+)\s*\(", src)))
    assert names == ["pq2_probe_clock", "pq2_probe_epilogue_mix", "pq2_probe_mfma_i8",
                     "pq2_probe_stream_read"]
    lib = probe_lib()
    for name in names:
        assert hasattr(lib, name), name


def test_probe_validation():
    lib = probe_lib()
    f = lib.pq2_probe_stream_read
    assert f(None, 1024, P, 256, None) == -1
    assert f(P, 1000, P, 256, None) == -1          # bytes a multiple of 16
    assert f(P + 8, 1024, P, 256, None) == -1      # src 16-byte aligned
    assert f(P, 1024, P, 0, None) == -1
    assert f(P, 1024, P, (1 << 20) + 1, None) == -1
    g = lib.pq2_probe_mfma_i8
    assert g(None, 10, 256, None) == -1
    assert g(P, 0, 256, None) == -1
    assert g(P, 10, 0, None) == -1
    e = lib.pq2_probe_epilogue_mix
    assert e(None, 10, 256, None) == -1
    assert e(P, 0, 256, None) == -1
    assert e(P, (1 << 24) + 1, 256, None) == -1
    assert e(P, 10, 0, None) == -1
    assert e(P + 2, 10, 256, None) == -1           # sink 4-byte aligned
    h = lib.pq2_probe_clock
    assert h(None, 100, None) == -1
    assert h(P + 4, 100, None) == -1
    assert h(P, 0, None) == -1
    assert h(P, (1 << 28) + 1, None) == -1


def test_noalloc_validation():
    f = pq2.lib.pq2_gemm_noalloc
    assert f(None, P, P, P, P, P, 1, 8, 128, None) == ERR_NULL
    assert f(P, P, P, P, P, None, 1, 8, 128, None) == ERR_NULL
    assert f(P, P, P, P, P, P, 1, 8, 129, None) == ERR_SHAPE
    assert f(P, P, P, P, P, P, 0, 8, 128, None) == ERR_SHAPE
    assert f(P, P, P, P + 8, P, P, 1, 8, 128, None) == ERR_ALIGN   # codes needs 16 B
    assert f(P, P, P, P, P, P + 2, 1, 8, 128, None) == ERR_ALIGN   # y needs 4 B
