"""Python access to the plain CPU oracle (``pq2_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it to check the GPU library. The GPU library never
imports this package, and this package never imports the GPU library.

``build()`` compiles the C file with gcc (-O2, no fast-math, no FP
contraction, OpenMP over independent output rows). The wrappers take and
return numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "pq2_oracle.c")
LIB = os.path.join(_HERE, "liboracle_pq2.so")
GROUP = 128

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle_pq2.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
               "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build(force=True)
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_version.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_weight.argtypes = [P, I64, I64, I64]
    lib.oracle_weight.restype = ctypes.c_int
    lib.oracle_quantize.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_quantize.restype = None
    lib.oracle_plane_order.argtypes = [P, I64, I64, P]
    lib.oracle_plane_order.restype = None
    lib.oracle_group_dots.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_group_dots.restype = None
    lib.oracle_gemm_f64.argtypes = [P, P, P, P, I64, I64, I64, P, P, ctypes.c_int]
    lib.oracle_gemm_f64.restype = None
    lib.oracle_gemm_f64_sampled.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P, P,
                                            ctypes.c_int]
    lib.oracle_gemm_f64_sampled.restype = None
    lib.oracle_group_dots_sampled.argtypes = [P, P, I64, P, P, I64, P, ctypes.c_int]
    lib.oracle_group_dots_sampled.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check_k(K: int) -> None:
    if K <= 0 or K % GROUP:
        raise ValueError("K must be a positive multiple of 128")


_MAX_THREADS = []


def max_threads() -> int:
    """OpenMP's thread count as the process started (read once: a call with
    threads = n sets OpenMP's count for the calls after it)."""
    if not _MAX_THREADS:
        _MAX_THREADS.append(int(_load().oracle_max_threads()))
    return _MAX_THREADS[0]


def half_to_double(bits: int) -> float:
    return float(_load().oracle_half_to_double(int(bits)))


def weight(codes: np.ndarray, K: int, n: int, k: int) -> int:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    return int(_load().oracle_weight(_ptr(codes), K, n, k))


def quantize(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """x float32 [M][K] -> (q int8 [M][K] natural order, s float32 [M][G], t int32 [M][G])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    _check_k(K)
    G = K // GROUP
    q = np.empty((M, K), np.int8)
    s = np.empty((M, G), np.float32)
    t = np.empty((M, G), np.int32)
    _load().oracle_quantize(_ptr(x), M, K, _ptr(q), _ptr(s), _ptr(t))
    return q, s, t


def plane_order(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    _check_k(K)
    qp = np.empty_like(q)
    _load().oracle_plane_order(_ptr(q), M, K, _ptr(qp))
    return qp


def group_dots(q: np.ndarray, codes: np.ndarray, threads: int = 0) -> np.ndarray:
    """q int8 [M][K] natural order, codes uint8 [N][K/4] -> D int32 [M][N][G]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    M, K = q.shape
    N = codes.shape[0]
    _check_k(K)
    assert codes.shape == (N, K // 4)
    D = np.empty((M, N, K // GROUP), np.int32)
    _load().oracle_group_dots(_ptr(q), _ptr(codes), M, N, K, _ptr(D), threads)
    return D


def gemm_f64(q: np.ndarray, s: np.ndarray, codes: np.ndarray, wscale: np.ndarray,
             threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """-> (y float64 [M][N], sum_g |term| float64 [M][N])."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ws = np.ascontiguousarray(wscale).view(np.uint16)
    M, K = q.shape
    N = codes.shape[0]
    _check_k(K)
    G = K // GROUP
    assert s.shape == (M, G) and codes.shape == (N, K // 4) and ws.shape == (N, G)
    y = np.empty((M, N), np.float64)
    tabs = np.empty((M, N), np.float64)
    _load().oracle_gemm_f64(_ptr(q), _ptr(s), _ptr(codes), _ptr(ws), M, N, K,
                            _ptr(y), _ptr(tabs), threads)
    return y, tabs


def gemm_f64_sampled(q, s, codes, wscale, mm, nn, threads: int = 0):
    """Outputs (mm[i], nn[i]) only -> (y float64 [P], sum|term| float64 [P])."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ws = np.ascontiguousarray(wscale).view(np.uint16)
    mm = np.ascontiguousarray(mm, dtype=np.int64)
    nn = np.ascontiguousarray(nn, dtype=np.int64)
    M, K = q.shape
    N = codes.shape[0]
    _check_k(K)
    assert mm.shape == nn.shape and mm.ndim == 1
    assert (mm >= 0).all() and (mm < M).all() and (nn >= 0).all() and (nn < N).all()
    P = mm.shape[0]
    y = np.empty(P, np.float64)
    tabs = np.empty(P, np.float64)
    _load().oracle_gemm_f64_sampled(_ptr(q), _ptr(s), _ptr(codes), _ptr(ws), M, N, K,
                                    _ptr(mm), _ptr(nn), P, _ptr(y), _ptr(tabs), threads)
    return y, tabs


def group_dots_sampled(q, codes, mm, nn, threads: int = 0) -> np.ndarray:
    """D for the outputs (mm[i], nn[i]) -> int32 [P][G]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    mm = np.ascontiguousarray(mm, dtype=np.int64)
    nn = np.ascontiguousarray(nn, dtype=np.int64)
    M, K = q.shape
    N = codes.shape[0]
    _check_k(K)
    assert (mm >= 0).all() and (mm < M).all() and (nn >= 0).all() and (nn < N).all()
    P = mm.shape[0]
    D = np.empty((P, K // GROUP), np.int32)
    _load().oracle_group_dots_sampled(_ptr(q), _ptr(codes), K, _ptr(mm), _ptr(nn), P,
                                      _ptr(D), threads)
    return D


def forward(x: np.ndarray, codes: np.ndarray, wscale: np.ndarray, threads: int = 0):
    """Whole path on the CPU: quantise, group dots, float64 epilogue."""
    q, s, t = quantize(x)
    y, tabs = gemm_f64(q, s, codes, wscale, threads)
    return y, tabs, (q, s, t)


def rel_err(y: np.ndarray, y_ref: np.ndarray, tabs: np.ndarray) -> float:
    """max |y - y*| / sum_g |term_g|, the per-output error measure the tests use.

    Outputs whose every term is zero must match exactly (error 0 or inf)."""
    y = np.asarray(y, np.float64)
    diff = np.abs(y - y_ref)
    scale = np.where(tabs > 0, tabs, 1.0)
    err = np.where(tabs > 0, diff / scale, np.where(diff > 0, np.inf, 0.0))
    return float(err.max()) if err.size else 0.0
