"""Thin Python binding of the PQ2_0 C ABI (include/pq2.h), for PyTorch tensors.

Argument marshalling only: tensors are checked for dtype, shape, device and
contiguity, their device pointers and the current HIP stream are passed to
``libpq2.so``, and a non-zero status raises :class:`PQ2Error`. Every step of
the computation runs in the library's gfx950 kernels; there is no fallback.
Importing this package raises if ``libpq2.so`` has not been built
(``python gemm_pq2_w2a8_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpq2.so")

GROUP = 128
PATH_AUTO, PATH_GEMV, PATH_SMALL, PATH_PREFILL, PATH_PANEL = 0, 1, 2, 3, 4
ACT_BF16, ACT_F16 = 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python gemm_pq2_w2a8_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
lib.pq2_abi_version.restype = ctypes.c_int
lib.pq2_abi_version.argtypes = []
lib.pq2_status_str.restype = ctypes.c_char_p
lib.pq2_status_str.argtypes = [ctypes.c_int]
lib.pq2_quantize_act.restype = ctypes.c_int
lib.pq2_quantize_act.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
lib.pq2_quantize_act_16.restype = ctypes.c_int
lib.pq2_quantize_act_16.argtypes = [_P, ctypes.c_int, _P, _P, _P, _I64, _I64, _P]
_SZ = ctypes.c_size_t
lib.pq2_gemm_workspace_bytes.restype = _SZ
lib.pq2_gemm_workspace_bytes.argtypes = [_I64, _I64, _I64]
lib.pq2_gemm.restype = ctypes.c_int
lib.pq2_gemm.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
lib.pq2_gemm_bf16.restype = ctypes.c_int
lib.pq2_gemm_bf16.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
lib.pq2_gemm_noalloc.restype = ctypes.c_int
lib.pq2_gemm_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
lib.pq2_gemm_kernel_path.restype = ctypes.c_int
lib.pq2_gemm_kernel_path.argtypes = [_I64, _I64, _I64, _SZ]
lib.pq2_gemm_path.restype = ctypes.c_int
lib.pq2_gemm_path.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _SZ,
                              _P]
lib.pq2_gemm_group_dots.restype = ctypes.c_int
lib.pq2_gemm_group_dots.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P]
lib.pq2_linear.restype = ctypes.c_int
lib.pq2_linear.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]
lib.pq2_linear_workspace_bytes.restype = _SZ
lib.pq2_linear_workspace_bytes.argtypes = [_I64, _I64, _I64]
lib.pq2_linear_kernel_path.restype = ctypes.c_int
lib.pq2_linear_kernel_path.argtypes = [_I64, _I64, _I64, _SZ]

LINEAR_MAX_M = 16   # PQ2_LINEAR_MAX_M

# Every extern "C" symbol declared in include/pq2.h.
ABI_SYMBOLS = ("pq2_abi_version", "pq2_status_str", "pq2_quantize_act", "pq2_quantize_act_16",
               "pq2_gemm_workspace_bytes", "pq2_gemm", "pq2_gemm_noalloc", "pq2_gemm_bf16",
               "pq2_gemm_kernel_path", "pq2_gemm_path", "pq2_linear", "pq2_linear_workspace_bytes",
               "pq2_linear_kernel_path", "pq2_gemm_group_dots")

NOALLOC_SCRATCH_BYTES = 16 << 20    # PQ2_NOALLOC_SCRATCH_BYTES

PATH_NAMES = {PATH_GEMV: "gemv_dot4", PATH_SMALL: "small_mfma", PATH_PREFILL: "prefill_mfma",
              PATH_PANEL: "small_panel"}


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes of pq2_gemm's fastest plan for this shape (0: none needed)."""
    return int(lib.pq2_gemm_workspace_bytes(M, N, K))


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes of pq2_linear's plan for this shape (0: none needed)."""
    return int(lib.pq2_linear_workspace_bytes(M, N, K))


def linear_kernel_path(M: int, N: int, K: int, workspace_bytes: Optional[int] = None) -> int:
    """PATH_GEMV or PATH_PANEL: the kernel pq2_linear takes for this shape given
    a workspace of that many bytes (None: what linear_workspace_bytes asks
    for); -1 where pq2_linear rejects the shape."""
    if workspace_bytes is None:
        workspace_bytes = linear_workspace_bytes(M, N, K)
    return int(lib.pq2_linear_kernel_path(M, N, K, int(workspace_bytes)))


def gemm_kernel_path(M: int, N: int, K: int, workspace_bytes: Optional[int] = None) -> int:
    """PATH_* that pq2_gemm takes for this shape on the current device given a
    workspace of that many bytes (None: the size gemm_workspace_bytes asks
    for); -1 for a bad shape."""
    if workspace_bytes is None:
        workspace_bytes = gemm_workspace_bytes(M, N, K)
    return int(lib.pq2_gemm_kernel_path(M, N, K, int(workspace_bytes)))


class PQ2Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(lib.pq2_status_str(status).decode())


def _check(status: int) -> None:
    if status != 0:
        raise PQ2Error(status)


def abi_version() -> int:
    return int(lib.pq2_abi_version())


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mk(x: torch.Tensor) -> Tuple[int, int]:
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    return int(x.shape[0]), int(x.shape[1])


def pq2_quantize_act(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, t: torch.Tensor,
                     stream=None) -> None:
    """x float32, bfloat16 or float16 [M][K] -> q int8 [M][K] (plane order),
    s float32 [M][G], t int32 [M][G]; 16-bit x is widened exactly first."""
    M, K = _mk(x)
    G = K // GROUP
    _need(q, "q", torch.int8, (M, K))
    _need(s, "s", torch.float32, (M, G))
    _need(t, "t", torch.int32, (M, G))
    if x.dtype in (torch.bfloat16, torch.float16):
        _need(x, "x", x.dtype, (M, K))
        fmt = ACT_BF16 if x.dtype == torch.bfloat16 else ACT_F16
        _check(lib.pq2_quantize_act_16(x.data_ptr(), fmt, q.data_ptr(), s.data_ptr(),
                                       t.data_ptr(), M, K, _stream(x, stream)))
        return
    _need(x, "x", torch.float32, (M, K))
    _check(lib.pq2_quantize_act(x.data_ptr(), q.data_ptr(), s.data_ptr(), t.data_ptr(), M, K,
                                _stream(x, stream)))


def _workspace(workspace, M: int, N: int, K: int, device, stream,
               query=None) -> Tuple[int, int, object]:
    """(pointer, bytes, keep-alive) of the split-K workspace argument: "auto"
    allocates the size pq2_gemm_workspace_bytes (or `query`) asks for with
    torch (none when 0), None passes no workspace, a device tensor passes its storage. An
    "auto" buffer is tied to the launch stream, so torch's allocator does not
    hand it out again before the kernels on that stream are done with it."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        n = (query or gemm_workspace_bytes)(M, N, K)
        if n == 0:
            return 0, 0, None
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
        if stream is not None:
            st = stream if isinstance(stream, torch.cuda.Stream) else \
                torch.cuda.ExternalStream(int(stream), device=device)
            workspace.record_stream(st)
    if workspace is None:
        return 0, 0, None
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def pq2_gemm(q: torch.Tensor, s: torch.Tensor, t: torch.Tensor, codes: torch.Tensor,
             wscale: torch.Tensor, y: torch.Tensor, workspace="auto", stream=None) -> None:
    """y [M][N] = PQ2_0 product of plane-order q/s/t and codes/wscale; y float32,
    or bfloat16 (pq2_gemm_bf16: the float32 result rounded to nearest-even).
    workspace: "auto" (torch allocates what the fastest plan needs), None (no
    workspace: plans that do not split K) or a device tensor."""
    M, K = _mk(q)
    N = int(codes.shape[0])
    G = K // GROUP
    _need(q, "q", torch.int8, (M, K))
    _need(s, "s", torch.float32, (M, G))
    _need(t, "t", torch.int32, (M, G))
    _need(codes, "codes", torch.uint8, (N, K // 4))
    if wscale.dtype == torch.float16:
        wscale = wscale.view(torch.int16)
    _need(wscale, "wscale", torch.int16, (N, G))
    wp, wn, _keep = _workspace(workspace, M, N, K, q.device, stream)
    if y.dtype == torch.bfloat16:
        _need(y, "y", torch.bfloat16, (M, N))
        _check(lib.pq2_gemm_bf16(q.data_ptr(), s.data_ptr(), t.data_ptr(), codes.data_ptr(),
                                 wscale.data_ptr(), y.data_ptr(), M, N, K, wp, wn,
                                 _stream(q, stream)))
        return
    _need(y, "y", torch.float32, (M, N))
    _check(lib.pq2_gemm(q.data_ptr(), s.data_ptr(), t.data_ptr(), codes.data_ptr(),
                        wscale.data_ptr(), y.data_ptr(), M, N, K, wp, wn, _stream(q, stream)))


def pq2_gemm_noalloc(q: torch.Tensor, s: torch.Tensor, t: torch.Tensor, codes: torch.Tensor,
                     wscale: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """pq2_gemm with the library's own per-device split-K scratch: no workspace,
    no allocation (calls that overlap on one device race on the scratch)."""
    M, K = _mk(q)
    N = int(codes.shape[0])
    G = K // GROUP
    _need(q, "q", torch.int8, (M, K))
    _need(s, "s", torch.float32, (M, G))
    _need(t, "t", torch.int32, (M, G))
    _need(codes, "codes", torch.uint8, (N, K // 4))
    if wscale.dtype == torch.float16:
        wscale = wscale.view(torch.int16)
    _need(wscale, "wscale", torch.int16, (N, G))
    _need(y, "y", torch.float32, (M, N))
    _check(lib.pq2_gemm_noalloc(q.data_ptr(), s.data_ptr(), t.data_ptr(), codes.data_ptr(),
                                wscale.data_ptr(), y.data_ptr(), M, N, K, _stream(q, stream)))


def pq2_gemm_path(q: torch.Tensor, s: torch.Tensor, t: torch.Tensor, codes: torch.Tensor,
                  wscale: torch.Tensor, y: torch.Tensor, path: int, workspace="auto",
                  stream=None) -> None:
    """pq2_gemm through the selected kernel path (PATH_*); workspace as for pq2_gemm."""
    M, K = _mk(q)
    N = int(codes.shape[0])
    G = K // GROUP
    _need(q, "q", torch.int8, (M, K))
    _need(s, "s", torch.float32, (M, G))
    _need(t, "t", torch.int32, (M, G))
    _need(codes, "codes", torch.uint8, (N, K // 4))
    if wscale.dtype == torch.float16:
        wscale = wscale.view(torch.int16)
    _need(wscale, "wscale", torch.int16, (N, G))
    _need(y, "y", torch.float32, (M, N))
    wp, wn, _keep = _workspace(workspace, M, N, K, q.device, stream)
    _check(lib.pq2_gemm_path(q.data_ptr(), s.data_ptr(), t.data_ptr(), codes.data_ptr(),
                             wscale.data_ptr(), y.data_ptr(), M, N, K, int(path), wp, wn,
                             _stream(q, stream)))


def pq2_linear(x: torch.Tensor, codes: torch.Tensor, wscale: torch.Tensor, y: torch.Tensor,
               workspace="auto", stream=None) -> None:
    """y float32 [M][N] from float32 x [M][K] with the quantisation inside the
    GEMM kernel (M <= LINEAR_MAX_M). workspace as for pq2_gemm, sized by
    linear_workspace_bytes."""
    M, K = _mk(x)
    N = int(codes.shape[0])
    G = K // GROUP
    _need(x, "x", torch.float32, (M, K))
    _need(codes, "codes", torch.uint8, (N, K // 4))
    if wscale.dtype == torch.float16:
        wscale = wscale.view(torch.int16)
    _need(wscale, "wscale", torch.int16, (N, G))
    _need(y, "y", torch.float32, (M, N))
    wp, wn, _keep = _workspace(workspace, M, N, K, x.device, stream, linear_workspace_bytes)
    _check(lib.pq2_linear(x.data_ptr(), codes.data_ptr(), wscale.data_ptr(), y.data_ptr(),
                          M, N, K, wp, wn, _stream(x, stream)))


def pq2_gemm_group_dots(q: torch.Tensor, t: torch.Tensor, codes: torch.Tensor,
                        d: torch.Tensor, path: int = PATH_AUTO, stream=None) -> None:
    """d int32 [M][N][G] = exact group dots through the selected kernel path."""
    M, K = _mk(q)
    N = int(codes.shape[0])
    G = K // GROUP
    _need(q, "q", torch.int8, (M, K))
    _need(t, "t", torch.int32, (M, G))
    _need(codes, "codes", torch.uint8, (N, K // 4))
    _need(d, "d", torch.int32, (M, N, G))
    _check(lib.pq2_gemm_group_dots(q.data_ptr(), t.data_ptr(), codes.data_ptr(), d.data_ptr(),
                                   M, N, K, int(path), _stream(q, stream)))


# ---------------------------------------------------------------- allocating helpers

def quantize_act(x: torch.Tensor, stream=None):
    """Allocate q/s/t with torch and run pq2_quantize_act."""
    M, K = _mk(x)
    G = K // GROUP
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty((M, G), dtype=torch.float32, device=x.device)
    t = torch.empty((M, G), dtype=torch.int32, device=x.device)
    pq2_quantize_act(x, q, s, t, stream)
    return q, s, t


def linear(x: torch.Tensor, codes: torch.Tensor, wscale: torch.Tensor,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Whole path, y float32 [M][N]: pq2_linear for float32 x with one token
    row (where quantising inside the GEMV beats the separate launch), else
    pq2_quantize_act (float32, bfloat16 or float16 x) into torch-allocated
    q/s/t followed by pq2_gemm."""
    M = int(x.shape[0])
    N = int(codes.shape[0])
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=x.device)
    if M == 1 and x.dtype == torch.float32:
        pq2_linear(x, codes, wscale, y, stream=stream)
        return y
    q, s, t = quantize_act(x, stream)
    pq2_gemm(q, s, t, codes, wscale, y, stream=stream)
    return y
