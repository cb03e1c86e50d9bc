"""Seeded synthetic inputs for the PQ2_0 ternary-weight GEMM.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It draws random numbers and lays them out in the buffer formats the
library consumes; it holds none of the method's arithmetic (no quantisation,
no decoding, no dot products).

Buffer formats produced (from the weight format described on the page
"Making a ternary reasoning model fast in vLLM", section "One token at a
time: plain Triton is enough"):

* codes: uint8 [N][K/4]. Each 2-bit code c in {0,1,2} stands for the weight
  c-1. The code of weight k of row n sits in byte n*K/4 + k//4 at bits
  2*(k%4) .. 2*(k%4)+1.
* wscale: float16 [N][K/128], one scale per 128-weight group (stored as the
  raw uint16 bit patterns when handed to the C ABI).
* x: float32 [M][K] activations, row-major.

Distributions follow the workload definitions: codes iid with a given
probability per code value, group scales float16(U(0.01, 0.1)) rounded to
nearest even, activations N(0, 1) in float32, optionally with a fraction of
outliers multiplied by 10.
"""

from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

GROUP = 128

# Probabilities of code values 0, 1, 2 (weights -1, 0, +1).
UNIFORM_CODES = (1.0 / 3.0, 1.0 / 3.0, 1.0 / 3.0)
# Prefill workload: weight -1 with p=0.4, weight 0 and +1 with p=0.3 each.
PREFILL_CODES = (0.4, 0.3, 0.3)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def pack_codes(c: np.ndarray) -> np.ndarray:
    """Pack a uint8 code array [N][K] (values 0..3) into bytes [N][K/4].

    Code of column 4*b+s goes to bits 2s..2s+1 of byte b.
    """
    c = np.asarray(c, dtype=np.uint8)
    n, k = c.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    c4 = c.reshape(n, k // 4, 4)
    out = (c4[:, :, 0] | (c4[:, :, 1] << 2) | (c4[:, :, 2] << 4) | (c4[:, :, 3] << 6))
    return out.astype(np.uint8)


# All 81 bytes whose four 2-bit fields lie in {0,1,2}; drawing one of them
# uniformly is the same as drawing four iid uniform codes.
_VALID_BYTES = np.array(
    [a | (b << 2) | (c << 4) | (d << 6)
     for d in range(3) for c in range(3) for b in range(3) for a in range(3)],
    dtype=np.uint8)


def draw_codes(n: int, k: int, rng: np.random.Generator,
               probs: Sequence[float] = UNIFORM_CODES) -> np.ndarray:
    """Packed codes uint8 [n][k/4], codes iid with P(code=v) = probs[v]."""
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    if tuple(probs) == UNIFORM_CODES:
        idx = rng.integers(0, 81, size=(n, k // 4), dtype=np.uint8)
        return _VALID_BYTES[idx]
    c = rng.choice(3, size=(n, k), p=np.asarray(probs, dtype=np.float64)).astype(np.uint8)
    return pack_codes(c)


def draw_wscale(n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """float16 [n][k/128] drawn as float16(U(0.01, 0.1)), round to nearest even."""
    u = rng.uniform(0.01, 0.1, size=(n, k // GROUP))
    return u.astype(np.float16)


def draw_x(m: int, k: int, rng: np.random.Generator, outlier_frac: float = 0.0,
           outlier_mult: float = 10.0) -> np.ndarray:
    """float32 [m][k] from N(0,1); each element is multiplied by outlier_mult
    with independent probability outlier_frac."""
    x = rng.standard_normal(size=(m, k), dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random(size=(m, k)) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return x


@dataclasses.dataclass
class Weights:
    codes: np.ndarray   # uint8 [N][K/4]
    wscale: np.ndarray  # float16 [N][K/128]

    @property
    def wscale_bits(self) -> np.ndarray:
        return self.wscale.view(np.uint16)


def weights(n: int, k: int, seed: int, probs: Sequence[float] = UNIFORM_CODES) -> Weights:
    """One weight matrix: codes then scales from one PCG64 stream."""
    rng = _rng(seed)
    codes = draw_codes(n, k, rng, probs)
    ws = draw_wscale(n, k, rng)
    return Weights(codes, ws)


def activations(m: int, k: int, seed: int, outlier_frac: float = 0.0) -> np.ndarray:
    return draw_x(m, k, _rng(seed), outlier_frac)


# Seed convention: activations use seed 0; weight matrix i of a set uses
# seed 1000 + i (matrix 0 of the tiny case uses seed 0 together with x).
def matrix_seed(i: int) -> int:
    return 1000 + i


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    k: int
    probs: tuple = UNIFORM_CODES
    outlier_frac: float = 0.0
    rotate: int = 1          # distinct weight matrices cycled per call


def tiny() -> Workload:
    return Workload("tiny_m1_n256_k512", 1, 256, 512)


def decode_gemv() -> Workload:
    return Workload("decode_gemv_m1_n5120_k6144", 1, 5120, 6144, rotate=64)


SMALL_SHAPES = ((5120, 6144), (17408, 5120), (5120, 17408))
SMALL_MS = (2, 4, 8, 16)


def small_batch(m: int, n: int, k: int) -> Workload:
    nbytes = n * k // 4 + 2 * n * (k // GROUP)
    rot = max(2, -(-512 * 1000 * 1000 // nbytes))   # at least 512 MB per set
    rot = min(rot, 64)
    return Workload(f"small_m{m}_n{n}_k{k}", m, n, k, outlier_frac=0.01, rotate=rot)


PREFILL_MS = (128, 512, 4096)
PREFILL_SHAPES = ((5120, 5120), (17408, 5120))


def prefill(m: int, n: int, k: int) -> Workload:
    return Workload(f"prefill_m{m}_n{n}_k{k}", m, n, k, probs=PREFILL_CODES)


# One synthetic decoder layer: (N, K) of its projections, in order: 5120 ->
# 6144, 6144 -> 5120, the gate and up projections 5120 -> 17408 stacked into
# one 34816-row matrix (both read the same activations; gate rows first, then
# up rows), and 17408 -> 5120. Five projections, four GEMMs.
LAYER_SHAPES = ((6144, 5120), (5120, 6144), (2 * 17408, 5120), (5120, 17408))
N_LAYERS = 64
