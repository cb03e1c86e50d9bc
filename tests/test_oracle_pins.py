"""Pins for the CPU oracle: checks against facts the pages and the mathematics fix.

None of these re-types the oracle's own loops. They use the pages' worked
example, closed forms, invariants, an independent numpy unpack + library
matmul on tiny shapes, and the page's plane-trick description executed on
32-bit words.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import pq2_synth as synth
from conftest import golden

G = 128


def np_unpack_codes(codes: np.ndarray, K: int) -> np.ndarray:
    """Independent unpack via numpy's bit unpacking: uint8 [N][K/4] -> codes [N][K]."""
    bits = np.unpackbits(codes[..., None], axis=-1, bitorder="little")  # [N][K/4][8]
    c = bits[..., 0::2].astype(np.int64) + 2 * bits[..., 1::2].astype(np.int64)
    return c.reshape(codes.shape[0], K)


def dense_dots(q: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Brute force group dots: unpack to ternary, one int64 matmul per group."""
    M, K = q.shape
    N = codes.shape[0]
    w = np_unpack_codes(codes, K) - 1
    Gn = K // G
    D = np.empty((M, N, Gn), np.int64)
    for g in range(Gn):
        D[:, :, g] = q[:, g * G:(g + 1) * G].astype(np.int64) @ w[:, g * G:(g + 1) * G].T
    return D


# ---------------------------------------------------------------- weight decode

def test_worked_example_decode():
    fx = golden("decode_worked_example.txt")
    codes = fx["codes"]
    # selector construction: code s in nibble s
    sel = sum(c << (4 * s) for s, c in enumerate(codes))
    assert sel == fx["selector"][0]
    lut = fx["lut"][0].to_bytes(4, "little")
    assert [lut[c] for c in codes] == fx["selected_bytes"]
    signed = [b - 256 if b >= 128 else b for b in fx["selected_bytes"]]
    assert signed == fx["weights"]
    # the byte whose bit fields 2s..2s+1 hold these codes decodes to the weights
    byte = sum(c << (2 * s) for s, c in enumerate(codes))
    row = np.full((1, 32), 0x55, np.uint8)  # all codes 1 (weight 0)
    row[0, 5] = byte
    got = [oracle.weight(row, 128, 0, 4 * 5 + s) for s in range(4)]
    assert got == fx["weights"]


def test_code3_and_lut_agree():
    """The lookup table maps every 2-bit code c to the signed byte c-1 (code 3 -> +2)."""
    fx = golden("decode_worked_example.txt")
    lut = fx["lut"][0].to_bytes(4, "little")
    for c in range(4):
        b = lut[c]
        want = b - 256 if b >= 128 else b
        row = np.zeros((1, 32), np.uint8)
        row[0, 0] = c << 6                # column 3 of byte 0
        assert oracle.weight(row, 128, 0, 3) == want


def test_one_hot_reads_every_weight():
    """With q = e_k, the group dot returns the weight of column k (bit layout pin)."""
    rng = np.random.default_rng(5)
    K, N = 256, 3
    c = rng.integers(0, 3, size=(N, K)).astype(np.uint8)
    codes = synth.pack_codes(c)
    q = np.eye(K, dtype=np.int8)           # M = K rows, row k is e_k
    D = oracle.group_dots(q, codes)       # [K][N][G]
    for k in range(K):
        assert (D[k, :, k // G] == c[:, k].astype(np.int32) - 1).all()
        other = [g for g in range(K // G) if g != k // G]
        assert (D[k][:, other] == 0).all()


# ---------------------------------------------------------------- group dots

@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (1, 7, 128), (3, 33, 256), (16, 5, 640),
                                   (2, 1, 128)])
def test_group_dots_bruteforce(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    codes = synth.draw_codes(N, K, rng)
    np.testing.assert_array_equal(oracle.group_dots(q, codes), dense_dots(q, codes))


def test_group_dots_bruteforce_tiny_workload():
    wl = synth.tiny()
    w = synth.weights(wl.n, wl.k, 0)
    x = synth.activations(wl.m, wl.k, 0)
    q, s, t = oracle.quantize(x)
    np.testing.assert_array_equal(oracle.group_dots(q, w.codes), dense_dots(q, w.codes))


def test_offset_identity():
    """dot(codes, q) - sum(q) == dot(codes - 1, q) per group, with t from the quantiser."""
    rng = np.random.default_rng(11)
    M, N, K = 4, 9, 384
    x = synth.draw_x(M, K, rng, outlier_frac=0.01)
    q, s, t = oracle.quantize(x)
    codes = synth.draw_codes(N, K, rng)
    c = np_unpack_codes(codes, K)
    raw = np.einsum("mgk,ngk->mng", q.reshape(M, -1, G).astype(np.int64),
                    c.reshape(N, -1, G))
    np.testing.assert_array_equal(oracle.group_dots(q, codes), raw - t[:, None, :])


@pytest.mark.parametrize("code,expect", [(1, "zero"), (2, "t"), (0, "-t")])
def test_constant_code_special_cases(code, expect):
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 256
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    t = q.reshape(M, -1, G).astype(np.int64).sum(-1)
    codes = synth.pack_codes(np.full((N, K), code, np.uint8))
    D = oracle.group_dots(q, codes)
    want = {"zero": 0 * t, "t": t, "-t": -t}[expect]
    np.testing.assert_array_equal(D, np.broadcast_to(want[:, None, :], D.shape))


def test_extreme_group_dot():
    q = np.full((1, 128), 127, np.int8)
    codes = synth.pack_codes(np.full((1, 128), 2, np.uint8))
    assert oracle.group_dots(q, codes)[0, 0, 0] == 16256
    q = np.full((1, 128), -127, np.int8)
    assert oracle.group_dots(q, codes)[0, 0, 0] == -16256
    codes = synth.pack_codes(np.zeros((1, 128), np.uint8))
    assert oracle.group_dots(q, codes)[0, 0, 0] == 16256


# ---------------------------------------------------------------- plane order

def test_plane_order_is_the_page_layout():
    """Position 32*s+b of each group holds natural element 4*b+s; checked element by element."""
    rng = np.random.default_rng(1)
    M, K = 2, 384
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qp = oracle.plane_order(q)
    for g in range(K // G):
        for s in range(4):
            for b in range(32):
                assert (qp[:, g * G + 32 * s + b] == q[:, g * G + 4 * b + s]).all()
    # bijection: the permutation applied to distinct labels yields all labels once
    lab = np.arange(K, dtype=np.int64).reshape(1, K) % 256 - 128
    assert sorted(oracle.plane_order(lab.astype(np.int8))[0].tolist()) == sorted(
        lab[0].astype(np.int8).tolist())


def test_plane_trick_matches_natural_dot():
    """Execute the page's plane trick on 32-bit words: plane s of word j is
    (w >> 2s) & 0x03030303 against plane-q word 8s+j of the group; subtract sum(q)."""
    fx = golden("plane_layout.txt")
    mask = np.uint32(fx["plane_mask"][0])
    rng = np.random.default_rng(2)
    M, N, K = 3, 6, 512
    x = synth.draw_x(M, K, rng)
    q, s, t = oracle.quantize(x)
    qp = oracle.plane_order(q)
    codes = synth.draw_codes(N, K, rng)
    Gn = K // G
    words = codes.view("<u4").reshape(N, Gn, 8)
    for m in range(M):
        qw = qp[m].reshape(Gn, 128)
        for n in range(N):
            for g in range(Gn):
                acc = 0
                for j in range(8):
                    w = words[n, g, j]
                    for sp in range(4):
                        planes = np.array([(w >> np.uint32(2 * sp)) & mask],
                                          dtype="<u4").view(np.uint8)
                        qb = qw[g, 32 * sp + 4 * j: 32 * sp + 4 * j + 4].astype(np.int64)
                        acc += int((planes.astype(np.int64) * qb).sum())
                assert acc - int(t[m, g]) == oracle.group_dots(q[m:m + 1], codes[n:n + 1])[0, 0, g]


# ---------------------------------------------------------------- quantiser

def test_quantize_hand_case():
    """amax = 127 gives s = 1 exactly, so q is x rounded half to even."""
    x = np.zeros((1, 128), np.float32)
    vals = [0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5, 127.0, -126.5, 0.49999997]
    x[0, :len(vals)] = vals
    q, s, t = oracle.quantize(x)
    assert s[0, 0] == np.float32(1.0)
    assert q[0, :len(vals)].tolist() == [0, 2, 2, -2, 126, 0, 4, 127, -126, 0]
    assert t[0, 0] == sum([0, 2, 2, -2, 126, 0, 4, 127, -126, 0])


def test_quantize_zero_and_underflow_groups():
    x = np.zeros((2, 256), np.float32)
    x[1, 128] = np.float32(1.4e-45)       # smallest subnormal: amax/127 underflows to 0
    x[1, 129] = -np.float32(1.4e-45)
    q, s, t = oracle.quantize(x)
    assert (q == 0).all() and (s == 0).all() and (t == 0).all()


def test_quantize_subnormal_scale_clamps():
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = np.float32(3e-39)           # s is subnormal; quotients may exceed 127
    x[0, 1:64] = np.float32(2.9e-39)
    x[0, 64:] = -np.float32(1e-39)
    q, s, t = oracle.quantize(x)
    assert 0 < s[0, 0] < np.finfo(np.float32).tiny
    assert np.abs(q).max() <= 127 and q[0, 0] == 127
    assert t[0, 0] == int(q.astype(np.int64).sum())


@pytest.mark.parametrize("outliers", [0.0, 0.01])
def test_quantize_invariants(outliers):
    rng = np.random.default_rng(7)
    M, K = 5, 1024
    x = synth.draw_x(M, K, rng, outlier_frac=outliers)
    q, s, t = oracle.quantize(x)
    Gn = K // G
    xg = x.reshape(M, Gn, G)
    qg = q.reshape(M, Gn, G).astype(np.int64)
    assert np.abs(qg).max() <= 127
    np.testing.assert_array_equal(qg.sum(-1), t)
    # the element attaining amax maps to +-127
    arg = np.abs(xg).argmax(-1)
    top = np.take_along_axis(qg, arg[..., None], -1)[..., 0]
    sign = np.sign(np.take_along_axis(xg, arg[..., None], -1)[..., 0])
    np.testing.assert_array_equal(top, 127 * sign)
    # odd symmetry
    qn, sn, tn = oracle.quantize(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)
    np.testing.assert_array_equal(tn, -t)
    # power-of-two scaling leaves q and t unchanged and scales s exactly
    q2, s2, t2 = oracle.quantize(x * np.float32(8.0))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s * np.float32(8.0))
    # exact-rational checks on a few groups: s is amax/127 correctly rounded, and
    # q is within half a unit (plus one float32 rounding of the quotient) of x/s
    for m in range(2):
        for g in range(2):
            amax = Fraction(float(np.abs(xg[m, g]).max()))
            sv = Fraction(float(s[m, g]))
            ulp = Fraction(float(np.spacing(s[m, g])))
            assert abs(sv - amax / 127) <= ulp / 2
            for i in range(G):
                r = Fraction(float(xg[m, g, i])) / sv
                assert abs(Fraction(int(qg[m, g, i])) - r) <= Fraction(1, 2) + Fraction(1, 1 << 16)


def test_quantize_rounds_ties_to_even_at_scale():
    """Quotients exactly halfway: with amax = 127*2^e the scale is 2^e and x = (k+1/2)*2^e."""
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 127 * 0.25
    x[0, 1:7] = np.array([0.5, 1.5, 2.5, 3.5, -4.5, -5.5], np.float32) * 0.25
    q, s, t = oracle.quantize(x)
    assert s[0, 0] == np.float32(0.25)
    assert q[0, :7].tolist() == [127, 0, 2, 2, 4, -4, -6]


# ---------------------------------------------------------------- epilogue

def test_half_to_double_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits[::37]])
    r = ref[::37]
    both_nan = np.isnan(got) & np.isnan(r)
    assert ((got == r) | both_nan).all()
    for b in [0x0001, 0x03ff, 0x0400, 0x3c00, 0x7bff, 0x8001, 0xfbff, 0x2e66, 0x7c00, 0xfc00]:
        v = oracle.half_to_double(b)
        assert v == float(np.uint16(b).view(np.float16))


def test_epilogue_one_hot_scales_give_group_dot():
    rng = np.random.default_rng(4)
    M, N, K = 3, 5, 512
    x = synth.draw_x(M, K, rng)
    q, s, t = oracle.quantize(x)
    codes = synth.draw_codes(N, K, rng)
    D = dense_dots(q, codes)
    ones_s = np.ones_like(s)
    for g0 in range(K // G):
        ws = np.zeros((N, K // G), np.float16)
        ws[:, g0] = 1.0
        y, tabs = oracle.gemm_f64(q, ones_s, codes, ws)
        np.testing.assert_array_equal(y, D[:, :, g0].astype(np.float64))
        np.testing.assert_array_equal(tabs, np.abs(D[:, :, g0]).astype(np.float64))
    y, _ = oracle.gemm_f64(q, ones_s, codes, np.ones((N, K // G), np.float16))
    np.testing.assert_array_equal(y, D.sum(-1).astype(np.float64))


def test_epilogue_distinct_scales_pick_the_right_indices():
    """Scale of (m, g) and (n, g) as distinct powers of two: a transposed or
    shifted scale index changes the result."""
    rng = np.random.default_rng(8)
    M, N, K = 2, 3, 384
    Gn = K // G
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    codes = synth.draw_codes(N, K, rng)
    D = dense_dots(q, codes)
    s = np.array([[2.0 ** (m * Gn + g) for g in range(Gn)] for m in range(M)], np.float32)
    ws = np.array([[2.0 ** -(n * Gn + g + 1) for g in range(Gn)] for n in range(N)], np.float16)
    y, _ = oracle.gemm_f64(q, s, codes, ws)
    for m in range(M):
        for n in range(N):
            want = sum(int(D[m, n, g]) * 2.0 ** (m * Gn + g) * 2.0 ** -(n * Gn + g + 1)
                       for g in range(Gn))
            assert y[m, n] == want


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (4, 17, 640), (16, 8, 1024)])
def test_gemm_matches_dense_dequantized_matmul(M, N, K):
    """Dequantise both operands to dense float64 and use one library matmul."""
    rng = np.random.default_rng(M + N + K)
    x = synth.draw_x(M, K, rng, outlier_frac=0.01)
    q, s, t = oracle.quantize(x)
    w = synth.weights(N, K, 99)
    a = q.astype(np.float64) * np.repeat(s.astype(np.float64), G, axis=1)
    b = (np_unpack_codes(w.codes, K) - 1).astype(np.float64) * np.repeat(
        w.wscale.astype(np.float64), G, axis=1)
    y_dense = a @ b.T
    y, tabs = oracle.gemm_f64(q, s, w.codes, w.wscale)
    assert np.all(np.abs(y - y_dense) <= 1e-12 * np.maximum(tabs, 1e-300))


def test_sampled_entry_points_agree_with_full():
    rng = np.random.default_rng(9)
    M, N, K = 5, 40, 384
    x = synth.draw_x(M, K, rng)
    q, s, t = oracle.quantize(x)
    w = synth.weights(N, K, 5)
    y, tabs = oracle.gemm_f64(q, s, w.codes, w.wscale)
    D = oracle.group_dots(q, w.codes)
    mm = rng.integers(0, M, 30)
    nn = rng.integers(0, N, 30)
    ys, ts = oracle.gemm_f64_sampled(q, s, w.codes, w.wscale, mm, nn)
    np.testing.assert_array_equal(ys, y[mm, nn])
    np.testing.assert_array_equal(ts, tabs[mm, nn])
    np.testing.assert_array_equal(oracle.group_dots_sampled(q, w.codes, mm, nn), D[mm, nn])


def test_tolerance_measure_catches_a_dropped_term():
    """A result missing one group's term fails the 1e-5 bound; fp32 rounding passes it."""
    rng = np.random.default_rng(10)
    M, N, K = 2, 16, 17408
    x = synth.draw_x(M, K, rng)
    q, s, t = oracle.quantize(x)
    w = synth.weights(N, K, 6)
    y, tabs = oracle.gemm_f64(q, s, w.codes, w.wscale)
    # float32 evaluation in a different order stays within the bound
    D = oracle.group_dots(q, w.codes).astype(np.float32)
    terms = D * (s[:, None, :] * w.wscale.astype(np.float32)[None, :, :])
    y32 = np.zeros((M, N), np.float32)
    for g in reversed(range(K // G)):
        y32 += terms[:, :, g]
    assert oracle.rel_err(y32, y, tabs) < 1e-5
    y_bad = y - (D[:, :, 3].astype(np.float64) * s[:, None, 3] *
                 w.wscale[None, :, 3].astype(np.float64))
    assert oracle.rel_err(y_bad, y, tabs) > 1e-5


def test_quantize_divides_rather_than_multiplies_by_reciprocal():
    """amax = 127 * 1070/1024 gives s = 1070/1024 exactly, and x = (k + 1/2) * s are
    exact ties under a correctly rounded division (-> even). fl(1/s) * x lands off the
    tie for k = 62 and 126, so a reciprocal multiply (or x * (127/amax)) fails here."""
    sv = 1070.0 / 1024.0
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 127 * sv
    ks = np.arange(0, 127)
    x[0, 1:128] = ((ks + 0.5) * sv).astype(np.float32)
    assert np.all(x[0, 1:128].astype(np.float64) == (ks + 0.5) * sv)   # exact ties
    q, s, t = oracle.quantize(x)
    assert s[0, 0] == np.float32(sv)
    want = [int(k + 1) if (k % 2) else int(k) for k in ks]   # ties to even
    assert q[0, 1:128].tolist() == want
    recip = np.rint(x[0, 1:128] * (np.float32(1) / np.float32(sv))).astype(int).tolist()
    assert recip != want                   # the fixture really separates the two readings
