"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer work (q, s bits, t, per-group dots) must match bit for bit. The float32
output y must satisfy max |y - y*| / sum_g |term_g| < 1e-5, with y* the
oracle's float64 result; with unit or one-hot scales every partial sum is an
integer below 2^24, so y must then match exactly.
"""

import numpy as np
import pytest
import torch

import oracle
import pq2_synth as synth

pytestmark = pytest.mark.gpu

G = 128
TOL = 1e-5


@pytest.fixture(scope="module")
def pq2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_pq2_w2a8_amd as lib   # raises if libpq2.so is missing
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def plane(q):
    """Natural -> plane order (position 32*s+b <- element 4*b+s), numpy reshape."""
    M, K = q.shape
    return np.ascontiguousarray(q.reshape(M, K // G, 32, 4).transpose(0, 1, 3, 2).reshape(M, K))


def rand_q(M, K, rng):
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    t = q.reshape(M, -1, G).astype(np.int32).sum(-1).astype(np.int32)
    return q, t


def gpu_dots(pq2, qn, t, codes, path):
    M, K = qn.shape
    N = codes.shape[0]
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(dev(plane(qn)), dev(t), dev(codes), d, path=path)
    return host(d)


def gpu_gemm(pq2, qp, s, t, codes, ws):
    M = qp.shape[0]
    N = codes.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(dev(qp), dev(s), dev(t), dev(codes), dev(ws.view(np.int16)), y)
    return host(y)


# ---------------------------------------------------------------- K1 quantise

def edge_rows():
    x = np.zeros((4, 640), np.float32)
    x[0, 0:10] = [0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5, 127.0, -126.5, 0.49999997]   # s = 1
    x[0, 128] = 1.4e-45                      # underflowing scale -> zeros
    x[0, 256:384] = np.float32(3e-39)        # subnormal scale
    x[0, 300] = -np.float32(1e-39)
    sv = 1070.0 / 1024.0                     # division vs reciprocal ties
    x[1, 0] = 127 * sv
    x[1, 1:128] = ((np.arange(127) + 0.5) * sv).astype(np.float32)
    x[1, 128:256] = -x[1, 0:128]
    x[2, :] = np.float32(3.0e38) * np.sign(np.sin(np.arange(640)))
    x[3, 128:256] = 1e-20 * np.arange(128, dtype=np.float32)
    return x


def edge_rows_many():
    """The edge rows repeated past 16384 groups (the launch then takes 8 lanes
    per group instead of 32), between rows of random activations."""
    e = edge_rows()
    reps = 16384 // (e.shape[0] * e.shape[1] // 128) + 2
    x = np.tile(e, (reps, 1))
    x[1::5] = synth.activations(x[1::5].shape[0], x.shape[1], 11, outlier_frac=0.01)
    return x


QUANT_CASES = {
    "tiny": lambda: synth.activations(1, 512, 0),
    "decode": lambda: synth.activations(1, 6144, 0),
    "small_outliers": lambda: synth.activations(16, 17408, 0, outlier_frac=0.01),
    "ragged": lambda: synth.activations(3, 640, 5, outlier_frac=0.01),
    "prefill": lambda: synth.activations(4096, 5120, 0),
    "edge": edge_rows,
    "edge_many": edge_rows_many,
    "layouts_boundary": lambda: synth.activations(409, 5120, 3),   # 16360 groups: 32 lanes
    "layouts_boundary_8": lambda: synth.activations(410, 5120, 3), # 16400 groups: 8 lanes
}


@pytest.mark.parametrize("case", list(QUANT_CASES))
def test_quantize_bitexact(pq2, case):
    x = QUANT_CASES[case]()
    print(f"quantize case={case} shape={x.shape}", flush=True)
    q, s, t = pq2.quantize_act(dev(x))
    qo, so, to = oracle.quantize(x)
    np.testing.assert_array_equal(host(q), oracle.plane_order(qo))
    np.testing.assert_array_equal(host(s).view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(host(t), to)


# ---------------------------------------------------------------- exact group dots

def edge_rows_16(dtype):
    """Values a 16-bit activation can hold at the ends of its range."""
    x = np.zeros((3, 384), np.float32)
    if dtype == torch.float16:
        x[0, 0:6] = [6e-8, -6e-8, 65504.0, -65504.0, 1e-5, 0.5]    # subnormal, max, tie-prone
        x[1, 128:256] = np.float32(6e-8) * np.arange(128)         # a group of subnormals
    else:
        x[0, 0:4] = [3.0e38, -3.0e38, 1e-38, 126.5]
        x[1, 128:256] = np.float32(1e-30) * np.arange(128)
    x[2, :] = np.sin(np.arange(384, dtype=np.float32)) * 1000
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("case", ["decode", "small_outliers", "ragged", "edge", "prefill"])
def test_quantize_16bit_bitexact(pq2, dtype, case):
    """bfloat16 / float16 activations: q, s, t bit for bit those the oracle gives
    for the same values widened to float32 (the widening is exact)."""
    print(f"quantize 16-bit {dtype} {case}", flush=True)
    if case == "edge":
        xf = edge_rows_16(dtype)
    else:
        xf = QUANT_CASES[case]()
    x16 = torch.from_numpy(xf).to(dtype)
    xw = x16.float().numpy()                      # exact widening, on the CPU
    q, s, t = pq2.quantize_act(x16.cuda())
    qo, so, to = oracle.quantize(xw)
    np.testing.assert_array_equal(host(q), oracle.plane_order(qo))
    np.testing.assert_array_equal(host(s).view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(host(t), to)


# the last three span several LDS windows of one token row (40960 activations):
# 32 or 2 chunk lanes per row, the windows' offsets in the loads' uniform part
GEMV_SHAPES = [(1, 128), (7, 384), (64, 512), (300, 640), (33, 2048), (130, 5120), (257, 6144),
               (65, 8192), (33, 45056), (5, 42368), (2, 90112)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_group_dots_gemv(pq2, N, K):
    print(f"dots gemv N={N} K={K}", flush=True)
    rng = np.random.default_rng(N * 7 + K)
    qn, t = rand_q(1, K, rng)
    codes = synth.draw_codes(N, K, rng)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, pq2.PATH_GEMV),
                                  oracle.group_dots(qn, codes))


GEMV_TOKEN_SHAPES = [(M, N, K) for M in (2, 3, 4)
                     for (N, K) in ((1, 128), (7, 384), (300, 640), (130, 5120), (257, 6144),
                                    (65, 8320), (33, 17408))]


@pytest.mark.parametrize("M,N,K", GEMV_TOKEN_SHAPES)
def test_group_dots_gemv_tokens(pq2, M, N, K):
    """The dot4 GEMV with 2 to 4 token rows (M = 3 runs as 4 with a padded row);
    K = 8320 and 17408 span several LDS windows."""
    print(f"dots gemv M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 100 + N * 7 + K)
    qn, t = rand_q(M, K, rng)
    codes = synth.draw_codes(N, K, rng)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, pq2.PATH_GEMV),
                                  oracle.group_dots(qn, codes))


SMALL_SHAPES = [(M, N, K) for M in (1, 2, 3, 8, 16) for (N, K) in ((1, 128), (17, 640), (100, 5120))]


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_group_dots_small(pq2, M, N, K):
    print(f"dots small M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 1000 + N + K)
    qn, t = rand_q(M, K, rng)
    codes = synth.draw_codes(N, K, rng, synth.PREFILL_CODES)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, pq2.PATH_SMALL),
                                  oracle.group_dots(qn, codes))


PANEL_SHAPES = [(1, 40, 2048), (2, 7, 2048), (3, 300, 2176), (5, 4100, 2304), (8, 4130, 5120),
                (16, 8200, 2048), (8, 520, 8192), (11, 5000, 3200), (16, 4097, 6144),
                (4, 1030, 17408), (5, 300, 18432), (3, 200, 17536), (16, 700, 17408),
                (9, 5000, 16384), (16, 33, 18432),
                (2, 300, 9344), (3, 100, 9344),   # G = 73: the register-operand variant
                # ring variant: 3 and 12 tokens, N of one tile and one row past a tile,
                # chunks of 6 and 4 groups per wave (K split in two: 7168 = 32 + 24)
                (3, 1000, 5120), (12, 2100, 6144), (7, 16, 2048), (13, 17, 4096),
                (6, 900, 7168),
                # 2 and 4 token tiles; K split so that the M-row panel fits LDS
                (17, 300, 2048), (20, 1000, 5120), (24, 4100, 3200), (32, 700, 17408),
                (33, 500, 2176), (40, 300, 6144), (48, 1030, 16384), (64, 4097, 5120),
                (64, 129, 18432), (57, 33, 2048)]


@pytest.mark.parametrize("M,N,K", PANEL_SHAPES)
def test_group_dots_panel(pq2, M, N, K):
    """The persistent small-batch kernel: odd G (a half-empty last group pair),
    ragged K slices (pairs not a multiple of the wave count), several tiles per
    block with a ragged last tile, N below one tile, K split into chunks (the
    panel of 16 x 17408 bytes does not fit one block's LDS), and 17..64 tokens
    in 2 or 4 token tiles with a partly padded last tile and chunks of 8 groups."""
    print(f"dots panel M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 1000 + N + K + 2)
    qn, t = rand_q(M, K, rng)
    codes = synth.draw_codes(N, K, rng, synth.PREFILL_CODES)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, pq2.PATH_PANEL),
                                  oracle.group_dots(qn, codes))


PREFILL_SHAPES = [(1, 1, 128), (17, 129, 384), (130, 300, 1024), (257, 129, 640), (128, 128, 128),
                  (20, 300, 4096), (130, 1000, 3200)]


@pytest.mark.parametrize("M,N,K", PREFILL_SHAPES)
def test_group_dots_prefill(pq2, M, N, K):
    print(f"dots prefill M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 1000 + N + K + 1)
    qn, t = rand_q(M, K, rng)
    codes = synth.draw_codes(N, K, rng, synth.PREFILL_CODES)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, pq2.PATH_PREFILL),
                                  oracle.group_dots(qn, codes))


@pytest.mark.parametrize("M,N,K", [(4000, 4200, 1024), (4100, 8300, 2048), (4001, 4203, 1024),
                                   (4096, 4100, 1152), (2000, 2100, 2048), (2048, 2100, 1152)])
def test_prefill_large_tiles_sampled(pq2, M, N, K):
    """Shapes with at least two 256 x 128 tiles per CU and G a multiple of 8
    (the first three: the wide tile, ragged in M and N, the last token tile 4
    tokens wide in the second, N odd in the third so y is stored element by
    element), four 128 x 128 tiles per CU (the fourth) or two 64 x 64 tiles
    per CU (the last two): G a multiple of 8 takes the variants whose stages
    arrive by buffer -> LDS copies (scale chunks of 8 groups), G = 9 the
    register-staged ones. Exact sampled group dots, sampled y within
    tolerance, exact y with unit scales."""
    print(f"prefill large tiles M={M} N={N} K={K}", flush=True)
    assert pq2.gemm_kernel_path(M, N, K) == pq2.PATH_PREFILL
    x = synth.activations(M, K, M + K, outlier_frac=0.0)
    w = synth.weights(N, K, synth.matrix_seed(N), synth.PREFILL_CODES)
    qo, so, to = oracle.quantize(x)
    qd, sd, td = dev(oracle.plane_order(qo)), dev(so), dev(to)
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    rng = np.random.default_rng(M + N)
    P = 512
    mm = np.concatenate([rng.integers(0, M, P - 4), [0, M - 1, 0, M - 1]])
    nn = np.concatenate([rng.integers(0, N, P - 4), [0, N - 1, N - 1, 0]])
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(qd, td, cd, d, path=pq2.PATH_PREFILL)
    ds = host(d[torch.from_numpy(mm).cuda(), torch.from_numpy(nn).cuda()])
    del d
    np.testing.assert_array_equal(ds, oracle.group_dots_sampled(qo, w.codes, mm, nn))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(qd, sd, td, cd, wd, y)
    ys, ts = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(host(y)[mm, nn], ys, ts) < TOL
    ones_w = torch.full((N, K // G), 0x3C00, dtype=torch.int16, device="cuda")
    pq2.pq2_gemm(qd, torch.ones_like(sd), td, cd, ones_w, y)
    np.testing.assert_array_equal(host(y)[mm, nn], ds.sum(-1).astype(np.float32))


@pytest.mark.parametrize("path,M", [(1, 1), (1, 4), (2, 5), (3, 20), (4, 7)])
def test_code3_is_plus_two(pq2, path, M):
    """Code 3 is not a PQ2_0 code; both sides decode it as +2."""
    rng = np.random.default_rng(path)
    N, K = 40, 2048 if path == 4 else 256     # the panel kernel needs K >= 2048
    qn, t = rand_q(M, K, rng)
    c = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    codes = synth.pack_codes(c)
    np.testing.assert_array_equal(gpu_dots(pq2, qn, t, codes, path), oracle.group_dots(qn, codes))


@pytest.mark.parametrize("path,M", [(1, 1), (1, 3), (2, 16), (3, 130), (4, 16)])
def test_extreme_dots(pq2, path, M):
    """q = +-127 everywhere with codes 2 or 0: |D| = 16256, the int32 extreme of a group."""
    N, K = 20, 2048 if path == 4 else 384
    qn = np.full((M, K), 127, np.int8)
    qn[::2] = -127
    t = qn.reshape(M, -1, G).astype(np.int32).sum(-1).astype(np.int32)
    c = np.zeros((N, K), np.uint8)
    c[::2] = 2
    codes = synth.pack_codes(c)
    d = gpu_dots(pq2, qn, t, codes, path)
    np.testing.assert_array_equal(d, oracle.group_dots(qn, codes))
    assert np.abs(d).max() == 16256


# ---------------------------------------------------------------- float32 output

Y_SHAPES = [(1, 256, 512), (1, 100, 640), (2, 300, 1024), (3, 300, 1024), (4, 257, 6144),
            (4, 33, 17408), (5, 129, 384), (16, 64, 5120),
            (17, 200, 640), (128, 256, 1024), (200, 130, 384)]


@pytest.mark.parametrize("M,N,K", Y_SHAPES)
def test_gemm_y_within_tolerance(pq2, M, N, K):
    print(f"gemm y M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, M + N, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N + K))
    y = host(pq2.linear(dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16))))
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(y, yo, tabs) < TOL


PATH_Y = [(1, 3, 300, 1024), (2, 5, 130, 1024), (4, 5, 4100, 2176), (4, 16, 8200, 2048),
          (4, 8, 300, 8192), (4, 16, 5000, 7168), (4, 5, 700, 17408), (4, 16, 1000, 17408),
          (4, 12, 5120, 18432), (4, 1, 33, 2048), (3, 16, 130, 640), (3, 40, 700, 5120),
          (3, 200, 520, 2048), (4, 17, 300, 2048), (4, 32, 1000, 5120), (4, 48, 700, 17408),
          (4, 64, 4100, 6144), (1, 1, 33, 45056), (1, 1, 70, 42368)]


@pytest.mark.parametrize("path,M,N,K", PATH_Y)
def test_gemm_path_y(pq2, path, M, N, K):
    """y through each kernel path (pq2_gemm_path) against the oracle; with unit scales
    every partial sum is an integer below 2^24, so y is then exact."""
    print(f"gemm path={path} M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, M + N + path, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N + K + path))
    qo, so, to = oracle.quantize(x)
    qd, td, cd = dev(oracle.plane_order(qo)), dev(to), dev(w.codes)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm_path(qd, dev(so), td, cd, dev(w.wscale_bits.view(np.int16)), y, path)
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(host(y), yo, tabs) < TOL
    ones_w = torch.full((N, K // G), 0x3C00, dtype=torch.int16, device="cuda")
    pq2.pq2_gemm_path(qd, torch.ones((M, K // G), device="cuda"), td, cd, ones_w, y, path)
    D = oracle.group_dots(qo, w.codes)
    np.testing.assert_array_equal(host(y), D.sum(-1).astype(np.float32))


@pytest.mark.parametrize("K", [2048, 2304])
def test_auto_path_every_m(pq2, K):
    """pq2_gemm's own kernel choice for every M from 1 to 72 on one weight matrix:
    the group dots of the chosen path are exact, y is within tolerance, and the
    sweep crosses every routing boundary (G = 16 takes the ring kernel at 3..16
    tokens, G = 18 the 16-token kernel at 3..7)."""
    N = 520
    w = synth.weights(N, K, synth.matrix_seed(K))
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    x_all = synth.activations(72, K, K, outlier_frac=0.01)
    seen = set()
    for M in range(1, 73):
        path = pq2.gemm_kernel_path(M, N, K)
        seen.add(path)
        print(f"auto M={M} N={N} K={K} path={path}", flush=True)
        x = x_all[:M]
        qo, so, to = oracle.quantize(x)
        qd, td = dev(oracle.plane_order(qo)), dev(to)
        d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
        pq2.pq2_gemm_group_dots(qd, td, cd, d)
        np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        pq2.pq2_gemm(qd, dev(so), td, cd, wd, y)
        yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
        assert oracle.rel_err(host(y), yo, tabs) < TOL
    want = {pq2.PATH_GEMV, pq2.PATH_PANEL, pq2.PATH_PREFILL}
    if K == 2304:
        want.add(pq2.PATH_SMALL)
    assert seen == want


def test_graph_replay_with_spins(pq2):
    """The power-proxy replay's pattern: quantise + pq2_gemm for projections on
    every kernel path (GEMV, panel ring, panel with split K and the caller's
    workspace, token tiles, tiled GEMM and its ring form), each followed by a
    spin kernel, captured in one HIP graph with no eager call before the
    capture. Three replays, with eager work (a larger split-K call on another
    workspace, poisoned outputs) and synchronisations between them: every
    replay's y is within tolerance of the oracle, and identical to the eager
    calls made afterwards."""
    shapes = [(1, 300, 2048), (4, 520, 2048), (16, 300, 17408), (40, 200, 2048), (130, 260, 1024),
              (256, 8192, 1024)]
    cap = torch.cuda.Stream()
    bufs, refs = [], []
    for i, (M, N, K) in enumerate(shapes):
        w = synth.weights(N, K, synth.matrix_seed(500 + i))
        xh = synth.activations(M, K, 500 + i, outlier_frac=0.01)
        yo, tabs, _ = oracle.forward(xh, w.codes, w.wscale)
        refs.append((yo, tabs))
        G_ = K // G
        bufs.append((M, N, K, dev(xh), dev(w.codes), dev(w.wscale_bits.view(np.int16)),
                     torch.empty((M, K), dtype=torch.int8, device="cuda"),
                     torch.empty((M, G_), dtype=torch.float32, device="cuda"),
                     torch.empty((M, G_), dtype=torch.int32, device="cuda"),
                     torch.empty((M, N), dtype=torch.float32, device="cuda")))
    wsz = max(pq2.gemm_workspace_bytes(M, N, K) for (M, N, K) in shapes)
    assert wsz > 0                               # the K = 17408 projection splits K
    work = torch.empty(wsz, dtype=torch.uint8, device="cuda")

    def step():
        for (M, N, K, x, cd, wd, q, s, t, y) in bufs:
            pq2.pq2_quantize_act(x, q, s, t, stream=cap)
            pq2.pq2_gemm(q, s, t, cd, wd, y, workspace=work, stream=cap)
            torch.cuda._sleep(1000)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    # a larger split-K problem, eager, on a workspace of its own
    wb = synth.weights(2048, 17408, synth.matrix_seed(599))
    qb, sb, tb = pq2.quantize_act(dev(synth.activations(16, 17408, 599)))
    cb, wbd = dev(wb.codes), dev(wb.wscale_bits.view(np.int16))
    yb = torch.empty((16, 2048), dtype=torch.float32, device="cuda")
    outs = []
    for rep in range(3):
        for b in bufs:                           # eager work between replays
            b[-1].fill_(float("nan"))
        pq2.pq2_gemm(qb, sb, tb, cb, wbd, yb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        outs.append([host(b[-1]).copy() for b in bufs])
        for i, b in enumerate(bufs):
            print(f"graph replay {rep} shape {shapes[i]}", flush=True)
            assert oracle.rel_err(outs[-1][i], *refs[i]) < TOL
            np.testing.assert_array_equal(outs[-1][i], outs[0][i])
    with torch.cuda.stream(cap):
        step()
    torch.cuda.synchronize()
    for i, b in enumerate(bufs):
        np.testing.assert_array_equal(host(b[-1]), outs[0][i])


BF16_OUT = [(1, 300, 2048), (2, 5120, 6144), (4, 520, 2048), (5, 70, 2304), (16, 300, 17408),
            (40, 200, 2048), (130, 260, 1024), (256, 8192, 1024), (300, 129, 640)]


def bf16_half_ulp(v):
    """Half a bfloat16 ulp at magnitude v (8 significand bits; v > 0), float64."""
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


@pytest.mark.parametrize("M,N,K", BF16_OUT)
def test_gemm_bf16_output(pq2, M, N, K):
    """pq2_gemm_bf16 on every kernel path (GEMV, 16-token kernel, panel with and
    without split K, token tiles, tiled GEMM and its ring form), against the
    oracle: |y - y*| <= half a bfloat16 ulp at |y*| + the float32 bound, plus
    the float32 bound itself (1e-5 of sum_g |term_g|). Also, as the header
    states, y is exactly pq2_gemm's float32 y rounded to nearest-even."""
    print(f"gemm bf16 out M={M} N={N} K={K} path={pq2.gemm_kernel_path(M, N, K)}", flush=True)
    x = synth.activations(M, K, M + N + K, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N + 2 * K))
    q, s, t = pq2.quantize_act(dev(x))
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    pq2.pq2_gemm(q, s, t, cd, wd, y32)
    pq2.pq2_gemm(q, s, t, cd, wd, y16)
    yb = host(y16.float()).astype(np.float64)
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    f32_bound = TOL * tabs
    bound = bf16_half_ulp(np.abs(yo) + f32_bound) + f32_bound
    over = np.abs(yb - yo) - bound
    assert (over <= 0).all(), f"worst excess {over.max():.3g} at {np.unravel_index(over.argmax(), over.shape)}"
    ref = y32.cpu().to(torch.bfloat16).view(torch.int16).numpy()   # RNE on the CPU
    np.testing.assert_array_equal(host(y16.view(torch.int16)), ref)


def random_shapes(seed, count=24, budget=1.5e9):
    """Log-uniform M in [1, 300], N in [1, 3000], K = 128 g with g in [1, 160],
    at most `budget` multiply-adds (the oracle's share), from a fixed seed."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        M = int(np.exp(rng.uniform(0, np.log(300))))
        N = int(np.exp(rng.uniform(0, np.log(3000))))
        K = 128 * int(rng.integers(1, 161))
        if M * N * K <= budget:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", random_shapes(11))
def test_random_shapes_auto_path(pq2, M, N, K):
    """Seeded random shapes (single weight rows, single tokens, K up to 20480,
    nothing a multiple of any tile) through pq2_gemm's own kernel choice: exact
    group dots and y within tolerance."""
    print(f"random M={M} N={N} K={K} path={pq2.gemm_kernel_path(M, N, K)}", flush=True)
    x = synth.activations(M, K, M * 7 + N, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N * 3 + K))
    qo, so, to = oracle.quantize(x)
    qd, td, cd = dev(oracle.plane_order(qo)), dev(to), dev(w.codes)
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(qd, td, cd, d)
    np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(qd, dev(so), td, cd, dev(w.wscale_bits.view(np.int16)), y)
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(host(y), yo, tabs) < TOL


def random_gemv_shapes(seed, count=16, budget=2e8):
    """One or two token rows: log-uniform N in [1, 40000], K = 128 g with g in
    [1, 512] (up to two LDS windows of one row), at most `budget` multiply-adds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        M = int(rng.integers(1, 3))
        N = int(np.exp(rng.uniform(0, np.log(40000))))
        K = 128 * int(rng.integers(1, 513))
        if M * N * K <= budget:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", random_gemv_shapes(23))
def test_random_gemv_shapes(pq2, M, N, K):
    """Seeded random one- and two-row shapes through pq2_gemm's own kernel choice
    (every GEMV launch plan: persistent and windowed, one block or two per CU,
    ragged row groups): exact group dots, y within tolerance, and pq2_linear
    identical to quantise + pq2_gemm."""
    print(f"random gemv M={M} N={N} K={K} path={pq2.gemm_kernel_path(M, N, K)}", flush=True)
    x = synth.activations(M, K, M * 11 + N, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N * 5 + K))
    qo, so, to = oracle.quantize(x)
    qd, td, cd = dev(oracle.plane_order(qo)), dev(to), dev(w.codes)
    wd = dev(w.wscale_bits.view(np.int16))
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(qd, td, cd, d)
    np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(qd, dev(so), td, cd, wd, y)
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(host(y), yo, tabs) < TOL
    y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q, s_, t = pq2.quantize_act(dev(x))
    pq2.pq2_gemm(q, s_, t, cd, wd, y2)
    y3 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_linear(dev(x), cd, wd, y3)
    np.testing.assert_array_equal(host(y3), host(y2))


def test_tiny_workload(pq2):
    wl = synth.tiny()
    w = synth.weights(wl.n, wl.k, 0)
    x = synth.activations(wl.m, wl.k, 0)
    y = host(pq2.linear(dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16))))
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(y, yo, tabs) < TOL
    # scale of the error relative to the output, for the record
    print("tiny: max|y-y*|/max|y*| =", np.abs(y - yo).max() / np.abs(yo).max())


@pytest.mark.parametrize("M", [1, 4, 16, 33])
def test_one_hot_scales_give_exact_dots(pq2, M):
    """s = 1 and ws[n][g] = [g == g0]: y equals the group dot exactly."""
    rng = np.random.default_rng(M)
    N, K = 70, 640
    qn, t = rand_q(M, K, rng)
    codes = synth.draw_codes(N, K, rng)
    D = oracle.group_dots(qn, codes)
    s = np.ones((M, K // G), np.float32)
    for g0 in (0, K // G - 1):
        ws = np.zeros((N, K // G), np.float16)
        ws[:, g0] = 1.0
        y = gpu_gemm(pq2, plane(qn), s, t, codes, ws)
        np.testing.assert_array_equal(y, D[:, :, g0].astype(np.float32))


@pytest.mark.parametrize("M", [1, 3, 16, 40])
def test_degenerate_inputs(pq2, M):
    """All-zero activations and all-zero-weight codes give exactly zero."""
    N, K = 33, 384
    w = synth.weights(N, K, 3)
    y = host(pq2.linear(torch.zeros((M, K), device="cuda"), dev(w.codes),
                        dev(w.wscale_bits.view(np.int16))))
    assert (y == 0).all()
    x = synth.activations(M, K, 4)
    zero_codes = synth.pack_codes(np.ones((N, K), np.uint8))
    y = host(pq2.linear(dev(x), dev(zero_codes), dev(w.wscale_bits.view(np.int16))))
    assert (y == 0).all()


def test_smallest_problem(pq2):
    x = synth.activations(1, 128, 9)
    w = synth.weights(1, 128, 9)
    y = host(pq2.linear(dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16))))
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(y, yo, tabs) < TOL


# ---------------------------------------------------------------- fused quantise + GEMM

LINEAR_SHAPES = ([(M, N, K) for M in (1, 2, 3, 4)
                  for (N, K) in ((1, 128), (300, 640), (257, 6144), (65, 8320), (40, 17408))]
                 + [(M, N, K) for M in (5, 8, 13, 16)
                    for (N, K) in ((300, 2048), (257, 6144), (33, 3072), (40, 17408),
                                   (1000, 5120))])


def linear_reference(pq2, xd, cd, wd, M, N, K, wsz):
    """pq2_quantize_act + pq2_gemm_path on the kernel pq2_linear reports for
    this shape and workspace (same plan, same float arithmetic)."""
    path = pq2.linear_kernel_path(M, N, K, wsz)
    assert path in (pq2.PATH_GEMV, pq2.PATH_PANEL)
    q, s, t = pq2.quantize_act(xd)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    work = torch.empty(max(wsz, 16), dtype=torch.uint8, device="cuda") if wsz else None
    pq2.pq2_gemm_path(q, s, t, cd, wd, y, path, workspace=work)
    return y


@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
def test_linear_equals_quantize_then_gemm(pq2, M, N, K):
    """pq2_linear quantises with the quantiser's own arithmetic, so y is
    bit-identical to pq2_quantize_act + pq2_gemm on the kernel path it takes
    (the dot4 GEMV, or the panel kernel's ring variant with the same K chunks),
    and within tolerance of the oracle."""
    print(f"linear M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, M * 31 + N, outlier_frac=0.01)
    x[0, :128] = 0.0                                   # a zero group (s = 0)
    x[M - 1, 128:256] *= np.float32(1e-39)             # subnormal x, tiny s
    w = synth.weights(N, K, synth.matrix_seed(M + N))
    xd, cd, wd = dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16))
    wsz = pq2.linear_workspace_bytes(M, N, K)
    expect = pq2.PATH_PANEL if (M >= 3 and K % 1024 == 0 and 2048 <= K <= 18432) else pq2.PATH_GEMV
    assert pq2.linear_kernel_path(M, N, K, wsz) == expect
    y1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_linear(xd, cd, wd, y1)
    yh = host(y1)
    np.testing.assert_array_equal(yh, host(linear_reference(pq2, xd, cd, wd, M, N, K, wsz)))
    yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
    assert oracle.rel_err(yh, yo, tabs) < TOL
    # unit scales, through the float path of the same kernel: exact integers
    ones_w = torch.full((N, K // G), 0x3C00, dtype=torch.int16, device="cuda")
    xs = np.repeat(np.float32(127.0) * np.sign(x.reshape(M, -1, G)[:, :, :1]), G, -1)
    xs = np.where(xs == 0, np.float32(127.0), xs).reshape(M, K)   # amax 127 -> s = 1
    xs[:, 1::3] = np.float32(-3.0)
    xs[:, 2::7] = np.float32(2.5)                      # exact ties: the IEEE division decides
    pq2.pq2_linear(dev(xs), cd, ones_w, y1)
    qo, so, to = oracle.quantize(xs)
    assert (so == 1.0).all()
    D = oracle.group_dots(qo, w.codes)
    np.testing.assert_array_equal(host(y1), D.sum(-1).astype(np.float32))


@pytest.mark.parametrize("M,N,K,wsz", [(5, 64, 640, 0), (16, 64, 128, 0), (17, 64, 2048, 0),
                                      (8, 40, 17408, 0), (8, 40, 17408, 1024)])
def test_linear_rejects_shapes_without_fused_kernel(pq2, M, N, K, wsz):
    """5..16 rows need the panel kernel's ring plan (K a multiple of 1024 in
    [2048, 18432], K chunks within the workspace); above 16 rows there is no
    fused kernel: PQ2_ERR_ARG, nothing written."""
    assert pq2.linear_kernel_path(M, N, K, wsz) == -1
    x = dev(synth.activations(M, K, 5))
    w = synth.weights(N, K, 5)
    y = torch.full((M, N), 7.0, device="cuda")
    work = torch.empty(max(wsz, 16), dtype=torch.uint8, device="cuda") if wsz else None
    with pytest.raises(pq2.PQ2Error) as e:
        pq2.pq2_linear(x, dev(w.codes), dev(w.wscale_bits.view(np.int16)), y, workspace=work)
    assert e.value.status == 5    # PQ2_ERR_ARG
    torch.cuda.synchronize()
    assert (host(y) == 7.0).all()


# ---------------------------------------------------------------- full workload sizes

FULL = [
    ("decode_gemv", 1, 5120, 6144, synth.UNIFORM_CODES, 0.0),
    ("layer_qkv", 1, 6144, 5120, synth.UNIFORM_CODES, 0.0),
    ("small_m2_oproj", 2, 5120, 6144, synth.UNIFORM_CODES, 0.01),
    ("small_m4_up", 4, 17408, 5120, synth.UNIFORM_CODES, 0.01),
    ("small_m3_down", 3, 5120, 17408, synth.UNIFORM_CODES, 0.01),
    ("small_m16_up", 16, 17408, 5120, synth.UNIFORM_CODES, 0.01),
    ("small_m8_up", 8, 17408, 5120, synth.UNIFORM_CODES, 0.01),
    ("small_m8_down", 8, 5120, 17408, synth.UNIFORM_CODES, 0.01),
    ("small_m16_down", 16, 5120, 17408, synth.UNIFORM_CODES, 0.01),
    ("tokens_m32_up", 32, 17408, 5120, synth.UNIFORM_CODES, 0.01),
    ("tokens_m64_down", 64, 5120, 17408, synth.UNIFORM_CODES, 0.01),
    ("tokens_m32_oproj", 32, 5120, 6144, synth.UNIFORM_CODES, 0.01),
    ("prefill_m512", 512, 5120, 5120, synth.PREFILL_CODES, 0.0),
    ("prefill_m4096_up", 4096, 17408, 5120, synth.PREFILL_CODES, 0.0),
]


# 17..64 token rows: the panel kernel in token tiles where the tiled GEMM would
# launch fewer than two blocks per CU, else the tiled GEMM.
TOKENS_PATH = {"tokens_m32_up": "PATH_PREFILL", "tokens_m64_down": "PATH_PANEL",
               "tokens_m32_oproj": "PATH_PANEL"}


@pytest.mark.parametrize("M,N,K", [(1, 5120, 6144), (4, 300, 17408), (2, 1000, 2048), (3, 70, 128),
                                   (16, 700, 5120), (8, 300, 17408)])
def test_linear_back_to_back_and_streams(pq2, M, N, K):
    """Calls of pq2_linear issued back to back with no host synchronisation, on
    one stream and alternating over two (each call with its own workspace),
    each give y bit-identical to pq2_quantize_act + pq2_gemm on the same
    kernel path for their own input; so do a larger call (K doubled, four
    rows) and a smaller one after it."""
    print(f"linear back-to-back M={M} N={N} K={K}", flush=True)
    w = synth.weights(N, K, synth.matrix_seed(K + M))
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    wsz = pq2.linear_workspace_bytes(M, N, K)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    xs, ys, works = [], [], []
    for i in range(12):
        x = dev(synth.activations(M, K, 100 + i, outlier_frac=0.01))
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        xs.append(x)
        ys.append(y)
        works.append(torch.empty(max(wsz, 16), dtype=torch.uint8, device="cuda") if wsz else None)
    torch.cuda.synchronize()
    for i in range(6):                       # one stream, back to back
        pq2.pq2_linear(xs[i], cd, wd, ys[i], workspace=works[i])
    for i in range(6, 12):                   # two streams, interleaved
        st = streams[i % 2]
        with torch.cuda.stream(st):
            pq2.pq2_linear(xs[i], cd, wd, ys[i], workspace=works[i], stream=st)
    torch.cuda.synchronize()
    for i in range(12):
        yr = linear_reference(pq2, xs[i], cd, wd, M, N, K, wsz)
        np.testing.assert_array_equal(host(ys[i]), host(yr), err_msg=f"call {i}")
    # a larger call, then a smaller one
    xb = dev(synth.activations(4, 2 * K, 7, outlier_frac=0.01))
    wb = synth.weights(N, 2 * K, synth.matrix_seed(2 * K))
    cb, wbd = dev(wb.codes), dev(wb.wscale_bits.view(np.int16))
    yb = torch.empty((4, N), dtype=torch.float32, device="cuda")
    pq2.pq2_linear(xb, cb, wbd, yb)
    pq2.pq2_linear(xs[0], cd, wd, ys[0], workspace=works[0])
    yr = linear_reference(pq2, xb, cb, wbd, 4, N, 2 * K, pq2.linear_workspace_bytes(4, N, 2 * K))
    np.testing.assert_array_equal(host(yb), host(yr))
    yr = linear_reference(pq2, xs[0], cd, wd, M, N, K, wsz)
    np.testing.assert_array_equal(host(ys[0]), host(yr))


@pytest.mark.parametrize("M,N,K", [(1, 5120, 6144), (2, 17408, 5120), (4, 5120, 17408),
                                   (16, 17408, 5120), (16, 5120, 17408), (8, 6144, 5120)])
def test_linear_full_size_sampled(pq2, M, N, K):
    """pq2_linear at the decode and small-batch sizes against sampled oracle outputs."""
    print(f"linear full M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, 0, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(0))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_linear(dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16)), y)
    yh = host(y)
    qo, so, to = oracle.quantize(x)
    rng = np.random.default_rng(2)
    P = 384
    mm = np.concatenate([rng.integers(0, M, P - 2), [0, M - 1]])
    nn = np.concatenate([rng.integers(0, N, P - 2), [N - 1, 0]])
    ys, ts = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(yh[mm, nn], ys, ts) < TOL


@pytest.mark.parametrize("name,M,N,K,probs,outl", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(pq2, name, M, N, K, probs, outl):
    print(f"full {name} M={M} N={N} K={K}", flush=True)
    if name in TOKENS_PATH:
        assert pq2.gemm_kernel_path(M, N, K) == getattr(pq2, TOKENS_PATH[name])
    x = synth.activations(M, K, 0, outlier_frac=outl)
    w = synth.weights(N, K, synth.matrix_seed(0), probs)
    xd, cd, wd = dev(x), dev(w.codes), dev(w.wscale_bits.view(np.int16))
    q, s, t = pq2.quantize_act(xd)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(q, s, t, cd, wd, y)
    yh = host(y)
    qo, so, to = oracle.quantize(x)
    np.testing.assert_array_equal(host(q), oracle.plane_order(qo))
    rng = np.random.default_rng(1)
    P = 384
    mm = np.concatenate([rng.integers(0, M, P - 2), [0, M - 1]])
    nn = np.concatenate([rng.integers(0, N, P - 2), [N - 1, 0]])
    ys, ts = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(yh[mm, nn], ys, ts) < TOL
    # unit scales: y = sum_g D, an integer below 2^24, exact in any order
    ones_s = torch.ones_like(s)
    ones_w = torch.full((N, K // G), 0x3C00, dtype=torch.int16, device="cuda")
    pq2.pq2_gemm(q, ones_s, t, cd, ones_w, y)
    yu = host(y)
    Ds = oracle.group_dots_sampled(qo, w.codes, mm, nn)
    np.testing.assert_array_equal(yu[mm, nn], Ds.sum(-1).astype(np.float32))


@pytest.mark.parametrize("M,N,K,path", [(1, 5120, 6144, 1), (4, 5120, 6144, 1),
                                        # one row: the persistent plans with several
                                        # batches per wave and a ragged last row group
                                        (1, 34821, 5120, 1), (1, 17411, 5120, 1),
                                        (1, 5123, 17408, 1),
                                        (2, 2048, 17408, 1), (16, 5120, 6144, 2),
                                        (16, 2048, 17408, 2), (256, 1024, 5120, 3),
                                        (16, 4100, 5120, 4), (9, 17408, 8192, 4),
                                        (24, 5120, 5120, 4), (64, 4100, 5120, 4)])
def test_full_row_dots(pq2, M, N, K, path):
    """Exact per-group dots over whole decode-size weight matrices."""
    print(f"full dots M={M} N={N} K={K} path={path}", flush=True)
    x = synth.activations(M, K, 0, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(1))
    qo, so, to = oracle.quantize(x)
    np.testing.assert_array_equal(gpu_dots(pq2, qo, to, w.codes, path),
                                  oracle.group_dots(qo, w.codes))


@pytest.mark.parametrize("M,N,K", [(5, 4100, 5120), (16, 4160, 640), (8, 4160, 17408),
                                   (16, 4096, 16384)])
def test_small_multi_tile_blocks(pq2, M, N, K):
    """Small-batch blocks of 64 (K <= 16384) or 32 weight rows (larger K), with ragged
    last blocks: exact group dots and float outputs."""
    print(f"small multi-tile M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    x = synth.draw_x(M, K, rng, outlier_frac=0.01)
    w = synth.weights(N, K, 7)
    qo, so, to = oracle.quantize(x)
    np.testing.assert_array_equal(gpu_dots(pq2, qo, to, w.codes, pq2.PATH_SMALL),
                                  oracle.group_dots(qo, w.codes))
    y = gpu_gemm(pq2, oracle.plane_order(qo), so, to, w.codes, w.wscale)
    mm = np.repeat(np.arange(M), 40)
    nn = np.concatenate([rng.integers(0, N, 38), [0, N - 1]] * M)
    ys, ts = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(y[mm, nn], ys, ts) < TOL


# Shapes whose code bytes or outputs lie past 2^31 (byte or element offsets), one
# per kernel path: 2.7 GB of codes for the GEMV, 16-token and panel kernels,
# 4.3 G outputs (17 GB of y) for the tiled GEMM.
BIG = [("gemv", 1, (1 << 21) + (1 << 19) + 3, 4096, "PATH_GEMV"),
       ("small", 5, (1 << 21) + (1 << 19) + 3, 4096, "PATH_SMALL"),
       ("panel", 16, (1 << 21) + (1 << 19) + 3, 4096, "PATH_PANEL"),
       ("prefill", 4096, (1 << 20) + 37, 1024, "PATH_PREFILL")]


@pytest.mark.parametrize("name,M,N,K,path", BIG, ids=[b[0] for b in BIG])
def test_offsets_beyond_2_31(pq2, name, M, N, K, path):
    """Random codes, scales and activations drawn on the GPU (seeded); sampled
    outputs, including the last rows and tokens, against the oracle."""
    print(f"big {name} M={M} N={N} K={K}", flush=True)
    G_ = K // G
    gen = torch.Generator(device="cuda").manual_seed(M + N)
    codes = torch.randint(0, 256, (N, K // 4), dtype=torch.uint8, device="cuda", generator=gen)
    wsc = (torch.rand((N, G_), device="cuda", generator=gen) * 0.09 + 0.01).half().view(torch.int16)
    x = torch.randn((M, K), device="cuda", generator=gen)
    q, s, t = pq2.quantize_act(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pid = getattr(pq2, path)
    if path == "PATH_SMALL":
        pq2.pq2_gemm_path(q, s, t, codes, wsc, y, pid)
    else:
        assert pq2.gemm_kernel_path(M, N, K) == pid
        pq2.pq2_gemm(q, s, t, codes, wsc, y)
    rng = np.random.default_rng(5)
    P = 256
    mm = np.concatenate([rng.integers(0, M, P - 4), [M - 1, M - 1, 0, M // 2]])
    nn = np.concatenate([rng.integers(0, N, P - 4), [N - 1, N - 2, N - 1, N - 3]])
    if name == "prefill":       # outputs past 2^31 elements: the upper half of the tokens
        mm[: P // 2] = rng.integers(M // 2, M, P // 2)
    else:                       # code bytes past 2^31: rows from 2^21 on
        nn[: P // 2] = rng.integers(1 << 21, N, P // 2)
    ys = y[torch.from_numpy(mm).cuda(), torch.from_numpy(nn).cuda()].cpu().numpy()
    um, im = np.unique(mm, return_inverse=True)
    un, inn = np.unique(nn, return_inverse=True)
    xs = x[torch.from_numpy(um).cuda()].cpu().numpy()
    cs = codes[torch.from_numpy(un).cuda()].cpu().numpy()
    ws_h = wsc[torch.from_numpy(un).cuda()].cpu().numpy()
    del codes, wsc, x, q, s, t, y
    torch.cuda.empty_cache()
    qo, so, _ = oracle.quantize(xs)
    yo, tabs = oracle.gemm_f64_sampled(qo, so, cs, ws_h, im, inn)
    assert oracle.rel_err(ys, yo, tabs) < TOL


def test_quantize_beyond_2_31(pq2):
    """The quantiser over 2^32 + 2^14 activations (17 GB of x): sampled rows on
    both sides of element 2^31 bit-exact against the oracle."""
    M, K = (1 << 18) + 1, 16384
    print(f"big quantize M={M} K={K}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((M, K), device="cuda", generator=gen)
    q, s, t = pq2.quantize_act(x)
    rows = np.array([0, 1, (1 << 17) - 1, 1 << 17, (1 << 17) + 5, M - 2, M - 1])
    ri = torch.from_numpy(rows).cuda()
    xs, qs, ss, ts = (a[ri].cpu().numpy() for a in (x, q, s, t))
    del x, q, s, t
    torch.cuda.empty_cache()
    qo, so, to = oracle.quantize(xs)
    np.testing.assert_array_equal(qs, oracle.plane_order(qo))
    np.testing.assert_array_equal(ss.view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(ts, to)


# K = 17408 at 3..16 rows: the ring plan in 3 chunks; 40 and 64 rows: the
# token-tiled plan in 3 chunks (one or two chunks exceed LDS or the groups a
# wave can hold)
WS_SHAPES = [(16, 300, 17408), (4, 5120, 17408), (8, 1000, 17408), (12, 2100, 17408),
             (40, 300, 6144), (64, 700, 5120)]


@pytest.mark.parametrize("M,N,K", WS_SHAPES)
def test_workspace_size_and_fallbacks(pq2, M, N, K):
    """The size query matches the plan: pq2_gemm_workspace_bytes is a whole
    number (2..16) of M x N float32 partial-sum planes; a workspace of exactly
    that size gives y bit-identical to a larger one; a byte less, a NULL
    workspace and a misaligned-size buffer take plans with fewer or no K
    chunks (pq2_gemm_kernel_path reports them). Every result within
    tolerance of the oracle, exact dots through the split and unsplit plans."""
    wsz = pq2.gemm_workspace_bytes(M, N, K)
    plane = M * N * 4
    print(f"workspace M={M} N={N} K={K} bytes={wsz} path={pq2.gemm_kernel_path(M, N, K)} "
          f"no-ws path={pq2.gemm_kernel_path(M, N, K, 0)}", flush=True)
    assert wsz % plane == 0 and 2 <= wsz // plane <= 16
    assert pq2.gemm_kernel_path(M, N, K) == pq2.PATH_PANEL
    x = synth.activations(M, K, M + N, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(N + M))
    q, s, t = pq2.quantize_act(dev(x))
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    yo, tabs, (qo, _, _) = oracle.forward(x, w.codes, w.wscale)
    outs = {}
    for name, nbytes in (("exact", wsz), ("larger", 2 * wsz + 48), ("short", wsz - 1),
                         ("one_plane", plane), ("none", None)):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        work = None if nbytes is None else torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        pq2.pq2_gemm(q, s, t, cd, wd, y, workspace=work)
        outs[name] = host(y)
        assert oracle.rel_err(outs[name], yo, tabs) < TOL, name
    np.testing.assert_array_equal(outs["exact"], outs["larger"])
    # the unsplit plan's kernel, read through its exact group dots
    p0 = pq2.gemm_kernel_path(M, N, K, 0)
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(q, t, cd, d, path=p0)
    np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))


SPLIT_SHAPES = [(1100, 17408, 3072), (2100, 8200, 4096), (600, 17300, 5120)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_prefill_tail_split(pq2, M, N, K):
    """The wide prefill tiles (256 weight rows x 128 tokens for the first two
    shapes, x 64 tokens for the third) with the K range of their last round's
    tiles split across blocks (partial sums in the workspace, added in chunk
    order): the size query is a whole number of partial tiles per split tile;
    the tiles computed whole are bit-identical with and without a workspace;
    every sampled output (the split tiles' token rows and their ragged edges
    included) within tolerance of the oracle; with unit scales y is the exact
    sum of the group dots; the allocation-free entry, whose scratch array is
    smaller than these partial sums, gives the result of a workspace of the
    scratch size."""
    wsz = pq2.gemm_workspace_bytes(M, N, K)
    tiles_n = -(-N // 256)
    # the library's tile rule: 128 tokens where those tiles fill 7/8 of a
    # round of two blocks per CU (256 CUs assumed by the rule), else 64
    BM = 128 if tiles_n * -(-M // 128) >= 448 else 64
    tile = BM * 256 * 4
    tiles_m = -(-M // BM)
    T = tiles_n * tiles_m
    P = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    tail = T % P
    print(f"tail split M={M} N={N} K={K} tile={BM} tiles={T} tail={tail} workspace={wsz}",
          flush=True)
    assert pq2.gemm_kernel_path(M, N, K) == pq2.PATH_PREFILL
    assert wsz > 0 and wsz % tile == 0 and (wsz // tile) % tail == 0
    x = synth.activations(M, K, M + K, outlier_frac=0.0)
    w = synth.weights(N, K, synth.matrix_seed(N), synth.PREFILL_CODES)
    qo, so, to = oracle.quantize(x)
    qd, sd, td = dev(oracle.plane_order(qo)), dev(so), dev(to)
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    work = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    ys = torch.empty((M, N), dtype=torch.float32, device="cuda")
    yw = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(qd, sd, td, cd, wd, ys, workspace=work)
    pq2.pq2_gemm(qd, sd, td, cd, wd, yw, workspace=None)
    full_rows = ((T - tail) // tiles_n) * BM           # token panels computed whole
    hs, hw = host(ys), host(yw)
    np.testing.assert_array_equal(hs[:full_rows], hw[:full_rows])
    rng = np.random.default_rng(M + N)
    P_ = 768
    lo = (T - tail) // tiles_n * BM                      # first row of a split tile
    mm = np.concatenate([rng.integers(lo, M, P_ // 2), rng.integers(0, M, P_ // 2 - 4),
                         [lo, M - 1, M - 1, lo]])
    nn = np.concatenate([rng.integers(0, N, P_ - 4), [0, N - 1, 0, N - 1]])
    yo, tabs = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(hs[mm, nn], yo, tabs) < TOL
    assert oracle.rel_err(hw[mm, nn], yo, tabs) < TOL
    ones_w = torch.full((N, K // G), 0x3C00, dtype=torch.int16, device="cuda")
    pq2.pq2_gemm(qd, torch.ones_like(sd), td, cd, ones_w, ys, workspace=work)
    dots = oracle.group_dots_sampled(qo, w.codes, mm, nn)
    np.testing.assert_array_equal(host(ys)[mm, nn], dots.sum(-1).astype(np.float32))
    # scratch smaller than the partial sums: the plan of a workspace of the
    # scratch size (fewer chunks, or none)
    assert wsz > pq2.NOALLOC_SCRATCH_BYTES
    yn = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm_noalloc(qd, sd, td, cd, wd, yn)
    small = torch.empty(pq2.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    pq2.pq2_gemm(qd, sd, td, cd, wd, ys, workspace=small)
    np.testing.assert_array_equal(host(yn), host(ys))
    assert oracle.rel_err(host(yn)[mm, nn], yo, tabs) < TOL


def test_workspace_two_streams(pq2):
    """Split-K calls on two streams at once, each with its own workspace,
    different inputs: y identical to the same calls run one at a time."""
    M, K = 16, 17408
    probs = []
    for N in (700, 300):
        assert pq2.gemm_kernel_path(M, N, K) == pq2.PATH_PANEL
        assert pq2.gemm_workspace_bytes(M, N, K) > 0
        x = synth.activations(M, K, N, outlier_frac=0.01)
        w = synth.weights(N, K, synth.matrix_seed(N))
        q, s, t = pq2.quantize_act(dev(x))
        cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        pq2.pq2_gemm(q, s, t, cd, wd, y)
        yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
        y0 = host(y)
        assert oracle.rel_err(y0, yo, tabs) < TOL
        work = torch.empty(pq2.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        probs.append((q, s, t, cd, wd, work, y0, N))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ya = torch.empty((M, 700), dtype=torch.float32, device="cuda")
    yb = torch.empty((M, 300), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        (q, s, t, cd, wd, work, _, _) = probs[0]
        pq2.pq2_gemm(q, s, t, cd, wd, ya, workspace=work, stream=sa)
        (q, s, t, cd, wd, work, _, _) = probs[1]
        pq2.pq2_gemm(q, s, t, cd, wd, yb, workspace=work, stream=sb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ya), probs[0][6])
    np.testing.assert_array_equal(host(yb), probs[1][6])
