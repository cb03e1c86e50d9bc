"""The five benchmark workloads, each at its own sizes and value distributions,
through pq2_gemm's own kernel choice (with the workspace pq2_gemm_workspace_bytes
asks for), against the CPU oracle on the same seeded inputs.

* tiny (M = 1, N = 256, K = 512): everything in full;
* decode GEMV (1 x 5120 x 6144) and all twelve small-batch points
  (M = 2, 4, 8, 16 on 5120 x 6144, 17408 x 5120, 5120 x 17408, 1 % outliers):
  q/s/t bit for bit, exact int32 group dots over the whole matrix, y within
  the tolerance on every output;
* all six prefill points (M = 128, 512, 4096 on 5120 x 5120 and 17408 x 5120,
  weights -1 / 0 / +1 with p = 0.4 / 0.3 / 0.3): exact dots and y on at least
  4096 sampled outputs that include every 32-row and 32-column tile edge
  (hence every 64- and 128-tile edge), and y in full at 128 rows;
* the 64-layer decode step at M = 1 and 16: the step as the benchmark issues
  it (one stream, gate and up stacked into one matrix, one workspace), with
  sampled outputs of every one of its 256 GEMMs against the oracle.

The tolerance is max |y - y*| / sum_g |term_g| < 1e-5 with y* the oracle's
float64 result (group dots exact, float32 summation of G terms); integer work
must match bit for bit.
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


def run_gemm(pq2, x, w):
    """Quantise on the GPU, then pq2_gemm with the workspace it asks for."""
    M, K = x.shape
    N = w.codes.shape[0]
    q, s, t = pq2.quantize_act(dev(x))
    cd, wd = dev(w.codes), dev(w.wscale_bits.view(np.int16))
    work = torch.empty(max(pq2.gemm_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                       device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pq2.pq2_gemm(q, s, t, cd, wd, y, workspace=work)
    return q, s, t, cd, y


def check_qst(q, s, t, qo, so, to):
    np.testing.assert_array_equal(host(q), oracle.plane_order(qo))
    np.testing.assert_array_equal(host(s).view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(host(t), to)


def test_tiny_config_in_full(pq2):
    wl = synth.tiny()
    x = synth.activations(wl.m, wl.k, 0)
    w = synth.weights(wl.n, wl.k, 0)
    print(f"config tiny M={wl.m} N={wl.n} K={wl.k} path={pq2.gemm_kernel_path(wl.m, wl.n, wl.k)}",
          flush=True)
    q, s, t, cd, y = run_gemm(pq2, x, w)
    qo, so, to = oracle.quantize(x)
    check_qst(q, s, t, qo, so, to)
    d = torch.empty((wl.m, wl.n, wl.k // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(q, t, cd, d)
    np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))
    yo, tabs = oracle.gemm_f64(qo, so, w.codes, w.wscale)
    assert oracle.rel_err(host(y), yo, tabs) < TOL


DECODE_SMALL = [("decode", 1, 5120, 6144, 0.0)] + [
    (f"small_m{m}_n{n}_k{k}", m, n, k, 0.01) for m in synth.SMALL_MS for (n, k) in synth.SMALL_SHAPES]


@pytest.mark.parametrize("name,M,N,K,outl", DECODE_SMALL, ids=[c[0] for c in DECODE_SMALL])
def test_decode_and_small_batch_configs(pq2, name, M, N, K, outl):
    """Whole weight matrix: exact group dots through the kernel pq2_gemm takes,
    and every output of pq2_gemm within tolerance."""
    path = pq2.gemm_kernel_path(M, N, K)
    print(f"config {name} M={M} N={N} K={K} path={path} "
          f"workspace={pq2.gemm_workspace_bytes(M, N, K)}", flush=True)
    x = synth.activations(M, K, 0, outlier_frac=outl)
    w = synth.weights(N, K, synth.matrix_seed(0))
    q, s, t, cd, y = run_gemm(pq2, x, w)
    qo, so, to = oracle.quantize(x)
    check_qst(q, s, t, qo, so, to)
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(q, t, cd, d, path=path)
    np.testing.assert_array_equal(host(d), oracle.group_dots(qo, w.codes))
    del d
    yo, tabs = oracle.gemm_f64(qo, so, w.codes, w.wscale)
    assert oracle.rel_err(host(y), yo, tabs) < TOL


def edge_sample(M, N, rng, uniform=4096):
    """(mm, nn): every 32-row tile edge paired with a random column edge, every
    32-column tile edge paired with a random row edge, the four corners, and
    `uniform` uniformly drawn outputs."""
    def edges(n):
        e = np.concatenate([np.arange(0, n, 32), np.arange(31, n, 32), [n - 1]])
        return np.unique(e)
    re_, ce = edges(M), edges(N)
    mm = np.concatenate([re_, rng.choice(re_, ce.size), [0, 0, M - 1, M - 1],
                         rng.integers(0, M, uniform)])
    nn = np.concatenate([rng.choice(ce, re_.size), ce, [0, N - 1, 0, N - 1],
                         rng.integers(0, N, uniform)])
    return mm.astype(np.int64), nn.astype(np.int64)


PREFILL = [(m, n, k) for m in synth.PREFILL_MS for (n, k) in synth.PREFILL_SHAPES]


@pytest.mark.parametrize("M,N,K", PREFILL, ids=[f"prefill_m{m}_n{n}" for (m, n, _) in PREFILL])
def test_prefill_configs(pq2, M, N, K):
    """Exact group dots and y on sampled outputs covering every tile edge; y in
    full at 128 rows."""
    path = pq2.gemm_kernel_path(M, N, K)
    print(f"config prefill M={M} N={N} K={K} path={path}", flush=True)
    x = synth.activations(M, K, 0)
    w = synth.weights(N, K, synth.matrix_seed(0), synth.PREFILL_CODES)
    q, s, t, cd, y = run_gemm(pq2, x, w)
    qo, so, to = oracle.quantize(x)
    check_qst(q, s, t, qo, so, to)
    mm, nn = edge_sample(M, N, np.random.default_rng(M + N))
    assert mm.size >= 4096
    mi, ni = torch.from_numpy(mm).cuda(), torch.from_numpy(nn).cuda()
    ys = host(y[mi, ni])
    d = torch.empty((M, N, K // G), dtype=torch.int32, device="cuda")
    pq2.pq2_gemm_group_dots(q, t, cd, d, path=path)
    ds = host(d[mi, ni])
    del d
    torch.cuda.empty_cache()
    np.testing.assert_array_equal(ds, oracle.group_dots_sampled(qo, w.codes, mm, nn))
    yo, tabs = oracle.gemm_f64_sampled(qo, so, w.codes, w.wscale, mm, nn)
    assert oracle.rel_err(ys, yo, tabs) < TOL
    if M == 128:
        yo, tabs = oracle.gemm_f64(qo, so, w.codes, w.wscale)
        assert oracle.rel_err(host(y), yo, tabs) < TOL


def layer_weights(gen, n, k):
    """One projection's weights drawn on the GPU: every packed byte is one of the
    81 bytes whose four 2-bit fields are codes 0..2 (four iid uniform codes);
    scales float16(U(0.01, 0.1))."""
    table = torch.from_numpy(synth._VALID_BYTES).cuda()
    codes = table[torch.randint(0, 81, (n, k // 4), generator=gen, device="cuda")]
    ws = (torch.rand((n, k // G), generator=gen, device="cuda") * 0.09 + 0.01).half()
    return codes, ws.view(torch.int16)


@pytest.mark.parametrize("M", [1, 16])
def test_layer64_step(pq2, M):
    """The 64-layer decode step as the benchmark issues it: per layer the
    projections 5120 -> 6144, 6144 -> 5120, gate and up (5120 -> 17408 each)
    stacked into one 34816 x 5120 matrix, and 17408 -> 5120, back to back on
    one stream with one workspace, one token row's small K <= 6144 matrices
    through the one-launch pq2_linear; 32 sampled outputs of every GEMM (the
    last row and column included) against the oracle."""
    print(f"config layer64 M={M}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(M)
    shapes = synth.LAYER_SHAPES
    xs = {k: synth.activations(M, k, k + M) for (_, k) in shapes}
    xd = {k: dev(v) for k, v in xs.items()}
    qst = {k: (torch.empty((M, k), dtype=torch.int8, device="cuda"),
               torch.empty((M, k // G), dtype=torch.float32, device="cuda"),
               torch.empty((M, k // G), dtype=torch.int32, device="cuda")) for (_, k) in shapes}
    wsz = max(pq2.gemm_workspace_bytes(M, n, k) for (n, k) in shapes)
    work = torch.empty(max(wsz, 16), dtype=torch.uint8, device="cuda")
    projs = []
    for layer in range(synth.N_LAYERS):
        for i, (n, k) in enumerate(shapes):
            codes, ws = layer_weights(gen, n, k)
            y = torch.empty((M, n), dtype=torch.float32, device="cuda")
            projs.append((layer, i, n, k, codes, ws, y))
    fused = [M == 1 and k <= 6144 and n * k <= (1 << 25) for (n, k) in shapes]
    torch.cuda.synchronize()
    for (layer, i, n, k, codes, ws, y) in projs:         # the step, no host syncs
        if fused[i]:
            pq2.pq2_linear(xd[k], codes, ws, y)
            continue
        q, s, t = qst[k]
        pq2.pq2_quantize_act(xd[k], q, s, t)
        pq2.pq2_gemm(q, s, t, codes, ws, y, workspace=work)
    torch.cuda.synchronize()
    qso = {k: oracle.quantize(v) for k, v in xs.items()}
    for i, (_, k) in enumerate(shapes):
        if not fused[i]:
            check_qst(*qst[k], *qso[k])
    rng = np.random.default_rng(64 + M)
    worst = 0.0
    for (layer, i, n, k, codes, ws, y) in projs:
        P = 32
        mm = np.concatenate([rng.integers(0, M, P - 2), [M - 1, 0]]).astype(np.int64)
        nn = np.concatenate([rng.integers(0, n, P - 2), [0, n - 1]]).astype(np.int64)
        un, inv = np.unique(nn, return_inverse=True)
        ui = torch.from_numpy(un).cuda()
        cs = host(codes[ui])
        wh = host(ws[ui]).view(np.uint16)
        ys = host(y[torch.from_numpy(mm).cuda(), torch.from_numpy(nn).cuda()])
        qo, so, _ = qso[k]
        yo, tabs = oracle.gemm_f64_sampled(qo, so, cs, wh, mm, inv.astype(np.int64))
        err = oracle.rel_err(ys, yo, tabs)
        worst = max(worst, err)
        assert err < TOL, f"layer {layer} GEMM {i} ({n} x {k}): error {err:.3g}"
    print(f"layer64 M={M}: worst error {worst:.3g} over {len(projs)} GEMMs", flush=True)
