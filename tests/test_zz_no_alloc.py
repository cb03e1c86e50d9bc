"""pq2_gemm_noalloc through the C ABI: y bit-identical to pq2_gemm given the
workspace pq2_gemm_workspace_bytes asks for, and within tolerance of the
oracle, on two calls in a row with the second one smaller (split-K shapes
whose partial sums live in the library's scratch, and a shape that needs
none); a shape whose partial sums exceed the scratch is rejected with
PQ2_ERR_SCRATCH before anything is enqueued."""

import numpy as np
import pytest
import torch

import oracle
import pq2_synth as synth

pytestmark = pytest.mark.gpu

G = 128
TOL = 1e-5
ERR_SCRATCH = 6


@pytest.fixture(scope="module")
def pq2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_pq2_w2a8_amd as lib
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def problem(pq2, M, N, K, seed):
    x = synth.activations(M, K, seed, outlier_frac=0.01)
    w = synth.weights(N, K, synth.matrix_seed(seed))
    q, s, t = pq2.quantize_act(dev(x))
    return x, w, q, s, t, dev(w.codes), dev(w.wscale_bits.view(np.int16))


def c_noalloc(pq2, q, s, t, cd, wd, y):
    M, K = q.shape
    N = cd.shape[0]
    return pq2.lib.pq2_gemm_noalloc(q.data_ptr(), s.data_ptr(), t.data_ptr(), cd.data_ptr(),
                                    wd.data_ptr(), y.data_ptr(), M, N, K,
                                    torch.cuda.current_stream().cuda_stream)


def c_gemm(pq2, q, s, t, cd, wd, y, work, nbytes):
    M, K = q.shape
    N = cd.shape[0]
    return pq2.lib.pq2_gemm(q.data_ptr(), s.data_ptr(), t.data_ptr(), cd.data_ptr(),
                            wd.data_ptr(), y.data_ptr(), M, N, K,
                            work.data_ptr() if work is not None else None, nbytes,
                            torch.cuda.current_stream().cuda_stream)


# (large, then smaller): the ring plan in 3 chunks; 64 then 40 rows in token
# tiles (9 and 3 chunks); a GEMV shape with no split
PAIRS = [((16, 5120, 17408), (4, 700, 17408)),
         ((64, 5120, 17408), (40, 300, 6144)),
         ((1, 5120, 6144), (1, 256, 512))]


@pytest.mark.parametrize("big,small", PAIRS, ids=["ring", "token_tiles", "gemv"])
def test_noalloc_matches_pq2_gemm(pq2, big, small):
    probs = []
    for i, (M, N, K) in enumerate((big, small)):
        need = pq2.gemm_workspace_bytes(M, N, K)
        print(f"noalloc M={M} N={N} K={K} workspace={need} path={pq2.gemm_kernel_path(M, N, K)}",
              flush=True)
        assert need <= pq2.NOALLOC_SCRATCH_BYTES
        probs.append(problem(pq2, M, N, K, 700 + 10 * i + M))
    ys = []
    for (x, w, q, s, t, cd, wd) in probs:          # two calls in a row, no sync between
        y = torch.full((q.shape[0], cd.shape[0]), float("nan"), device="cuda")
        assert c_noalloc(pq2, q, s, t, cd, wd, y) == 0
        ys.append(y)
    for (x, w, q, s, t, cd, wd), y in zip(probs, ys):
        M, K = q.shape
        N = cd.shape[0]
        need = pq2.gemm_workspace_bytes(M, N, K)
        work = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        yr = torch.empty((M, N), dtype=torch.float32, device="cuda")
        assert c_gemm(pq2, q, s, t, cd, wd, yr, work, need) == 0
        yn = host(y)
        np.testing.assert_array_equal(yn, host(yr))
        yo, tabs, _ = oracle.forward(x, w.codes, w.wscale)
        assert oracle.rel_err(yn, yo, tabs) < TOL


def test_noalloc_rejects_scratch_overflow(pq2):
    M, N, K = 64, 7800, 17408
    need = pq2.gemm_workspace_bytes(M, N, K)
    print(f"noalloc overflow M={M} N={N} K={K} workspace={need}", flush=True)
    assert need > pq2.NOALLOC_SCRATCH_BYTES
    x, w, q, s, t, cd, wd = problem(pq2, M, N, K, 790)
    y = torch.full((M, N), float("nan"), device="cuda")
    torch.cuda.synchronize()
    assert c_noalloc(pq2, q, s, t, cd, wd, y) == ERR_SCRATCH
    assert np.isnan(host(y)).all()          # nothing was enqueued
    with pytest.raises(pq2.PQ2Error):
        pq2.pq2_gemm_noalloc(q, s, t, cd, wd, y)
