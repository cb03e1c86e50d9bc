"""bench.py's command-line contract and workload definitions, on the CPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr
    assert r.stdout == ""


def test_workloads_cover_the_configurations():
    import bench
    wls = bench.workload_list()
    assert "decode" in wls
    kinds = {kind for kind, _ in wls.values()}
    assert kinds == {"gemm", "layers"}
    # small batches at 2, 4, 8 and 16 rows on the three decode shapes, prefill at
    # 128, 512 and 4096 rows, and the 64-layer step at 1 and 16 rows
    for m in (2, 4, 8, 16):
        for n, k in ((5120, 6144), (17408, 5120), (5120, 17408)):
            assert f"small_m{m}_n{n}_k{k}" in wls
    for m in (128, 512, 4096):
        for n in (5120, 17408):
            assert f"prefill_m{m}_n{n}_k5120" in wls
    assert {"layer64_m1", "layer64_m16"} <= set(wls)


@pytest.mark.parametrize("m,us", [(1, 25000 / 1.5 / 1000), (2, 25000 / 1.5 / 1000),
                                  (16, 55000 / 1.5 / 1000), (64, 55000 / 1.5 / 1000)])
def test_proxy_spin_length(m, us):
    """25k spin cycles at 2 tokens up to 55k at 16, at 1.5 cycles per ns of other
    work, held at the ends of that range."""
    import bench
    assert bench.proxy_spin_us(m) == pytest.approx(us)


def test_proxy_spin_length_is_linear_between_2_and_16():
    import bench
    a, b = bench.proxy_spin_us(2), bench.proxy_spin_us(16)
    assert bench.proxy_spin_us(9) == pytest.approx((a + b) / 2)


def test_bad_counts_are_rejected():
    for flags in (["--steps", "0"], ["--trials", "0"], ["--warmup", "-1"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, flags


def test_power_sampler_parses_and_stops(tmp_path, monkeypatch):
    """The proxy's power sampler reads socket power and the first graphics
    clock from amd-smi's JSON (a stand-in script here), and returns when the
    tool's output is not what it expects."""
    import threading
    import time

    import bench
    tool = tmp_path / "amd-smi"
    tool.write_text("#!/bin/sh\n"
                    "echo '{\"gpu_data\": [{\"gpu\": 0, \"power\": {\"socket_power\": "
                    "{\"value\": 321, \"unit\": \"W\"}}, \"clock\": {\"gfx_0\": {\"clk\": "
                    "{\"value\": 2100, \"unit\": \"MHz\"}}}}]}'\n")
    tool.chmod(0o755)
    monkeypatch.setenv("PATH", f"{tmp_path}{os.pathsep}{os.environ['PATH']}")
    stop, out = threading.Event(), []
    th = threading.Thread(target=bench.power_sampler, args=(stop, out), daemon=True)
    th.start()
    time.sleep(0.5)
    stop.set()
    th.join(timeout=20)
    assert not th.is_alive() and out
    assert all(p == 321.0 and c == 2100.0 and s0 <= s1 for (s0, s1, p, c) in out)
    tool.write_text("#!/bin/sh\necho not json\n")
    stop2, out2 = threading.Event(), []
    bench.power_sampler(stop2, out2)          # returns at the first bad sample
    assert out2 == []
