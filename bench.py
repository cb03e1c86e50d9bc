"""Benchmark of the PQ2_0 ternary GEMM path on one MI355X.

A step is one pass of the hot path over one batch: pq2_quantize_act on the
activations, then pq2_gemm against the next weight matrix of a rotating set
(the set is larger than the 256 MB Infinity Cache, so weights stream from
HBM). Inputs are resident in HBM before the timed region starts. For
M <= 4 the single-launch pq2_linear (quantisation inside the GEMV) is timed
too and reported in the config (fused_step_us).

Default workload: decode GEMV, M = 1, N = 5120, K = 6144, 64 rotating
matrices. ``--workload`` selects another configuration; ``--sweep`` prints
one line per configuration (small-batch, prefill, 64-layer decode step).

Printed JSON line: metric/value/unit (algorithmic HBM GB/s of the whole step,
or int8 TOP/s for prefill), the roofline of the dominant kernel measured with
HIP events around each of its launches, and the CPU oracle timed on a bounded
sample of the same workload on the host's cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, published
GROUP = 128
METRIC = "PQ2 GEMM: HBM GB/s (% peak) at M=1..16; int8 TOPS (% peak) prefill"


# ---------------------------------------------------------------- algorithmic work

def gemm_bytes(M, N, K):
    """codes + fp16 group scales + plane-order q + s and t + y (float32)."""
    G = K // GROUP
    return N * K // 4 + 2 * N * G + M * K + 8 * M * G + 4 * M * N


def quant_bytes(M, K):
    G = K // GROUP
    return 4 * M * K + M * K + 8 * M * G


LINEAR_MAX_M = 4   # PQ2_LINEAR_MAX_M


def step_bytes(M, N, K):
    """Algorithmic HBM bytes of quantise + GEMM (q, s, t written and read back)."""
    return gemm_bytes(M, N, K) + quant_bytes(M, K)


def gemm_ops(M, N, K):
    return 2 * M * N * K


# ---------------------------------------------------------------- workloads

def workload_list():
    import pq2_synth as synth
    out = {"decode": ("gemm", synth.decode_gemv())}
    for m in synth.SMALL_MS:
        for n, k in synth.SMALL_SHAPES:
            w = synth.small_batch(m, n, k)
            out[w.name] = ("gemm", w)
    for m in synth.PREFILL_MS:
        for n, k in synth.PREFILL_SHAPES:
            w = synth.prefill(m, n, k)
            out[w.name] = ("gemm", w)
    for m in (1, 16):
        out[f"layer64_m{m}"] = ("layers", m)
    return out


def make_weight_set(wl, torch, dev):
    """Rotating set of distinct matrices, generated on the host (numpy PCG64)."""
    import pq2_synth as synth
    codes, scales = [], []
    for i in range(wl.rotate):
        w = synth.weights(wl.n, wl.k, synth.matrix_seed(i), wl.probs)
        codes.append(torch.from_numpy(w.codes).to(dev))
        scales.append(torch.from_numpy(w.wscale_bits.view(np.int16)).to(dev))
    return codes, scales


def make_layer_set(torch, dev, n_layers, gen):
    """64 synthetic layers x 5 projections; generated on the device from a seeded
    torch generator (5.6 GB of packed weights would take minutes with numpy).
    Each packed byte is one of the 81 bytes whose four 2-bit fields are codes
    0..2, drawn uniformly, i.e. four iid uniform codes."""
    import pq2_synth as synth
    table = torch.from_numpy(synth._VALID_BYTES).to(dev)
    layers = []
    for _ in range(n_layers):
        projs = []
        for (n, k) in synth.LAYER_SHAPES:
            idx = torch.randint(0, 81, (n, k // 4), generator=gen, device=dev)
            codes = table[idx]
            ws = (torch.rand((n, k // GROUP), generator=gen, device=dev) * 0.09 + 0.01)
            projs.append((codes, ws.to(torch.float16).view(torch.int16), n, k))
        layers.append(projs)
    return layers


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(wl, budget_s=10.0):
    """The oracle (as is) on a bounded sample of the workload, all host cores."""
    import oracle
    import pq2_synth as synth
    oracle.build(force=False)
    threads = oracle.max_threads()
    x = synth.activations(wl.m, wl.k, 0, wl.outlier_frac)
    n_mats = min(wl.rotate, 4)
    mats = [synth.weights(wl.n, wl.k, synth.matrix_seed(i), wl.probs) for i in range(n_mats)]
    calls = 0
    t0 = time.perf_counter()
    while True:
        w = mats[calls % n_mats]
        oracle.forward(x, w.codes, w.wscale, threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_call = el / calls
    return {
        "value": step_bytes(wl.m, wl.n, wl.k) / per_call / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{calls} full calls (quantise + all {wl.m}x{wl.n} outputs) over {n_mats} "
                  f"of the workload's matrices, {el:.1f} s, {per_call * 1e3:.1f} ms/call",
    }


def cpu_baseline_prefill(wl, budget_s=10.0):
    import oracle
    import pq2_synth as synth
    oracle.build(force=False)
    threads = oracle.max_threads()
    x = synth.activations(wl.m, wl.k, 0)
    w = synth.weights(wl.n, wl.k, synth.matrix_seed(0), wl.probs)
    q, s, t = oracle.quantize(x)
    rng = np.random.default_rng(0)
    P = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        mm = rng.integers(0, wl.m, 4096)
        nn = rng.integers(0, wl.n, 4096)
        oracle.gemm_f64_sampled(q, s, w.codes, w.wscale, mm, nn, threads=threads)
        P += 4096
    el = time.perf_counter() - t0
    return {"value": 2 * P * wl.k / el / 1e12, "unit": "TOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{P} sampled outputs of the {wl.m}x{wl.n} product, {el:.1f} s"}


# ---------------------------------------------------------------- GPU timing

def traffic_record(kernel_tag):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    import hashlib
    rec = json.load(open(path))
    root = os.path.dirname(os.path.abspath(__file__))
    for src, sha in rec["source_sha256"].items():
        if hashlib.sha256(open(os.path.join(root, src), "rb").read()).hexdigest() != sha:
            return None        # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def spin_cycles_per_ms(torch):
    """Calibrate torch.cuda._sleep (a one-thread spin kernel) against HIP events."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def queue_ahead(torch, host_ms, cyc_per_ms):
    """Hold the stream with a spin kernel long enough for the host to enqueue
    the whole timed region, so HIP events time the GPU and not Python."""
    torch.cuda._sleep(int(cyc_per_ms * (2.0 * host_ms + 5.0)))


def run_gemm(args, wl, torch, pq2):
    dev = torch.device("cuda:0")
    import pq2_synth as synth
    codes, scales = make_weight_set(wl, torch, dev)
    x = torch.from_numpy(synth.activations(wl.m, wl.k, 0, wl.outlier_frac)).to(dev)
    M, N, K = wl.m, wl.n, wl.k
    G = K // GROUP
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s = torch.empty((M, G), dtype=torch.float32, device=dev)
    t = torch.empty((M, G), dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    R = len(codes)
    # raw pointers: the timed loop calls the C ABI directly (no per-call checks)
    lib = pq2.lib
    stream = torch.cuda.current_stream(dev).cuda_stream
    xp, qp, sp, tp, yp = x.data_ptr(), q.data_ptr(), s.data_ptr(), t.data_ptr(), y.data_ptr()
    cps = [c.data_ptr() for c in codes]
    wps = [w.data_ptr() for w in scales]
    quant, gemm, linear = lib.pq2_quantize_act, lib.pq2_gemm, lib.pq2_linear
    fused = M <= LINEAR_MAX_M

    def step_unfused(i):
        st1 = quant(xp, qp, sp, tp, M, K, stream)
        st2 = gemm(qp, sp, tp, cps[i % R], wps[i % R], yp, M, N, K, stream)
        if st1 or st2:
            raise pq2.PQ2Error(st1 or st2)

    def step_fused(i):
        st = linear(xp, cps[i % R], wps[i % R], yp, M, N, K, stream)
        if st:
            raise pq2.PQ2Error(st)

    step = step_unfused
    for i in range(args.warmup):
        step(i)
        if fused:
            step_fused(i)
    torch.cuda.synchronize()
    cyc_per_ms = spin_cycles_per_ms(torch)

    def timed(body):
        """Run body(i) for the K timed iterations between two HIP events, with
        the stream held by a spin kernel while the host enqueues them."""
        h0 = time.perf_counter()
        for i in range(args.steps):
            body(i)
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - h0) * 1e3
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        queue_ahead(torch, host_ms, cyc_per_ms)
        a.record()
        h0 = time.perf_counter()
        for i in range(args.steps):
            body(i)
        enq_ms = (time.perf_counter() - h0) * 1e3
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b), enq_ms, host_ms

    # the whole step
    wall0 = time.perf_counter()
    total_ms, enq_ms, _ = timed(step)
    wall = time.perf_counter() - wall0
    # pq2_gemm alone, back to back on the same stream (average launch duration
    # including the dispatch gap between launches)
    gemm_total, _, _ = timed(lambda i: gemm(qp, sp, tp, cps[i % R], wps[i % R], yp, M, N, K, stream))
    out = dict(ms_step=total_ms / args.steps, gemm_ms=gemm_total / args.steps, wall=wall,
               path=pq2.PATH_NAMES[pq2.gemm_kernel_path(M, N, K)],
               M=M, N=N, K=K, host_enqueue_ms=enq_ms, gpu_ms=total_ms, fused=fused)
    out["kernel_ms"] = out["gemm_ms"]
    if fused:
        fus_total, _, _ = timed(step_fused)
        out["fused_ms_step"] = fus_total / args.steps
    return out


def report_gemm(args, wl, r, torch):
    M, N, K = r["M"], r["N"], r["K"]
    sbytes = step_bytes(M, N, K)
    prefill = M > 16
    fused = r["fused"]
    path = r["path"]
    if prefill:
        value = gemm_ops(M, N, K) / (r["ms_step"] * 1e-3) / 1e12
        unit = "TOP/s"
        achieved = gemm_ops(M, N, K) / (r["kernel_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": achieved / I8_PEAK_TOPS}
    else:
        value = sbytes / (r["ms_step"] * 1e-3) / 1e9
        unit = "GB/s"
        achieved = gemm_bytes(M, N, K) / (r["kernel_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["kernel"] = path
    roof["kernel_us"] = r["kernel_ms"] * 1e3
    roof["timing"] = ("HIP events around K back-to-back pq2_gemm launches (rotating weights); the "
                      "stream is held by a spin kernel while the host enqueues, so the events see "
                      "GPU time; includes the dispatch gap between launches")
    roof["traffic"] = traffic_record(f"{path}_{wl.name}")
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "N": N, "K": K, "rotating_matrices": wl.rotate,
                   "step": "pq2_quantize_act + pq2_gemm",
                   "algorithmic_bytes_per_step": sbytes,
                   "gemm_bytes_per_call": gemm_bytes(M, N, K),
                   "gemm_int_ops_per_call": gemm_ops(M, N, K),
                   "host_enqueue_ms": r["host_enqueue_ms"], "gpu_ms": r["gpu_ms"],
                   "pq2_gemm_us": r["gemm_ms"] * 1e3},
        "roofline": roof,
    }
    if fused:
        line["config"]["fused_step_us"] = r["fused_ms_step"] * 1e3
    if not args.no_cpu:
        line["cpu_baseline"] = (cpu_baseline_prefill(wl, args.cpu_seconds) if prefill
                                else cpu_baseline(wl, args.cpu_seconds))
    return line


def layer_step(m, torch, pq2, stream):
    """The 64-layer synthetic decode step as a list of launches on `stream`:
    returns (step, shares_input); step(after=None) enqueues every projection
    (quantise where the input is new, then pq2_gemm) and calls after() behind
    each projection's GEMM."""
    import pq2_synth as synth
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    layers = make_layer_set(torch, dev, synth.N_LAYERS, gen)
    xs, bufs = {}, {}
    for (n, k) in synth.LAYER_SHAPES:
        if k not in xs:
            xs[k] = torch.from_numpy(synth.activations(m, k, 0)).to(dev)
            bufs[k] = (torch.empty((m, k), dtype=torch.int8, device=dev),
                       torch.empty((m, k // GROUP), dtype=torch.float32, device=dev),
                       torch.empty((m, k // GROUP), dtype=torch.int32, device=dev))
    ys = {n: torch.empty((m, n), dtype=torch.float32, device=dev) for (n, _) in synth.LAYER_SHAPES}
    lib = pq2.lib
    # the gate and up projections (the two 5120 -> 17408 ones) read the same
    # activations, so one quantisation serves both; every other projection
    # quantises its own input
    shares_input = tuple(i > 0 and synth.LAYER_SHAPES[i] == synth.LAYER_SHAPES[i - 1]
                         for i in range(len(synth.LAYER_SHAPES)))
    calls = []
    for projs in layers:
        for i, (codes, ws, n, k) in enumerate(projs):
            q, s, t = bufs[k]
            calls.append((not shares_input[i], xs[k].data_ptr(), q.data_ptr(), s.data_ptr(),
                          t.data_ptr(), codes.data_ptr(), ws.data_ptr(), ys[n].data_ptr(), n, k))
    quant, gemm = lib.pq2_quantize_act, lib.pq2_gemm

    def step(after=None):
        for (qz, xp, qp, sp, tp, cp, wp, yp, n, k) in calls:
            if qz:
                quant(xp, qp, sp, tp, m, k, stream)
            gemm(qp, sp, tp, cp, wp, yp, m, n, k, stream)
            if after is not None:
                after()

    step.buffers = (layers, xs, bufs, ys)     # the launches hold raw pointers into these
    return step, shares_input


def run_layers(args, m, torch, pq2):
    """64-layer synthetic decode step: 5 PQ2_0 projections per layer, back to back."""
    import pq2_synth as synth
    stream = torch.cuda.current_stream(torch.device("cuda:0")).cuda_stream
    step, shares_input = layer_step(m, torch, pq2, stream)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    steps = max(1, args.steps // 20)
    cyc_per_ms = spin_cycles_per_ms(torch)
    h0 = time.perf_counter()
    step()
    host_ms = (time.perf_counter() - h0) * 1e3 * steps
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    queue_ahead(torch, host_ms, cyc_per_ms)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    total = 0
    for i, (n, k) in enumerate(synth.LAYER_SHAPES):
        total += gemm_bytes(m, n, k) + (0 if shares_input[i] else quant_bytes(m, k))
    total *= synth.N_LAYERS
    gbs = total / (ms * 1e-3) / 1e9
    return {"metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": 2, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
            "config": {"workload": f"layer64_m{m}", "M": m, "layers": synth.N_LAYERS,
                       "gemms_per_step": 5 * synth.N_LAYERS,
                       "quantisations_per_step": (5 - sum(shares_input)) * synth.N_LAYERS,
                       "projection": "pq2_quantize_act + pq2_gemm (gate and up share one quantisation)",
                       "algorithmic_bytes_per_step": total},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                         "note": "whole step incl. quantise launches and launch gaps"}}


# The pages' power proxy: a low-power spin after every projection stands in for
# the decode step's other work (norms, attention, recurrent updates, sampling),
# so that a replay of the projections runs at the clock and power state of
# serving rather than of back-to-back memory-bound kernels. The pages sized
# the spin from a serving trace (page "Making a ternary reasoning model fast
# in vLLM", section "A power proxy for the rest of the model"): 25k cycles at
# 2 tokens rising to 55k at 16, which they relate to the non-GEMM time of the
# trace at roughly 1.5 spin cycles per ns. Here the spin is that much time
# per projection.
def proxy_spin_us(m):
    cycles = 25000.0 + (min(max(m, 2), 16) - 2) * (55000.0 - 25000.0) / 14.0
    return cycles / 1.5 / 1000.0


def run_proxy(args, m, torch, pq2):
    """The 64-layer step with a spin after every projection, captured once in a
    HIP graph and replayed back to back for --proxy-seconds. Kernel durations
    under the proxy come from a kernel trace of this run (the spin's wall time
    follows the clock, so the step time mixes the two); this line reports the
    replay itself."""
    dev = torch.device("cuda:0")
    cap = torch.cuda.Stream(dev)
    spin_us = proxy_spin_us(m) if args.proxy_spin_us is None else args.proxy_spin_us
    cyc_per_ms = spin_cycles_per_ms(torch)
    spin = int(cyc_per_ms * spin_us / 1000.0)
    step, _ = layer_step(m, torch, pq2, cap.cuda_stream)
    after = (lambda: torch.cuda._sleep(spin)) if spin > 0 else None
    with torch.cuda.stream(cap):
        step(after)                 # eager first: any per-stream workspace exists before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(after)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    replays, t0 = 0, time.perf_counter()
    a.record()
    while time.perf_counter() - t0 < args.proxy_seconds:
        for _ in range(10):
            g.replay()
        replays += 10
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / replays
    return {"proxy": {"workload": f"layer64_m{m}", "M": m, "spin_us_per_projection": spin_us,
                      "spin_cycles": spin, "projections_per_step": 5 * 64,
                      "replays": replays, "ms_per_replay": ms,
                      "note": "HIP-graph replay of the 64-layer step with a spin after every "
                              "projection; GEMM kernel durations from a kernel trace of this run"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--sweep", action="store_true", help="one line per configuration")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--proxy", type=int, default=0, metavar="M",
                    help="power-proxy replay of the 64-layer step at M token rows "
                         "(one JSON line of its own, not the bench line)")
    ap.add_argument("--proxy-seconds", type=float, default=5.0)
    ap.add_argument("--proxy-spin-us", type=float, default=None,
                    help="spin per projection (default: the pages' calibration for M; 0: none)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise kernel (y = 2x, float32) over MIB MiB, "
                         "the calibration for HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the PQ2_0 path is measured on a single MI355X; run with --gpus 1 "
              "(no multi-GPU path is built).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        reps = 10
        for _ in range(reps):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe": {"kernel": "torch.mul(src, 2.0, out=dst)",
                                         "read_bytes_per_launch": 4 * n,
                                         "write_bytes_per_launch": 4 * n, "launches": reps}}))
        return

    import gemm_pq2_w2a8_amd as pq2

    if args.proxy:
        print(json.dumps(run_proxy(args, args.proxy, torch, pq2)), flush=True)
        return

    wls = workload_list()
    names = list(wls) if args.sweep else [args.workload]
    for name in names:
        kind, wl = wls[name]
        print(f"# running {name}", file=sys.stderr, flush=True)
        if kind == "gemm":
            r = run_gemm(args, wl, torch, pq2)
            line = report_gemm(args, wl, r, torch)
        else:
            line = run_layers(args, wl, torch, pq2)
        print(json.dumps(line), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
