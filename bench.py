"""Benchmark of the PQ2_0 ternary GEMM path on one MI355X.

A step is one pass of the hot path over one batch: pq2_quantize_act on the
activations, then pq2_gemm against the next weight matrix of a rotating set
(the set is larger than the 256 MB Infinity Cache, so weights stream from
HBM). Inputs are resident in HBM before the timed region starts. For
M <= 16 the step without the quantiser launch, pq2_linear (quantisation
inside the GEMM kernel), is timed too where it has a kernel for the shape and
reported in the config (fused_step_us).

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


LINEAR_MAX_M = 16   # PQ2_LINEAR_MAX_M


def linear_bytes(M, N, K):
    """Algorithmic HBM bytes of pq2_linear: codes + fp16 group scales +
    float32 x + y (q, s and t never leave the kernel)."""
    G = K // GROUP
    return N * K // 4 + 2 * N * G + 4 * M * K + 4 * M * N


def one_launch(M, N, K):
    """Where the one-launch pq2_linear (quantisation inside the GEMV) measured
    faster than pq2_quantize_act + pq2_gemm on MI355X: one token row with
    K <= 6144 and N * K <= 2^25 (decode 5120 x 6144: 5.07 against 6.57 us).
    The 64-layer step takes it there: with it on every GEMM of a layer, or
    on the stacked 34816 x 5120 gate and up too, the step measured slower.
    From two rows on it is slower than the two launches except on the
    decode shape (7.21 against 7.53 us at two rows). The bench line reports
    it beside the two-launch step."""
    return M == 1 and K <= 6144 and N * K <= (1 << 25)


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
    """The oracle (as is) on a bounded sample of the workload: all host cores
    for budget_s, then one core for half of that."""
    import oracle
    import pq2_synth as synth
    oracle.build(force=False)
    threads = oracle.max_threads()
    x = synth.activations(wl.m, wl.k, 0, wl.outlier_frac)
    n_mats = min(wl.rotate, 4)
    mats = [synth.weights(wl.n, wl.k, synth.matrix_seed(i), wl.probs) for i in range(n_mats)]

    def timed(nthreads, budget):
        calls = 0
        t0 = time.perf_counter()
        while True:
            w = mats[calls % n_mats]
            oracle.forward(x, w.codes, w.wscale, threads=nthreads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return calls, el
    calls, el = timed(threads, budget_s)
    calls1, el1 = timed(1, budget_s / 2)
    per_call, per_call1 = el / calls, el1 / calls1
    return {
        "value": step_bytes(wl.m, wl.n, wl.k) / per_call / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{calls} full calls (quantise + all {wl.m}x{wl.n} outputs) over {n_mats} "
                  f"of the workload's matrices, {el:.1f} s, {per_call * 1e3:.1f} ms/call",
        "one_core_value": step_bytes(wl.m, wl.n, wl.k) / per_call1 / 1e9,
        "one_core_sample": f"{calls1} calls on one core, {el1:.1f} s, {per_call1 * 1e3:.1f} ms/call",
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

    def timed(nthreads, budget):
        P = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:
            mm = rng.integers(0, wl.m, 4096)
            nn = rng.integers(0, wl.n, 4096)
            oracle.gemm_f64_sampled(q, s, w.codes, w.wscale, mm, nn, threads=nthreads)
            P += 4096
        return P, time.perf_counter() - t0
    P, el = timed(threads, budget_s)
    P1, el1 = timed(1, budget_s / 2)
    return {"value": 2 * P * wl.k / el / 1e12, "unit": "TOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{P} sampled outputs of the {wl.m}x{wl.n} product, {el:.1f} s",
            "one_core_value": 2 * P1 * wl.k / el1 / 1e12,
            "one_core_sample": f"{P1} sampled outputs on one core, {el1:.1f} s"}


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


class Timer:
    """HIP events around `steps` calls of a body on the current stream. The
    stream is first held by a spin kernel long enough for the host to enqueue
    the whole region, so the events time the GPU and not Python. Each call of
    the body takes its own weight matrix from a running index (the bodies keep
    it), so no pass re-reads a matrix sooner than a whole rotation later."""

    def __init__(self, torch, steps):
        self.torch = torch
        self.steps = steps
        self.cyc_per_ms = spin_cycles_per_ms(torch)

    def host_ms(self, body):
        t0 = time.perf_counter()
        for _ in range(self.steps):
            body()
        self.torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    def run(self, body, host_ms, side=None):
        """GPU ms of `steps` calls of body; side(event) is called right after
        the first event is recorded (work for another stream that waits for
        that event, so it runs alongside the timed region)."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(self.cyc_per_ms * (2.0 * host_ms + 5.0)))
        a.record()
        if side is not None:
            side(a)
        for _ in range(self.steps):
            body()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)


def median(v):
    return float(np.median(np.asarray(v, dtype=np.float64)))


class Probes:
    """The measurement probes (libpq2_probe.so): streaming-read and int8 MFMA
    ceilings, and the shader clock read in-band while other work runs."""

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_pq2_w2a8_amd",
                            "libpq2_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python gemm_pq2_w2a8_amd/build.py`")
        lib = ctypes.CDLL(path)
        P, SZ = ctypes.c_void_p, ctypes.c_size_t
        lib.pq2_probe_stream_read.argtypes = [P, SZ, P, ctypes.c_int, P]
        lib.pq2_probe_mfma_i8.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        lib.pq2_probe_epilogue_mix.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        lib.pq2_probe_clock.argtypes = [P, ctypes.c_uint64, P]
        for f in (lib.pq2_probe_stream_read, lib.pq2_probe_mfma_i8, lib.pq2_probe_epilogue_mix,
                  lib.pq2_probe_clock):
            f.restype = ctypes.c_int
        self.lib = lib
        dev = torch.device("cuda:0")
        self.sink = torch.empty(1 << 20, dtype=torch.int32, device=dev)
        self.clk = torch.zeros(2, dtype=torch.int64, device=dev)
        self.side = torch.cuda.Stream(dev)
        # first launch on the side stream outside any timed region (a stream's
        # first launch costs far more than later ones)
        self._ok(self.lib.pq2_probe_clock(self.clk.data_ptr(), 1000, self.side.cuda_stream),
                 "clock")
        torch.cuda.synchronize()
        props = torch.cuda.get_device_properties(dev)
        self.cus = props.multi_processor_count
        # wall clock counter rate (hipDeviceAttributeWallClockRate): 100 MHz on CDNA
        self.wall_mhz = 100.0

    def _ok(self, st, what):
        if st != 0:
            raise RuntimeError(f"probe {what} failed with status {st}")

    def clock_side(self, ms):
        """A side(event) for Timer.run: the clock probe on a side stream (default
        priority), started when the timed region starts and spinning ~ms."""
        side = self.side
        ticks = max(1, min(int(ms * 1e3 * self.wall_mhz), (1 << 28)))

        def go(event):
            side.wait_event(event)
            self._ok(self.lib.pq2_probe_clock(self.clk.data_ptr(), ticks, side.cuda_stream),
                     "clock")
        return go

    def sclk_mhz(self):
        self.torch.cuda.synchronize()
        cyc, wall = (int(v) for v in self.clk.cpu())
        return cyc / wall * self.wall_mhz if wall > 0 else None

    def stream_read(self, nbytes, rotate_bytes, calls, trials=5):
        """Best time per launch (median over trials, best over launch shapes)
        of a plain read of nbytes, the slices cycling through a buffer of
        rotate_bytes (above the Infinity Cache, like the rotating weights)."""
        torch = self.torch
        n16 = (nbytes + 15) // 16 * 16
        slices = max(2, rotate_bytes // n16)
        buf = torch.empty(slices * n16, dtype=torch.uint8, device="cuda:0")
        buf.fill_(1)
        stream = torch.cuda.current_stream().cuda_stream
        tm = Timer(torch, calls)
        best = None
        for blocks in (self.cus * 2, self.cus * 4, self.cus * 8):
            ctr = [0]

            def body():
                off = (ctr[0] % slices) * n16
                ctr[0] += 1
                self._ok(self.lib.pq2_probe_stream_read(buf.data_ptr() + off, n16,
                                                        self.sink.data_ptr(), blocks, stream),
                         "stream_read")
            h = tm.host_ms(body)
            us = median([tm.run(body, h) for _ in range(trials)]) / calls * 1e3
            if best is None or us < best[0]:
                best = (us, blocks)
        del buf
        return {"bytes": n16, "us": best[0], "GB/s": n16 / (best[0] * 1e-6) / 1e9,
                "blocks": best[1], "rotating_bytes": slices * n16}

    def launch_floor(self, calls=400, trials=5):
        """Time per launch of a one-block kernel that reads 16 bytes, launched
        back to back: the fixed cost of every launch on this stack (dispatch,
        the in-order wait for the previous kernel, its cache write-back)."""
        torch = self.torch
        buf = torch.ones(16, dtype=torch.uint8, device="cuda:0")
        stream = torch.cuda.current_stream().cuda_stream
        tm = Timer(torch, calls)

        def body():
            self._ok(self.lib.pq2_probe_stream_read(buf.data_ptr(), 16, self.sink.data_ptr(), 1,
                                                    stream), "stream_read")
        h = tm.host_ms(body)
        return median([tm.run(body, h) for _ in range(trials)]) / calls * 1e3

    def mfma_i8(self, trials=5):
        torch = self.torch
        stream = torch.cuda.current_stream().cuda_stream
        blocks, iters = self.cus * 8, 2000
        tm = Timer(torch, 4)

        def body():
            self._ok(self.lib.pq2_probe_mfma_i8(self.sink.data_ptr(), iters, blocks, stream),
                     "mfma")
        h = tm.host_ms(body)
        ms = median([tm.run(body, h) for _ in range(trials)]) / 4
        ops = blocks * 4 * iters * 8 * 2 * 16 * 16 * 64
        return {"TOP/s": ops / (ms * 1e-3) / 1e12, "us": ms * 1e3, "blocks": blocks,
                "waves_per_cu": 4 * blocks // self.cus,
                "instruction": "v_mfma_i32_16x16x64_i8, 8 independent chains per wave"}


    def epilogue_mix(self, trials=5):
        """The int8 MFMA rate left once an exact float32 per-group epilogue
        runs beside it (per 16 x 16 tile and group: 2 int8 MFMAs, one float32
        4x4x1 outer-product MFMA, 4 conversions and 4 FMAs per lane)."""
        torch = self.torch
        stream = torch.cuda.current_stream().cuda_stream
        blocks, iters = self.cus * 8, 1000
        tm = Timer(torch, 4)

        def body():
            self._ok(self.lib.pq2_probe_epilogue_mix(self.sink.data_ptr(), iters, blocks, stream),
                     "epilogue mix")
        h = tm.host_ms(body)
        ms = median([tm.run(body, h) for _ in range(trials)]) / 4
        ops = blocks * 4 * iters * 8 * 2 * 2 * 16 * 16 * 64
        return {"TOP/s": ops / (ms * 1e-3) / 1e12, "us": ms * 1e3, "blocks": blocks,
                "waves_per_cu": 4 * blocks // self.cus,
                "mix": "per 16x16 tile and group: 2 v_mfma_i32_16x16x64_i8, 1 "
                       "v_mfma_f32_4x4x1_16b_f32, 4 v_cvt_f32_i32, 4 v_fmac_f32"}


def run_gemm(args, wl, torch, pq2, steps, trials, probes=None):
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
    wsz = pq2.gemm_workspace_bytes(M, N, K)
    lwsz = pq2.linear_workspace_bytes(M, N, K) if M <= LINEAR_MAX_M else 0
    work = torch.empty(max(wsz, lwsz, 16), dtype=torch.uint8, device=dev)
    R = len(codes)
    # raw pointers: the timed loop calls the C ABI directly (no per-call checks)
    lib = pq2.lib
    stream = torch.cuda.current_stream(dev).cuda_stream
    xp, qp, sp, tp, yp = x.data_ptr(), q.data_ptr(), s.data_ptr(), t.data_ptr(), y.data_ptr()
    wkp = work.data_ptr() if wsz else None
    lwkp = work.data_ptr() if lwsz else None
    cps = [c.data_ptr() for c in codes]
    wps = [w.data_ptr() for w in scales]
    quant, gemm, linear = lib.pq2_quantize_act, lib.pq2_gemm, lib.pq2_linear
    fused = M <= LINEAR_MAX_M and pq2.linear_kernel_path(M, N, K, lwsz) >= 0
    ctr = [0]          # one running matrix index over every pass

    def nxt():
        i = ctr[0] % R
        ctr[0] += 1
        return i

    def step():
        i = nxt()
        st1 = quant(xp, qp, sp, tp, M, K, stream)
        st2 = gemm(qp, sp, tp, cps[i], wps[i], yp, M, N, K, wkp, wsz, stream)
        if st1 or st2:
            raise pq2.PQ2Error(st1 or st2)

    def gemm_only():
        i = nxt()
        st = gemm(qp, sp, tp, cps[i], wps[i], yp, M, N, K, wkp, wsz, stream)
        if st:
            raise pq2.PQ2Error(st)

    def step_fused():
        i = nxt()
        st = linear(xp, cps[i], wps[i], yp, M, N, K, lwkp, lwsz, stream)
        if st:
            raise pq2.PQ2Error(st)

    def quant_only():
        st = quant(xp, qp, sp, tp, M, K, stream)
        if st:
            raise pq2.PQ2Error(st)

    for _ in range(args.warmup):
        step()
        if fused:
            step_fused()
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    h_step = tm.host_ms(step)
    h_gemm = tm.host_ms(gemm_only)
    h_fused = tm.host_ms(step_fused) if fused else 0.0
    step_ms, gemm_ms, fused_ms, sclk = [], [], [], []
    wall0 = time.perf_counter()
    for _ in range(trials):
        step_ms.append(tm.run(step, h_step))
        # the clock probe spins for about half of the step region just timed,
        # which is shorter than the GEMM-only region
        side = probes.clock_side(0.5 * step_ms[-1]) if probes is not None else None
        gemm_ms.append(tm.run(gemm_only, h_gemm, side))
        if probes is not None:
            sclk.append(probes.sclk_mhz())
        if fused:
            fused_ms.append(tm.run(step_fused, h_fused))
    wall = time.perf_counter() - wall0
    per = lambda v: median(v) / steps
    wbytes = N * K // 4 + 2 * N * G          # one matrix: codes + float16 scales
    out = dict(ms_step=per(step_ms), gemm_ms=per(gemm_ms), wall=wall,
               path=pq2.PATH_NAMES[pq2.gemm_kernel_path(M, N, K)], M=M, N=N, K=K,
               host_enqueue_ms=h_step, fused=fused, trials=trials, steps=steps,
               workspace_bytes=wsz,
               trial_step_us=[v / steps * 1e3 for v in step_ms],
               trial_gemm_us=[v / steps * 1e3 for v in gemm_ms],
               bytes_between_reuse=(R - 1) * wbytes if R > 1 else None,
               rotate=R)
    out["kernel_ms"] = out["gemm_ms"]
    # the quantiser alone (K1), back to back on the same activations
    h_quant = tm.host_ms(quant_only)
    out["quant_ms"] = per([tm.run(quant_only, h_quant) for _ in range(trials)])
    if probes is not None and M <= LINEAR_MAX_M:
        # the same launches on one matrix, whose bytes then stay in the caches:
        # what the kernel takes when no byte has to come from HBM
        def resident():
            st = gemm(qp, sp, tp, cps[0], wps[0], yp, M, N, K, wkp, wsz, stream)
            if st:
                raise pq2.PQ2Error(st)
        resident()
        h_res = tm.host_ms(resident)
        out["resident_gemm_ms"] = per([tm.run(resident, h_res) for _ in range(trials)])
    if sclk and all(v is not None for v in sclk):
        out["sclk_mhz"] = median(sclk)
    if fused:
        out["fused_ms_step"] = per(fused_ms)
        out["trial_fused_us"] = [v / steps * 1e3 for v in fused_ms]
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
    if not prefill:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = traffic_record(f"{path}_{wl.name}")
    roof["kernel"] = path
    roof["kernel_us"] = r["kernel_ms"] * 1e3
    roof["timing"] = (f"HIP events around {r['steps']} back-to-back pq2_gemm launches, median "
                      f"of {r['trials']} trials; one running matrix index over every pass; the "
                      "stream is held by a spin kernel while the host enqueues, so the events see "
                      "GPU time; includes the dispatch gap between launches")
    cfg = {"workload": wl.name, "M": M, "N": N, "K": K, "rotating_matrices": r["rotate"],
           "bytes_between_matrix_reuse": r["bytes_between_reuse"],
           "step": "pq2_quantize_act + pq2_gemm",
           "algorithmic_bytes_per_step": sbytes,
           "gemm_bytes_per_call": gemm_bytes(M, N, K),
           "gemm_int_ops_per_call": gemm_ops(M, N, K),
           "workspace_bytes": r["workspace_bytes"],
           "trials": r["trials"], "steps_per_trial": r["steps"],
           "trial_step_us": [round(v, 3) for v in r["trial_step_us"]],
           "trial_pq2_gemm_us": [round(v, 3) for v in r["trial_gemm_us"]],
           "host_enqueue_ms": r["host_enqueue_ms"],
           "pq2_gemm_us": r["gemm_ms"] * 1e3,
           "pq2_quantize_act_us": r["quant_ms"] * 1e3}
    if "sclk_mhz" in r:
        cfg["sclk_mhz_during_pq2_gemm"] = r["sclk_mhz"]
    if "resident_gemm_ms" in r:
        cfg["pq2_gemm_cache_resident_us"] = r["resident_gemm_ms"] * 1e3
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": r["steps"],
        "warmup": args.warmup, "ms_per_step": r["ms_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": cfg,
        "roofline": roof,
    }
    if fused:
        cfg["fused_step_us"] = r["fused_ms_step"] * 1e3
        cfg["trial_fused_step_us"] = [round(v, 3) for v in r["trial_fused_us"]]
        if one_launch(M, N, K):
            cfg["one_launch_GB/s"] = linear_bytes(M, N, K) / (r["fused_ms_step"] * 1e-3) / 1e9
    if not args.no_cpu:
        line["cpu_baseline"] = (cpu_baseline_prefill(wl, args.cpu_seconds) if prefill
                                else cpu_baseline(wl, args.cpu_seconds))
    return line


def layer_step(m, torch, pq2, stream):
    """The 64-layer synthetic decode step as a list of launches on `stream`:
    step(after=None) enqueues every GEMM of the step (pq2_linear, or
    pq2_quantize_act then pq2_gemm) and calls after() behind each."""
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
    # one split-K workspace serves every projection: they run in order on one stream
    wsz = max(max(pq2.gemm_workspace_bytes(m, n, k), pq2.linear_workspace_bytes(m, n, k))
              for (n, k) in synth.LAYER_SHAPES)
    work = torch.empty(max(wsz, 16), dtype=torch.uint8, device=dev)
    wkp = work.data_ptr() if wsz else None
    lib = pq2.lib
    # one launch (pq2_linear, quantisation inside the GEMV) where one_launch
    # says it measured faster; the two-launch step elsewhere (MI355X, M = 1
    # step: 2.28 ms this way, 2.34 with every projection in one launch, 2.39
    # with the down projection's as well as the two K <= 6144 ones)
    fused = tuple(one_launch(m, n, k) for (n, k) in synth.LAYER_SHAPES)
    calls = []
    for projs in layers:
        for i, (codes, ws, n, k) in enumerate(projs):
            q, s, t = bufs[k]
            calls.append((fused[i], xs[k].data_ptr(), q.data_ptr(), s.data_ptr(), t.data_ptr(),
                          codes.data_ptr(), ws.data_ptr(), ys[n].data_ptr(), n, k))
    quant, gemm, linear = lib.pq2_quantize_act, lib.pq2_gemm, lib.pq2_linear

    def step(after=None):
        for (fz, xp, qp, sp, tp, cp, wp, yp, n, k) in calls:
            if fz:
                linear(xp, cp, wp, yp, m, n, k, wkp, wsz, stream)
            else:
                quant(xp, qp, sp, tp, m, k, stream)
                gemm(qp, sp, tp, cp, wp, yp, m, n, k, wkp, wsz, stream)
            if after is not None:
                after()

    step.buffers = (layers, xs, bufs, ys, work)   # the launches hold raw pointers into these
    step.workspace_bytes = wsz
    step.fused = fused
    return step


def run_layers(args, m, torch, pq2, steps, trials):
    """64-layer synthetic decode step: per layer 4 PQ2_0 GEMMs (5 projections,
    gate and up stacked into one matrix), back to back on one stream (every
    weight matrix is read once per step, 5.6 GB)."""
    import pq2_synth as synth
    stream = torch.cuda.current_stream(torch.device("cuda:0")).cuda_stream
    step = layer_step(m, torch, pq2, stream)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    h = tm.host_ms(step)
    runs = [tm.run(step, h) for _ in range(trials)]
    ms = median(runs) / steps
    total = 0
    for i, (n, k) in enumerate(synth.LAYER_SHAPES):
        total += linear_bytes(m, n, k) if step.fused[i] else gemm_bytes(m, n, k) + quant_bytes(m, k)
    total *= synth.N_LAYERS
    gbs = total / (ms * 1e-3) / 1e9
    n_quant = sum(not f for f in step.fused)
    return {"metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": 2, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
            "config": {"workload": f"layer64_m{m}", "M": m, "layers": synth.N_LAYERS,
                       "projections_per_layer": 5,
                       "gemms_per_step": len(synth.LAYER_SHAPES) * synth.N_LAYERS,
                       "quantiser_launches_per_step": n_quant * synth.N_LAYERS,
                       "projection": "pq2_quantize_act + pq2_gemm, or pq2_linear where that "
                                     "is faster; gate and up stacked into one 34816 x 5120 "
                                     "matrix (they read the same activations)",
                       "fused_projections_per_layer": int(sum(step.fused)),
                       "algorithmic_bytes_per_step": total, "trials": trials,
                       "trial_ms": [round(v / steps, 4) for v in runs],
                       "workspace_bytes": step.workspace_bytes},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                         "note": "whole step incl. quantise launches and launch gaps"}}


# The pages' power proxy: a low-power spin after every matrix multiply stands in
# for the decode step's other work (norms, attention, recurrent updates,
# sampling), so that a replay of the projections runs at the clock and power state of
# serving rather than of back-to-back memory-bound kernels. The pages sized
# the spin from a serving trace (page "Making a ternary reasoning model fast
# in vLLM", section "A power proxy for the rest of the model"): 25k cycles at
# 2 tokens rising to 55k at 16, which they relate to the non-GEMM time of the
# trace at roughly 1.5 spin cycles per ns. Here the spin is that much time
# after each GEMM launch (the stacked gate and up projections are one).
def proxy_spin_us(m):
    cycles = 25000.0 + (min(max(m, 2), 16) - 2) * (55000.0 - 25000.0) / 14.0
    return cycles / 1.5 / 1000.0


def power_sampler(stop, out):
    """(start, end, socket power W, first graphics clock MHz) read with
    amd-smi, a child process per sample, until stop is set (nothing if it is
    missing)."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi")
    while exe and not stop.is_set():
        try:
            t0 = time.perf_counter()
            r = subprocess.run([exe, "metric", "-p", "-c", "--json"], capture_output=True,
                               text=True, timeout=10)
            d = json.loads(r.stdout)
            g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
            out.append((t0, time.perf_counter(), float(g["power"]["socket_power"]["value"]),
                        float(g["clock"]["gfx_0"]["clk"]["value"])))
        except (OSError, ValueError, KeyError, IndexError, TypeError,
                subprocess.SubprocessError):
            return


def run_proxy(args, m, torch, pq2):
    """The 64-layer step with a spin after every GEMM, captured once in a
    HIP graph and replayed back to back for --proxy-seconds. Kernel durations
    under the proxy come from a kernel trace of this run (the spin's wall time
    follows the clock, so the step time mixes the two); this line reports the
    replay itself."""
    dev = torch.device("cuda:0")
    cap = torch.cuda.Stream(dev)
    spin_us = proxy_spin_us(m) if args.proxy_spin_us is None else args.proxy_spin_us
    cyc_per_ms = spin_cycles_per_ms(torch)
    spin = int(cyc_per_ms * spin_us / 1000.0)
    import pq2_synth as synth
    step = layer_step(m, torch, pq2, cap.cuda_stream)
    after = (lambda: torch.cuda._sleep(spin)) if spin > 0 else None
    with torch.cuda.stream(cap):
        step(after)                 # eager run before capture (checks the launches)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(after)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    import threading
    stop, samples = threading.Event(), []
    sampler = threading.Thread(target=power_sampler, args=(stop, samples), daemon=True)
    sampler.start()
    replays, t0 = 0, time.perf_counter()
    a.record()
    while time.perf_counter() - t0 < args.proxy_seconds:
        for _ in range(10):
            g.replay()
        replays += 10
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = a.elapsed_time(b) / replays
    stop.set()
    sampler.join()
    inside = [(p, c) for (s0, s1, p, c) in samples if s0 >= t0 and s1 <= t1]
    power = None
    if inside:
        power = {"samples": len(inside), "socket_W_median": median([p for p, _ in inside]),
                 "gfx_MHz_median": median([c for _, c in inside]),
                 "source": "amd-smi metric -p -c, polled during the replay"}
    return {"proxy": {"workload": f"layer64_m{m}", "M": m, "spin_us_per_gemm": spin_us,
                      "spin_cycles": spin,
                      "gemms_per_step": len(synth.LAYER_SHAPES) * synth.N_LAYERS,
                      "replays": replays, "ms_per_replay": ms, "power": power,
                      "note": "HIP-graph replay of the 64-layer step with a spin after every "
                              "GEMM; GEMM kernel durations from a kernel trace of this run"}}


def layer_read_floor(torch, probes, m, steps=5, trials=5):
    """The 64-layer step's practical ceiling when every GEMM is its own launch:
    the step's launches in the step's order on one stream, each replaced by a
    plain streaming read of that launch's algorithmic bytes (a projection's
    codes, scales, activations and y; the quantiser's float32 activations),
    every projection reading its own slice of one buffer as large as the
    step's weights (so the reads come from HBM), with no arithmetic."""
    import pq2_synth as synth
    dev = torch.device("cuda:0")
    r16 = lambda b: (b + 15) // 16 * 16
    sizes = []
    for (n, k) in synth.LAYER_SHAPES:
        fused = one_launch(m, n, k)
        sizes.append((r16(linear_bytes(m, n, k) if fused else gemm_bytes(m, n, k)),
                      0 if fused else r16(4 * m * k)))
    per_layer = sum(g for g, _ in sizes)
    buf = torch.empty(per_layer * synth.N_LAYERS, dtype=torch.uint8, device=dev)
    small = torch.empty(r16(max(q for _, q in sizes) + 16), dtype=torch.uint8, device=dev)
    buf.fill_(1)
    small.fill_(1)
    big_blocks = probes.cus * 4
    launches, off = [], 0
    for _ in range(synth.N_LAYERS):
        for g, q in sizes:
            if q:
                launches.append((small.data_ptr(), q, max(1, min(big_blocks, q // 32768))))
            launches.append((buf.data_ptr() + off, g, big_blocks))
            off += g
    stream = torch.cuda.current_stream(dev).cuda_stream
    lib, sink = probes.lib, probes.sink.data_ptr()

    def step():
        for ptr, nb, blocks in launches:
            probes._ok(lib.pq2_probe_stream_read(ptr, nb, sink, blocks, stream), "stream_read")
    step()
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    h = tm.host_ms(step)
    ms = median([tm.run(step, h) for _ in range(trials)]) / steps
    total = sum(nb for _, nb, _ in launches)
    del buf, small
    return {"ms_per_step": ms, "GB/s": total / (ms * 1e-3) / 1e9, "bytes_per_step": total,
            "launches_per_step": len(launches)}


def run_ceiling(torch):
    """Practical ceilings of one MI355X: a plain streaming read at several
    sizes (slices cycling through 1 GiB), the 64-layer step's launches as
    plain reads, the launch floor, the int8 MFMA loop and the exact-epilogue
    instruction mix."""
    probes = Probes(torch)
    reads = []
    for mib in (8, 24, 64, 256):
        nbytes = mib << 20
        print(f"# stream read {mib} MiB", file=sys.stderr, flush=True)
        reads.append(probes.stream_read(nbytes, 1 << 30, calls=max(4, 800 // mib)))
    floors = {}
    for m in (1, 16):
        print(f"# 64-layer step read floor, M = {m}", file=sys.stderr, flush=True)
        floors[f"layer64_m{m}"] = layer_read_floor(torch, probes, m)
        torch.cuda.empty_cache()
    print("# launch floor", file=sys.stderr, flush=True)
    lf = probes.launch_floor()
    print("# int8 MFMA loop", file=sys.stderr, flush=True)
    mf = probes.mfma_i8()
    print("# int8 MFMA with the float32 epilogue mix", file=sys.stderr, flush=True)
    em = probes.epilogue_mix()
    return {"ceiling": {"stream_read": reads, "layer_read_floor": floors, "launch_floor_us": lf,
                        "mfma_i8": mf,
                        "epilogue_mix": em,
                        "hbm_peak_GB/s": HBM_PEAK_GBS, "i8_peak_TOP/s": I8_PEAK_TOPS}}


def extras(args, wl, r, torch, pq2, probes):
    """Figures the default line carries beside its own workload: the prefill
    half of the metric (M = 4096, N = 17408, K = 5120, int8 TOP/s), the
    64-layer decode step at one token row (whole-step HBM GB/s), and the
    practical ceilings the kernels are compared with."""
    import pq2_synth as synth
    out = {}
    print("# extras: prefill m4096 n17408", file=sys.stderr, flush=True)
    pw = synth.prefill(4096, 17408, 5120)
    pr = run_gemm(args, pw, torch, pq2, max(1, min(args.steps, 20)), args.trials, probes)
    ops = gemm_ops(pw.m, pw.n, pw.k)
    tops = ops / (pr["kernel_ms"] * 1e-3) / 1e12
    out[pw.name] = {"pq2_gemm_us": pr["kernel_ms"] * 1e3, "kernel": pr["path"],
                    "TOP/s": tops, "frac_i8_peak": tops / I8_PEAK_TOPS,
                    "step_us": pr["ms_step"] * 1e3,
                    "sclk_mhz_during_pq2_gemm": pr.get("sclk_mhz"),
                    "trial_pq2_gemm_us": [round(v, 2) for v in pr["trial_gemm_us"]]}
    torch.cuda.empty_cache()
    print("# extras: layer64 m1", file=sys.stderr, flush=True)
    lr = run_layers(args, 1, torch, pq2, 5, args.trials)
    out["layer64_m1"] = {"ms_per_step": lr["ms_per_step"], "GB/s": lr["value"],
                         "frac_hbm_peak": lr["value"] / HBM_PEAK_GBS,
                         "algorithmic_bytes_per_step": lr["config"]["algorithmic_bytes_per_step"],
                         "trial_ms": lr["config"]["trial_ms"]}
    torch.cuda.empty_cache()
    print("# extras: layer64 m1 read floor", file=sys.stderr, flush=True)
    fl = layer_read_floor(torch, probes, 1)
    out["layer64_m1"]["read_floor_ms"] = fl["ms_per_step"]
    out["layer64_m1"]["read_floor_launches"] = fl["launches_per_step"]
    out["layer64_m1"]["step_time_over_read_floor"] = lr["ms_per_step"] / fl["ms_per_step"]
    torch.cuda.empty_cache()
    if r is not None and r["M"] <= 16:
        print("# extras: ceilings", file=sys.stderr, flush=True)
        nb = gemm_bytes(r["M"], r["N"], r["K"])
        sr = probes.stream_read(nb, 1 << 30, calls=max(20, min(args.steps, 200)))
        sr["pq2_gemm_time_over_read_time"] = r["kernel_ms"] * 1e3 / sr["us"]
        out["stream_read_same_bytes"] = sr
        out["launch_floor_us"] = probes.launch_floor()
    out["mfma_i8_loop"] = probes.mfma_i8()
    out["mfma_i8_with_epilogue_mix"] = probes.epilogue_mix()
    return out


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
                    help="spin per GEMM (default: the pages' calibration for M; 0: none)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise kernel (y = 2x, float32) over MIB MiB, "
                         "the calibration for HBM byte counters")
    ap.add_argument("--trials", type=int, default=5, help="timed trials (the median is reported)")
    ap.add_argument("--no-extras", action="store_true",
                    help="default line only: skip the prefill, 64-layer and ceiling figures")
    ap.add_argument("--ceiling", action="store_true",
                    help="only print the practical ceilings: streaming reads of several sizes "
                         "and the int8 MFMA loop (libpq2_probe.so)")
    args = ap.parse_args()
    if args.steps < 1 or args.trials < 1 or args.warmup < 0:
        ap.error("--steps and --trials must be positive, --warmup not negative")

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

    if args.ceiling:
        print(json.dumps(run_ceiling(torch)), flush=True)
        return

    import gemm_pq2_w2a8_amd as pq2

    if args.proxy:
        print(json.dumps(run_proxy(args, args.proxy, torch, pq2)), flush=True)
        return

    wls = workload_list()
    names = list(wls) if args.sweep else [args.workload]
    probes = Probes(torch)
    for name in names:
        kind, wl = wls[name]
        print(f"# running {name}", file=sys.stderr, flush=True)
        if kind == "gemm":
            r = run_gemm(args, wl, torch, pq2, args.steps, args.trials, probes)
            line = report_gemm(args, wl, r, torch)
        else:
            line = run_layers(args, wl, torch, pq2, max(1, args.steps // 40), args.trials)
        torch.cuda.empty_cache()
        if not args.sweep and not args.no_extras:
            line["config"]["also"] = extras(args, wl, r if kind == "gemm" else None, torch, pq2,
                                            probes)
        print(json.dumps(line), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
