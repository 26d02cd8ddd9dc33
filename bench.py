"""Benchmark: TFLOP/s and fraction of the MI355X dense fp16 MFMA peak for the fp16 GEMM
(fp32 accumulation, optional fused bias + erf-GELU epilogue).

One step = one ``mi355gemm_gemm`` call on the headline workload (M = N = K = 2048, A, B ~
N(0, 1), no epilogue), inputs resident in HBM.  The JSON line also carries the other
workloads (2048^3 + bias + GELU, the ragged 1000 x 3000 x 777 case, 8192^3 with and without
the epilogue, 256^3), the roofline of the kernel and the CPU oracle timed on this host.

TFLOP/s counts 2*M*N*K per GEMM, as the tutorial does (thecryptopost.io page, section 2:
flops = 2 * M * N * K); the epilogue's arithmetic is not counted.  Latency is measured
with device events on the stream the kernels run on, as the tutorial's bench() measures
with CUDA events (aitrending.vip page, "Benchmarking & Verification").  The step time
(`value`, `ms_per_step`) is wall clock between synchronisations around back-to-back calls,
launch gaps included; the roofline uses the kernel's own mean duration from the pair of
HIP events each launch records as its kernel starts and ends (mi355gemm_gemm_timed), the
duration a rocprofv3 kernel trace reports.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-extra] [--config NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = ("TFLOP/s and % of MI355X fp16 MFMA peak, fp16 GEMM 2048³ & 8192³ "
          "(+bias+GELU)")
HEADLINE = "gemm_2048"

# HBM bytes per dispatch of the headline kernel: rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE,
# each scaled by what the same counter reads for a plain copy of known size (the
# --calibrate-copy run).  Reported only while the kernel sources hash to the version the
# counters were taken on (profiles/ holds the summary); otherwise null.
TRAFFIC = {"kernel_config": "d128x128x32_w2x2_l4_s4", "sources_sha256_16": "770356e2ca61873a",
           "bytes": 58810743}


# The files whose text defines the GEMM kernels (the configuration name fixes the template
# arguments); the counters above stand only while their code is unchanged.
GEMM_KERNEL_SOURCES = ("gemm_common.hpp", "gemm_direct.hpp", "gemm_staged.hpp", "gemm_pingpong.hpp")


def code_text(source: str) -> str:
    """The source with // comments, trailing blanks and empty lines removed, so that a
    change to the comments alone keeps the hash (the kernels have no string literal
    holding //)."""
    lines = (line.split("//", 1)[0].rstrip() for line in source.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_fp16_gemm_fp32_amd", "csrc", name)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


# The same counters for the other tiles of the same area a calibrated run may take at
# 2048^3 (each forced with --config; profiles/ holds the summary).
TRAFFIC_OTHER = {"sources_sha256_16": "770356e2ca61873a",
                 "bytes": {"d128x128x64_w2x2_l4_s4": 58839365, "d128x128x64_w2x2_s4": 58900814,
                           "d128x128x64_w2x2k2_s4": 58831249, "d128x128x32_w2x2_s4": 58848567,
                           "d128x128x64_w2x4_s4": 58836317, "d64x256x32_w1x4_s4": 58841467}}


def traffic_for(kernel_config: str):
    h = kernel_sources_hash()
    if TRAFFIC and TRAFFIC["kernel_config"] == kernel_config and TRAFFIC["sources_sha256_16"] == h:
        return TRAFFIC["bytes"]
    if TRAFFIC_OTHER["sources_sha256_16"] == h:
        return TRAFFIC_OTHER["bytes"].get(kernel_config)
    return None


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-ms", type=float, default=MIN_WARMUP_MS,
                    help="keep warming up past --warmup calls until this many milliseconds "
                         "have passed (0: exactly --warmup calls)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--epilogue", default=None, help="override the workload's epilogue")
    ap.add_argument("--dist", default=None,
                    help="override the headline workload's operand distribution (e.g. zeros, to "
                         "show what the operand values cost under the power limit)")
    ap.add_argument("--config", default=None, help="force a kernel configuration by name")
    ap.add_argument("--no-calibrate", dest="calibrate", action="store_false",
                    help="time the selector's own choice; by default each GEMM workload first "
                         "times the configurations of its tile area on this device and installs the "
                         "fastest (tune.calibrate), since some tiles run up to 25%% slower on "
                         "some MI355X boxes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--gemm-only", action="store_true",
                    help="extra GEMM workloads only (no vector add, softmax, attention, cold run)")
    ap.add_argument("--no-gemm-extras", action="store_true",
                    help="skip the extra GEMM workloads and the cold run (profiling the other kernels)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-clock", dest="clock", action="store_false",
                    help="skip the sustained window per GEMM workload that reads the engine "
                         "clock and socket power from amd-smi (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration for rocprofv3)")
    return ap.parse_args(argv)


# Untimed warm-up lasts at least this long by default.  After a pause the engine clock
# needs tens of milliseconds of load to settle: on MI355X the 2048^3 step took 25.2 us
# after 20 warm-up calls (0.5 ms) and 21.6 us after 2000 (45 ms); 8192^3 926 us after 20
# and 902 us after 2000.
MIN_WARMUP_MS = 100.0


def warm_up(fn, calls, min_ms):
    """`calls` untimed calls of fn, then more until at least `min_ms` milliseconds have
    passed since the first, so the timed region starts on a settled clock.  Returns the
    number of calls made."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(calls):
        fn()
        n += 1
    torch.cuda.synchronize()
    while True:
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms:
            return n
        batch = 1 if n == 0 else max(1, min(100000, int((min_ms - el) / (el / n)) + 1))
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()


def time_gemm(lib, A, B, bias, epi, out, steps, warmup, config=None, min_warm_ms=0.0):
    """Three timed passes of `steps` calls each, after `warmup` untimed calls (and more,
    up to `min_warm_ms` milliseconds of them, see warm_up).

    Pass 1 (the step and kernel time): wall clock between synchronisations around the
    back-to-back calls, and HIP events at both ends of the same region on the stream the
    kernels are launched on; the event time per call is the kernel's average launch
    duration, which the roofline uses (a rocprofv3 kernel trace of the same back-to-back
    calls reads within a few percent of it).
    Pass 2: every launch records its own pair of HIP events from the kernel dispatch
    (mi355gemm_gemm_timed), as the kernel starts and as it ends.  Kept for reference
    only: the per-launch signalling it adds has read from 1% to 17% above the
    back-to-back time from run to run, and over 60% above it under a profiler.
    Pass 3: an event pair recorded on the stream around every call; it also counts the
    dispatch latency of each launch.
    Returns (ms per step by wall clock, ms per step by events, mean, median and minimum
    ms per launch from pass 2, mean ms per call from pass 3, warm-up calls made)."""
    import torch
    stream = torch.cuda.current_stream()
    warm = warm_up(lambda: lib.gemm(A, B, bias, epi, out=out, config=config), warmup, min_warm_ms)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        lib.gemm(A, B, bias, epi, out=out, config=config)
    stop.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    event_ms = start.elapsed_time(stop) / steps

    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for a, b in pairs:              # creates the HIP events the launches re-record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for a, b in pairs:
        lib.gemm(A, B, bias, epi, out=out, config=config, events=(a, b))
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in pairs)
    kernel_ms = sum(per) / steps

    for a, b in pairs:
        a.record(stream)
        lib.gemm(A, B, bias, epi, out=out, config=config)
        b.record(stream)
    torch.cuda.synchronize()
    call_ms = sum(a.elapsed_time(b) for a, b in pairs) / steps
    return wall_ms, event_ms, kernel_ms, per[len(per) // 2], per[0], call_ms, warm


def time_graph(lib, A, B, bias, epi, out, calls=100, replays=20, min_warm_ms=MIN_WARMUP_MS):
    """`calls` back-to-back calls captured in one HIP graph, replayed `replays` times
    after a warm-up: ms per call without the per-call host work of the binding."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.gemm(A, B, bias, epi, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            lib.gemm(A, B, bias, epi, out=out)
    warm_up(graph.replay, 1, min_warm_ms)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * calls)


def _sha16(t) -> str:
    """First 16 hex digits of the sha256 of a CPU fp16 tensor's bytes."""
    import hashlib
    import torch
    return hashlib.sha256(t.contiguous().view(-1).view(torch.int16).numpy().tobytes()).hexdigest()[:16]


def inputs_sha256(w, epi) -> dict:
    """sha256 (first 16 hex digits) of the fp16 bytes of every input of the workload."""
    import workloads
    A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=(epi != "none"), seed=w.seed)
    out = {"A": _sha16(A), "B": _sha16(B)}
    if bias is not None:
        out["bias"] = _sha16(bias)
    return out


def run_cold(lib, w, steps, min_warm_ms=MIN_WARMUP_MS, min_bytes=256 << 20):
    """The workload with cold caches: enough copies of A and B (more than min_bytes in
    all, past the L2s and the Infinity Cache) that each call reads operands the previous
    calls did not touch; kernel time per launch from HIP events around back-to-back calls."""
    import torch
    import workloads
    A, B, _ = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=False, seed=w.seed)
    per_copy = 2 * (A.numel() + B.numel())
    n = max(2, -(-min_bytes // per_copy) + 1)
    As = [A.to("cuda:0") for _ in range(n)]
    Bs = [B.to("cuda:0") for _ in range(n)]
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda:0")
    stream = torch.cuda.current_stream()
    turn = [0]

    def call():
        lib.gemm(As[turn[0] % n], Bs[turn[0] % n], out=out)
        turn[0] += 1
    warm_up(call, n, min_warm_ms)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    stop.record(stream)
    torch.cuda.synchronize()
    mean = start.elapsed_time(stop) / steps
    return {"workload": w.name + "_cold", "copies": n, "bytes_rotated": n * per_copy,
            "kernel_us": mean * 1e3, "tflops": w.flops / (mean * 1e-3) / 1e12}


RESIDENCY_KEYS = ("accumulation_counter", "ppt_residency_acc", "socket_thm_residency_acc",
                  "vr_thm_residency_acc", "hbm_thm_residency_acc", "prochot_residency_acc")


class ClockSampler:
    """Engine clock and socket power as the driver reports them (amd-smi's GPU metrics:
    current_gfxclks per XCD in MHz, current_socket_power in W, and the power limit),
    sampled from a background thread while GEMM calls run.  The driver refreshes these
    metrics only every few hundred milliseconds, so a reading needs a sustained window of
    calls (measure()), not the short timed region.  None where amd-smi is unavailable."""

    def __init__(self):
        self.smi = None
        self.handle = None
        self.power_limit_w = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self.smi = amdsmi
            info = amdsmi.amdsmi_get_power_info(self.handle)
            lim = info.get("power_limit")
            if isinstance(lim, (int, float)) and lim > 0:
                # reported in microwatts by this driver
                self.power_limit_w = lim / 1e6 if lim > 1e5 else float(lim)
        except Exception:
            self.smi = None

    def read(self):
        if self.smi is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        except Exception:
            return None
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        power = m.get("current_socket_power")
        num = lambda v: v if isinstance(v, (int, float)) else None
        return {"ts": m.get("firmware_timestamp") or m.get("system_clock_counter"),
                "gfxclk_mhz": sum(clks) / len(clks) if clks else None,
                "gfxclk_mhz_min": min(clks) if clks else None,
                "gfxclk_mhz_max": max(clks) if clks else None,
                "socket_power_w": num(power),
                # cumulative counters: time in power-limit (PPT) and thermal throttling,
                # on the firmware's accumulation time base
                "acc": {k: num(m.get(k)) for k in RESIDENCY_KEYS}}

    def measure(self, fn, seconds=3.0, per_call_s=1e-5):
        """Runs fn back to back for about `seconds` while sampling every 10 ms; returns the
        median of the readings the driver refreshed after the first third of the window
        (the clock has settled by then; a reading still unchanged from before is dropped),
        or None."""
        import statistics
        import threading
        import torch
        if self.smi is None:
            return None
        stop = [False]
        samples = []

        def sampler():
            t0 = time.perf_counter()
            while not stop[0]:
                r = self.read()
                if r is not None:
                    samples.append((time.perf_counter() - t0, r))
                time.sleep(0.01)
        th = threading.Thread(target=sampler, daemon=True)
        th.start()
        t0 = time.perf_counter()
        batch = max(1, int(0.02 / per_call_s))
        while time.perf_counter() - t0 < seconds:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
        stop[0] = True
        th.join()
        key = lambda r: (r["ts"], r["gfxclk_mhz"], r["socket_power_w"])
        early = {key(r) for t, r in samples if t < seconds / 3}
        late = [r for t, r in samples if t >= seconds / 3 and r["gfxclk_mhz"] is not None]
        fresh, seen = [], set(early)
        for r in late:                      # one reading per driver refresh after settling
            if key(r) not in seen:
                seen.add(key(r))
                fresh.append(r)
        if not fresh:
            return None
        med = lambda k: statistics.median(r[k] for r in fresh if r[k] is not None)
        # fraction of the settled part of the window spent throttled, by cause: the
        # residency counters' increase over the accumulation counter's
        residency = None
        first = next((r for t, r in samples if t >= seconds / 3), None)
        last = samples[-1][1] if samples else None
        if first is not None and last is not None:
            a0, a1 = first["acc"], last["acc"]
            span = (a1["accumulation_counter"] or 0) - (a0["accumulation_counter"] or 0)
            if span > 0:
                residency = {k.replace("_residency_acc", ""): (a1[k] - a0[k]) / span
                             for k in RESIDENCY_KEYS[1:]
                             if a0[k] is not None and a1[k] is not None}
        return {"gfxclk_mhz": med("gfxclk_mhz"), "gfxclk_mhz_min": min(r["gfxclk_mhz_min"] for r in fresh),
                "gfxclk_mhz_max": max(r["gfxclk_mhz_max"] for r in fresh),
                "socket_power_w": med("socket_power_w"), "power_limit_w": self.power_limit_w,
                "throttle_residency": residency,
                "readings": len(fresh), "window_s": seconds}


def clock_text(clock) -> str:
    if not clock:
        return ""
    return "; held %.0f MHz at %s W (limit %s W), kernel at %.2f of the held-clock peak" % (
        clock["gfxclk_mhz"], clock["socket_power_w"], clock["power_limit_w"],
        clock.get("kernel_frac_of_held_clock_peak") or float("nan"))


def held_clock_peak(cus, mhz):
    """Dense fp16 MFMA peak at the engine clock held under load: CUs x 4096 flop/clk."""
    return cus * 4096 * mhz * 1e6 / 1e12 if mhz else None


def derived_peak():
    """CUs x 4096 flop/clk x the highest engine clock the driver lists (sysfs
    pp_dpm_sclk), next to the published 2.5 PFLOP/s; None where unreadable."""
    import glob
    import re
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mhz = None
    for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            vals = [int(m) for m in re.findall(r"(\d+)\s*Mhz", open(f).read(), flags=re.I)]
        except OSError:
            continue
        if vals:
            mhz = max(mhz or 0, max(vals))
    return {"cus": cus, "max_sclk_mhz": mhz,
            "tflops": cus * 4096 * mhz * 1e6 / 1e12 if mhz else None,
            "published_tflops": PEAK_FP16_TFLOPS}


def cpu_oracle_by_workload(max_gflop=20.0):
    """The CPU oracle on every workload: the full product where it costs at most
    max_gflop, else the first rows of A (a row block, the same per-row work) scaled to
    GFLOP/s; plus one-thread timings of the small and the ragged workload."""
    import oracle
    import workloads
    lib = oracle.load()
    threads = oracle.num_threads(lib)
    out = []
    for w in workloads.WORKLOADS:
        epi = w.epilogues[-1]
        A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=(epi != "none"), seed=w.seed)
        rows = w.M if w.flops <= max_gflop * 1e9 else max(1, int(max_gflop * 1e9 // (2 * w.N * w.K)))
        runs = [(threads, "threads")]
        if w.name in ("gemm_256", "gemm_ragged_1000x3000x777"):
            runs.append((1, "one_thread"))
        rec = {"workload": w.name, "epilogue": epi, "rows": rows}
        for n, key in runs:
            oracle.set_num_threads(n, lib)
            t0 = time.perf_counter()
            oracle.gemm(A[:rows].contiguous(), B, bias, epi, lib=lib)
            el = time.perf_counter() - t0
            rec[key] = {"threads": n, "seconds": el, "gflops": 2.0 * rows * w.N * w.K / el / 1e9}
        oracle.set_num_threads(threads, lib)
        out.append(rec)
    return out


def run_workload(lib, w, epi, steps, warmup, config=None, min_warm_ms=MIN_WARMUP_MS,
                 calibrate=False, sampler=None):
    import torch
    import workloads
    A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=(epi != "none"), seed=w.seed)
    dev = torch.device("cuda:0")
    A, B = A.to(dev), B.to(dev)
    bias = bias.to(dev) if bias is not None else None
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    calibration = None
    if calibrate and config is None:
        from dense_fp16_gemm_fp32_amd import tune
        calibration = tune.calibrate(A, B, bias, epi, out=out)[1]
    cid = lib.select(A, B, bias, epi, out=out) if config is None else lib.config_id(config)
    wall_ms, event_ms, disp_ms, disp_med, disp_min, call_ms, warm = time_gemm(
        lib, A, B, bias, epi, out, steps, warmup, config, min_warm_ms)
    kernel_ms = event_ms   # the back-to-back event time per launch
    tflops = w.flops / (wall_ms * 1e-3) / 1e12
    # launch-bound sizes: the same calls replayed from a captured graph
    graph_ms = time_graph(lib, A, B, bias, epi, out, min_warm_ms=min_warm_ms) if w.M <= 256 else None
    clock = None
    if sampler is not None and w.M > 256:
        clock = sampler.measure(lambda: lib.gemm(A, B, bias, epi, out=out, config=config),
                                per_call_s=kernel_ms * 1e-3)
        if clock is not None:
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            clock["held_clock_peak_tflops"] = held_clock_peak(cus, clock["gfxclk_mhz"])
            clock["kernel_frac_of_held_clock_peak"] = (
                w.flops / (kernel_ms * 1e-3) / 1e12 / clock["held_clock_peak_tflops"])
    return {
        "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": epi,
        "kernel_config": lib.mi355gemm_config_name(cid),
        "calibration_us": calibration,
        "ms": wall_ms, "us": wall_ms * 1e3, "tflops": tflops,
        "pct_of_peak": 100.0 * tflops / PEAK_FP16_TFLOPS,
        "event_us": event_ms * 1e3,
        "kernel_us": kernel_ms * 1e3,
        "dispatch_event_us": disp_ms * 1e3,
        "dispatch_event_median_us": disp_med * 1e3,
        "dispatch_event_min_us": disp_min * 1e3,
        "call_event_pair_us": call_ms * 1e3,
        "warmup_calls": warm,
        "graph_us_per_call": graph_ms * 1e3 if graph_ms is not None else None,
        # engine clock and socket power over a sustained window of the same calls
        "clock": clock,
        "inputs_sha256_16": inputs_sha256(w, epi),
        "kernel_tflops": w.flops / (kernel_ms * 1e-3) / 1e12,
        "algorithmic_GBps": w.algorithmic_bytes(epi) / (kernel_ms * 1e-3) / 1e9,
        "steps": steps,
    }


def run_vector_add(lib, n, steps, warmup, min_warm_ms=MIN_WARMUP_MS):
    """The tutorial's first kernel at n elements: c = a + b (fp16), 6 bytes per element.
    Its GB/s is the measured HBM roofline the GEMM's traffic figures are read against;
    torch's own a + b on the same tensors is timed beside it as context."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(0)
    a = torch.randn(n, generator=gen, dtype=torch.float32).to(torch.float16).to("cuda:0")
    b = torch.randn(n, generator=gen, dtype=torch.float32).to(torch.float16).to("cuda:0")
    c = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    out = {"workload": "vector_add", "n": n, "bytes": 6 * n}
    for name, fn in (("mi355gemm", lambda: lib.vector_add(a, b, out=c)),
                     ("torch", lambda: torch.add(a, b, out=c))):
        warm_up(fn, warmup, min_warm_ms)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = 6.0 * n / (ms * 1e-3) / 1e9
        if name == "mi355gemm":
            out.update({"us": ms * 1e3, "GBps": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS})
        else:
            out["torch_GBps"] = gbs
    return out


def run_softmax(lib, M, N, steps, warmup, min_warm_ms=MIN_WARMUP_MS):
    """The tutorial's row-wise softmax on an M x N fp16 matrix (N(0, 3^2) entries, seed 0):
    4 bytes move per element (one read, one write), so its GB/s reads against HBM peak."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(0)
    x = (torch.randn(M, N, generator=gen, dtype=torch.float32) * 3).to(torch.float16).to("cuda:0")
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    fn = lambda: lib.softmax(x, out=y)
    warm_up(fn, warmup, min_warm_ms)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = 4.0 * M * N / (ms * 1e-3) / 1e9
    return {"workload": "softmax", "M": M, "N": N, "bytes": 4 * M * N, "us": ms * 1e3,
            "GBps": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


def attention_flops(B, H, Sq, Sk, D, causal):
    """4 D flops (two products) per query-key pair the mask allows; causal allows
    min(i + 1, Sk) keys to query i (upper-left aligned)."""
    if causal:
        n = min(Sq, Sk)
        pairs = n * (n + 1) // 2 + max(0, Sq - Sk) * Sk
    else:
        pairs = Sq * Sk
    return 4.0 * B * H * D * pairs


def run_attention(lib, B, H, S, D, causal, steps, warmup, min_warm_ms=MIN_WARMUP_MS):
    """The tutorial's FlashAttention forward on (B, H, S, D) fp16 tensors, N(0,1) seed 0,
    scale 1/sqrt(D)."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(0)
    q, k, v = (torch.randn((B, H, S, D), generator=gen).to(torch.float16).to("cuda:0")
               for _ in range(3))
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    flops = attention_flops(B, H, S, S, D, causal)
    fn = lambda: lib.attention(q, k, v, causal=causal, out=o)
    warm_up(fn, warmup, min_warm_ms)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "attention", "batch": B, "heads": H, "seq": S, "head_dim": D,
            "causal": causal, "flops": flops, "us": ms * 1e3, "tflops": tf,
            "frac_of_fp16_peak": tf / PEAK_FP16_TFLOPS}


def host_info():
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": cpu, "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def calibrate_copy(reps=5, mib=256):
    """A plain device-to-device copy of known size (mib MiB read, mib MiB written), for
    scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("bench: calibration copy of %d MiB x %d done" % (mib, reps), file=sys.stderr, flush=True)


def cpu_baseline(w, epi, seconds):
    """The CPU oracle (untuned) on this host: the full product of the workload, repeated
    for about `seconds` of wall time."""
    import oracle
    import workloads
    A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=(epi != "none"), seed=w.seed)
    lib = oracle.load()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(A, B, bias, epi, lib=lib)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tflops = w.flops * reps / el / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(lib),
            "kind": "oracle",
            "sample": "full %dx%dx%d product (%s), %d repetition(s) in %.1f s, fp64 accumulation"
                      % (w.M, w.N, w.K, epi, reps, el)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import dense_fp16_gemm_fp32_amd as lib
    import workloads

    lib.library()  # fails loudly if the HIP library is not built
    w = workloads.BY_NAME[args.workload]
    if args.dist:
        import dataclasses
        w = dataclasses.replace(w, dist=args.dist)
    epi = args.epilogue or w.epilogues[0]
    print("bench: %s epilogue=%s steps=%d warmup=%d" % (w.name, epi, args.steps, args.warmup),
          file=sys.stderr, flush=True)
    sampler = ClockSampler() if args.clock else None
    head = run_workload(lib, w, epi, args.steps, args.warmup, args.config, args.min_warmup_ms,
                        args.calibrate, sampler)
    print("bench: headline %.2f us/step (events %.2f us per launch), %.1f TFLOP/s; per-launch "
          "dispatch events %.2f us%s"
          % (head["us"], head["event_us"], head["tflops"], head["dispatch_event_us"],
             clock_text(head["clock"])),
          file=sys.stderr, flush=True)
    if args.calibrate_copy:
        calibrate_copy()

    extra = []
    if not args.no_extra and not args.no_gemm_extras:
        for ew in workloads.WORKLOADS:
            for e in ew.epilogues:
                if ew.name == w.name and e == epi:
                    continue
                steps = 20 if ew.M >= 8192 else (1000 if ew.M <= 256 else 200)
                r = run_workload(lib, ew, e, steps, 10, min_warm_ms=args.min_warmup_ms,
                                 calibrate=args.calibrate, sampler=sampler)
                print("bench: %s %s %.2f us/step, kernel %.2f us, %.1f TFLOP/s%s%s"
                      % (ew.name, e, r["us"], r["kernel_us"], r["tflops"],
                         "" if r["graph_us_per_call"] is None
                         else ", %.2f us/call from a graph" % r["graph_us_per_call"],
                         clock_text(r["clock"])),
                      file=sys.stderr, flush=True)
                extra.append(r)

    others = not args.no_extra and not args.gemm_only
    vadd = None
    if others:
        vadd = run_vector_add(lib, 1 << 28, 50, 5, args.min_warmup_ms)
        print("bench: vector_add n=2^28 %.2f us %.1f GB/s (torch %.1f GB/s)"
              % (vadd["us"], vadd["GBps"], vadd["torch_GBps"]), file=sys.stderr, flush=True)

    softmax = []
    if others:
        for (M, N) in ((8192, 8192), (4096, 4096), (64, 65536)):
            r = run_softmax(lib, M, N, 100, 5, args.min_warmup_ms)
            print("bench: softmax %dx%d %.2f us %.1f GB/s" % (M, N, r["us"], r["GBps"]),
                  file=sys.stderr, flush=True)
            softmax.append(r)

    attention = []
    if others:
        for (D, causal) in ((128, False), (128, True), (64, False), (64, True)):
            r = run_attention(lib, 4, 32, 4096, D, causal, 20, 3, args.min_warmup_ms)
            print("bench: attention 4x32x4096 d%d %s %.1f us %.1f TFLOP/s"
                  % (D, "causal" if causal else "full", r["us"], r["tflops"]),
                  file=sys.stderr, flush=True)
            attention.append(r)

    cold = None
    if others and not args.no_gemm_extras:
        cold = run_cold(lib, w, 200, args.min_warmup_ms)
        print("bench: %s %.2f us/launch over %d input copies (%.0f MiB)"
              % (cold["workload"], cold["kernel_us"], cold["copies"], cold["bytes_rotated"] / 2**20),
              file=sys.stderr, flush=True)

    cpu = None
    cpu_all = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, epi, args.cpu_seconds)
        if others:
            cpu_all = cpu_oracle_by_workload()

    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "min_warmup_ms": args.min_warmup_ms,
        "warmup_calls": head["warmup_calls"],
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": epi,
                   "inputs": "%s seed %d" % (w.dist, w.seed),
                   "kernel_config": head["kernel_config"],
                   "calibrated": head["calibration_us"] is not None},
        "pct_of_peak": head["pct_of_peak"],
        "event_ms_per_step": head["event_us"] * 1e-3,
        "kernel_us": head["kernel_us"],
        "calibration_us": head["calibration_us"],
        "dispatch_event_us": head["dispatch_event_us"],
        "dispatch_event_median_us": head["dispatch_event_median_us"],
        "dispatch_event_min_us": head["dispatch_event_min_us"],
        "call_event_pair_us": head["call_event_pair_us"],
        # the dominant (only) kernel: 2*M*N*K flops per launch over its average launch
        # duration, HIP events around the timed back-to-back launches on their stream
        "roofline": {"bound": "mfma", "achieved": head["kernel_tflops"],
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": head["kernel_tflops"] / PEAK_FP16_TFLOPS,
                     "traffic": traffic_for(head["kernel_config"]),
                     # the same kernel against the MFMA peak at the engine clock the part
                     # held under this load (power-limited with random fp16 operands)
                     "held_clock_mhz": (head["clock"] or {}).get("gfxclk_mhz"),
                     "held_clock_peak": (head["clock"] or {}).get("held_clock_peak_tflops"),
                     "frac_of_held_clock_peak": (head["clock"] or {}).get("kernel_frac_of_held_clock_peak")},
        "clock": head["clock"],
        "cpu_baseline": cpu,
        "cpu_oracle_by_workload": cpu_all,
        "host": host_info(),
        "cold": cold,
        "peak_derived": derived_peak(),
        "memory_roofline": vadd,
        "softmax": softmax,
        "attention": attention,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count},
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
