"""Benchmark: TFLOP/s and fraction of the MI355X dense fp16 MFMA peak for the fp16 GEMM
(fp32 accumulation, optional fused bias + erf-GELU epilogue).

One step = one ``mi355gemm_gemm`` call on the headline workload (M = N = K = 2048, A, B ~
N(0, 1), no epilogue), inputs resident in HBM.  The JSON line also carries the other
workloads (2048^3 + bias + GELU, the ragged 1000 x 3000 x 777 case, 8192^3 with and without
the epilogue, 256^3), the roofline of the kernel and the CPU oracle timed on this host.

TFLOP/s counts 2*M*N*K per GEMM, as the tutorial does (thecryptopost.io page, section 2:
flops = 2 * M * N * K); the epilogue's arithmetic is not counted.  Latency is measured
with device events on the stream the kernels run on, as the tutorial's bench() measures
with CUDA events (aitrending.vip page, "Benchmarking & Verification").

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

# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE per dispatch of the headline kernel, KiB, and
# the copy-kernel calibration factor; filled from the committed profiles (None until the
# counters are taken on the current kernel).
TRAFFIC_BYTES = None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--epilogue", default=None, help="override the workload's epilogue")
    ap.add_argument("--config", default=None, help="force a kernel configuration by name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def time_gemm(lib, A, B, bias, epi, out, steps, warmup, config=None):
    """Average device time per call (ms) over `steps` back-to-back calls, bracketed by
    synchronisations, measured with events on the launch stream."""
    import torch
    for _ in range(warmup):
        lib.gemm(A, B, bias, epi, out=out, config=config)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        lib.gemm(A, B, bias, epi, out=out, config=config)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def run_workload(lib, w, epi, steps, warmup, config=None):
    import torch
    import workloads
    A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=(epi != "none"), seed=w.seed)
    dev = torch.device("cuda:0")
    A, B = A.to(dev), B.to(dev)
    bias = bias.to(dev) if bias is not None else None
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    cid = lib.select(A, B, bias, epi, out=out) if config is None else lib.config_id(config)
    ms, wall = time_gemm(lib, A, B, bias, epi, out, steps, warmup, config)
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes(epi) / (ms * 1e-3) / 1e9
    return {
        "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": epi,
        "kernel_config": lib.mi355gemm_config_name(cid),
        "ms": ms, "us": ms * 1e3, "tflops": tflops,
        "pct_of_peak": 100.0 * tflops / PEAK_FP16_TFLOPS,
        "algorithmic_GBps": gbs, "steps": steps, "wall_s": wall,
    }


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
    epi = args.epilogue or w.epilogues[0]
    print("bench: %s epilogue=%s steps=%d warmup=%d" % (w.name, epi, args.steps, args.warmup),
          file=sys.stderr, flush=True)
    head = run_workload(lib, w, epi, args.steps, args.warmup, args.config)
    print("bench: headline %.2f us  %.1f TFLOP/s" % (head["us"], head["tflops"]),
          file=sys.stderr, flush=True)

    extra = []
    if not args.no_extra:
        for ew in workloads.WORKLOADS:
            for e in ew.epilogues:
                if ew.name == w.name and e == epi:
                    continue
                steps = 50 if ew.M >= 8192 else 300
                r = run_workload(lib, ew, e, steps, 10)
                print("bench: %s %s %.2f us %.1f TFLOP/s" % (ew.name, e, r["us"], r["tflops"]),
                      file=sys.stderr, flush=True)
                extra.append(r)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, epi, args.cpu_seconds)

    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": epi,
                   "inputs": "%s seed %d" % (w.dist, w.seed),
                   "kernel_config": head["kernel_config"]},
        "pct_of_peak": head["pct_of_peak"],
        "roofline": {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["tflops"] / PEAK_FP16_TFLOPS,
                     "traffic": TRAFFIC_BYTES},
        "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count},
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
