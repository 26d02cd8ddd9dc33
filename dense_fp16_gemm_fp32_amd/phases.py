"""Where the direct kernel's time goes: per-workgroup phase timestamps from the
phase-clock build of the library (``libmi355gemm_phases.so``, built with
MI355_PHASE_CLOCK=1 by the package build; its kernels are the regular ones plus the
stamps).

For each shape and configuration: warm-up calls, then three calls of which the last one's
stamps are read.  Thread 0 of each workgroup stamps s_memrealtime (100 MHz) and s_memtime
(shader clock cycles) at entry, once the first stage has landed, after the K loop, after
the epilogue has written the tile to LDS, after the following barrier, after the C stores
are issued and once they are complete.  Printed per phase: min / median / 90th percentile /
max over the workgroups in microseconds, the clock the cycle counter implies and the K
loop's cycles per stage.

Usage (on the GPU):
  python -m dense_fp16_gemm_fp32_amd.phases --shapes MxNxK[:epilogue[:dist]] ... --configs NAME ...
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TILES = 8192      # workgroups the build records (kPhaseClockTiles)
PHASES = ("entry", "first stage", "K loop", "epilogue", "barrier", "C stores issued", "C stores done")


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", nargs="+", required=True)
    ap.add_argument("--configs", nargs="+", required=True)
    ap.add_argument("--warmup", type=int, default=200)
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    import dense_fp16_gemm_fp32_amd as g
    import workloads
    from dense_fp16_gemm_fp32_amd import build
    if not os.path.exists(build.PHASE_LIBRARY):
        raise ImportError("%s is not built (python -m dense_fp16_gemm_fp32_amd.build)" % build.PHASE_LIBRARY)
    g.LIBRARY = build.PHASE_LIBRARY
    lib = g.library()
    lib.mi355gemm_phase_clock_read.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    lib.mi355gemm_phase_clock_read.restype = ctypes.c_int
    lib.mi355gemm_phase_clock_clear.restype = ctypes.c_int
    buf = (ctypes.c_ulonglong * (TILES * 16))()
    for text in args.shapes:
        parts = text.split(":")
        M, N, K = (int(x) for x in parts[0].split("x"))
        epi = parts[1] if len(parts) > 1 and parts[1] else "none"
        dist = parts[2] if len(parts) > 2 and parts[2] else "normal"
        A, B, bias = workloads.make_inputs(M, N, K, dist, with_bias=True, seed=0)
        A, B, bias = A.cuda(), B.cuda(), bias.cuda()
        b_arg = bias if epi != "none" else None
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        for name in args.configs:
            cid = g.config_id(name)
            info = g.mi355gemm_config_info(cid)
            if not info["direct"]:
                print("%s %s: not a direct-kernel configuration, skipped" % (text, name))
                continue
            tiles = -(-M // info["block_m"]) * -(-N // info["block_n"])
            if tiles > TILES:
                print("%s %s: %d workgroups, more than the %d recorded" % (text, name, tiles, TILES))
                continue
            for _ in range(args.warmup):
                g.gemm(A, B, b_arg, epi, out=out, config=cid)
            torch.cuda.synchronize()
            if lib.mi355gemm_phase_clock_clear() != 0:
                raise RuntimeError(g.mi355gemm_last_error())
            for _ in range(3):
                g.gemm(A, B, b_arg, epi, out=out, config=cid)
            torch.cuda.synchronize()
            if lib.mi355gemm_phase_clock_read(buf, TILES * 16) != 0:
                raise RuntimeError(g.mi355gemm_last_error())
            rt = [[buf[t * 16 + s] for s in range(7)] for t in range(tiles)]
            cy = [[buf[t * 16 + 8 + s] for s in range(7)] for t in range(tiles)]
            t0 = min(r[0] for r in rt)
            ghz = statistics.median((c[6] - c[0]) / ((r[6] - r[0]) * 10.0) for r, c in zip(rt, cy) if r[6] > r[0])
            nk = -(-K // info["block_k"])
            loop = statistics.median(c[2] - c[1] for c in cy)
            print("%s %s: %d workgroups, span %.2f us, clock %.2f GHz, K loop %d cycles = %.0f per %d-deep stage"
                  % (text, name, tiles, max(r[6] - t0 for r in rt) / 100.0, ghz, loop, loop / max(nk, 1),
                     info["block_k"]))
            rows = [("start (from the first)", [(r[0] - t0) / 100.0 for r in rt])]
            rows += [("-> " + PHASES[s], [(r[s] - r[s - 1]) / 100.0 for r in rt]) for s in range(1, 7)]
            rows.append(("end (from the first start)", [(r[6] - t0) / 100.0 for r in rt]))
            for label, v in rows:
                print("   %-28s min %6.2f  p50 %6.2f  p90 %6.2f  max %6.2f us"
                      % (label, min(v), _pct(v, 0.5), _pct(v, 0.9), max(v)))
            sys.stdout.flush()
    return 0


if __name__ == "__main__":
    sys.exit(main())
