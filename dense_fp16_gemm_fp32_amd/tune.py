"""Shape-keyed autotuning: time every configuration that can serve a shape and write the
selector's table of measured winners.

The tutorial's schedule sweep (thecryptopost.io page, section 3, "Knobs - sweeping the
schedule by hand") builds each candidate schedule, checks it numerically, times it and
keeps the fastest, noting that the best schedule depends on the architecture and the
shape; its autotuning section searches the same space per target.  Here the candidates
are the library's compiled configurations, forced one at a time through
``mi355gemm_gemm_config`` (a configuration that cannot serve the shape is skipped, as the
sweep skips schedules over the shared-memory budget), and each one is first checked
against the rule-chosen configuration's output (relative Frobenius distance below 5e-3,
as a wrong kernel would fail the sweep's numerical check).

MI355X runs these GEMMs at its power limit, so single timings move by several percent
from run to run: candidates are timed in interleaved rounds and compared by their median.
The engine clock reacts to load within milliseconds, so the candidate timed first after
a pause runs on a cooler part: the order reverses every other round, and each timing
covers ``--ms`` milliseconds of back-to-back calls (default 20), long enough for the
clock to settle.
A shape gets a table entry only when its winner beats the configuration the selector's
rules would pick by at least ``--margin`` (default 3%); otherwise the rules stand.

The table is C source, ``csrc/tuned_table.inc``, compiled into the library (rebuild after
writing it); ``mi355gemm_select`` consults it for an exact (M, N, K, epilogue, alignment)
match before the rules.  Tune on a library built with an empty table: the rule choice the
winners are compared with comes from ``mi355gemm_select``, so a shape that already has an
entry would be compared with that entry and lose it.

Usage (on the GPU):
  python -m dense_fp16_gemm_fp32_amd.tune [--shapes MxNxK[:epilogue[:dist]] ...]
         [--rounds 7] [--margin 0.03] [--write]
With no --shapes, the benchmark's workloads are tuned.
"""
from __future__ import annotations

import argparse
import datetime
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TABLE = os.path.join(PKG, "csrc", "tuned_table.inc")


def parse_shape(text: str):
    parts = text.split(":")
    M, N, K = (int(x) for x in parts[0].split("x"))
    epi = parts[1] if len(parts) > 1 and parts[1] else "none"
    dist = parts[2] if len(parts) > 2 and parts[2] else "normal"
    return M, N, K, epi, dist


def default_shapes():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import workloads
    out = []
    for w in workloads.WORKLOADS:
        for e in w.epilogues:
            out.append((w.M, w.N, w.K, e, w.dist))
    return out


def _aligned(t, n):
    return t is None or t.data_ptr() % n == 0


def alignment_class(A, B, out, bias, K, N):
    """(A rows 16-byte friendly, B and C rows 16-byte friendly), as the library defines
    them (K % 8 == 0 and A 16-byte aligned; N % 8 == 0, B and C 16-byte aligned and the
    bias 8-byte aligned)."""
    av = K % 8 == 0 and _aligned(A, 16)
    bv = N % 8 == 0 and _aligned(B, 16) and _aligned(out, 16) and _aligned(bias, 8)
    return int(av), int(bv)


def _time(fn, steps):
    import torch
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(steps):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1e3   # us per call


def tune(shapes, rounds=7, margin=0.03, log=print, ms=20.0):
    """Returns a list of dicts, one per shape: the rule choice, every candidate's median
    time, the winner and whether it earns a table entry."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import dense_fp16_gemm_fp32_amd as g
    import workloads

    results = []
    for (M, N, K, epi, dist) in shapes:
        A, B, bias = workloads.make_inputs(M, N, K, dist, with_bias=True, seed=0)
        A, B, bias = A.cuda(), B.cuda(), bias.cuda()
        b_arg = bias if epi != "none" else None
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        rule = g.select(A, B, b_arg, epi, out=out)
        ref = g.gemm(A, B, b_arg, epi).float()
        ref_norm = float(ref.norm())
        flops = 2.0 * M * N * K
        # about `ms` milliseconds per timing at 1 PFLOP/s
        steps = max(3, min(20000, int(ms * 1e-3 / max(flops / 1e15, 1e-9))))
        cands = []
        for cfg in g.configs():
            st = g.mi355gemm_gemm_config(M, N, K, A.data_ptr(), B.data_ptr(), out.data_ptr(),
                                         b_arg.data_ptr() if b_arg is not None else None,
                                         g.EPILOGUES[epi], torch.cuda.current_stream().cuda_stream,
                                         cfg["id"])
            if st != g.OK:
                continue                                   # cannot serve this shape
            torch.cuda.synchronize()
            d = float((out.float() - ref).norm()) / max(ref_norm, 1e-30)
            if not d <= 5e-3:
                log("  %s: output differs from the rule choice (rel. Frobenius %.2e), skipped"
                    % (cfg["name"], d))
                continue
            cands.append(cfg)
        times = {c["name"]: [] for c in cands}
        for rnd in range(rounds):
            for c in (cands if rnd % 2 == 0 else cands[::-1]):
                cid = c["id"]
                for _ in range(2):
                    g.gemm(A, B, b_arg, epi, out=out, config=cid)
                torch.cuda.synchronize()
                times[c["name"]].append(_time(lambda: g.gemm(A, B, b_arg, epi, out=out, config=cid), steps))
        med = {k: statistics.median(v) for k, v in times.items()}
        rule_name = g.mi355gemm_config_name(rule)
        best = min(med, key=med.get)
        entry = best != rule_name and med[best] <= (1.0 - margin) * med[rule_name]
        log("%dx%dx%d %s (%s): rule %s %.2f us, best %s %.2f us%s"
            % (M, N, K, epi, dist, rule_name, med[rule_name], best, med[best],
               "  -> table entry" if entry else ""))
        av, bv = alignment_class(A, B, out, b_arg, K, N)
        results.append({"M": M, "N": N, "K": K, "epilogue": epi, "dist": dist,
                        "a_vector": av, "bc_vector": bv,
                        "rule": rule_name, "best": best, "entry": entry, "median_us": med})
    return results


def calibration_candidates(a, b, bias=None, epilogue="none", out=None):
    """The configurations ``calibrate`` may time and install for this call: the direct
    configurations whose tile area (block_m x block_n) equals the selector's choice's --
    about the same number of tiles, so the same share of the chip -- and that serve its K (the
    ping-pong ones need K % 8 == 0), or the selector's
    choice alone when it is not a direct kernel or when B and C rows are not 16-byte
    friendly (the library then splits the launch into a direct part and a narrow strip,
    which a forced configuration cannot do).  Returns (rule name, [candidate names])."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import dense_fp16_gemm_fp32_amd as g

    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    b_arg = bias if epilogue != "none" else None
    rule = g.select(a, b, b_arg, epilogue, out=out)
    if rule < 0:
        raise g.GemmError(g.EINVAL, g.mi355gemm_last_error())
    rule_name = g.mi355gemm_config_name(rule)
    info = g.mi355gemm_config_info(rule)
    _, bv = alignment_class(a, b, out, b_arg, K, N)
    if not info["direct"] or not bv:
        return rule_name, [rule_name]
    return rule_name, [c["name"] for c in g.configs()
                       if c["direct"] and c["block_m"] * c["block_n"] == info["block_m"] * info["block_n"]
                       and not (c["k_mult8"] and K % 8)]


def agrees(got, ref, rel_fro=5e-3, elem=1e-2) -> bool:
    """Candidate output against the selector's output, both fp16 on the device: relative
    Frobenius distance at most ``rel_fro`` and every element within ``elem * (1 + |ref|)``,
    no NaN or Inf where the reference is finite."""
    import torch
    g64, r64 = got.double(), ref.double()
    if not bool(torch.isfinite(g64[torch.isfinite(r64)]).all()):
        return False
    d = (g64 - r64).abs()
    if not bool((d <= elem * (1.0 + r64.abs())).all()):
        return False
    nr = float(r64.norm())
    return float(d.norm()) <= rel_fro * (nr if nr > 0 else max(r64.numel(), 1) ** 0.5)


def calibrate(a, b, bias=None, epilogue="none", out=None, candidates=None, ms=20.0,
              rounds=4, prewarm_ms=100.0):
    """Time candidate configurations for one call on the current device and install the
    fastest for its shape, epilogue and alignment class in this process
    (``mi355gemm_set_choice``).  The same tile can run up to 25% slower on one MI355X machine
    than on another, while a neighbouring tile does not, so the measured table and the
    rules cannot know the best tile for every box.

    ``candidates``: configuration names; by default ``calibration_candidates`` (the tile
    shapes, wave layouts, k-groups and ring depths of the selector's tile area).  Each must agree with
    the selector's output (``agrees``: relative Frobenius distance at most 5e-3 and every
    element within 1e-2 * (1 + |ref|)).  Timing as in ``tune``: ``prewarm_ms`` of calls
    first, then ``rounds`` interleaved rounds in alternating order, medians compared.
    Returns ``(name, {name: median us})``; with a single candidate nothing is timed or
    installed.
    """
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import dense_fp16_gemm_fp32_amd as g

    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    b_arg = bias if epilogue != "none" else None
    rule_name, default = calibration_candidates(a, b, bias, epilogue, out)
    if candidates is None:
        candidates = default
    if len(default) == 1 and candidates == default:
        return rule_name, {}
    ref = g.gemm(a, b, b_arg, epilogue)
    ids = {}
    for name in candidates:
        cid = g.config_id(name)
        try:
            g.gemm(a, b, b_arg, epilogue, out=out, config=cid)
        except g.GemmError:
            continue                                       # cannot serve this call
        torch.cuda.synchronize()
        if agrees(out, ref):
            ids[name] = cid
    if not ids:
        raise g.GemmError(g.EUNSUPPORTED, "no candidate configuration serves this call")
    if len(ids) == 1:
        return next(iter(ids)), {}
    flops = 2.0 * M * N * K
    steps = max(3, min(20000, int(ms * 1e-3 / max(flops / 1e15, 1e-9))))
    calls = {n: (lambda cid=cid: g.gemm(a, b, b_arg, epilogue, out=out, config=cid)) for n, cid in ids.items()}
    warm_steps = max(1, int(steps * prewarm_ms / ms / len(calls)))
    for fn in calls.values():
        for _ in range(warm_steps):
            fn()
    torch.cuda.synchronize()
    times = {n: [] for n in calls}
    items = list(calls.items())
    for rnd in range(rounds):
        for n, fn in (items if rnd % 2 == 0 else items[::-1]):
            fn()
            times[n].append(_time(fn, steps))
    med = {n: statistics.median(v) for n, v in times.items()}
    best = min(med, key=med.get)
    av, bv = alignment_class(a, b, out, b_arg, K, N)
    g.set_choice(M, N, K, epilogue, av, bv, best)
    return best, med


NOTE_PREFIX = "// note:"


def existing_notes(path: str = TABLE) -> list:
    """The hand-written note lines (``// note: ...``) of the current table, which a rewrite
    keeps: they record why a measured winner was left out or where a rule came from."""
    try:
        with open(path) as fh:
            return [line.rstrip("\n") for line in fh if line.startswith(NOTE_PREFIX)]
    except OSError:
        return []


def table_source(results, device: str, notes=()) -> str:
    lines = [
        "// Measured selector table, written by dense_fp16_gemm_fp32_amd/tune.py.  Lines that",
        "// start with '// note:' are written by hand and kept when the tuner rewrites the file;",
        "// every other line is the tuner's.",
        "// Device: %s; %s." % (device, datetime.date.today().isoformat()),
        "// Fields: M, N, K, epilogue, A 16-byte rows, B/C 16-byte rows, configuration name.",
        "// Shapes whose best configuration beat the rule choice by less than the margin have",
        "// no entry (the rules stand); their timings are listed for the record.",
    ]
    lines.extend(notes)
    epi_code = {"none": 0, "bias": 1, "bias_gelu": 2}
    for r in results:
        lines.append("// %dx%dx%d %s: %s" % (r["M"], r["N"], r["K"], r["epilogue"], ", ".join(
            "%s %.2f us" % (k, v) for k, v in sorted(r["median_us"].items(), key=lambda kv: kv[1]))))
        if r["entry"]:
            lines.append('{%d, %d, %d, %d, %d, %d, "%s"},' % (
                r["M"], r["N"], r["K"], epi_code[r["epilogue"]], r["a_vector"], r["bc_vector"],
                r["best"]))
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", nargs="*", default=None)
    ap.add_argument("--rounds", type=int, default=7)
    ap.add_argument("--margin", type=float, default=0.03)
    ap.add_argument("--ms", type=float, default=20.0, help="milliseconds per timing")
    ap.add_argument("--write", action="store_true", help="write csrc/tuned_table.inc")
    ap.add_argument("--output", default=TABLE)
    args = ap.parse_args(argv)
    import torch
    shapes = [parse_shape(s) for s in args.shapes] if args.shapes else default_shapes()
    res = tune(shapes, args.rounds, args.margin, log=lambda m: print(m, flush=True), ms=args.ms)
    src = table_source(res, torch.cuda.get_device_properties(0).name, existing_notes(args.output))
    if args.write:
        with open(args.output, "w") as f:
            f.write(src)
        print("wrote", args.output, "- rebuild the library to use it")
    else:
        sys.stdout.write(src)


if __name__ == "__main__":
    main()
