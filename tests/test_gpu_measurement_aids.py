"""The measurement aids run and report sane figures: the phase-clock build of the library
(the direct kernel's per-workgroup timestamps, read by dense_fp16_gemm_fp32_amd.phases)
and the per-CU bandwidth probe."""
import os
import re
import subprocess
import sys

import pytest

from dense_fp16_gemm_fp32_amd import build

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(cmd, timeout):
    print("run", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=timeout)
    assert r.returncode == 0, r.stdout[-2000:]
    return r.stdout


@pytest.mark.skipif(not os.path.exists(build.PHASE_LIBRARY), reason="phase-clock build not present")
def test_phase_clock_reports_every_workgroup_in_order():
    out = _run([sys.executable, "-m", "dense_fp16_gemm_fp32_amd.phases", "--shapes", "512x512x512",
                "--configs", "d64x128x32_w1x4_s4", "--warmup", "5"], 120)
    head = re.search(r"(\d+) workgroups, span ([\d.]+) us, clock ([\d.]+) GHz, K loop (\d+) cycles", out)
    assert head, out
    tiles, span, ghz, loop = int(head.group(1)), float(head.group(2)), float(head.group(3)), int(head.group(4))
    assert tiles == 8 * 4                      # 512 / 64 x 512 / 128
    assert 0.5 < span < 1000.0 and 0.5 < ghz < 3.0 and loop > 0
    # every phase row is non-negative (the stamps of each workgroup come in program order)
    rows = re.findall(r"->.*min\s+(-?[\d.]+)", out)
    assert len(rows) == 6 and all(float(v) >= 0.0 for v in rows), out


@pytest.mark.skipif(not os.path.exists(build.PROBE), reason="bandwidth probe not built")
def test_bandwidth_probe_rates_are_plausible():
    out = _run([build.PROBE], 120)
    assert out.strip().endswith("done"), out[-2000:]
    rates = {}
    for m in re.finditer(r"^(.+?)\s+waves/CU\s+(\d+)\s+([\d.]+) B/clk per CU", out, re.M):
        rates[(m.group(1).strip(), int(m.group(2)))] = float(m.group(3))
    assert len(rates) == 18, out
    # per CU and clock: no path beats the LDS's 256 B/clk by much, and every one moves data
    assert all(0.5 < v < 320.0 for v in rates.values()), rates
    # the transposing read moves fewer bytes per clock than the plain 16-byte read
    for w in (4, 8, 16):
        assert rates[("LDS ds_read_b64_tr_b16", w)] < rates[("LDS ds_read_b128", w)]
