"""Host checks of the benchmark's bookkeeping (CPU only)."""
from __future__ import annotations

import os
import sys
import time

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (4, 4), (5, 3), (3, 5), (17, 40), (256, 256)])
def test_attention_flops_count_the_allowed_pairs(Sq, Sk):
    """4 D flops per allowed (query, key) pair; the causal mask (key j <= query i) counted
    by brute force."""
    B, H, D = 2, 3, 64
    allowed = np.tril(np.ones((Sq, Sk), dtype=np.int64)).sum()
    assert bench.attention_flops(B, H, Sq, Sk, D, True) == 4.0 * B * H * D * allowed
    assert bench.attention_flops(B, H, Sq, Sk, D, False) == 4.0 * B * H * D * Sq * Sk


def test_gpus_above_one_exit_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code != 0
    assert "one GPU" in capsys.readouterr().err


def test_warm_up_runs_the_calls_then_tops_up_to_the_minimum_time(monkeypatch):
    """warm_up makes the requested calls, then more until the minimum time has passed;
    with no minimum it makes exactly the requested calls."""
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []

    def fn():
        calls.append(1)
        time.sleep(0.001)
    t0 = time.perf_counter()
    n = bench.warm_up(fn, 3, 30.0)
    assert n == len(calls) and n > 3
    assert (time.perf_counter() - t0) * 1e3 >= 30.0
    calls.clear()
    assert bench.warm_up(fn, 5, 0.0) == 5 == len(calls)
    calls.clear()
    assert bench.warm_up(fn, 0, 0.0) == 0 == len(calls)
    assert bench.warm_up(fn, 0, 5.0) >= 1


def test_kernel_hash_ignores_comments_but_not_code():
    """The traffic figure is keyed to the kernels' code: a comment or blank line changes
    nothing, a changed statement changes the text that is hashed."""
    src = "int a = 1;  // one\n\n// a note\nint b = a + 2;\n"
    assert bench.code_text(src) == bench.code_text("int a = 1;\nint b = a + 2;  // two\n")
    assert bench.code_text(src) != bench.code_text("int a = 1;\nint b = a + 3;\n")


def test_traffic_lookup_covers_the_calibration_family_only_for_the_measured_code():
    import bench
    h = bench.kernel_sources_hash()
    for name in ("d128x128x64_w2x2_s4", "d128x128x32_w2x2_s4", "d128x128x64_w2x2k2_s4",
                 "d128x128x64_w2x4_s4", "d64x256x32_w1x4_s4", "d128x128x64_w2x2_l4_s4",
                 "d128x128x32_w2x2_l4_s4"):
        got = bench.traffic_for(name)
        measured = (bench.TRAFFIC["sources_sha256_16"] == h if name == bench.TRAFFIC["kernel_config"]
                    else bench.TRAFFIC_OTHER["sources_sha256_16"] == h)
        assert (got is not None) == measured
        if got is not None:
            assert 25165824 <= got < 4 * 25165824   # A, B and C once, up to 4x that
    assert bench.traffic_for("d256x256x32_w2x2_s4") is None


def test_bench_calibrates_by_default():
    import bench
    assert bench.parse([]).calibrate is True
    assert bench.parse(["--no-calibrate"]).calibrate is False
    assert bench.parse(["--config", "d128x128x32_w2x2_s4"]).config == "d128x128x32_w2x2_s4"
