"""The timed GEMM entry point (mi355gemm_gemm_timed) on the GPU: the same output as the
untimed call, and events that bracket the kernels' own execution."""
import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import oracle
import workloads

pytestmark = pytest.mark.gpu


def _recorded_pair():
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("shape,epi", [((2048, 2048, 2048), "none"), ((1000, 3000, 777), "bias_gelu"),
                                       ((300, 1029, 136), "bias_gelu"), ((64, 5, 200), "bias")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_timed_call_matches_untimed_and_brackets_the_kernels(shape, epi):
    """Same configuration, same bits.  The events' interval is positive, and no longer
    than events recorded on the stream around the same call (which also count its
    dispatch).  1029 columns take a direct launch plus a narrow one: the interval then
    spans both; 5 columns take the narrow kernel alone."""
    M, N, K = shape
    print("timed", shape, epi, flush=True)
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=3)
    dev = torch.device("cuda:0")
    Ad, Bd, biasd = A.to(dev), B.to(dev), bias.to(dev)
    b_arg = biasd if epi != "none" else None
    plain = g.gemm(Ad, Bd, b_arg, epi)
    s0, s1 = _recorded_pair()
    k0, k1 = _recorded_pair()
    s0.record()
    timed = g.gemm(Ad, Bd, b_arg, epi, events=(k0, k1))
    s1.record()
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    kernel_ms, call_ms = k0.elapsed_time(k1), s0.elapsed_time(s1)
    assert 0.0 < kernel_ms <= call_ms + 1e-3, (kernel_ms, call_ms)
    ref = oracle.gemm(A, B, bias if epi != "none" else None, epi)
    got = timed.cpu().numpy().astype(np.float64)
    r = ref.view(np.float16).astype(np.float64)
    assert np.linalg.norm(got - r) <= 5e-3 * np.linalg.norm(r)
    assert np.all(np.abs(got - r) <= 1e-2 * (1 + np.abs(r)))


def test_timed_call_with_a_forced_config_and_one_event():
    M = N = K = 512
    A, B, _ = workloads.make_inputs(M, N, K, "normal", seed=4)
    Ad, Bd = A.cuda(), B.cuda()
    cid = g.config_id("d128x128x64_w2x2k2_s4")
    ref = g.gemm(Ad, Bd, config=cid)
    k0, _ = _recorded_pair()
    out = g.gemm(Ad, Bd, config=cid, events=(k0, None))
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))


def test_unrecorded_events_are_rejected_before_any_launch():
    A = torch.zeros((64, 64), dtype=torch.float16, device="cuda:0")
    fresh = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    with pytest.raises(ValueError):
        g.gemm(A, A, events=fresh)


def test_negative_config_ids_are_rejected_with_and_without_events():
    A = torch.zeros((64, 64), dtype=torch.float16, device="cuda:0")
    k0, k1 = _recorded_pair()
    for events in (None, (k0, k1)):
        with pytest.raises(g.GemmError):
            g.gemm(A, A, config=-1, events=events)
