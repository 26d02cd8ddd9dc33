"""Choices installed at run time on the GPU: calibrate() times one tile area's
configurations on the device and installs the fastest; mi355gemm_gemm then launches it."""
import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
from dense_fp16_gemm_fp32_amd import tune
import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_installed_choices():
    g.clear_choices()
    yield
    g.clear_choices()


@pytest.mark.parametrize("shape,epi", [((3000, 1000, 777), "bias_gelu"), ((2048, 2048, 512), "none")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_calibrate_installs_a_family_member_and_the_call_uses_it(shape, epi):
    M, N, K = shape
    print("calibrate", shape, epi, flush=True)
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=11)
    Ad, Bd, biasd = A.cuda(), B.cuda(), bias.cuda()
    b_arg = biasd if epi != "none" else None
    rule = g.select(Ad, Bd, b_arg, epi)
    info = g.mi355gemm_config_info(rule)
    best, med = tune.calibrate(Ad, Bd, b_arg, epi, ms=2.0, rounds=2, prewarm_ms=10.0)
    family = {c["name"] for c in g.configs() if c["direct"]
              and c["block_m"] * c["block_n"] == info["block_m"] * info["block_n"]}
    assert best in family and set(med) <= family and len(med) >= 2
    assert g.mi355gemm_config_name(g.select(Ad, Bd, b_arg, epi)) == best
    got = g.gemm(Ad, Bd, b_arg, epi)
    forced = g.gemm(Ad, Bd, b_arg, epi, config=g.config_id(best))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), forced.view(torch.int16))
    ref = oracle.gemm(A, B, bias if epi != "none" else None, epi).view(np.float16).astype(np.float64)
    out = got.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(out - ref) <= 5e-3 * np.linalg.norm(ref)
    assert np.all(np.abs(out - ref) <= 1e-2 * (1 + np.abs(ref)))
    g.clear_choices()
    assert g.select(Ad, Bd, b_arg, epi) == rule


def test_calibrate_with_a_one_member_tile_area_installs_nothing():
    """256^3 takes the 64x128 tile, the only configuration of its tile area: the
    calibration has nothing to time, installs nothing, and the call still matches the
    oracle."""
    M, N, K = 256, 256, 256
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=13)
    Ad, Bd, biasd = A.cuda(), B.cuda(), bias.cuda()
    rule = g.select(Ad, Bd, biasd, "bias_gelu")
    assert g.mi355gemm_config_name(rule) == "d64x128x32_w1x4_s4"
    assert [c["name"] for c in g.configs() if c["direct"] and c["block_m"] * c["block_n"] == 64 * 128] \
        == ["d64x128x32_w1x4_s4"]
    name, med = tune.calibrate(Ad, Bd, biasd, "bias_gelu", ms=2.0, rounds=2, prewarm_ms=10.0)
    assert name == "d64x128x32_w1x4_s4" and med == {}
    assert g.select(Ad, Bd, biasd, "bias_gelu") == rule
    got = g.gemm(Ad, Bd, biasd, "bias_gelu")
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, bias, "bias_gelu").view(np.float16).astype(np.float64)
    out = got.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(out - ref) <= 5e-3 * np.linalg.norm(ref)
    assert np.all(np.abs(out - ref) <= 1e-2 * (1 + np.abs(ref)))


def test_calibrate_with_one_candidate_installs_nothing():
    A, B, _ = workloads.make_inputs(256, 256, 256, "normal", seed=2)
    Ad, Bd = A.cuda(), B.cuda()
    rule = g.select(Ad, Bd)
    name, med = tune.calibrate(Ad, Bd, candidates=["d128x128x64_w2x2_s4"])
    assert name == "d128x128x64_w2x2_s4" and med == {}
    assert g.select(Ad, Bd) == rule


@pytest.mark.parametrize("shape", [(2048, 2047, 2048), (1000, 3001, 777)],
                         ids=lambda v: "x".join(map(str, v)))
def test_calibrate_on_rows_that_are_not_16_byte_friendly_installs_nothing(shape):
    """Odd N: the library splits the call into a direct launch and a narrow strip, which a
    forced configuration cannot do, so calibration has the selector's choice as its only
    candidate, times nothing and installs nothing; the call itself still serves the shape
    and matches the oracle."""
    M, N, K = shape
    print("calibrate odd N", shape, flush=True)
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=12)
    Ad, Bd, biasd = A.cuda(), B.cuda(), bias.cuda()
    rule = g.select(Ad, Bd, biasd, "bias_gelu")
    name, med = tune.calibrate(Ad, Bd, biasd, "bias_gelu", ms=2.0, rounds=2, prewarm_ms=10.0)
    assert name == g.mi355gemm_config_name(rule) and med == {}
    assert g.select(Ad, Bd, biasd, "bias_gelu") == rule
    got = g.gemm(Ad, Bd, biasd, "bias_gelu")
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, bias, "bias_gelu").view(np.float16).astype(np.float64)
    out = got.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(out - ref) <= 5e-3 * np.linalg.norm(ref)
    assert np.all(np.abs(out - ref) <= 1e-2 * (1 + np.abs(ref)))
