"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs come from ``workloads`` (seeded, host-side); the same fp16 bits go to both sides.
Random inputs are compared to the tolerance bar in ``parity.py``; structured inputs
whose sums are exact (all-ones, selection matrices, small integers) must match the
oracle bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import oracle
import workloads
from parity import assert_bitexact, assert_parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EPIS = ("none", "bias", "bias_gelu")


def _dev(t):
    return None if t is None else t.to(DEV)


def _run(A, B, bias, epi, config=None, out=None):
    C = g.gemm(_dev(A), _dev(B), _dev(bias) if epi != "none" else None, epilogue=epi,
               config=config, out=out)
    torch.cuda.synchronize()
    return C


def _compatible(cfg, M, N, K):
    if cfg["narrow"] and N > cfg["block_n"]:
        return False
    if cfg["a_vector"] and K % 8:
        return False
    if cfg["bc_vector"] and N % 8:
        return False
    if cfg["k_mult8"] and K % 8:
        return False
    return True


ALL_CONFIGS = None


def all_configs():
    global ALL_CONFIGS
    if ALL_CONFIGS is None:
        ALL_CONFIGS = g.configs()
    return ALL_CONFIGS


def test_device_is_gfx950():
    props = torch.cuda.get_device_properties(0)
    print("device:", props.name, getattr(props, "gcnArchName", "?"), props.multi_processor_count,
          "CUs", flush=True)
    assert "gfx950" in getattr(props, "gcnArchName", "gfx950")


# ---- one MFMA block: pins the operand and result lane maps ---------------------------

def _small_int_inputs(M, N, K):
    i = torch.arange(M).view(M, 1)
    k = torch.arange(K).view(1, K)
    A = ((i * 7 + k * 3) % 9 - 4).to(torch.float16)
    kk = torch.arange(K).view(K, 1)
    j = torch.arange(N).view(1, N)
    B = ((kk * 5 + j * 11) % 7 - 3).to(torch.float16)
    return A.contiguous(), B.contiguous()


@pytest.mark.parametrize("shape", [(32, 32, 16), (64, 64, 64), (96, 160, 48)])
def test_small_integer_products_bitexact_every_config(shape):
    """|C| <= K*4*3 stays an exactly representable fp16 integer, so every correct
    summation order gives the same bits; a wrong lane map does not."""
    M, N, K = shape
    A, B = _small_int_inputs(M, N, K)
    ref = oracle.gemm(A, B)
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        print("config", cfg["name"], shape, flush=True)
        C = _run(A, B, None, "none", config=cfg["id"])
        assert_bitexact(C, ref, "%s %s" % (cfg["name"], shape))


# ---- the kernels a run can take on a workload -------------------------------------------

def _members(w, epi):
    """Every configuration a benchmark run of workload w may launch: the selector's choice
    and each configuration run-time calibration may install in its place (tune's
    calibration_candidates, the direct configurations of the same tile area).  Names, the
    selector's first."""
    from dense_fp16_gemm_fp32_amd import tune
    A = torch.empty((w.M, w.K), dtype=torch.float16, device=DEV)
    B = torch.empty((w.K, w.N), dtype=torch.float16, device=DEV)
    bias = torch.empty((w.N,), dtype=torch.float16, device=DEV) if epi != "none" else None
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=DEV)
    rule, cands = tune.calibration_candidates(A, B, bias, epi, out)
    return [rule] + [c for c in cands if c != rule]


def test_members_cover_the_calibration_family():
    """The member list the full-size tests below walk is the selector's choice plus every
    direct configuration of its tile area (every workload's K is a multiple of 8, so the
    ping-pong kernel counts): several at 2048^3 and 8192^3, one where the area has a
    single configuration (256^3 on 64x128)."""
    areas = {}
    for c in g.configs():
        if c["direct"]:
            areas.setdefault(c["block_m"] * c["block_n"], set()).add(c["name"])
    for w in workloads.WORKLOADS:
        for e in w.epilogues:
            names = _members(w, e)
            print(w.name, e, names, flush=True)
            assert len(set(names)) == len(names)
            info = g.mi355gemm_config_info(g.config_id(names[0]))
            assert set(names) == areas[info["block_m"] * info["block_n"]]
            if w.M >= 2048:
                assert len(names) >= 2


# ---- structured inputs at every workload shape: exact results --------------------------

@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=[w.name for w in workloads.WORKLOADS])
def test_all_ones_gives_K_exactly(w):
    """All-ones operands: every partial sum is an integer below 2^11, exact in any order, so
    C must be K everywhere, for every configuration a run on this shape may take."""
    A = torch.ones((w.M, w.K), dtype=torch.float16, device=DEV)
    B = torch.ones((w.K, w.N), dtype=torch.float16, device=DEV)
    for name in _members(w, "none"):
        print("all-ones", w.name, name, flush=True)
        C = _run(A, B, None, "none", config=g.config_id(name))
        assert torch.all(C == float(w.K)).item(), "all-ones product is not K everywhere (%s)" % name


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=[w.name for w in workloads.WORKLOADS])
def test_selection_matrices_copy_rows_and_columns(w):
    """0/1 selection matrices: C[i, :] = B[i mod K, :] and C[:, j] = A[:, j mod K] exactly,
    for every configuration a run on this shape may take."""
    M, N, K = w.M, w.N, w.K
    Ar, Br, _ = workloads.make_inputs(M, N, K, w.dist, seed=11)
    A_sel = torch.zeros((M, K), dtype=torch.float16)
    A_sel[torch.arange(M), torch.arange(M) % K] = 1
    B_sel = torch.zeros((K, N), dtype=torch.float16)
    B_sel[torch.arange(N) % K, torch.arange(N)] = 1
    want_rows = Br[torch.arange(M) % K]
    want_cols = Ar[:, torch.arange(N) % K]
    A_sel_d, Br_d, Ar_d, B_sel_d = A_sel.to(DEV), Br.to(DEV), Ar.to(DEV), B_sel.to(DEV)
    for name in _members(w, "none"):
        cid = g.config_id(name)
        # A selects rows of B
        print("row selection", w.name, name, flush=True)
        C = _run(A_sel_d, Br_d, None, "none", config=cid)
        assert torch.equal(C.cpu(), want_rows), "row selection mismatch (%s)" % name
        # B selects columns of A
        print("column selection", w.name, name, flush=True)
        C = _run(Ar_d, B_sel_d, None, "none", config=cid)
        assert torch.equal(C.cpu(), want_cols), "column selection mismatch (%s)" % name


# ---- random inputs at small and ragged shapes, every config, every epilogue -----------

SMALL_SHAPES = [(1, 1, 1), (1, 8, 8), (7, 9, 5), (33, 65, 17), (64, 64, 64), (130, 264, 200),
                (257, 129, 72), (300, 500, 136), (129, 257, 777), (200, 96, 1), (500, 264, 1000)]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=["%dx%dx%d" % s for s in SMALL_SHAPES])
def test_random_parity_every_config_and_epilogue(shape):
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=M + N + K)
    refs = {e: oracle.gemm(A, B, bias, e) for e in EPIS}
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        for e in EPIS:
            print("config", cfg["name"], shape, e, flush=True)
            C = _run(A, B, bias, e, config=cfg["id"])
            assert_parity(C, refs[e], "%s %s %s" % (cfg["name"], shape, e))


def _seeded_shapes(n=40, seed=20261203):
    """Shapes drawn from a fixed seed: M and K anywhere in [1, 700) and [1, 1500), N a
    multiple of 8 (the direct kernels' column granularity) seven times in ten and any
    value otherwise."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        K = int(rng.integers(1, 1500))
        N = int(rng.integers(1, 88)) * 8 if rng.random() < 0.7 else int(rng.integers(1, 700))
        shapes.append((M, N, K))
    return shapes


RANDOM_SHAPES = _seeded_shapes()


@pytest.mark.parametrize("shape", RANDOM_SHAPES, ids=["%dx%dx%d" % s for s in RANDOM_SHAPES])
def test_seeded_random_shapes_every_config_and_epilogue(shape):
    """Breadth beyond the hand-picked shapes: every configuration that can serve the shape,
    and the selector's own choice (which splits columns past a multiple of 8 off to the
    narrow kernel), with every epilogue, against the oracle."""
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=3 * M + 5 * N + 7 * K)
    refs = {e: oracle.gemm(A, B, bias, e) for e in EPIS}
    for e in EPIS:
        print("selector", shape, e, flush=True)
        assert_parity(_run(A, B, bias, e), refs[e], "selector %s %s" % (shape, e))
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        for e in EPIS:
            print("config", cfg["name"], shape, e, flush=True)
            C = _run(A, B, bias, e, config=cfg["id"])
            assert_parity(C, refs[e], "%s %s %s" % (cfg["name"], shape, e))


# ---- the workloads at full size, in the launch configuration the benchmark uses --------

def _workload_cases():
    cases = []
    for w in workloads.WORKLOADS:
        for e in w.epilogues:
            cases.append((w, e))
        if w.name == "gemm_256" or w.name == "gemm_2048_bias_gelu":
            cases.append((w, "bias"))
    return cases


CASES = _workload_cases()


@pytest.mark.parametrize("w,epi", CASES, ids=["%s-%s" % (w.name, e) for w, e in CASES])
def test_workload_parity(w, epi):
    """Each workload at full size on its own inputs, through the selector and forced onto
    every configuration run-time calibration may install instead (the benchmark times
    whichever it installs).  Up to 2048^3 the whole output is compared with the oracle;
    at 8192^3 sampled elements, including every tile-boundary row and column."""
    A, B, bias = workloads.make_inputs(w.M, w.N, w.K, w.dist, with_bias=True, seed=w.seed)
    Ad, Bd, biasd = A.to(DEV), B.to(DEV), bias.to(DEV)
    full = w.M * w.N * w.K <= 2048 ** 3
    if full:
        ref = oracle.gemm(A, B, bias, epi)
    else:
        rng = np.random.default_rng(0)
        edge = np.array([0, 1, 127, 128, 255, 256, w.M - 1])
        rows = np.concatenate([rng.integers(0, w.M, 6000), np.repeat(edge, 64)])
        cols = np.concatenate([rng.integers(0, w.N, 6000), rng.integers(0, w.N, edge.size * 64)])
        rows2 = np.repeat(rng.integers(0, w.M, 64), edge.size)
        cols2 = np.tile(np.array([0, 1, 127, 128, 255, 256, w.N - 1]), 64)
        rows = np.concatenate([rows, rows2])
        cols = np.concatenate([cols, cols2])
        ref = oracle.gemm_sampled(A, B, rows, cols, bias, epi)
        ri, ci = torch.from_numpy(rows), torch.from_numpy(cols)
    members = [None] + _members(w, epi)
    for name in members:
        cid = None if name is None else g.config_id(name)
        print("workload", w.name, epi, "config", name or "(selector) " + g.mi355gemm_config_name(
            g.select(Ad, Bd, biasd if epi != "none" else None, epi)), flush=True)
        C = _run(Ad, Bd, biasd, epi, config=cid)
        if full:
            rep = assert_parity(C, ref, "%s %s %s" % (w.name, epi, name))
        else:
            rep = assert_parity(C.cpu()[ri, ci], ref, "%s %s %s (sampled)" % (w.name, epi, name))
        print("   ", rep, flush=True)


# ---- memory outside C is never touched -------------------------------------------------

@pytest.mark.parametrize("shape", [(1000, 3000, 777), (130, 264, 200), (33, 65, 17), (257, 136, 64)])
def test_guard_bands_untouched(shape):
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=3)
    pad = 4096
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        out = buf[pad:pad + M * N].view(M, N)
        print("guard", cfg["name"], shape, flush=True)
        _run(A, B, bias, "bias_gelu", config=cfg["id"], out=out)
        assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
        assert not torch.isnan(out).any().item()


# ---- degenerate shapes -------------------------------------------------------------------

def test_empty_and_zero_k():
    A = torch.zeros((0, 16), dtype=torch.float16, device=DEV)
    B = torch.zeros((16, 8), dtype=torch.float16, device=DEV)
    assert g.gemm(A, B).shape == (0, 8)
    A = torch.zeros((8, 16), dtype=torch.float16, device=DEV)
    B = torch.zeros((16, 0), dtype=torch.float16, device=DEV)
    assert g.gemm(A, B).shape == (8, 0)
    # K == 0: an empty sum, C = epi(bias or 0)
    _, _, bias = workloads.make_inputs(1, 40, 1, "normal", with_bias=True, seed=4)
    A0 = torch.zeros((24, 0), dtype=torch.float16)
    B0 = torch.zeros((0, 40), dtype=torch.float16)
    for e in EPIS:
        out = torch.full((24, 40), 7.0, dtype=torch.float16, device=DEV)
        C = _run(A0, B0, bias, e, out=out)
        ref = oracle.gemm(A0, B0, bias, e)
        assert_parity(C, ref, "K=0 " + e)


def test_misaligned_operands_use_narrow_loads():
    # few enough tiles (4 of 64x128) that the register-staged kernel serves the call
    M, N, K = 100, 136, 96
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=6)
    # views one element into larger buffers: 2-byte aligned only
    Ab = torch.zeros(M * K + 1, dtype=torch.float16, device=DEV)
    Ab[1:] = A.reshape(-1).to(DEV)
    Ad = Ab[1:].view(M, K)
    Cb = torch.zeros(M * N + 1, dtype=torch.float16, device=DEV)
    Cd = Cb[1:].view(M, N)
    cid = g.select(Ad, B.to(DEV), bias.to(DEV), "bias_gelu", out=Cd)
    info = g.mi355gemm_config_info(cid)
    assert info["a_vector"] == 0 and info["bc_vector"] == 0
    g.gemm(Ad, B.to(DEV), bias.to(DEV), "bias_gelu", out=Cd)
    torch.cuda.synchronize()
    assert_parity(Cd, oracle.gemm(A, B, bias, "bias_gelu"), "misaligned")


def test_runs_on_a_side_stream():
    M, N, K = 512, 512, 512
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=8)
    s = torch.cuda.Stream(device=DEV)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = g.gemm(Ad, Bd, bd, "bias_gelu")
    s.synchronize()
    assert_parity(C, oracle.gemm(A, B, bias, "bias_gelu"), "side stream")


def test_rejects_bad_tensors():
    A = torch.zeros((8, 16), dtype=torch.float16, device=DEV)
    B = torch.zeros((16, 8), dtype=torch.float16, device=DEV)
    with pytest.raises(TypeError):
        g.gemm(A.float(), B)
    with pytest.raises(ValueError):
        g.gemm(A, B.t())
    with pytest.raises(ValueError):
        g.gemm(A, torch.zeros((15, 8), dtype=torch.float16, device=DEV))
    with pytest.raises(g.GemmError):
        g.gemm(A, B, None, "bias_gelu")


# ---- several workgroups per compute unit ------------------------------------------------

@pytest.mark.parametrize("K", [1024, 1019])
def test_many_workgroups_per_cu_bitexact_every_config(K):
    """4096 x 4096 x K gives every tile shape several workgroups per compute unit (64
    of 256 x 256 up to 2048 of 64 x 128 per 256 CUs), so workgroups of the 64 KiB-ring
    tiles share a CU, its LDS and its memory pipes, and each ring slot is refilled 8 or
    more times per tile.  A copy that overtook a fragment read still queued for its slot
    would corrupt operands.  K = 1019 runs the K-tail variant: the last stage's straddling
    A chunk is patched in LDS (by the loader waves where the tile has them) between the
    copy landing and the barrier that releases it.  Integer inputs: every partial sum is
    an integer below 2^24, exact in fp32 in any order, so every configuration must give
    the oracle's bits, on two launches in a row (the second starting while the first
    drains)."""
    M = N = 4096
    A, B = _small_int_inputs(M, N, K)
    ref = oracle.gemm(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for cfg in all_configs():
        if not cfg["direct"] or not _compatible(cfg, M, N, K):
            continue
        print("many workgroups", cfg["name"], K, flush=True)
        outs = [torch.empty((M, N), dtype=torch.float16, device=DEV) for _ in range(2)]
        for o in outs:
            g.gemm(Ad, Bd, out=o, config=cfg["id"])
        torch.cuda.synchronize()
        for o in outs:
            assert_bitexact(o, ref, cfg["name"])


# ---- the direct kernel's two K loops --------------------------------------------------

def test_direct_kernel_full_turn_boundary_bitexact():
    """The direct kernel runs whole ring turns whose copies all lie below K with the
    copy's K offset in the scalar offset field, then the rest with masked copies.  The
    switch sits at K = (2 * stages - 1) * block_k; K just below, at and above it, a turn
    later, and with a K tail (K % 8 != 0) must give the oracle's bits.  Integer inputs:
    every partial sum is an integer below 2^24, exact in fp32 in any order, so the one
    rounding to fp16 is the oracle's."""
    for cfg in all_configs():
        if not cfg["direct"]:
            continue
        # the row-split ping-pong kernel copies one stage further ahead per turn
        rows_pp = cfg["pingpong"] and cfg["k_groups"] == 1
        kb = (2 * cfg["stages"] - (0 if rows_pp else 1)) * cfg["block_k"]
        M, N = cfg["block_m"] + 3, cfg["block_n"] + 8
        for K in (kb - 8, kb, kb + 3, kb + 8, kb + cfg["stages"] * cfg["block_k"]):
            if cfg["k_mult8"] and K % 8:
                continue
            print("turn boundary", cfg["name"], (M, N, K), flush=True)
            A, B = _small_int_inputs(M, N, K)
            C = _run(A, B, None, "none", config=cfg["id"])
            assert_bitexact(C, oracle.gemm(A, B), "%s K=%d" % (cfg["name"], K))


# ---- the fused GELU over every finite fp16 input -------------------------------------

def _ordered(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> integers in the same order as the values (+0 and -0 equal)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def test_gelu_epilogue_every_finite_fp16_input():
    """With A = 0 the kernel's output is C[i, j] = fp16(GELU(bias[j])), so putting every
    finite fp16 value in the bias runs the register epilogue's erf-GELU once on each.  The
    result must be within one fp16 step of the oracle's correctly rounded value
    everywhere and equal to it for almost all inputs (the kernel evaluates GELU in fp32)."""
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = all_bits[(all_bits & 0x7C00) != 0x7C00]
    N = finite.size                      # 63488, a multiple of 8
    M, K = 8, 16
    bias = torch.from_numpy(finite.view(np.float16).copy())
    A = torch.zeros((M, K), dtype=torch.float16)
    _, B, _ = workloads.make_inputs(M, N, K, "normal", seed=5)
    ref = oracle.gemm(A, B, bias, "bias_gelu")
    assert np.array_equal(ref[0], ref[M - 1])
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        print("gelu sweep", cfg["name"], flush=True)
        C = _run(A, B, bias, "bias_gelu", config=cfg["id"])
        got = C.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        d = np.abs(_ordered(got) - _ordered(ref))
        assert d.max() <= 1, "%s: GELU off by %d fp16 steps at bias %r" % (
            cfg["name"], d.max(), float(bias[int(np.argmax(d.max(axis=0)))]))
        assert (d == 0).mean() >= 0.99, "%s: only %.4f exact" % (cfg["name"], (d == 0).mean())


def test_gelu_epilogue_non_finite_inputs():
    """+inf, -inf and NaN in the bias reach the epilogue as GELU's input (A = 0): the result
    is what x * Phi(x) gives in IEEE arithmetic, as the oracle evaluates it -- +inf for
    +inf, NaN for -inf (-inf * 0) and for NaN -- and the finite columns beside them are
    unaffected, on every configuration."""
    M, N, K = 8, 64, 16
    vals = [float("inf"), float("-inf"), float("nan"), 65504.0, -65504.0, 0.0, -0.0, 1.0]
    bias = torch.tensor((vals * (N // len(vals)))[:N], dtype=torch.float16)
    A = torch.zeros((M, K), dtype=torch.float16)
    _, B, _ = workloads.make_inputs(M, N, K, "normal", seed=6)
    ref = oracle.gemm(A, B, bias, "bias_gelu").view(np.float16).astype(np.float64)
    assert np.isposinf(ref[0, 0]) and np.isnan(ref[0, 1]) and np.isnan(ref[0, 2])
    for cfg in all_configs():
        if not _compatible(cfg, M, N, K):
            continue
        print("gelu non-finite", cfg["name"], flush=True)
        got = _run(A, B, bias, "bias_gelu", config=cfg["id"]).cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), cfg["name"]
        assert np.array_equal(np.isposinf(got), np.isposinf(ref)), cfg["name"]
        assert np.array_equal(np.isneginf(got), np.isneginf(ref)), cfg["name"]
        fin = np.isfinite(ref)
        assert np.all(np.abs(got[fin] - ref[fin]) <= 1e-2 * (1 + np.abs(ref[fin]))), cfg["name"]


# ---- the direct kernel on A with any alignment and any K --------------------------------

@pytest.mark.parametrize("shape", [(300, 264, 777), (1000, 3000, 777), (130, 136, 9), (64, 128, 5),
                                   (257, 384, 1027), (128, 128, 65), (300, 264, 776),
                                   (1000, 3000, 784), (257, 520, 8), (600, 768, 1032)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_direct_kernel_k_tail_and_misaligned_a(shape):
    """K % 8 != 0 (the chunk of each A row that holds K is patched in LDS) and an A that is
    only 2-byte aligned, on every direct configuration that serves the K (the ping-pong
    ones need K % 8 == 0: the shapes with such K run them too), against the oracle; C sits
    between NaN guard bands."""
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=K)
    refs = {e: oracle.gemm(A, B, bias, e) for e in ("none", "bias_gelu")}
    Ab = torch.zeros(M * K + 1, dtype=torch.float16, device=DEV)
    Ab[1:] = A.reshape(-1).to(DEV)
    for cfg in all_configs():
        if not cfg["direct"] or (cfg["k_mult8"] and K % 8):
            continue
        for a_dev, how in ((A.to(DEV), "aligned"), (Ab[1:].view(M, K), "A+2 bytes")):
            for e in ("none", "bias_gelu"):
                pad = 4096
                buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
                out = buf[pad:pad + M * N].view(M, N)
                print("direct", cfg["name"], shape, how, e, flush=True)
                g.gemm(a_dev, B.to(DEV), bias.to(DEV) if e != "none" else None, e, out=out,
                       config=cfg["id"])
                torch.cuda.synchronize()
                assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
                assert_parity(out, refs[e], "%s %s %s %s" % (cfg["name"], shape, how, e))


# ---- rows of B and C that are not 16-byte friendly on large problems ---------------------
# The direct kernel takes the columns up to the last multiple of 8 (at any 2-byte
# alignment) and a narrow-load kernel the last N % 8 columns, on the same stream.

SPLIT_SHAPES = [(1024, 1031, 300), (2048, 2047, 2048), (1000, 3001, 777), (768, 2050, 64),
                (1300, 1029, 1001), (1040, 1031, 4999), (16389, 1027, 75)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=["x".join(map(str, s)) for s in SPLIT_SHAPES])
def test_odd_n_takes_the_direct_kernel_and_a_narrow_strip(shape):
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=M + N + K)
    Ad, Bd, biasd = _dev(A), _dev(B), _dev(bias)
    pad = 4096
    for e in EPIS:
        buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        out = buf[pad:pad + M * N].view(M, N)
        cid = g.select(Ad, Bd, biasd if e != "none" else None, e, out=out)
        assert g.mi355gemm_config_info(cid)["direct"] == 1, g.mi355gemm_config_name(cid)
        print("odd N", shape, e, g.mi355gemm_config_name(cid), flush=True)
        g.gemm(Ad, Bd, biasd if e != "none" else None, e, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
        rep = assert_parity(out, oracle.gemm(A, B, bias, e), "odd N %s %s" % (shape, e))
        print("   ", rep, flush=True)


@pytest.mark.parametrize("which", ["B", "C", "bias", "all"])
def test_misaligned_b_c_bias_on_the_direct_kernel(which):
    """N % 8 == 0 but B, C or the bias only 2-byte aligned: the direct kernel serves every
    column with unaligned 16-byte copies and stores."""
    M, N, K = 1024, 1024, 520
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=31)

    def shifted(t, on):
        t = t.to(DEV).reshape(-1)
        if not on:
            return t
        b = torch.zeros(t.numel() + 1, dtype=torch.float16, device=DEV)
        b[1:] = t
        return b[1:]
    Bd = shifted(B, which in ("B", "all")).view(K, N)
    biasd = shifted(bias, which in ("bias", "all"))
    pad = 4096 + (1 if which in ("C", "all") else 0)
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
    out = buf[pad:pad + M * N].view(M, N)
    cid = g.select(_dev(A), Bd, biasd, "bias_gelu", out=out)
    assert g.mi355gemm_config_info(cid)["direct"] == 1
    g.gemm(_dev(A), Bd, biasd, "bias_gelu", out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
    assert_parity(out, oracle.gemm(A, B, bias, "bias_gelu"), "misaligned " + which)


def test_odd_n_strip_ignores_the_next_rows_values():
    """The last N % 8 columns are read as 16-byte pieces whose padding comes from the start
    of the next row of B: an inf there must reach no stored output but its own column's."""
    M, N, K = 1000, 1029, 777
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=5)
    B = B.clone()
    B[:, 0] = float("inf")
    out = g.gemm(_dev(A), _dev(B), _dev(bias), "bias")
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, bias, "bias")
    got = out.cpu().numpy()
    ref16 = ref.view(np.float16)
    assert np.array_equal(np.isnan(got[:, 0]), np.isnan(ref16[:, 0]))
    assert np.array_equal(np.isinf(got[:, 0]), np.isinf(ref16[:, 0]))
    assert np.isfinite(got[:, 1:]).all()
    assert_parity(out[:, 1:].contiguous(), np.ascontiguousarray(ref.view(np.float16)[:, 1:]).view(np.uint16),
                  "strip after an inf column")


SPLIT_EDGES = [(1024, 1031, 0), (1024, 1031, 1), (1024, 1031, 5), (1024, 1031, 8), (1024, 1031, 9),
               (1024, 1031, 16), (1024, 1033, 517), (1, 8191, 64), (13, 8199, 40)]


@pytest.mark.parametrize("shape", SPLIT_EDGES, ids=["x".join(map(str, s)) for s in SPLIT_EDGES])
def test_split_path_edges(shape):
    """Through the direct + narrow split: K entirely inside the narrow kernel's element tail
    (K <= 8), at its boundaries (8, 9, 16), one k-block plus a tail, K = 0 (C = epilogue of
    the bias), and a single row or 13 rows of A."""
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=K + 7)
    Ad, Bd, biasd = _dev(A), _dev(B), _dev(bias)
    for e in ("bias", "bias_gelu"):
        pad = 1024
        buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        out = buf[pad:pad + M * N].view(M, N)
        cid = g.select(Ad, Bd, biasd, e, out=out)
        assert g.mi355gemm_config_info(cid)["direct"] == 1, g.mi355gemm_config_name(cid)
        print("split edge", shape, e, g.mi355gemm_config_name(cid), flush=True)
        g.gemm(Ad, Bd, biasd, e, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
        assert_parity(out, oracle.gemm(A, B, bias, e), "split edge %s %s" % (shape, e))



# ---- at most 8 columns: the narrow kernel -------------------------------------------------

NARROW_SHAPES = [(1, 1, 1), (7, 1, 8), (9, 2, 9), (64, 3, 15), (130, 4, 16), (1000, 5, 17),
                 (257, 6, 100), (64, 7, 511), (200, 8, 512), (33, 1, 513), (520, 3, 2055),
                 (1024, 8, 0), (1024, 7, 4097)]


@pytest.mark.parametrize("shape", NARROW_SHAPES, ids=["x".join(map(str, s)) for s in NARROW_SHAPES])
def test_narrow_kernel_parity(shape):
    """N <= 8 takes the narrow kernel: K inside its element tail (K < 16 with rows closer than
    8 elements), at block boundaries, several blocks per wave; ragged M; every epilogue;
    guard bands around C."""
    M, N, K = shape
    A, B, bias = workloads.make_inputs(M, N, K, "normal", with_bias=True, seed=M * 31 + N * 7 + K)
    Ad, Bd, biasd = _dev(A), _dev(B), _dev(bias)
    for e in EPIS:
        pad = 256
        buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        out = buf[pad:pad + M * N].view(M, N)
        cid = g.select(Ad, Bd, biasd if e != "none" else None, e, out=out)
        assert g.mi355gemm_config_info(cid)["narrow"] == 1, g.mi355gemm_config_name(cid)
        print("narrow", shape, e, flush=True)
        g.gemm(Ad, Bd, biasd if e != "none" else None, e, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
        ref = oracle.gemm(A, B, bias, e)
        assert_parity(out, ref, "narrow %s %s" % (shape, e))
        for cfg in all_configs():
            if not cfg["narrow"]:
                continue
            print("   forced", cfg["name"], flush=True)
            out.fill_(float("nan"))
            g.gemm(Ad, Bd, biasd if e != "none" else None, e, out=out, config=cfg["id"])
            torch.cuda.synchronize()
            assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + M * N:]).all().item()
            assert_parity(out, ref, "narrow %s %s %s" % (cfg["name"], shape, e))


@pytest.mark.parametrize("N", [1, 3, 8])
def test_narrow_kernel_at_any_alignment(N):
    """A, B, C and bias each shifted by one element (2-byte aligned only)."""
    M, K = 300, 1001
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=N)

    def shifted(t):
        t = t.to(DEV).reshape(-1)
        b = torch.zeros(t.numel() + 1, dtype=torch.float16, device=DEV)
        b[1:] = t
        return b[1:]
    Ad, Bd, biasd = shifted(A).view(M, K), shifted(B).view(K, N), shifted(bias)
    buf = torch.full((M * N + 2 * 65,), float("nan"), dtype=torch.float16, device=DEV)
    out = buf[65:65 + M * N].view(M, N)
    cid = g.select(Ad, Bd, biasd, "bias_gelu", out=out)
    assert g.mi355gemm_config_info(cid)["narrow"] == 1
    g.gemm(Ad, Bd, biasd, "bias_gelu", out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:65]).all().item() and torch.isnan(buf[65 + M * N:]).all().item()
    assert_parity(out, oracle.gemm(A, B, bias, "bias_gelu"), "narrow misaligned N=%d" % N)


def test_narrow_config_rejects_wide_problems():
    cid = [c["id"] for c in all_configs() if c["narrow"]][0]
    A = torch.zeros((16, 16), dtype=torch.float16, device=DEV)
    B = torch.zeros((16, 9), dtype=torch.float16, device=DEV)
    C = torch.zeros((16, 9), dtype=torch.float16, device=DEV)
    st = g.mi355gemm_gemm_config(16, 9, 16, A.data_ptr(), B.data_ptr(), C.data_ptr(), None, 0,
                                 torch.cuda.current_stream().cuda_stream, cid)
    assert st == g.EUNSUPPORTED and "at most 8 columns" in g.mi355gemm_last_error()
