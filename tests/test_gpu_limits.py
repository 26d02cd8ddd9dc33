"""GPU parity at the largest sizes each entry point accepts (the 32-bit buffer offsets
the kernels use) and past 4 GiB per operand (64-bit pointer arithmetic), on sampled
outputs the oracle computes one by one.

Inputs are seeded synthetic draws made on the device by torch's generator (the host
could not draw gigabytes quickly); only the slices the sampled outputs depend on are
copied back for the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import oracle
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
KMAX = (1 << 22) - 1          # K and N must stay below 2^22


def _randn(shape, seed, scale=1.0):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)
    if scale != 1.0:
        t *= scale
    return t.to(torch.float16)


def _check_sampled(A, B, C, rows, cols, bias=None, epi="none", what=""):
    """C[rows x cols] against the oracle's product of the matching A rows and B columns."""
    r = torch.as_tensor(rows, device=DEV)
    c = torch.as_tensor(cols, device=DEV)
    a = A.index_select(0, r).cpu()
    b = B.index_select(1, c).cpu().contiguous()
    bb = bias.index_select(0, c).cpu() if bias is not None else None
    ref = oracle.gemm(a, b, bb, epi)
    got = C.index_select(0, r).index_select(1, c)
    return assert_parity(got, ref, what)


@pytest.mark.parametrize("K", [KMAX, KMAX - 7])
def test_gemm_at_the_k_limit_every_config(K):
    """K just below 2^22 (odd, and a multiple of 8): A and B of 2 GiB each; every
    configuration that can serve the shape, forced."""
    M = N = 256
    print("gemm K limit", K, flush=True)
    A = _randn((M, K), 1, K ** -0.5)
    B = _randn((K, N), 2, 1.0)
    rows = [0, 1, 127, 128, 255]
    cols = [0, 7, 128, 200, 255]
    ran = 0
    for cfg in g.configs():
        if ((cfg["a_vector"] or cfg["k_mult8"]) and K % 8) or cfg["narrow"]:
            continue
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        st = g.mi355gemm_gemm_config(M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), None, 0,
                                     torch.cuda.current_stream().cuda_stream, cfg["id"])
        assert st == g.OK, (cfg["name"], g.mi355gemm_last_error())
        torch.cuda.synchronize()
        print("   ", cfg["name"], _check_sampled(A, B, C, rows, cols, what=cfg["name"]), flush=True)
        ran += 1
    assert ran >= 4


@pytest.mark.parametrize("N", [KMAX, KMAX - 7])
def test_gemm_at_the_n_limit(N):
    """N just below 2^22: C of 1 GiB, columns at the far end, with the fused epilogue."""
    M, K = 128, 96
    print("gemm N limit", N, flush=True)
    A = _randn((M, K), 3)
    B = _randn((K, N), 4, K ** -0.5)
    bias = _randn((N,), 5)
    C = g.gemm(A, B, bias, "bias_gelu")
    torch.cuda.synchronize()
    cols = [0, 1, 8 * (N // 8) - 1, N - 9, N - 2, N - 1, N // 2]
    print("   ", _check_sampled(A, B, C, [0, 63, 64, 127], cols, bias, "bias_gelu", "N limit"), flush=True)


def test_gemm_operands_past_4_gib():
    """M = 2^26 rows: A and C of 8 GiB each, so row offsets pass 2^32 bytes."""
    M, N, K = 1 << 26, 64, 64
    print("gemm M = 2^26", flush=True)
    A = _randn((M, K), 6)
    B = _randn((K, N), 7, 0.125)
    C = g.gemm(A, B)
    torch.cuda.synchronize()
    rows = [0, 1, (1 << 25) - 1, 1 << 25, M - 129, M - 2, M - 1]
    print("   ", _check_sampled(A, B, C, rows, [0, 31, 63], what="M past 4 GiB"), flush=True)
    del A, C


def test_attention_at_the_sequence_limit():
    """seq_k just below the 32-bit offset limit for head dim 128 (k and v 2 GiB each)."""
    D = 128
    Sk = (1 << 31) // (2 * D) - 1025
    Sq = 300
    print("attention seq_k", Sk, flush=True)
    q = _randn((1, 1, Sq, D), 8)
    k = _randn((1, 1, Sk, D), 9)
    v = _randn((1, 1, Sk, D), 10)
    lse = torch.empty((1, 1, Sq), dtype=torch.float32, device=DEV)
    for causal in (False, True):
        o = g.attention(q, k, v, causal=causal, lse=lse)
        torch.cuda.synchronize()
        rows = np.array([0, 255, 256, Sq - 1])
        ro, rl, re = oracle.attention_rows(q.cpu().numpy().reshape(1, Sq, D),
                                           k.cpu().numpy().reshape(1, Sk, D),
                                           v.cpu().numpy().reshape(1, Sk, D),
                                           np.zeros(rows.size, np.int64), rows, causal=causal)
        got = o.reshape(Sq, D)[torch.as_tensor(rows, device=DEV)].cpu().contiguous()
        gf = got.numpy().astype(np.float64)
        rf = ro.view(np.float16).astype(np.float64)
        tol = 2.0 ** -9 * re + 2.0 ** -10 * np.abs(rf) + 2.0 ** -20
        assert np.all(np.abs(gf - rf) <= tol), "causal %d max excess %g" % (causal, np.max(np.abs(gf - rf) - tol))
        assert np.allclose(lse.reshape(Sq)[torch.as_tensor(rows, device=DEV)].cpu().numpy(), rl, atol=1e-3)


def test_softmax_long_row_and_many_rows():
    """One row of 2^27 elements (softmax_long) and 2^22 + 3 rows of 1000 (8 GiB)."""
    print("softmax long row", flush=True)
    x = _randn((1, 1 << 27), 11, 3.0)
    y = g.softmax(x)
    torch.cuda.synchronize()
    ref = oracle.softmax(x.cpu().numpy()).view(np.float16)
    d = np.abs(y.cpu().numpy().view(np.int16).astype(np.int32) - ref.view(np.int16).astype(np.int32))
    assert d.max() <= 1 and (d == 0).mean() >= 0.99
    del x, y
    print("softmax many rows", flush=True)
    M, N = (1 << 22) + 3, 1000
    x = _randn((M, N), 12, 3.0)
    y = g.softmax(x)
    torch.cuda.synchronize()
    rows = torch.as_tensor([0, 1, M // 2, M - 2, M - 1], device=DEV)
    ref = oracle.softmax(x.index_select(0, rows).cpu().numpy()).view(np.int16).astype(np.int32)
    got = y.index_select(0, rows).cpu().numpy().view(np.int16).astype(np.int32)
    d = np.abs(got - ref)
    assert d.max() <= 1 and (d == 0).mean() >= 0.99


def test_vector_add_past_2_31_elements():
    """n = 2^31 + 1001 elements (4 GiB per operand): the head, the middle around 2^31 and
    the tail are bit-exact."""
    n = (1 << 31) + 1001
    print("vector add n", n, flush=True)
    a = _randn((n,), 13)
    b = _randn((n,), 14)
    c = torch.empty_like(a)
    g.vector_add(a, b, out=c)
    torch.cuda.synchronize()
    for lo in (0, (1 << 31) - 4096, n - 4096):
        sa, sb, sc = (t[lo:lo + 4096].cpu().numpy() for t in (a, b, c))
        assert np.array_equal(sc.view(np.uint16), oracle.vector_add(sa, sb)), lo


@pytest.mark.parametrize("K", [KMAX, KMAX - 7])
def test_narrow_gemm_at_the_k_limit(K):
    """Three columns (the narrow kernel), K just below 2^22: every output against the oracle."""
    M, N = 40, 3
    print("narrow K limit", K, flush=True)
    A = _randn((M, K), 3, K ** -0.5)
    B = _randn((K, N), 4, 1.0)
    C = g.gemm(A, B)
    torch.cuda.synchronize()
    _check_sampled(A, B, C, list(range(M)), list(range(N)), what="narrow K=%d" % K)
