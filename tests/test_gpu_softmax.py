"""GPU parity of the row-wise softmax (the tutorial's fused softmax) through the C ABI.

The kernel computes in fp32 and the oracle in fp64, both rounding once to fp16, so the
bar is: within one fp16 step everywhere, equal for at least 99% of the elements, and NaN
in exactly the same places."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _ordered(b):
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _isnan(b):
    return ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)


def _check(got, want, what, exact_frac=0.99):
    assert np.array_equal(_isnan(got), _isnan(want)), what + ": NaN positions differ"
    keep = ~_isnan(want)
    d = np.abs(_ordered(got[keep]) - _ordered(want[keep]))
    assert d.size == 0 or d.max() <= 1, "%s: off by %d fp16 steps" % (what, d.max())
    assert d.size == 0 or (d == 0).mean() >= exact_frac, "%s: %.4f exact" % (what, (d == 0).mean())


def _x(M, N, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, N)) * scale).astype(np.float16)


def _run(x, out=None):
    t = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(DEV)
    y = g.softmax(t, out=out)
    torch.cuda.synchronize()
    return y


SHAPES = [(1, 1), (3, 7), (5, 8), (64, 512), (33, 513), (4, 1000), (5, 2048), (5, 2049),
          (7, 4096), (6, 4097), (9, 8191), (4, 8193),
          (3, 16384), (2, 16385), (3, 32768), (2, 32769), (5, 65536), (2, 70001),
          (2, 131072), (2, 131073), (1000, 3000), (4096, 256)]


@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_softmax_parity(shape):
    M, N = shape
    x = _x(M, N, M * 7 + N)
    print("softmax", shape, flush=True)
    _check(_bits(_run(x)), oracle.softmax(x), "%dx%d" % shape)


@pytest.mark.parametrize("N", [6, 300, 20000, 100000, 200000])
def test_softmax_edge_rows(N):
    x = _x(6, N, N, scale=2.0)
    x[0, ::3] = -np.inf                 # some -inf: finite result
    x[1, :] = -np.inf                   # all -inf: NaN row
    x[2, N // 2] = np.inf               # +inf: NaN row
    x[3, N - 1] = np.nan                # NaN: NaN row
    x[4, :] = 5.0                       # constant: 1/N
    x[5, 0] = 60.0                      # dominant: one-hot
    _check(_bits(_run(x)), oracle.softmax(x), "edge rows N=%d" % N)


def test_softmax_in_place_and_guard_bands():
    M, N = 37, 1003                     # rows only 2-byte aligned
    x = _x(M, N, 99)
    want = oracle.softmax(x)
    t = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(DEV)
    g.softmax(t, out=t)
    torch.cuda.synchronize()
    _check(_bits(t), want, "in place")
    pad = 64
    for shift in (0, 1, 3):
        buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        out = buf[pad + shift:pad + shift + M * N].view(M, N)
        _run(x, out=out)
        _check(_bits(out), want, "output offset %d" % shift)
        assert torch.isnan(buf[:pad + shift]).all().item()
        assert torch.isnan(buf[pad + shift + M * N:]).all().item()


def test_softmax_rows_sum_to_one():
    x = _x(256, 4096, 5)
    y = _run(x).float()
    assert torch.allclose(y.sum(dim=1), torch.ones(256, device=DEV), atol=4096 * 2.0 ** -12)


def test_softmax_leading_dimensions():
    """Any leading dimensions: a 3-D tensor and a 1-D vector are softmaxed over the last
    dimension, row by row, exactly as the 2-D call on the same rows."""
    x = _x(12, 777, 9)
    y2 = _bits(_run(x))
    t3 = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(DEV).reshape(3, 4, 777)
    y3 = _bits(g.softmax(t3))
    t1 = torch.from_numpy(x[5].copy().view(np.int16)).view(torch.float16).to(DEV)
    y1 = _bits(g.softmax(t1))
    torch.cuda.synchronize()
    assert np.array_equal(y3.reshape(y2.shape), y2) and np.array_equal(y1, y2[5])
