"""GPU parity of the attention forward (the tutorial's FlashAttention) through the C ABI.

Tolerance, from the arithmetic: the kernel rounds every softmax weight p_j to fp16 before
the product with v (relative error <= 2^-11 per weight), accumulates scores, sums and
products in fp32 and rounds o to fp16 once (<= 2^-11 |o|).  The oracle computes in fp64
and also returns err = sum_j p_j |v_j| / l, the size of the first error term.  An element
passes when |o_gpu - o_ref| <= 2^-9 err + 2^-10 |o_ref| + 2^-20 (four and two times the
two rounding bounds; the fp32 score, sum and exp2 errors are orders of magnitude smaller
at these sizes); lse passes within 1e-3 absolute (values near log(seq_k) + O(1)).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(DEV)


def _np(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _qkv(B, H, Sq, Sk, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, H, Sq, D)) * scale).astype(np.float16)
    k = (rng.standard_normal((B, H, Sk, D)) * scale).astype(np.float16)
    v = rng.standard_normal((B, H, Sk, D)).astype(np.float16)
    return q, k, v


def _check(got_bits, ref_bits, err, what):
    got = got_bits.view(np.float16).astype(np.float64)
    ref = ref_bits.view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    tol = 2.0 ** -9 * err + 2.0 ** -10 * np.abs(ref) + 2.0 ** -20
    bad = np.abs(got - ref) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance, first at %s: got %r ref %r tol %r"
                             % (what, bad.sum(), tuple(i), got[tuple(i)], ref[tuple(i)], tol[tuple(i)]))
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= 5e-3, "%s: relative Frobenius distance %.2e" % (what, rel)


SHAPES = [  # B, H, Sq, Sk, D
    (1, 1, 1, 1, 64), (1, 2, 5, 7, 128), (2, 3, 256, 256, 128), (1, 2, 300, 300, 64),
    (1, 1, 513, 77, 128), (1, 1, 77, 513, 128), (2, 2, 1000, 1000, 128), (1, 3, 640, 1111, 64),
    (3, 1, 257, 64, 128), (1, 1, 64, 65, 64)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_attention_parity(shape, causal):
    B, H, Sq, Sk, D = shape
    print("attention", shape, "causal" if causal else "full", flush=True)
    q, k, v = _qkv(B, H, Sq, Sk, D, seed=sum(shape) * 3 + causal, scale=1.5)
    scale = 1.0 / np.sqrt(D)
    ro, rl, re = oracle.attention(q, k, v, scale=scale, causal=causal)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    o = g.attention(_t(q), _t(k), _t(v), causal=causal, lse=lse)
    torch.cuda.synchronize()
    _check(_np(o), ro, re, "o %s" % (shape,))
    assert np.allclose(lse.cpu().numpy(), rl, rtol=0, atol=1e-3), "lse %s" % (shape,)


@pytest.mark.parametrize("scale", [0.02, 0.3, 1.0])
def test_attention_scales(scale):
    """Flat to peaked softmax: small scales spread the weight over every key, large ones
    concentrate it on a few (fp16 inputs of spread 2 and scale 1 give score gaps of
    hundreds)."""
    B, H, Sq, Sk, D = 1, 2, 300, 520, 128
    print("attention scale", scale, flush=True)
    q, k, v = _qkv(B, H, Sq, Sk, D, seed=int(scale * 100), scale=2.0)
    for causal in (False, True):
        ro, _, re = oracle.attention(q, k, v, scale=scale, causal=causal)
        o = g.attention(_t(q), _t(k), _t(v), causal=causal, scale=scale)
        torch.cuda.synchronize()
        _check(_np(o), ro, re, "scale %g causal %d" % (scale, causal))


def test_attention_exact_cases():
    """One key: every weight is exactly 1, so o = v bit for bit.  One-hot keys with a large
    scale: every other weight is exactly 0 in fp32, so o = v[selected] bit for bit."""
    for D in (64, 128):
        print("attention exact D", D, flush=True)
        q, k, v = _qkv(2, 3, 77, 1, D, seed=D)
        for causal in (False, True):
            o = g.attention(_t(q), _t(k), _t(v), causal=causal)
            torch.cuda.synchronize()
            assert np.array_equal(_np(o), np.broadcast_to(v.view(np.uint16), o.shape))
        rng = np.random.default_rng(D + 1)
        Sk = D
        sigma = rng.permutation(D)
        k = np.zeros((1, 1, Sk, D), np.float16)
        k[0, 0, np.arange(Sk), sigma] = 4.0
        v = rng.standard_normal((1, 1, Sk, D)).astype(np.float16)
        pi = rng.integers(0, Sk, size=300)
        q = np.zeros((1, 1, 300, D), np.float16)
        q[0, 0, np.arange(300), sigma[pi]] = 8.0
        o = g.attention(_t(q), _t(k), _t(v), causal=False, scale=4.0)
        torch.cuda.synchronize()
        assert np.array_equal(_np(o)[0, 0], v[0, 0, pi].view(np.uint16))
        # causal: query i points at key min(i, Sk-1) (visible) -> that value row
        sel = np.minimum(np.arange(300), Sk - 1)
        q = np.zeros((1, 1, 300, D), np.float16)
        q[0, 0, np.arange(300), sigma[sel]] = 8.0
        o = g.attention(_t(q), _t(k), _t(v), causal=True, scale=4.0)
        torch.cuda.synchronize()
        assert np.array_equal(_np(o)[0, 0], v[0, 0, sel].view(np.uint16))


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_full_size_sampled(D, causal):
    """The benchmark's size (batch 4, 32 heads, 4096 queries and keys) in the launch the
    benchmark times; sampled rows (first and last of the sequence, of query blocks and of
    waves, random ones) against the oracle computed row by row."""
    B, H, S = 4, 32, 4096
    print("attention full size D", D, "causal" if causal else "full", flush=True)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(D + causal)
    q = torch.randn((B, H, S, D), generator=gen).to(torch.float16)
    k = torch.randn((B, H, S, D), generator=gen).to(torch.float16)
    v = torch.randn((B, H, S, D), generator=gen).to(torch.float16)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    o = g.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, lse=lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.concatenate([[0, 1, 31, 32, 255, 256, 257, 511, 2047, 2048, S - 2, S - 1],
                           rng.integers(0, S, size=36)])
    pairs = rng.integers(0, B * H, size=rows.size)
    pairs[:4] = [0, B * H - 1, 0, B * H - 1]
    qn, kn, vn = (t.numpy().reshape(B * H, S, D) for t in (q, k, v))
    ro, rl, re = oracle.attention_rows(qn, kn, vn, pairs, rows, causal=causal)
    got = _np(o).reshape(B * H, S, D)[pairs, rows]
    _check(got, ro, re, "full size D %d causal %d" % (D, causal))
    gl = lse.cpu().numpy().reshape(B * H, S)[pairs, rows]
    assert np.allclose(gl, rl, rtol=0, atol=1e-3)


def test_attention_guard_bands_and_side_stream():
    """Output written exactly in place: the neighbouring batches of a larger buffer keep
    their sentinel; the call runs on a side stream."""
    B, H, Sq, Sk, D = 2, 2, 300, 200, 128
    print("attention guard bands", flush=True)
    q, k, v = _qkv(B, H, Sq, Sk, D, seed=99)
    big = torch.full((B + 2, H, Sq, D), 7.0, dtype=torch.float16, device=DEV)
    lse_big = torch.full((B + 2, H, Sq), 7.0, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    qt, kt, vt = _t(q), _t(k), _t(v)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.attention(qt, kt, vt, causal=True, out=big[1:B + 1], lse=lse_big[1:B + 1], stream=s)
    s.synchronize()
    assert torch.all(big[0] == 7.0) and torch.all(big[B + 1] == 7.0)
    assert torch.all(lse_big[0] == 7.0) and torch.all(lse_big[B + 1] == 7.0)
    ro, rl, re = oracle.attention(q, k, v, causal=True)
    _check(_np(big[1:B + 1]), ro, re, "in place")
    assert np.allclose(lse_big[1:B + 1].cpu().numpy(), rl, rtol=0, atol=1e-3)


def test_attention_empty_and_errors():
    z = torch.empty((0, 2, 5, 64), dtype=torch.float16, device=DEV)
    assert g.attention(z, z, z).shape == z.shape
    q = torch.zeros((1, 1, 0, 64), dtype=torch.float16, device=DEV)
    k = torch.zeros((1, 1, 4, 64), dtype=torch.float16, device=DEV)
    assert g.attention(q, k, k).shape == q.shape
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float16, device=DEV)
    k0 = torch.zeros((1, 1, 0, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(g.GemmError) as e:
        g.attention(q, k0, k0)
    assert e.value.status == g.EINVAL
    q96 = torch.zeros((1, 1, 4, 96), dtype=torch.float16, device=DEV)
    with pytest.raises(g.GemmError) as e:
        g.attention(q96, q96, q96)
    assert e.value.status == g.EUNSUPPORTED


def test_attention_leading_dimensions():
    """Any leading dimensions: 3-D (heads, seq, d) and 5-D tensors give the same rows as
    the 4-D call on the same data."""
    q, k, v = _qkv(2, 3, 150, 170, 64, seed=123)
    o4 = _np(g.attention(_t(q), _t(k), _t(v), causal=True))
    q3, k3, v3 = (x.reshape(6, *x.shape[2:]) for x in (q, k, v))
    o3 = _np(g.attention(_t(q3), _t(k3), _t(v3), causal=True))
    q5, k5, v5 = (x.reshape(1, 2, 3, *x.shape[2:]) for x in (q, k, v))
    lse = torch.empty((1, 2, 3, 150), dtype=torch.float32, device=DEV)
    o5 = _np(g.attention(_t(q5), _t(k5), _t(v5), causal=True, lse=lse))
    torch.cuda.synchronize()
    assert np.array_equal(o3.reshape(o4.shape), o4) and np.array_equal(o5.reshape(o4.shape), o4)
    ro, rl, re = oracle.attention(q, k, v, causal=True)
    _check(o4, ro, re, "leading dims")
    assert np.allclose(lse.cpu().numpy().reshape(rl.shape), rl, atol=1e-3)
    q2 = _t(q[0, 0])          # (seq, d): one problem
    o2 = _np(g.attention(q2, _t(k[0, 0]), _t(v[0, 0]), causal=True))
    torch.cuda.synchronize()
    assert np.array_equal(o2, o4[0, 0])
