"""GPU parity of the element-wise fp16 vector add (the tutorial's first kernel) through the
C ABI: bit-exact against the oracle (the correctly rounded sum), NaN compared as NaN."""
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


def _check(got_bits, want_bits, what):
    nan_g = ((got_bits & 0x7C00) == 0x7C00) & ((got_bits & 0x3FF) != 0)
    nan_w = ((want_bits & 0x7C00) == 0x7C00) & ((want_bits & 0x3FF) != 0)
    assert np.array_equal(nan_g, nan_w), what + ": NaN positions differ"
    ok = (got_bits == want_bits) | nan_w
    if not ok.all():
        i = int(np.argmax(~ok))
        raise AssertionError("%s: element %d got %#06x want %#06x (%d differ)"
                             % (what, i, got_bits[i], want_bits[i], int((~ok).sum())))


def _random_bits(n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 1000, 4097, (1 << 20) + 3])
def test_vector_add_bitexact(n):
    a, b = _random_bits(n, n), _random_bits(n, n + 1)
    want = oracle.vector_add(a, b)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.float16).to(DEV)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.float16).to(DEV)
    print("vector_add n=%d" % n, flush=True)
    c = g.vector_add(ta, tb)
    torch.cuda.synchronize()
    _check(_bits(c), want, "n=%d" % n)


def test_vector_add_every_relative_alignment_with_guard_bands():
    n = 3001
    a, b = _random_bits(n, 11), _random_bits(n, 12)
    want = oracle.vector_add(a, b)
    pad = 64
    for sa in range(8):
        for sc in range(8):
            sb = (sa + sc) % 8
            ba = torch.zeros(n + 16, dtype=torch.float16, device=DEV)
            bb = torch.zeros(n + 16, dtype=torch.float16, device=DEV)
            bc = torch.full((n + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
            ba[sa:sa + n] = torch.from_numpy(a.view(np.int16)).view(torch.float16).to(DEV)
            bb[sb:sb + n] = torch.from_numpy(b.view(np.int16)).view(torch.float16).to(DEV)
            out = bc[pad + sc:pad + sc + n]
            g.vector_add(ba[sa:sa + n], bb[sb:sb + n], out=out)
            torch.cuda.synchronize()
            _check(_bits(out), want, "offsets a=%d b=%d c=%d" % (sa, sb, sc))
            assert torch.isnan(bc[:pad + sc]).all().item()
            assert torch.isnan(bc[pad + sc + n:]).all().item()


def test_vector_add_in_place_and_specials():
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF,
                         0x7C00, 0xFC00, 0x7E00, 0x3C00, 0xBC00, 0x3555, 0x7BFE], np.uint16)
    a = np.repeat(specials, specials.size)
    b = np.tile(specials, specials.size)
    want = oracle.vector_add(a, b)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.float16).to(DEV)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.float16).to(DEV)
    g.vector_add(ta, tb, out=ta)          # c aliases a
    torch.cuda.synchronize()
    _check(_bits(ta), want, "specials, in place")


def test_vector_add_empty_and_errors():
    e = torch.empty(0, dtype=torch.float16, device=DEV)
    assert g.vector_add(e, e).numel() == 0
    x = torch.zeros(8, dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        g.vector_add(x, torch.zeros(9, dtype=torch.float16, device=DEV))
    with pytest.raises(TypeError):
        g.vector_add(x.float(), x)
