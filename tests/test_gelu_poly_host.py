"""The fused GELU's arithmetic, checked on the CPU.

The GEMM kernels evaluate GELU(x) = max(x, 0) - |x| * 2^P(|x|), with P a degree-7
polynomial for log2 Phi(-z) (``gelu_erf`` in ``csrc/gemm_common.hpp``; the coefficients
come from ``dense_fp16_gemm_fp32_amd/gelu_poly.py``).  These tests read the coefficients
from the header, check them against scipy's log of the normal CDF, and run the kernel's
fp32 operations, emulated in numpy, over every finite fp16 input against the oracle's
correctly rounded GELU.  The GPU tests run the same inputs through the kernels.
"""
import os
import re

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_fp32_amd import gelu_poly

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "dense_fp16_gemm_fp32_amd", "csrc", "gemm_common.hpp")
F32_MAX = np.float32(3.4028234663852886e38)


def header_coefficients() -> np.ndarray:
    text = open(HEADER).read()
    body = text[text.index("float gelu_erf(float x)"):]
    body = body[:body.index("\n}\n")]
    found = dict((int(k), np.float32(float(v)))
                 for k, v in re.findall(r"\bc(\d) = ([-+0-9.e]+)f", body))
    assert sorted(found) == list(range(gelu_poly.DEGREE + 1)), found
    return np.array([found[k] for k in range(gelu_poly.DEGREE + 1)], dtype=np.float32)


def kernel_gelu_f16(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """fp16 bits of the kernel's GELU of fp32 inputs x: Horner in fp32 fused steps, exp2
    rounded to fp32, and the last multiply-add rounded once to fp16 (v_fma_mixlo_f16)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        q = gelu_poly.horner_f32(c, np.abs(x))
        h = np.exp2(q.astype(np.float64)).astype(np.float32)
        ax = np.abs(np.minimum(x, F32_MAX))
        r = -ax.astype(np.float64) * h.astype(np.float64) + np.maximum(x, np.float32(0)).astype(np.float64)
    return r.astype(np.float16).view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def test_header_holds_the_fitted_coefficients():
    pytest.importorskip("scipy")
    assert np.array_equal(header_coefficients(), gelu_poly.coefficients())


def test_polynomial_tracks_log2_of_the_normal_tail():
    """Within 8e-6 of log2 Phi(-z) on [0, 6] in fp32 Horner form (h within 6e-6
    relative); Phi(-0) = 1/2 gives P(0) = -1."""
    special = pytest.importorskip("scipy.special")
    c = header_coefficients()
    z = np.linspace(0.0, gelu_poly.Z_MAX, 600001)
    err = np.abs(gelu_poly.horner_f32(c, z).astype(np.float64) - special.log_ndtr(-z) / np.log(2.0))
    assert err.max() <= 8e-6, err.max()
    assert abs(float(gelu_poly.horner_f32(c, np.zeros(1))[0]) + 1.0) <= 1e-5


def test_polynomial_falls_to_minus_infinity_beyond_the_fit():
    """Past z = 6, P decreases from -29.9 (2^P < 1.1e-9, so |x| 2^P < 2^-25 rounds to
    zero in fp16 for 6 <= |x| <= 1000) and Horner's rule
    ends in -inf, never NaN, up to the largest float."""
    c = header_coefficients()
    near = gelu_poly.horner_f32(c, np.linspace(6.0, 1e3, 100001))
    assert np.all(np.diff(near.astype(np.float64)) < 0)
    assert near.max() <= -29.9
    far = np.logspace(np.log10(6.0), np.log10(float(F32_MAX)), 20001).astype(np.float32)
    far = far[np.isfinite(far)]
    q = gelu_poly.horner_f32(c, far)
    assert not np.isnan(q).any()
    q = q.astype(np.float64)
    first_inf = int(np.argmax(np.isneginf(q)))
    assert first_inf > 0 and np.all(np.isneginf(q[first_inf:]))
    assert np.all(np.diff(q[:first_inf]) <= 0)
    z = np.linspace(6.0, 1e3, 100001).astype(np.float32)
    assert np.all(z.astype(np.float64) * np.exp2(near.astype(np.float64)) < 2.0 ** -25)


def test_every_finite_fp16_input_against_the_oracle():
    """The emulated kernel arithmetic: within one fp16 step of the oracle's correctly
    rounded GELU everywhere, equal to it for at least 99% of the inputs (the GPU test
    asks the same of the kernels)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7C00) != 0x7C00]
    x = finite.view(np.float16).astype(np.float32)
    ref = oracle.f64_to_f16(oracle.gelu(x.astype(np.float64)))
    got = kernel_gelu_f16(x, header_coefficients())
    d = np.abs(ordered(got) - ordered(ref))
    assert d.max() <= 1, float(x[np.argmax(d)])
    assert (d == 0).mean() >= 0.99, (d == 0).mean()


def test_non_finite_inputs():
    """+inf gives +inf, -inf and NaN give NaN (x * Phi(x) in IEEE arithmetic: -inf * 0
    and NaN); the largest fp16 values and the signed zeros are exact."""
    x = np.array([np.inf, -np.inf, np.nan, 65504.0, -65504.0, 0.0, -0.0], dtype=np.float32)
    got = kernel_gelu_f16(x, header_coefficients()).view(np.float16).astype(np.float64)
    assert np.isposinf(got[0]) and np.isnan(got[1]) and np.isnan(got[2])
    assert got[3] == 65504.0 and got[4] == 0.0 and got[5] == 0.0 and got[6] == 0.0
