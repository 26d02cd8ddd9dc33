"""Derivation of the polynomial the GEMM kernels use for the normal tail in their fused
GELU epilogue (``gelu_erf`` in ``csrc/gemm_common.hpp``).

GELU(x) = x * Phi(x) (Phi the standard normal CDF) is evaluated as
max(x, 0) - |x| * Phi(-|x|), and Phi(-z) for z = |x| as 2^P(z), with P a polynomial of
degree 7 fitted to log2 Phi(-z) on [0, 6]: a least-squares fit on 4000 Chebyshev nodes of
that interval, converted to the power basis and rounded to fp32.

- On [0, 6], P evaluated by Horner's rule in fp32 is within 8e-6 of log2 Phi(-z), so
  2^P is within 6e-6 relative of Phi(-z), against the 2^-11 relative step of the fp16
  result.
- The leading coefficient is negative, and P decreases from -29.9 at z = 6 on: 2^P stays
  below 1.1e-9 there, so |x| * 2^P rounds to zero in fp16 for every x <= -6, as
  x * Phi(x) does. Horner's rule overflows to -inf (never NaN) for large z, and 2^-inf
  is 0.

Run as a script, it prints the fp32 coefficients in the form the kernel header holds
them; a CPU test checks that the header's values are these.  Needs numpy and scipy.
"""

import numpy as np

DEGREE = 7
Z_MAX = 6.0
NODES = 4000


def coefficients(degree: int = DEGREE, z_max: float = Z_MAX, nodes: int = NODES) -> np.ndarray:
    """Power-basis coefficients c[0..degree] of P, rounded to fp32."""
    from scipy.special import log_ndtr
    z = np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes) * (z_max / 2) + z_max / 2
    fit = np.polynomial.chebyshev.Chebyshev.fit(z, log_ndtr(-z) / np.log(2.0), degree,
                                                domain=[0.0, z_max])
    return fit.convert(kind=np.polynomial.Polynomial).coef.astype(np.float32)


def horner_f32(c: np.ndarray, z: np.ndarray) -> np.ndarray:
    """P(z) by Horner's rule with each step a fused multiply-add rounded to fp32, as the
    kernel evaluates it (an fp32 product is exact in fp64, so one fp64 multiply-add
    rounded to fp32 is the fused operation except for rare double roundings)."""
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    acc = np.full(z64.shape, c[-1], dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for k in range(len(c) - 2, -1, -1):
            acc = (acc.astype(np.float64) * z64 + np.float64(c[k])).astype(np.float32)
    return acc


if __name__ == "__main__":
    for k, v in enumerate(coefficients()):
        print("c%d = %.9ef" % (k, float(v)))
