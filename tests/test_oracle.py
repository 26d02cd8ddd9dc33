"""Pins for the CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself: numpy's own binary16
conversions (exhaustive), IEEE 754 rounding cases, normal-CDF table values and scipy's
``ndtr``, exact rational arithmetic (``fractions.Fraction``) on tiny shapes, numpy's
fp64 matmul, and closed forms (all-ones, selection and permutation matrices, zero
operands, transposition).  ``test_oracle_mutants.py`` checks that plausible mistakes
planted in the oracle's C source fail at least one of these pins.
"""
from __future__ import annotations

import bisect
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALL_BITS = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _lib(request):
    return getattr(request, "param", None) or oracle.load()


# ---------------------------------------------------------------- fp16 codec --------

def test_decode_exhaustive_matches_numpy(oracle_lib):
    got = oracle.f16_to_f64(ALL_BITS, lib=oracle_lib)
    ref = ALL_BITS.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zero too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_encode_roundtrip_every_finite_pattern(oracle_lib):
    vals = ALL_BITS.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    back = oracle.f64_to_f16(vals[finite], lib=oracle_lib)
    assert np.array_equal(back, ALL_BITS[finite])
    inf_bits = oracle.f64_to_f16(np.array([np.inf, -np.inf]), lib=oracle_lib)
    assert list(inf_bits) == [0x7C00, 0xFC00]
    assert oracle.f64_to_f16(np.array([np.nan]), lib=oracle_lib)[0] & 0x7FFF > 0x7C00


def _midpoints():
    """Midpoints between adjacent finite fp16 values (both signs), and each midpoint
    nudged one fp64 ulp either way."""
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16)
    v = pos.astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0          # exact in fp64
    mids = np.concatenate([mids, [65520.0]])
    allm = np.concatenate([mids, -mids])
    return np.concatenate([allm, np.nextafter(allm, np.inf), np.nextafter(allm, -np.inf)])


def test_encode_midpoints_match_numpy(oracle_lib):
    x = _midpoints()
    got = oracle.f64_to_f16(x, lib=oracle_lib)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_encode_random_doubles_match_numpy(oracle_lib):
    rng = np.random.default_rng(1234)
    mag = np.exp2(rng.uniform(-30, 17, size=400_000))
    x = mag * rng.choice([-1.0, 1.0], size=mag.size)
    got = oracle.f64_to_f16(x, lib=oracle_lib)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _parse_float(tok: str) -> float:
    return float.fromhex(tok) if "0x" in tok else float(tok)


def test_encode_ieee_golden_cases(oracle_lib):
    rows = []
    with open(os.path.join(GOLDEN, "f16_rounding_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tok = line.split()
            rows.append((_parse_float(tok[0]), int(tok[1], 16), line.strip()))
    assert len(rows) >= 15
    got = oracle.f64_to_f16(np.array([r[0] for r in rows]), lib=oracle_lib)
    for (x, want, line), g in zip(rows, got):
        assert int(g) == want, line


# ---------------------------------------------------------------- GELU --------------

def _gelu_points():
    pts = []
    with open(os.path.join(GOLDEN, "gelu_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            x, phi = (float(t) for t in line.split())
            pts.append((x, phi))
    return pts


def test_gelu_table_points(oracle_lib):
    pts = _gelu_points()
    x = np.array([p[0] for p in pts])
    want = x * np.array([p[1] for p in pts])
    got = oracle.gelu(x, lib=oracle_lib)
    assert got[x == 0.0][0] == 0.0
    np.testing.assert_allclose(got, want, rtol=4e-15, atol=0)  # a few ulp of libm erf


def test_gelu_matches_scipy_ndtr_on_a_dense_grid(oracle_lib):
    x = np.linspace(-12.0, 12.0, 200_001)
    got = oracle.gelu(x, lib=oracle_lib)
    want = x * ndtr(x)
    # relative agreement wherever the value is not deep in the underflowing tail
    big = np.abs(want) > 1e-300
    np.testing.assert_allclose(got[big], want[big], rtol=1e-13, atol=0)


def test_gelu_odd_part_identity_and_minimum(oracle_lib):
    x = np.linspace(0.0, 8.0, 4001)
    d = oracle.gelu(x, lib=oracle_lib) - oracle.gelu(-x, lib=oracle_lib)
    np.testing.assert_allclose(d, x, rtol=0, atol=4e-15)
    grid = np.linspace(-3, 0, 300_001)
    g = oracle.gelu(grid, lib=oracle_lib)
    i = int(np.argmin(g))
    assert abs(grid[i] - (-0.7517915)) < 2e-5
    assert abs(g[i] - (-0.1699712)) < 1e-6


def test_gelu_fp16_large_x_limits_exhaustive(oracle_lib):
    """Over every finite fp16 x: fp16(GELU(x)) == x for x >= 3.5, and -0 for x <=
    -5.7265625; everywhere, the oracle agrees with numpy's rounding of x*ndtr(x) except
    at fp16 near-ties."""
    x = ALL_BITS.view(np.float16).astype(np.float64)
    fin = np.isfinite(x)
    xs = x[fin]
    g = oracle.gelu(xs, lib=oracle_lib)
    bits = oracle.f64_to_f16(g, lib=oracle_lib)
    big = xs >= 3.5
    assert np.array_equal(bits[big], ALL_BITS[fin][big])
    neg = xs <= -5.7265625
    assert np.all(bits[neg] == 0x8000)
    ref = (xs * ndtr(xs)).astype(np.float16).view(np.uint16)
    diff = np.nonzero(bits != ref)[0]
    for i in diff:  # only near-ties may differ: check the two fp64 values straddle a midpoint
        a, b = g[i], xs[i] * ndtr(xs[i])
        assert abs(a - b) <= 1e-13 * max(abs(a), 1e-300), (xs[i], a, b)


# ---------------------------------------------------------------- GEMM core ---------

def _f16_table():
    bits = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = [Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64)]
    return vals, bits


_TABLE = None


def fraction_to_f16(x: Fraction):
    """Correctly rounded (ties to even) fp16 bits of an exact rational; also returns
    the distance to the nearest fp16 midpoint, relative to |x| (for near-tie checks)."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _f16_table()
    vals, bits = _TABLE
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    if a >= 65520:
        return sign | 0x7C00, Fraction(1)
    j = bisect.bisect_left(vals, a)
    if j < len(vals) and vals[j] == a:
        return sign | int(bits[j]), Fraction(1)
    lo, hi = vals[j - 1], (vals[j] if j < len(vals) else Fraction(65536))
    mid = (lo + hi) / 2
    if a < mid:
        pick = j - 1
    elif a > mid:
        pick = j
    else:
        pick = j - 1 if int(bits[j - 1]) % 2 == 0 else j
    out = int(bits[pick]) if pick < len(bits) else 0x7C00
    dist = abs(a - mid) / a if a else Fraction(1)
    return sign | out, dist


def _random_f16(rng, shape, with_subnormals=True):
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-6, 4, size=shape))
    h = x.astype(np.float16)
    if with_subnormals:
        sub = rng.random(shape) < 0.1
        h[sub] = (rng.integers(-1023, 1024, size=int(sub.sum())) * 2.0 ** -24).astype(np.float16)
    return h


def _exact_product(A, B, bias=None):
    A64 = A.astype(np.float64)
    B64 = B.astype(np.float64)
    M, K = A.shape
    N = B.shape[1]
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            m = 0.0
            for k in range(K):
                s += Fraction(float(A64[i, k])) * Fraction(float(B64[k, j]))
                m += abs(float(A64[i, k]) * float(B64[k, j]))
            if bias is not None:
                s += Fraction(float(bias.astype(np.float64)[j]))
                m += abs(float(bias.astype(np.float64)[j]))
            out[i][j] = s
            mag[i][j] = m
    return out, mag


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (3, 2, 7), (5, 7, 3), (7, 5, 16),
                                   (16, 16, 16), (3, 16, 1), (1, 7, 16)])
@pytest.mark.parametrize("epi", ["none", "bias"])
def test_gemm_matches_exact_rational_bruteforce(oracle_lib, shape, epi):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = _random_f16(rng, (M, K))
    B = _random_f16(rng, (K, N))
    bias = _random_f16(rng, (N,)) if epi == "bias" else None
    got = oracle.gemm(A, B, bias, epi, lib=oracle_lib)
    exact, mag = _exact_product(A, B, bias)
    for i in range(M):
        for j in range(N):
            want, dist = fraction_to_f16(exact[i][j])
            if int(got[i, j]) == want:
                continue
            # fp64 summation may only flip a correctly rounded result at a near-tie:
            # |fp64 sum - exact| <= (K+1) * 2^-53 * sum|terms|
            bound = (K + 2) * 2.0 ** -53 * mag[i][j]
            assert exact[i][j] != 0 and float(dist) * abs(float(exact[i][j])) <= bound, \
                (shape, i, j, hex(int(got[i, j])), hex(want))


def test_gemm_bias_gelu_against_exact_sum_and_ndtr(oracle_lib):
    rng = np.random.default_rng(99)
    M, N, K = 6, 9, 13
    A, B, bias = _random_f16(rng, (M, K)), _random_f16(rng, (K, N)), _random_f16(rng, (N,))
    got = oracle.gemm(A, B, bias, "bias_gelu", lib=oracle_lib)
    exact, _ = _exact_product(A, B, bias)
    for i in range(M):
        for j in range(N):
            x = float(exact[i][j])
            ref_val = x * float(ndtr(x))
            want = int(np.array([ref_val]).astype(np.float16).view(np.uint16)[0])
            if int(got[i, j]) != want:
                # allowed only when ref_val lies within 1e-12 (relative) of a midpoint
                _, dist = fraction_to_f16(Fraction(ref_val))
                assert float(dist) < 1e-12, (i, j, x)


@pytest.mark.parametrize("shape", [(256, 256, 256), (1000, 3000, 777)])
def test_gemm_matches_numpy_fp64_matmul(oracle_lib, shape):
    """Library special case: numpy's fp64 matmul rounded once to fp16.  Only near-ties
    (where the two fp64 sums straddle an fp16 midpoint) may differ."""
    import workloads
    M, N, K = shape
    A, B, _ = workloads.make_inputs(M, N, K, "uniform" if K == 777 else "normal", seed=3)
    A = A.numpy()
    B = B.numpy()
    got = oracle.gemm(A, B, lib=oracle_lib)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    s = A64 @ B64
    ref = s.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)
    n_bad = bad[0].size
    assert n_bad <= 1e-4 * M * N
    if n_bad:
        mag = np.abs(A64) @ np.abs(B64)
        g = got[bad].view(np.float16).astype(np.float64)
        r = ref[bad].view(np.float16).astype(np.float64)
        mid = (g + r) / 2.0
        assert np.all(np.abs(s[bad] - mid) <= 2 * K * 2.0 ** -53 * mag[bad])
        # and the two candidates are adjacent fp16 values
        assert np.all(np.abs(got[bad].astype(np.int32) - ref[bad].astype(np.int32)) == 1)


@pytest.mark.parametrize("K", [1, 256, 777, 2048, 8192])
def test_all_ones_gives_K(oracle_lib, K):
    M, N = 3, 5
    A = np.ones((M, K), np.float16)
    B = np.ones((K, N), np.float16)
    got = oracle.gemm(A, B, lib=oracle_lib).view(np.float16)
    assert np.all(got.astype(np.float64) == float(K))


def test_selection_matrices_copy_rows_and_columns(oracle_lib):
    rng = np.random.default_rng(7)
    M, N, K = 37, 29, 11
    B = _random_f16(rng, (K, N))
    A_sel = np.zeros((M, K), np.float16)
    A_sel[np.arange(M), np.arange(M) % K] = 1
    got = oracle.gemm(A_sel, B, lib=oracle_lib)
    assert np.array_equal(got, B.view(np.uint16)[np.arange(M) % K])
    A = _random_f16(rng, (M, K))
    B_sel = np.zeros((K, N), np.float16)
    B_sel[np.arange(N) % K, np.arange(N)] = 1
    got = oracle.gemm(A, B_sel, lib=oracle_lib)
    assert np.array_equal(got, A.view(np.uint16)[:, np.arange(N) % K])


def test_identity_and_permutation(oracle_lib):
    rng = np.random.default_rng(8)
    n = 24
    B = _random_f16(rng, (n, 17))
    eye = np.eye(n, dtype=np.float16)
    assert np.array_equal(oracle.gemm(eye, B, lib=oracle_lib), B.view(np.uint16))
    perm = rng.permutation(n)
    P = eye[perm]
    assert np.array_equal(oracle.gemm(P, B, lib=oracle_lib), B.view(np.uint16)[perm])
    A = _random_f16(rng, (9, n))
    assert np.array_equal(oracle.gemm(A, eye, lib=oracle_lib), A.view(np.uint16))


def test_zero_operand_and_empty_k(oracle_lib):
    rng = np.random.default_rng(9)
    A = np.zeros((5, 8), np.float16)
    B = _random_f16(rng, (8, 6))
    bias = _random_f16(rng, (6,))
    got = oracle.gemm(A, B, lib=oracle_lib).view(np.float16)
    assert np.all(got == 0)
    # A = 0 reduces the epilogue to a function of the bias alone: column j gets bias[j]
    got_b = oracle.gemm(A, B, bias, "bias", lib=oracle_lib)
    assert np.array_equal(got_b, np.broadcast_to(bias.view(np.uint16), (5, 6)))
    got_g = oracle.gemm(A, B, bias, "bias_gelu", lib=oracle_lib)
    bx = bias.astype(np.float64)
    want = (bx * ndtr(bx)).astype(np.float16).view(np.uint16)
    assert np.array_equal(got_g, np.broadcast_to(want, (5, 6)))
    # K = 0: an empty sum, C = epi(bias or 0)
    A0 = np.zeros((4, 0), np.float16)
    B0 = np.zeros((0, 6), np.float16)
    assert np.all(oracle.gemm(A0, B0, lib=oracle_lib) == 0)
    assert np.array_equal(oracle.gemm(A0, B0, bias, "bias_gelu", lib=oracle_lib),
                          np.broadcast_to(want, (4, 6)))


def test_transpose_and_row_permutation_invariance(oracle_lib):
    rng = np.random.default_rng(10)
    A = _random_f16(rng, (23, 31))
    B = _random_f16(rng, (31, 19))
    C = oracle.gemm(A, B, lib=oracle_lib)
    Ct = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), lib=oracle_lib)
    assert np.array_equal(C.T, Ct)
    perm = rng.permutation(23)
    assert np.array_equal(oracle.gemm(A[perm], B, lib=oracle_lib), C[perm])


def test_sampled_equals_full(oracle_lib):
    import workloads
    A, B, bias = workloads.make_inputs(70, 90, 130, "normal", with_bias=True, seed=5)
    for epi in ("none", "bias", "bias_gelu"):
        full = oracle.gemm(A, B, bias, epi, lib=oracle_lib)
        rng = np.random.default_rng(1)
        r = rng.integers(0, 70, 500)
        c = rng.integers(0, 90, 500)
        s = oracle.gemm_sampled(A, B, r, c, bias, epi, lib=oracle_lib)
        assert np.array_equal(s, full[r, c])


def test_rejects_bad_arguments(oracle_lib):
    A = np.zeros((2, 3), np.float16)
    B = np.zeros((3, 4), np.float16)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, None, "bias", lib=oracle_lib)
    with pytest.raises(ValueError):
        oracle.gemm(A, np.zeros((2, 4), np.float16), lib=oracle_lib)
    with pytest.raises(ValueError):
        oracle.gemm_sampled(A, B, [2], [0], lib=oracle_lib)


# ---------------------------------------------------------------- vector add --------

def _finite(bits):
    return (bits & 0x7C00) != 0x7C00


def test_vector_add_matches_numpy_float16_sums(oracle_lib):
    """numpy adds two float16 arrays in float32 and rounds once to float16, which is the
    correctly rounded sum (the float32 sum of two float16 values rounds to the same
    float16 as the exact sum); random bit patterns cover subnormals, zeros and the
    overflow boundary."""
    rng = np.random.default_rng(7)
    a = rng.integers(0, 1 << 16, 400_000, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 1 << 16, 400_000, dtype=np.uint32).astype(np.uint16)
    keep = _finite(a) & _finite(b)
    a, b = a[keep], b[keep]
    got = oracle.vector_add(a, b, lib=oracle_lib)
    with np.errstate(over="ignore"):
        ref = (a.view(np.float16) + b.view(np.float16)).view(np.uint16)
    assert np.array_equal(got, ref)


def test_vector_add_closed_forms(oracle_lib):
    f = ALL_BITS[_finite(ALL_BITS)]
    zero = np.zeros_like(f)
    # x + 0 = x (and -0 + +0 = +0)
    got = oracle.vector_add(f, zero, lib=oracle_lib)
    want = np.where(f == 0x8000, 0, f).astype(np.uint16)
    assert np.array_equal(got, want)
    # x + (-x) = +0
    assert np.all(oracle.vector_add(f, f ^ 0x8000, lib=oracle_lib) == 0)
    # x + x = 2x exactly while 2x is finite (exponent + 1, or a doubled subnormal)
    xv = f.view(np.float16).astype(np.float64)
    ok = np.abs(2 * xv) < 65504
    got = oracle.vector_add(f[ok], f[ok], lib=oracle_lib).view(np.float16).astype(np.float64)
    assert np.array_equal(got, 2 * xv[ok])
    # specials: inf + finite = inf, inf + -inf = nan, nan propagates
    inf, ninf, nan = np.uint16(0x7C00), np.uint16(0xFC00), np.uint16(0x7E00)
    r = oracle.vector_add(np.array([inf, inf, nan, 0x3C00], np.uint16),
                          np.array([0x3C00, ninf, 0x3C00, 0x7BFF], np.uint16), lib=oracle_lib)
    assert r[0] == 0x7C00 and (r[1] & 0x7C00) == 0x7C00 and (r[1] & 0x3FF) != 0
    assert (r[2] & 0x7C00) == 0x7C00 and (r[2] & 0x3FF) != 0
    assert r[3] == 0x7BFF     # 65504 + 1 rounds back to 65504


# ---------------------------------------------------------------- softmax -----------

def _sm(x, lib):
    return oracle.softmax(np.asarray(x, dtype=np.float16), lib=lib).view(np.float16).astype(np.float64)


def test_softmax_matches_scipy(oracle_lib):
    """scipy's fp64 softmax, rounded once to fp16 by numpy, must equal the oracle except
    at the rare near-ties of the final rounding (none expected at this size)."""
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(3)
    for (M, N, scale) in [(37, 1, 1.0), (23, 5, 3.0), (64, 333, 4.0), (8, 4096, 8.0)]:
        x = (rng.standard_normal((M, N)) * scale).astype(np.float16)
        got = oracle.softmax(x, lib=oracle_lib)
        ref = sp_softmax(x.astype(np.float64), axis=1).astype(np.float16).view(np.uint16)
        diff = (got != ref).sum()
        assert diff <= max(1, x.size // 100000), (M, N, diff)


def test_softmax_closed_forms(oracle_lib):
    # equal entries: 1/N everywhere
    for N in (1, 2, 3, 7, 64, 1000):
        y = _sm(np.full((3, N), 1.25), oracle_lib)
        assert np.all(y == np.float64(np.float16(1.0 / N)))
    # two entries: (sigmoid(a - b), sigmoid(b - a))
    from scipy.special import expit
    rng = np.random.default_rng(5)
    a = rng.standard_normal(200).astype(np.float16)
    b = rng.standard_normal(200).astype(np.float16)
    y = _sm(np.stack([a, b], axis=1), oracle_lib)
    d = a.astype(np.float64) - b.astype(np.float64)
    assert np.array_equal(y[:, 0], expit(d).astype(np.float16).astype(np.float64))
    assert np.array_equal(y[:, 1], expit(-d).astype(np.float16).astype(np.float64))
    # shift invariance by a power of two that keeps every value exact in fp16
    x = np.round(rng.standard_normal((16, 50)) * 4).astype(np.float16)
    assert np.array_equal(_sm(x, oracle_lib), _sm(x + np.float16(32), oracle_lib))
    # a dominant entry: one-hot (the rest underflow below fp16's smallest subnormal)
    x = np.zeros((4, 300), np.float16)
    x[np.arange(4), [0, 17, 150, 299]] = 60.0
    y = _sm(x, oracle_lib)
    assert np.all(y[np.arange(4), [0, 17, 150, 299]] == 1.0) and y.sum() == 4.0
    # rows sum to 1 within the fp16 rounding of each entry
    x = (rng.standard_normal((32, 777)) * 2).astype(np.float16)
    y = _sm(x, oracle_lib)
    assert np.all(np.abs(y.sum(axis=1) - 1.0) <= 777 * 2.0 ** -12)


def test_softmax_ieee_edge_cases(oracle_lib):
    ninf, pinf, nan = -np.inf, np.inf, np.nan
    x = np.array([[ninf, 0.0, 1.0], [ninf, ninf, ninf], [pinf, 0.0, 1.0], [nan, 0.0, 1.0]], np.float16)
    y = _sm(x, oracle_lib)
    assert y[0, 0] == 0.0 and np.isclose(y[0, 1] + y[0, 2], 1.0, atol=1e-3)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2])) and np.all(np.isnan(y[3]))
    assert oracle.softmax(np.zeros((0, 5), np.float16), lib=oracle_lib).shape == (0, 5)
    assert oracle.softmax(np.zeros((5, 0), np.float16), lib=oracle_lib).shape == (5, 0)


# ---------------------------------------------------------------- attention ---------

def _f16_of_fraction(fr: Fraction) -> np.float16:
    """The fp16 value nearest to an exact rational (ties to even), found among the
    neighbours of numpy's conversion of its nearest double."""
    h = np.float16(float(fr))
    cands = [h, np.nextafter(h, np.float16(np.inf)), np.nextafter(h, np.float16(-np.inf))]
    cands = [c for c in cands if np.isfinite(c)]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(c.view(np.uint16)) & 1))
    return best


def _qkv(rng, BH, Sq, Sk, D, scale=1.0):
    q = (rng.standard_normal((BH, Sq, D)) * scale).astype(np.float16)
    k = (rng.standard_normal((BH, Sk, D)) * scale).astype(np.float16)
    v = rng.standard_normal((BH, Sk, D)).astype(np.float16)
    return q, k, v


def _ulps(a_bits, b_bits):
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def test_attention_single_key(oracle_lib):
    """One key: every weight is 1, so o = v[0] exactly and lse = the single score."""
    rng = np.random.default_rng(11)
    q, k, v = _qkv(rng, 3, 5, 1, 16)
    for causal in (False, True):
        o, lse, err = oracle.attention(q, k, v, scale=0.37, causal=causal, lib=oracle_lib)
        assert np.array_equal(o, np.broadcast_to(v.view(np.uint16), o.shape))
        assert np.array_equal(err, np.abs(np.broadcast_to(v.astype(np.float64), o.shape)))
        for b in range(3):
            for i in range(5):
                dot = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(q[b, i], k[b, 0]))
                assert lse[b, i] == pytest.approx(0.37 * float(dot), rel=1e-14, abs=1e-14)


def test_attention_uniform_weights(oracle_lib):
    """q = 0 (or scale = 0) makes every allowed weight equal: o is the exact mean of the
    allowed value rows, rounded once, and lse = log(number of allowed keys)."""
    rng = np.random.default_rng(12)
    BH, Sq, Sk, D = 2, 9, 13, 4
    _, k, v = _qkv(rng, BH, Sq, Sk, D)
    qz = np.zeros((BH, Sq, D), np.float16)
    qr = rng.standard_normal((BH, Sq, D)).astype(np.float16)
    for causal in (False, True):
        for (q, scale) in ((qz, 0.5), (qr, 0.0)):
            o, lse, _ = oracle.attention(q, k, v, scale=scale, causal=causal, lib=oracle_lib)
            of = o.view(np.float16)
            for b in range(BH):
                for i in range(Sq):
                    n = min(i + 1, Sk) if causal else Sk
                    assert lse[b, i] == pytest.approx(np.log(n), abs=1e-14)
                    for d in range(D):
                        mean = sum(Fraction(float(x)) for x in v[b, :n, d]) / n
                        assert of[b, i, d] == _f16_of_fraction(mean), (causal, b, i, d)


def test_attention_selection(oracle_lib):
    """Keys are scaled one-hot rows along a permutation sigma of the head dimensions and
    query i points at key pi(i): with a large scale the softmax is one-hot within far less
    than fp16's resolution, so o[i] = v[pi(i)] exactly (a transposed k or v, a swapped
    operand or a wrong row picks another value row)."""
    rng = np.random.default_rng(13)
    Sk = D = 16
    sigma = rng.permutation(D)
    k = np.zeros((1, Sk, D), np.float16)
    k[0, np.arange(Sk), sigma] = 4.0
    v = rng.standard_normal((1, Sk, D)).astype(np.float16)
    pi = rng.permutation(Sk)[:12]
    q = np.zeros((1, 12, D), np.float16)
    q[0, np.arange(12), sigma[pi]] = 8.0
    o, _, _ = oracle.attention(q, k, v, scale=2.0, causal=False, lib=oracle_lib)
    assert np.array_equal(o[0], v[0, pi].view(np.uint16))
    # causal: query i selects key i (on the diagonal, always visible)
    qd = np.zeros((1, Sk, D), np.float16)
    qd[0, np.arange(Sk), sigma] = 8.0
    o, _, _ = oracle.attention(qd, k, v, scale=2.0, causal=True, lib=oracle_lib)
    assert np.array_equal(o[0], v[0].view(np.uint16))


def test_attention_two_keys_logistic(oracle_lib):
    """Two keys: the weights are the logistic function of the score difference, o =
    v0 expit(s0 - s1) + v1 expit(s1 - s0) and lse = logaddexp(s0, s1)."""
    from scipy.special import expit
    rng = np.random.default_rng(14)
    n = 300
    x = rng.standard_normal((1, n, 1)).astype(np.float16)
    k = np.array([[[1.0], [0.0]]], np.float16)
    v = rng.standard_normal((1, 2, 1)).astype(np.float16)
    scale = 1.7
    o, lse, _ = oracle.attention(x, k, v, scale=scale, causal=False, lib=oracle_lib)
    s0 = scale * x[0, :, 0].astype(np.float64)
    v0, v1 = float(v[0, 0, 0]), float(v[0, 1, 0])
    ref = (v0 * expit(s0) + v1 * expit(-s0)).astype(np.float16).view(np.uint16)
    d = _ulps(o[0, :, 0], ref)
    assert d.max() <= 1 and (d == 0).mean() >= 0.99
    assert np.allclose(lse[0], np.logaddexp(s0, 0.0), rtol=0, atol=1e-13)


def _scipy_attention(q, k, v, scale, causal):
    from scipy.special import logsumexp, softmax
    s = scale * np.matmul(q.astype(np.float64), np.swapaxes(k.astype(np.float64), -1, -2))
    if causal:
        Sq, Sk = s.shape[-2:]
        s = np.where(np.tril(np.ones((Sq, Sk), bool)), s, -np.inf)
    p = softmax(s, axis=-1)
    return p @ v.astype(np.float64), logsumexp(s, axis=-1), p @ np.abs(v.astype(np.float64))


@pytest.mark.parametrize("BH,Sq,Sk,D,causal", [
    (2, 17, 17, 16, False), (2, 17, 17, 16, True), (3, 40, 23, 8, True),
    (1, 23, 40, 32, True), (2, 64, 96, 64, False), (1, 5, 200, 128, True)])
def test_attention_matches_scipy(oracle_lib, BH, Sq, Sk, D, causal):
    """scipy's softmax and numpy's fp64 matmul (an independent formulation): o within one
    fp16 step and almost always equal, lse and err to fp64 accuracy."""
    rng = np.random.default_rng(BH * 1000 + Sq * 10 + Sk)
    q, k, v = _qkv(rng, BH, Sq, Sk, D, scale=1.5)
    scale = 1.0 / np.sqrt(D)
    o, lse, err = oracle.attention(q, k, v, scale=scale, causal=causal, lib=oracle_lib)
    ro, rl, re = _scipy_attention(q, k, v, scale, causal)
    d = _ulps(o, ro.astype(np.float16).view(np.uint16))
    assert d.max() <= 1 and (d == 0).mean() >= 0.995
    assert np.allclose(lse, rl, rtol=0, atol=1e-12)
    assert np.allclose(err, re, rtol=1e-12, atol=1e-15)


def test_attention_causal_is_the_prefix(oracle_lib):
    """Causal row i is the non-causal attention of query i over keys 0..i only."""
    rng = np.random.default_rng(15)
    q, k, v = _qkv(rng, 2, 12, 12, 8)
    o, lse, err = oracle.attention(q, k, v, scale=0.4, causal=True, lib=oracle_lib)
    for i in range(12):
        oi, li, ei = oracle.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], scale=0.4,
                                      causal=False, lib=oracle_lib)
        assert np.array_equal(o[:, i], oi[:, 0]) and np.array_equal(lse[:, i], li[:, 0])
        assert np.array_equal(err[:, i], ei[:, 0])


def test_attention_shift_invariance_without_overflow(oracle_lib):
    """A score offset common to every key of a row (an extra head dimension where every
    key holds 1 and the query holds 1000) leaves o unchanged and moves lse by exactly the
    offset; without the row-maximum shift exp(1000) would overflow."""
    rng = np.random.default_rng(16)
    q, k, v = _qkv(rng, 2, 10, 30, 7)
    o, lse, _ = oracle.attention(q, k, v, scale=1.0, causal=False, lib=oracle_lib)
    q2 = np.concatenate([q, np.full((2, 10, 1), 1000.0, np.float16)], axis=-1)
    k2 = np.concatenate([k, np.ones((2, 30, 1), np.float16)], axis=-1)
    v2 = np.concatenate([v, np.zeros((2, 30, 1), np.float16)], axis=-1)
    o2, lse2, _ = oracle.attention(q2, k2, v2, scale=1.0, causal=False, lib=oracle_lib)
    d = _ulps(o2[..., :7], o)
    assert d.max() <= 1 and (d == 0).mean() >= 0.99
    assert np.allclose(lse2 - 1000.0, lse, rtol=0, atol=1e-9)


def test_attention_convex_hull(oracle_lib):
    """Every output is a weighted mean of the allowed values: within their min and max."""
    rng = np.random.default_rng(17)
    q, k, v = _qkv(rng, 3, 33, 33, 16, scale=2.0)
    for causal in (False, True):
        o, _, _ = oracle.attention(q, k, v, scale=0.25, causal=causal, lib=oracle_lib)
        of = o.view(np.float16)
        for i in range(33):
            n = i + 1 if causal else 33
            assert np.all(of[:, i] >= v[:, :n].min(axis=1)) and np.all(of[:, i] <= v[:, :n].max(axis=1))


def test_attention_rows_and_edges(oracle_lib):
    rng = np.random.default_rng(18)
    q, k, v = _qkv(rng, 4, 21, 19, 8)
    o, lse, err = oracle.attention(q, k, v, causal=True, lib=oracle_lib)
    pairs = np.array([0, 3, 2, 1, 3]); rows = np.array([0, 20, 7, 18, 19])
    ro, rl, re = oracle.attention_rows(q, k, v, pairs, rows, causal=True, lib=oracle_lib)
    assert np.array_equal(ro, o[pairs, rows]) and np.array_equal(rl, lse[pairs, rows])
    assert np.array_equal(re, err[pairs, rows])
    with pytest.raises(ValueError):
        oracle.attention(q, k[:, :0], v[:, :0], lib=oracle_lib)   # no keys: undefined
    assert oracle.attention(q[:, :0], k, v, lib=oracle_lib)[0].shape == (4, 0, 8)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, [4], [0], lib=oracle_lib)
