"""CPU oracle for the fp16 GEMM (+ bias, + erf-GELU) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``gemm_oracle.c`` (plain C, fp64 accumulation, its own
binary16 codec, ``erf``/``erfc`` from the host libm); this module only builds it with
gcc and marshals numpy arrays through ctypes.  What it computes follows "Designing
High-Performance GPU Kernels with TileLang: Tensor-Core GEMM, Fused Softmax,
FlashAttention, and Autotuning": the thecryptopost.io page, section 2 ("Memory
hierarchy - tiled tensor-core GEMM", ``make_matmul``: A (M, K), B (K, N), C (M, N)
float16 row-major) for the product, and the ainovat.com page's fused-epilogue
paragraph for ``GELU(acc + bias)`` before the single fp16 write; ``vector_add`` is the
same tutorial's first kernel (the ainovat.com page's first paragraph), ``softmax`` its
row-wise softmax (the same page's third paragraph) and ``attention`` the plain definition
its FlashAttention forward kernel computes (the same page's FlashAttention paragraph).

Every function here is pinned by ``tests/test_oracle.py`` (closed forms, exhaustive
codec checks against numpy, exact rational brute force); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gemm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_gemm.so")

EPI_NONE, EPI_BIAS, EPI_BIAS_GELU = 0, 1, 2
EPILOGUES = {"none": EPI_NONE, "bias": EPI_BIAS, "bias_gelu": EPI_BIAS_GELU}

_lib = None


def compile_command(source: str = SOURCE, output: str = LIBRARY, extra=()) -> list[str]:
    return ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
            "-std=c11", "-Wall", "-Wextra", *extra, source, "-o", output, "-lm"]


def build(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile the oracle into a shared library (always recompiles); ``extra`` adds
    compiler flags (the sanitizer build of the tests)."""
    tmp = output + ".tmp%d" % os.getpid()
    subprocess.run(compile_command(source, tmp, extra), check=True)
    os.replace(tmp, output)
    return output


def load(path: str | None = None, rebuild_if_missing: bool = True) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is not there)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    target = path or LIBRARY
    if not os.path.exists(target):
        if not rebuild_if_missing:
            raise FileNotFoundError(target)
        build(output=target)
    lib = ctypes.CDLL(target)
    _declare(lib)
    if path is None:
        _lib = lib
    return lib


def _declare(lib: ctypes.CDLL) -> None:
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int, p]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_sampled.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int, i64, p, p, p]
    lib.oracle_gemm_sampled.restype = ctypes.c_int
    lib.oracle_vector_add.argtypes = [i64, p, p, p]
    lib.oracle_vector_add.restype = ctypes.c_int
    lib.oracle_softmax.argtypes = [i64, i64, p, p]
    lib.oracle_softmax.restype = ctypes.c_int
    d = ctypes.c_double
    lib.oracle_attention.argtypes = [i64, i64, i64, i64, p, p, p, d, ctypes.c_int, p, p, p]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [i64, i64, i64, i64, p, p, p, d, ctypes.c_int, i64,
                                          p, p, p, p, p]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    for name in ("oracle_f16_to_f64_array", "oracle_f64_to_f16_array", "oracle_gelu_array"):
        getattr(lib, name).argtypes = [i64, p, p]
        getattr(lib, name).restype = None


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits(a) -> np.ndarray:
    """Accept a numpy float16/uint16 array or a CPU torch float16 tensor; return the
    contiguous uint16 bit pattern."""
    if hasattr(a, "detach"):  # torch tensor, kept optional so numpy-only callers work
        a = a.detach().cpu().contiguous().view(dtype=_torch_int16()).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    elif a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 / uint16 bit patterns, got %s" % a.dtype)
    return a


def _torch_int16():
    import torch
    return torch.int16


def f16_to_f64(bits, lib=None) -> np.ndarray:
    lib = lib or load()
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_f16_to_f64_array(b.size, _ptr(b), _ptr(out))
    return out


def f64_to_f16(x, lib=None) -> np.ndarray:
    """Round fp64 values to fp16 (RNE); returns uint16 bit patterns."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_f64_to_f16_array(x.size, _ptr(x), _ptr(out))
    return out


def gelu(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    lib.oracle_gelu_array(x.size, _ptr(x), _ptr(out))
    return out


def set_num_threads(n: int, lib=None) -> None:
    """Threads the oracle's OpenMP loops use from now on in this process."""
    (lib or load()).oracle_set_num_threads(int(n))


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's loops use."""
    return (lib or load()).oracle_num_threads()


def _epi_code(epilogue) -> int:
    if isinstance(epilogue, str):
        return EPILOGUES[epilogue]
    return int(epilogue)


def gemm(A, B, bias=None, epilogue="none", lib=None) -> np.ndarray:
    """C = fp16(epi(A @ B [+ bias])) with fp64 accumulation; returns uint16 bits (M, N)."""
    lib = lib or load()
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("shape mismatch %s x %s" % (a.shape, b.shape))
    M, K = a.shape
    N = b.shape[1]
    epi = _epi_code(epilogue)
    bb = _bits(bias) if bias is not None else None
    if epi != EPI_NONE and (bb is None or bb.size != N):
        raise ValueError("bias of length N required for epilogue %r" % (epilogue,))
    out = np.empty((M, N), dtype=np.uint16)
    rc = lib.oracle_gemm(M, N, K, _ptr(a), _ptr(b), _ptr(bb), epi, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments (rc=%d)" % rc)
    return out


def vector_add(a, b, lib=None) -> np.ndarray:
    """c = fp16(a + b) element-wise (one rounding); returns uint16 bits of a's shape."""
    lib = lib or load()
    x, y = _bits(a), _bits(b)
    if x.shape != y.shape:
        raise ValueError("shape mismatch %s vs %s" % (x.shape, y.shape))
    out = np.empty(x.shape, dtype=np.uint16)
    rc = lib.oracle_vector_add(x.size, _ptr(x), _ptr(y), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_vector_add rejected its arguments (rc=%d)" % rc)
    return out


def softmax(x, lib=None) -> np.ndarray:
    """Row-wise softmax of a 2-D fp16 array (fp64 inside, one rounding); uint16 bits."""
    lib = lib or load()
    a = _bits(x)
    if a.ndim != 2:
        raise ValueError("softmax expects a 2-D array, got %s" % (a.shape,))
    out = np.empty(a.shape, dtype=np.uint16)
    rc = lib.oracle_softmax(a.shape[0], a.shape[1], _ptr(a), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_softmax rejected its arguments (rc=%d)" % rc)
    return out


def _attn_operands(q, k, v):
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    if qb.ndim < 2 or kb.shape != vb.shape or qb.shape[:-2] != kb.shape[:-2] \
            or qb.shape[-1] != kb.shape[-1]:
        raise ValueError("attention expects q (..., Sq, D), k and v (..., Sk, D); got %s %s %s"
                         % (qb.shape, kb.shape, vb.shape))
    return qb, kb, vb


def attention(q, k, v, scale=None, causal=False, lib=None):
    """Attention forward over the leading (batch, head) dimensions, fp64 inside, one
    rounding: returns (o bits uint16 shaped like q, lse fp64 (..., Sq), err fp64 like q),
    err being sum_j p_j |v_j| / l per output element (the tolerance scale)."""
    lib = lib or load()
    qb, kb, vb = _attn_operands(q, k, v)
    Sq, D = qb.shape[-2:]
    Sk = kb.shape[-2]
    BH = int(np.prod(qb.shape[:-2], dtype=np.int64))
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty(qb.shape, dtype=np.uint16)
    lse = np.empty(qb.shape[:-1], dtype=np.float64)
    err = np.empty(qb.shape, dtype=np.float64)
    rc = lib.oracle_attention(BH, Sq, Sk, D, _ptr(qb), _ptr(kb), _ptr(vb), float(scale),
                              int(bool(causal)), _ptr(o), _ptr(lse), _ptr(err))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments (rc=%d)" % rc)
    return o, lse, err


def attention_rows(q, k, v, pairs, rows, scale=None, causal=False, lib=None):
    """Selected output rows o[pair[t], row[t], :] (pairs index the flattened leading
    dimensions), each computed exactly as ``attention`` computes it: (o bits (n, D),
    lse (n,), err (n, D))."""
    lib = lib or load()
    qb, kb, vb = _attn_operands(q, k, v)
    Sq, D = qb.shape[-2:]
    Sk = kb.shape[-2]
    BH = int(np.prod(qb.shape[:-2], dtype=np.int64))
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pr = np.ascontiguousarray(pairs, dtype=np.int64)
    rw = np.ascontiguousarray(rows, dtype=np.int64)
    if pr.shape != rw.shape or pr.ndim != 1:
        raise ValueError("pairs and rows must be 1-D and of one length")
    n = pr.size
    o = np.empty((n, D), dtype=np.uint16)
    lse = np.empty(n, dtype=np.float64)
    err = np.empty((n, D), dtype=np.float64)
    rc = lib.oracle_attention_rows(BH, Sq, Sk, D, _ptr(qb), _ptr(kb), _ptr(vb), float(scale),
                                   int(bool(causal)), n, _ptr(pr), _ptr(rw), _ptr(o), _ptr(lse),
                                   _ptr(err))
    if rc != 0:
        raise ValueError("oracle_attention_rows rejected its arguments (rc=%d)" % rc)
    return o, lse, err


def gemm_sampled(A, B, rows, cols, bias=None, epilogue="none", lib=None) -> np.ndarray:
    """Selected output elements C[rows[s], cols[s]] (uint16 bits), each computed exactly
    as the full product computes it."""
    lib = lib or load()
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N = b.shape[1]
    if b.shape[0] != K:
        raise ValueError("shape mismatch %s x %s" % (a.shape, b.shape))
    epi = _epi_code(epilogue)
    bb = _bits(bias) if bias is not None else None
    if epi != EPI_NONE and (bb is None or bb.size != N):
        raise ValueError("bias of length N required for epilogue %r" % (epilogue,))
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in shape")
    out = np.empty(r.shape, dtype=np.uint16)
    rc = lib.oracle_gemm_sampled(M, N, K, _ptr(a), _ptr(b), _ptr(bb), epi, r.size,
                                 _ptr(r), _ptr(c), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gemm_sampled rejected its arguments (rc=%d)" % rc)
    return out
