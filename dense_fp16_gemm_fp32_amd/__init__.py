"""Python binding of the mi355gemm C ABI (``include/mi355gemm.h``).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libmi355gemm.so``.  The ``mi355gemm_*`` functions mirror the C entry points one to one
(raw integers for pointers and the stream); ``gemm()`` is the torch-tensor convenience
wrapper that allocates ``out`` when it is not given, as the tutorial's kernels allocate
their output (thecryptopost.io page, section 2, ``out_idx=[-1]``).

There is no fallback: if the library is not built, or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first, so the library binds to the same HIP runtime as torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libmi355gemm.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
EPI_NONE, EPI_BIAS, EPI_BIAS_GELU = 0, 1, 2
EPILOGUES = {"none": EPI_NONE, "bias": EPI_BIAS, "bias_gelu": EPI_BIAS_GELU}
STATUS_NAMES = {OK: "OK", EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP"}

# Every symbol include/mi355gemm.h declares.
EXPORTS = (
    "mi355gemm_gemm", "mi355gemm_gemm_config", "mi355gemm_gemm_timed", "mi355gemm_select",
    "mi355gemm_num_configs",
    "mi355gemm_config_name", "mi355gemm_config_info", "mi355gemm_lds_budget",
    "mi355gemm_last_error", "mi355gemm_version", "mi355gemm_vector_add", "mi355gemm_softmax",
    "mi355gemm_attention", "mi355gemm_set_choice", "mi355gemm_clear_choices",
)


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


class ConfigDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "block_m", "block_n", "block_k", "stages", "waves_m", "waves_n", "k_groups", "threads",
        "lds_bytes", "a_vector", "bc_vector", "group_m", "direct", "narrow", "k_mult8",
        "pingpong", "loader_waves", "mfma_block")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def library() -> ctypes.CDLL:
    """The loaded ``libmi355gemm.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(
                "%s is not built; run `python -m dense_fp16_gemm_fp32_amd.build` "
                "(or __graft_entry__.build()) first" % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        i64, p, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.mi355gemm_gemm.argtypes = [i64, i64, i64, p, p, p, p, ci, p]
        lib.mi355gemm_gemm.restype = ci
        lib.mi355gemm_gemm_config.argtypes = [i64, i64, i64, p, p, p, p, ci, p, ci]
        lib.mi355gemm_gemm_config.restype = ci
        lib.mi355gemm_gemm_timed.argtypes = [i64, i64, i64, p, p, p, p, ci, p, ci, p, p]
        lib.mi355gemm_gemm_timed.restype = ci
        lib.mi355gemm_select.argtypes = [i64, i64, i64, ci, p, p, p, p]
        lib.mi355gemm_select.restype = ci
        lib.mi355gemm_num_configs.argtypes = []
        lib.mi355gemm_num_configs.restype = ci
        lib.mi355gemm_config_name.argtypes = [ci]
        lib.mi355gemm_config_name.restype = ctypes.c_char_p
        lib.mi355gemm_config_info.argtypes = [ci, ctypes.POINTER(ConfigDesc)]
        lib.mi355gemm_config_info.restype = ci
        lib.mi355gemm_lds_budget.argtypes = []
        lib.mi355gemm_lds_budget.restype = ci
        lib.mi355gemm_last_error.argtypes = []
        lib.mi355gemm_last_error.restype = ctypes.c_char_p
        lib.mi355gemm_vector_add.argtypes = [i64, p, p, p, p]
        lib.mi355gemm_vector_add.restype = ci
        lib.mi355gemm_softmax.argtypes = [i64, i64, p, p, p]
        lib.mi355gemm_softmax.restype = ci
        lib.mi355gemm_attention.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p,
                                            ctypes.c_float, ci, p]
        lib.mi355gemm_attention.restype = ci
        lib.mi355gemm_set_choice.argtypes = [i64, i64, i64, ci, ci, ci, ci]
        lib.mi355gemm_set_choice.restype = ci
        lib.mi355gemm_clear_choices.argtypes = []
        lib.mi355gemm_clear_choices.restype = None
        lib.mi355gemm_version.argtypes = []
        lib.mi355gemm_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


# ---- the C entry points, same names, raw arguments --------------------------------

def mi355gemm_gemm(M, N, K, A, B, C, bias, epi, stream) -> int:
    return library().mi355gemm_gemm(M, N, K, A, B, C, bias, epi, stream)


def mi355gemm_gemm_config(M, N, K, A, B, C, bias, epi, stream, config_id) -> int:
    return library().mi355gemm_gemm_config(M, N, K, A, B, C, bias, epi, stream, config_id)


def mi355gemm_gemm_timed(M, N, K, A, B, C, bias, epi, stream, config_id, start_event,
                         stop_event) -> int:
    return library().mi355gemm_gemm_timed(M, N, K, A, B, C, bias, epi, stream, config_id,
                                          start_event, stop_event)


def mi355gemm_vector_add(n, a, b, c, stream) -> int:
    return library().mi355gemm_vector_add(n, a, b, c, stream)


def mi355gemm_softmax(M, N, x, y, stream) -> int:
    return library().mi355gemm_softmax(M, N, x, y, stream)


def mi355gemm_select(M, N, K, epi, A, B, C, bias) -> int:
    return library().mi355gemm_select(M, N, K, epi, A, B, C, bias)


def mi355gemm_set_choice(M, N, K, epi, a_vector, bc_vector, config_id) -> int:
    return library().mi355gemm_set_choice(M, N, K, epi, a_vector, bc_vector, config_id)


def mi355gemm_clear_choices() -> None:
    library().mi355gemm_clear_choices()


def mi355gemm_num_configs() -> int:
    return library().mi355gemm_num_configs()


def mi355gemm_config_name(config_id: int) -> str | None:
    r = library().mi355gemm_config_name(config_id)
    return None if r is None else r.decode()


def mi355gemm_config_info(config_id: int) -> dict:
    d = ConfigDesc()
    st = library().mi355gemm_config_info(config_id, ctypes.byref(d))
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())
    return d.as_dict()


def mi355gemm_lds_budget() -> int:
    return library().mi355gemm_lds_budget()


def mi355gemm_last_error() -> str:
    return library().mi355gemm_last_error().decode()


def mi355gemm_version() -> str:
    return library().mi355gemm_version().decode()


# ---- torch convenience layer -------------------------------------------------------

def configs() -> list[dict]:
    out = []
    for i in range(mi355gemm_num_configs()):
        d = mi355gemm_config_info(i)
        d["id"] = i
        d["name"] = mi355gemm_config_name(i)
        out.append(d)
    return out


_config_ids: dict | None = None


def config_id(name: str) -> int:
    global _config_ids
    if _config_ids is None:
        _config_ids = {mi355gemm_config_name(i): i for i in range(mi355gemm_num_configs())}
    return _config_ids[name]


_F16 = torch.float16


def _check_tensor(t, name, ndim):
    # the cheap attribute reads first: this runs three times per call on the launch path
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype is not _F16:
        raise TypeError("%s must be float16, got %s" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-D tensor" % (name, ndim))


def _epi(epilogue) -> int:
    if isinstance(epilogue, str):
        if epilogue not in EPILOGUES:
            raise ValueError("epilogue must be one of %s" % sorted(EPILOGUES))
        return EPILOGUES[epilogue]
    return int(epilogue)


try:   # the raw handle of the current stream without building a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover - older torch
    def _raw_stream(index):
        return torch.cuda.current_stream(index).cuda_stream

try:   # the current device index, without torch.cuda's Python-level checks
    _current_device = torch._C._cuda_getDevice
except AttributeError:  # pragma: no cover - older torch
    _current_device = torch.cuda.current_device


def gemm(a: torch.Tensor, b: torch.Tensor, bias: torch.Tensor | None = None,
         epilogue="none", out: torch.Tensor | None = None, config: int | str | None = None,
         stream: torch.cuda.Stream | None = None, events=None) -> torch.Tensor:
    """``out = epilogue(a @ b [+ bias])`` on the GPU; a (M,K), b (K,N), bias (N,), fp16.

    Runs on `stream` (default: the current stream of a's device) and returns without
    synchronising, like any other torch GPU op.  `events`, a (start, stop) pair of
    timing-enabled ``torch.cuda.Event`` that have been recorded at least once (so that
    their HIP events exist), makes the kernels record them as they start and end
    (``mi355gemm_gemm_timed``): ``start.elapsed_time(stop)`` is then the kernel time."""
    _check_tensor(a, "a", 2)
    _check_tensor(b, "b", 2)
    M, K = a.shape
    if b.shape[0] != K:
        raise ValueError("inner dimensions differ: a %s, b %s" % (tuple(a.shape), tuple(b.shape)))
    N = b.shape[1]
    dev = a.device
    if b.device != dev:
        raise ValueError("a and b are on different devices")
    epi = _epi(epilogue)
    bptr = None
    if bias is not None:
        _check_tensor(bias, "bias", 1)
        if bias.shape[0] != N or bias.device != dev:
            raise ValueError("bias must have N=%d elements on %s" % (N, dev))
        bptr = bias.data_ptr()
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    else:
        _check_tensor(out, "out", 2)
        if tuple(out.shape) != (M, N) or out.device != dev:
            raise ValueError("out must be (%d, %d) on %s" % (M, N, dev))
    lib = _lib if _lib is not None else library()
    cur = _current_device()
    idx = dev.index if dev.index is not None else cur
    sptr = stream.cuda_stream if stream is not None else _raw_stream(idx)
    args = (M, N, K, a.data_ptr(), b.data_ptr(), out.data_ptr(), bptr, epi, sptr)
    if config is None and events is None and idx == cur:
        # the common call: the selector's choice on the current device
        st = lib.mi355gemm_gemm(*args)
        if st != OK:
            raise GemmError(st, mi355gemm_last_error())
        return out
    # config None: the selector's choice; any given id goes to the library, which rejects
    # ids out of range (the timed entry reads -1 as the selector's choice, so a negative
    # id given here is rejected before it)
    cid = None if config is None else (config_id(config) if isinstance(config, str) else int(config))
    if events is not None:
        ev = tuple(e.cuda_event if e is not None else None for e in events)
        if len(ev) != 2 or any(h == 0 for h in ev):
            raise ValueError("events must be a (start, stop) pair of torch.cuda.Event (or None), "
                             "each recorded once before")
        if cid is not None and cid < 0:
            raise GemmError(EINVAL, "unknown config id %d" % cid)

    def call():
        if events is not None:
            return lib.mi355gemm_gemm_timed(*args, -1 if cid is None else cid, ev[0], ev[1])
        return lib.mi355gemm_gemm(*args) if cid is None else lib.mi355gemm_gemm_config(*args, cid)
    # the library launches on the calling thread's current HIP device
    if idx == cur:
        st = call()
    else:
        with torch.cuda.device(idx):
            st = call()
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())
    return out


def vector_add(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """``out = a + b`` element-wise on the GPU (fp16, one rounding), any shape, contiguous."""
    for t, name in ((a, "a"), (b, "b")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16:
            raise TypeError("%s must be a float16 torch.Tensor" % name)
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor on a GPU device" % name)
    if a.shape != b.shape or a.device != b.device:
        raise ValueError("a and b must have the same shape and device")
    if out is None:
        out = torch.empty_like(a)
    elif (out.shape != a.shape or out.dtype != torch.float16 or out.device != a.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous float16 tensor shaped like a")
    lib = _lib if _lib is not None else library()
    idx = a.device.index if a.device.index is not None else torch.cuda.current_device()
    sptr = stream.cuda_stream if stream is not None else _raw_stream(idx)
    args = (a.numel(), a.data_ptr(), b.data_ptr(), out.data_ptr(), sptr)
    if idx == torch.cuda.current_device():
        st = lib.mi355gemm_vector_add(*args)
    else:
        with torch.cuda.device(idx):
            st = lib.mi355gemm_vector_add(*args)
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())
    return out


def softmax(x: torch.Tensor, out: torch.Tensor | None = None,
            stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Softmax over the last dimension of a contiguous fp16 tensor on the GPU (every
    leading index is one row)."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float16:
        raise TypeError("x must be a float16 torch.Tensor")
    if x.device.type != "cuda" or x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous tensor of at least 1 dimension on a GPU device")
    if out is None:
        out = torch.empty_like(x)
    elif (not isinstance(out, torch.Tensor) or out.dtype != torch.float16 or out.shape != x.shape
          or out.device != x.device or not out.is_contiguous()):
        raise ValueError("out must be a contiguous float16 tensor shaped like x on its device")
    lib = _lib if _lib is not None else library()
    idx = x.device.index if x.device.index is not None else torch.cuda.current_device()
    sptr = stream.cuda_stream if stream is not None else _raw_stream(idx)
    N = x.shape[-1]
    M = x.numel() // N if N > 0 else 0
    if idx == torch.cuda.current_device():
        st = lib.mi355gemm_softmax(M, N, x.data_ptr(), out.data_ptr(), sptr)
    else:
        with torch.cuda.device(idx):
            st = lib.mi355gemm_softmax(M, N, x.data_ptr(), out.data_ptr(), sptr)
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())
    return out


def mi355gemm_attention(batch, heads, seq_q, seq_k, head_dim, q, k, v, o, lse, scale, causal,
                        stream) -> int:
    return library().mi355gemm_attention(batch, heads, seq_q, seq_k, head_dim, q, k, v, o, lse,
                                         scale, causal, stream)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None,
              stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Attention forward of contiguous fp16 tensors on the GPU: q (..., seq_q, head_dim),
    k and v (..., seq_k, head_dim) with the same leading dimensions (typically batch and
    heads; every leading index is one independent problem).  ``scale`` defaults to
    1/sqrt(head_dim).  ``lse`` (optional, fp32, shaped like q without its last
    dimension) receives the natural-log sum of exp of each query row's scores."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % n)
        if t.dtype != torch.float16:
            raise TypeError("%s must be float16, got %s" % (n, t.dtype))
        if t.device.type != "cuda":
            raise ValueError("%s must be on a GPU device" % n)
        if t.dim() < 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor of at least 2 dimensions" % n)
    lead, (Sq, D) = tuple(q.shape[:-2]), tuple(q.shape[-2:])
    Sk = k.shape[-2]
    if k.shape != lead + (Sk, D) or v.shape != k.shape:
        raise ValueError("k and v must be (..., seq_k, head_dim) with q's leading dimensions; "
                         "got %s %s %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.dim())
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must be shaped like q on its device")
    lse_ptr = None
    if lse is not None:
        if (lse.dtype != torch.float32 or lse.device != q.device or tuple(lse.shape) != lead + (Sq,)
                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 tensor shaped like q without "
                             "its last dimension, on q's device")
        lse_ptr = lse.data_ptr()
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    pairs = 1
    for d in lead:
        pairs *= d
    lib = _lib if _lib is not None else library()
    idx = q.device.index if q.device.index is not None else torch.cuda.current_device()
    sptr = stream.cuda_stream if stream is not None else _raw_stream(idx)
    args = (pairs, 1, Sq, Sk, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
            float(scale), int(bool(causal)), sptr)
    if idx == torch.cuda.current_device():
        st = lib.mi355gemm_attention(*args)
    else:
        with torch.cuda.device(idx):
            st = lib.mi355gemm_attention(*args)
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())
    return out


def set_choice(M: int, N: int, K: int, epilogue="none", a_vector: bool = True,
               bc_vector: bool = True, config=None) -> None:
    """Install ``config`` (a name or id) for requests of exactly this shape, epilogue and
    alignment class in this process (``mi355gemm_set_choice``)."""
    cid = config_id(config) if isinstance(config, str) else int(config)
    st = mi355gemm_set_choice(M, N, K, _epi(epilogue), int(bool(a_vector)), int(bool(bc_vector)), cid)
    if st != OK:
        raise GemmError(st, mi355gemm_last_error())


def clear_choices() -> None:
    """Remove every installed choice (``mi355gemm_clear_choices``)."""
    mi355gemm_clear_choices()


def select(a: torch.Tensor, b: torch.Tensor, bias=None, epilogue="none", out=None) -> int:
    """Configuration id ``gemm`` would use for these tensors (host-only decision)."""
    M, K = a.shape
    N = b.shape[1]
    cid = mi355gemm_select(M, N, K, _epi(epilogue), a.data_ptr(), b.data_ptr(),
                           out.data_ptr() if out is not None else 256,
                           bias.data_ptr() if bias is not None else None)
    return cid
