"""Python binding of libqgemv.so, the MI355X (gfx950) quantized GEMV library.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels. torch supplies device memory and the current stream. The binding
raises if the compiled library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "qgemv.h")

MAX_BATCH = 8
SMALLN_MAX = 32

_lib = None


class QGError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str):
        super().__init__(f"{func}: status {status}: {detail}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


class _GemmProblem(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("X", ctypes.c_void_p), ("ldx", ctypes.c_int64),
                ("Y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64)]


class _GemmQ81Problem(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("xq", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64), ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


class _LaunchOverride(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("gemv_waves", "smalln_form", "smalln_waves", "smalln_tiles",
                                            "smalln_depth", "verify_form", "verify_waves", "verify_tiles")]


# kernel forms a launch override can force (include/qgemv.h)
FORM_AUTO = 0
FORM_SMALLN_REGS, FORM_SMALLN_LDS, FORM_SMALLN_LDS1, FORM_SMALLN_DOT, FORM_SMALLN_STREAM, FORM_SMALLN_WALK, \
    FORM_SMALLN_SPLIT, FORM_SMALLN_SLICE = 1, 2, 3, 4, 5, 6, 7, 8
FORM_VERIFY_MFMA, FORM_VERIFY_DOT, FORM_VERIFY_STREAM = 1, 2, 3


class _TopkOut(ctypes.Structure):
    _fields_ = [("index", ctypes.c_void_p), ("logit", ctypes.c_void_p), ("logprob", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("token", ctypes.c_void_p)]


class _Sampler(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float), ("min_p", ctypes.c_float),
                ("u", ctypes.c_void_p)]


_P, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int

_SIGS = {
    "qg_abi_version": (_I, []),
    "qg_status_string": (ctypes.c_char_p, [_I]),
    "qg_last_error": (ctypes.c_char_p, []),
    "qg_q4k_bytes": (_SZ, [_I64, _I64]),
    "qg_q8_0_bytes": (_SZ, [_I64, _I64]),
    "qg_q6k_bytes": (_SZ, [_I64, _I64]),
    "qg_pack_q4k": (_I, [_P, _P, _I64, _I64, _P]),
    "qg_pack_q8_0": (_I, [_P, _P, _I64, _I64, _P]),
    "qg_pack_q6k": (_I, [_P, _P, _I64, _I64, _P]),
    "qg_workspace_clear": (_I, [_P, _SZ, _P]),
    "qgemv_q4k": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "qgemv_q4k_batch": (_I, [ctypes.POINTER(_Problem), _I, _P]),
    "qgemv_q8_0": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "qg_q8_1_bytes": (_SZ, [_I64]),
    "qg_quantize_q8_1": (_I, [_P, _I64, _P, _P]),
    "qg_quantize_q8_1_columns": (_I, [_P, _I64, _I64, _I64, _P, _P]),
    "qgemv_q4k_q8_1": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "qgemv_q4k_q8_1_batch": (_I, [ctypes.POINTER(_Problem), _I, _P]),
    "qgemm_q4k_q8_1_smalln": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "qgemm_q4k_q8_1_smalln_batch": (_I, [ctypes.POINTER(_GemmQ81Problem), _I, _P]),
    "qgemv_q6k": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "qgemm_q4k_smalln": (_I, [_P, _P, _I64, _P, _I64, _I64, _I64, _I64, _P]),
    "qgemm_q4k_smalln_batch": (_I, [ctypes.POINTER(_GemmProblem), _I, _P]),
    "qgemm_q4k_smalln_batch_workspace_bytes": (_SZ, [ctypes.POINTER(_GemmProblem), _I]),
    "qgemm_q4k_smalln_batch_ws": (_I, [ctypes.POINTER(_GemmProblem), _I, _P, _SZ, _P]),
    "qg_set_launch_override": (_I, [ctypes.c_void_p]),
    "qg_get_launch_override": (_I, [ctypes.c_void_p]),
    "lmhead_argmax_verify_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "lmhead_argmax_verify": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P, _P, _P]),
    "lmhead_argmax_verify_q8_1_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "lmhead_argmax_verify_q8_1": (_I, [_P, _P, _I64, _I64, _I64, _P, _SZ, _P, _P, _P]),
    "lmhead_argmax_workspace_bytes": (_SZ, [_I64, _I64]),
    "logits_topk_workspace_bytes": (_SZ, [_I64]),
    "logits_topk": (_I, [_P, _I64, _I, ctypes.POINTER(_Sampler), _P, _SZ, ctypes.POINTER(_TopkOut), _P]),
    "lmhead_topk_workspace_bytes": (_SZ, [_I64, _I64]),
    "lmhead_topk": (_I, [_P, _P, _I64, _I64, _I, _P, ctypes.POINTER(_Sampler), _P, _SZ, ctypes.POINTER(_TopkOut),
                         _P]),
    "lmhead_argmax": (_I, [_P, _P, _I64, _I64, _P, _SZ, _P, _P, _P]),
    "lmhead_argmax_noalloc": (_I, [_P, _P, _I64, _I64, _P, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libqgemv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with quantized_gemv_argmax_amd.build.build() "
                               "(hipcc, gfx950); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/qgemv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def status_string(s: int) -> str:
    return lib().qg_status_string(int(s)).decode()


def last_error() -> str:
    return lib().qg_last_error().decode()


def _check(func: str, status: int):
    if status != 0:
        raise QGError(func, status, f"{status_string(status)}: {last_error()}")


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


# ------------------------------------------------------------------ workspace
class Workspace:
    """A device scratch buffer reused across calls on one stream (grown on demand).
    It starts all-zero, as the library requires, and every call leaves it so."""

    def __init__(self, device=None, nbytes: int = 0):
        self.device = torch.device(device if device is not None else "cuda")
        self.buf = None
        if nbytes:
            self.ensure(nbytes)

    def ensure(self, nbytes: int):
        if nbytes and (self.buf is None or self.buf.numel() < nbytes):
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=self.device)
        return self

    def ptr(self) -> int | None:
        return None if self.buf is None else self.buf.data_ptr()

    def nbytes(self) -> int:
        return 0 if self.buf is None else self.buf.numel()


_default_ws: dict = {}


def default_workspace(device=None) -> Workspace:
    dev = torch.device(device if device is not None else "cuda")
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    if key not in _default_ws:
        _default_ws[key] = Workspace(dev)
    return _default_ws[key]


def _ws(ws: Workspace | None, need: int, device) -> Workspace:
    ws = ws if ws is not None else default_workspace(device)
    ws.ensure(need)
    return ws


# ------------------------------------------------------------------ sizes / packing
def q4k_bytes(M: int, K: int) -> int:
    return int(lib().qg_q4k_bytes(M, K))


def q8_0_bytes(M: int, K: int) -> int:
    return int(lib().qg_q8_0_bytes(M, K))


def q6k_bytes(M: int, K: int) -> int:
    return int(lib().qg_q6k_bytes(M, K))


def pack_q4k(canonical: torch.Tensor, M: int, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Repack canonical Q4_K bytes (uint8 device tensor) into the library's layout."""
    _need_cuda(canonical)
    n = q4k_bytes(M, K)
    if canonical.numel() != n or canonical.dtype != torch.uint8:
        raise ValueError(f"expected {n} uint8 bytes of Q4_K blocks")
    out = out if out is not None else torch.empty(n, dtype=torch.uint8, device=canonical.device)
    _check("qg_pack_q4k", lib().qg_pack_q4k(_ptr(canonical), _ptr(out), M, K, _stream(canonical.device)))
    return out


def pack_q8_0(canonical: torch.Tensor, M: int, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    _need_cuda(canonical)
    n = q8_0_bytes(M, K)
    if canonical.numel() != n or canonical.dtype != torch.uint8:
        raise ValueError(f"expected {n} uint8 bytes of Q8_0 blocks")
    out = out if out is not None else torch.empty(n, dtype=torch.uint8, device=canonical.device)
    _check("qg_pack_q8_0", lib().qg_pack_q8_0(_ptr(canonical), _ptr(out), M, K, _stream(canonical.device)))
    return out


def pack_q6k(canonical: torch.Tensor, M: int, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Repack canonical Q6_K bytes (uint8 device tensor) into the library's layout."""
    _need_cuda(canonical)
    n = q6k_bytes(M, K)
    if canonical.numel() != n or canonical.dtype != torch.uint8:
        raise ValueError(f"expected {n} uint8 bytes of Q6_K blocks")
    out = out if out is not None else torch.empty(n, dtype=torch.uint8, device=canonical.device)
    _check("qg_pack_q6k", lib().qg_pack_q6k(_ptr(canonical), _ptr(out), M, K, _stream(canonical.device)))
    return out


# ------------------------------------------------------------------ launch override
class launch_override:
    """Context manager (or plain call through .set()) that forces kernel forms or
    launch shapes on this host thread for tests and measurements, through
    qg_set_launch_override; fields not given keep the automatic choice. Example:
    `with qg.launch_override(smalln_form=qg.FORM_SMALLN_LDS, smalln_tiles=2): ...`"""

    def __init__(self, **fields):
        self.o = _LaunchOverride()
        for k, v in fields.items():
            if k not in dict(_LaunchOverride._fields_):
                raise TypeError(f"unknown launch override field {k!r}")
            setattr(self.o, k, int(v))
        self._prev = None

    def set(self):
        _check("qg_set_launch_override", lib().qg_set_launch_override(ctypes.byref(self.o)))

    def __enter__(self):
        self._prev = _LaunchOverride()
        _check("qg_get_launch_override", lib().qg_get_launch_override(ctypes.byref(self._prev)))
        self.set()
        return self

    def __exit__(self, *exc):
        _check("qg_set_launch_override", lib().qg_set_launch_override(ctypes.byref(self._prev)))
        return False


def get_launch_override() -> dict:
    o = _LaunchOverride()
    _check("qg_get_launch_override", lib().qg_get_launch_override(ctypes.byref(o)))
    return {n: getattr(o, n) for n, _ in _LaunchOverride._fields_}


# ------------------------------------------------------------------ products
def qgemv_q4k(w: torch.Tensor, x: torch.Tensor, M: int, K: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[M] = W x for a packed Q4_K matrix (fp32 x, y)."""
    _need_cuda(w, x, y)
    y = y if y is not None else torch.empty(M, dtype=torch.float32, device=x.device)
    _check("qgemv_q4k", lib().qgemv_q4k(_ptr(w), _ptr(x), _ptr(y), M, K, _stream(x.device)))
    return y


def qgemv_q4k_batch(problems):
    """problems: list of (w_packed, x, y, M, K); one launch for all of them."""
    arr = (_Problem * len(problems))()
    dev = None
    for i, (w, x, y, M, K) in enumerate(problems):
        _need_cuda(w, x, y)
        dev = x.device
        arr[i] = _Problem(_ptr(w), _ptr(x), _ptr(y), M, K)
    _check("qgemv_q4k_batch", lib().qgemv_q4k_batch(arr, len(problems), _stream(dev)))
    return [p[2] for p in problems]


def qgemv_q8_0(w: torch.Tensor, x: torch.Tensor, M: int, K: int, y: torch.Tensor | None = None) -> torch.Tensor:
    _need_cuda(w, x, y)
    y = y if y is not None else torch.empty(M, dtype=torch.float32, device=x.device)
    _check("qgemv_q8_0", lib().qgemv_q8_0(_ptr(w), _ptr(x), _ptr(y), M, K, _stream(x.device)))
    return y


def q8_1_bytes(K: int) -> int:
    return int(lib().qg_q8_1_bytes(K))


def q8_1_views(xq: torch.Tensor, K: int):
    """(d float32[K/32], q int8[K], s int16[K/32]) views of a quantized-activation buffer."""
    nc = K // 32
    q_off = -(-4 * nc // 16) * 16
    s_off = -(-(q_off + K) // 16) * 16
    return (xq[:4 * nc].view(torch.float32), xq[q_off:q_off + K].view(torch.int8),
            xq[s_off:s_off + 2 * nc].view(torch.int16))


def quantize_q8_1(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Int8 activations with a float32 scale and a block sum per 32 (uint8 buffer)."""
    _need_cuda(x, out)
    K = x.numel()
    n = q8_1_bytes(K)
    out = out if out is not None else torch.empty(n, dtype=torch.uint8, device=x.device)
    _check("qg_quantize_q8_1", lib().qg_quantize_q8_1(_ptr(x), K, _ptr(out), _stream(x.device)))
    return out


def qgemv_q4k_q8_1(w: torch.Tensor, xq: torch.Tensor, M: int, K: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[M] = W xq for a packed Q4_K matrix and quantized activations."""
    _need_cuda(w, xq, y)
    y = y if y is not None else torch.empty(M, dtype=torch.float32, device=xq.device)
    _check("qgemv_q4k_q8_1", lib().qgemv_q4k_q8_1(_ptr(w), _ptr(xq), _ptr(y), M, K, _stream(xq.device)))
    return y


def qgemv_q4k_q8_1_batch(problems):
    """problems: list of (w_packed, xq, y, M, K); one launch for all of them."""
    arr = (_Problem * len(problems))()  # same field layout as qg_gemv_q8_1_problem
    dev = None
    for i, (w, xq, y, M, K) in enumerate(problems):
        _need_cuda(w, xq, y)
        dev = xq.device
        arr[i] = _Problem(_ptr(w), _ptr(xq), _ptr(y), M, K)
    _check("qgemv_q4k_q8_1_batch", lib().qgemv_q4k_q8_1_batch(arr, len(problems), _stream(dev)))
    return [p[2] for p in problems]


def quantize_q8_1_columns(X: torch.Tensor, out: torch.Tensor | None = None, K: int | None = None) -> torch.Tensor:
    """X (N, ldx) fp32, row n = column n (its first K = ldx entries unless K is
    given) -> N consecutive Q8_1 buffers of q8_1_bytes(K) bytes, in one launch."""
    _need_cuda(X, out)
    N, ldx = X.shape
    if X.stride(1) != 1 or X.stride(0) != ldx:
        raise ValueError("X must be a contiguous (N, ldx) tensor")
    K = ldx if K is None else K
    nb = q8_1_bytes(K)
    out = out if out is not None else torch.empty(N * nb, dtype=torch.uint8, device=X.device)
    _check("qg_quantize_q8_1_columns",
           lib().qg_quantize_q8_1_columns(_ptr(X), ldx, K, N, _ptr(out), _stream(X.device)))
    return out


def qgemm_q4k_q8_1_smalln(w: torch.Tensor, xq: torch.Tensor, M: int, K: int, N: int,
                          Y: torch.Tensor | None = None) -> torch.Tensor:
    """Y (N, ldy) = W Xq for N <= 8 quantized columns (quantize_q8_1_columns)."""
    _need_cuda(w, xq, Y)
    Y = Y if Y is not None else torch.empty((N, (M + 3) // 4 * 4), dtype=torch.float32, device=xq.device)
    if Y.shape[0] != N or Y.stride(1) != 1:
        raise ValueError("Y must be a contiguous (N, ldy) tensor")
    _check("qgemm_q4k_q8_1_smalln", lib().qgemm_q4k_q8_1_smalln(_ptr(w), _ptr(xq), _ptr(Y), Y.stride(0), M, K, N,
                                                                _stream(xq.device)))
    return Y


def qgemm_q4k_q8_1_smalln_batch(problems):
    """problems: list of (w_packed, xq, Y, M, K) with Y (N, ldy) and xq holding N
    quantized columns; one launch for all of them."""
    arr = (_GemmQ81Problem * len(problems))()
    dev = None
    for i, (w, xq, Y, M, K) in enumerate(problems):
        _need_cuda(w, xq, Y)
        dev = xq.device
        if Y.stride(1) != 1:
            raise ValueError("Y must be a contiguous (N, ldy) tensor")
        arr[i] = _GemmQ81Problem(_ptr(w), _ptr(xq), _ptr(Y), Y.stride(0), M, K, Y.shape[0])
    _check("qgemm_q4k_q8_1_smalln_batch", lib().qgemm_q4k_q8_1_smalln_batch(arr, len(problems), _stream(dev)))
    return [p[2] for p in problems]


def qgemv_q6k(w: torch.Tensor, x: torch.Tensor, M: int, K: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[M] = W x for a packed Q6_K matrix (fp32 x, y)."""
    _need_cuda(w, x, y)
    y = y if y is not None else torch.empty(M, dtype=torch.float32, device=x.device)
    _check("qgemv_q6k", lib().qgemv_q6k(_ptr(w), _ptr(x), _ptr(y), M, K, _stream(x.device)))
    return y


def qgemm_q4k_smalln(w: torch.Tensor, X: torch.Tensor, M: int, K: int, Y: torch.Tensor | None = None) -> torch.Tensor:
    """X: (N, ldx) fp32, row n = column n of the K x N operand (ldx >= K, ldx % 4 == 0).
    Returns Y as (N, ldy) with Y[n, :M] = W X[n, :K]."""
    _need_cuda(w, X, Y)
    N, ldx = X.shape
    if X.stride(1) != 1 or X.stride(0) != ldx:
        raise ValueError("X must be a contiguous (N, ldx) tensor")
    if Y is None:
        ldy = (M + 3) // 4 * 4
        Y = torch.empty((N, ldy), dtype=torch.float32, device=X.device)
    ldy = Y.shape[1]
    _check("qgemm_q4k_smalln", lib().qgemm_q4k_smalln(_ptr(w), _ptr(X), ldx, _ptr(Y), ldy, M, K, N,
                                                        _stream(X.device)))
    return Y


def _gemm_problems(problems):
    arr = (_GemmProblem * len(problems))()
    dev = None
    for i, (w, X, Y, M, K) in enumerate(problems):
        _need_cuda(w, X, Y)
        dev = X.device
        N, ldx = X.shape
        if X.stride(1) != 1 or X.stride(0) != ldx or Y.stride(1) != 1 or Y.shape[0] != N:
            raise ValueError("X and Y must be contiguous (N, ld) tensors with the same N")
        arr[i] = _GemmProblem(_ptr(w), _ptr(X), ldx, _ptr(Y), Y.stride(0), M, K, N)
    return arr, dev


def qgemm_q4k_smalln_batch(problems):
    """problems: list of (w_packed, X, Y, M, K) with X (N, ldx) and Y (N, ldy) as in
    qgemm_q4k_smalln; one launch for all of them. Returns the Y tensors."""
    arr, dev = _gemm_problems(problems)
    _check("qgemm_q4k_smalln_batch", lib().qgemm_q4k_smalln_batch(arr, len(problems), _stream(dev)))
    return [p[2] for p in problems]


def qgemm_q4k_smalln_batch_workspace_bytes(problems) -> int:
    arr, _ = _gemm_problems(problems)
    return lib().qgemm_q4k_smalln_batch_workspace_bytes(arr, len(problems))


def qgemm_q4k_smalln_batch_ws(problems, ws: Workspace | None = None):
    """qgemm_q4k_smalln_batch with a workspace (sized by
    qgemm_q4k_smalln_batch_workspace_bytes; a per-device scratch buffer if None),
    which lets the library split few-tile, many-column products over K slices. One
    workspace serves batches of any shapes; its counters come back zero and the rest
    of it undefined. Calls sharing a workspace (the scratch one included) must not
    overlap: calls on concurrent streams pass workspaces of their own."""
    arr, dev = _gemm_problems(problems)
    need = lib().qgemm_q4k_smalln_batch_workspace_bytes(arr, len(problems))
    if ws is None:  # scratch contents: never the zero-kept workspace of the LM-head calls
        key = ("scratch", str(dev))
        ws = _default_ws.setdefault(key, Workspace(dev))
    ws.ensure(need)
    _check("qgemm_q4k_smalln_batch_ws",
           lib().qgemm_q4k_smalln_batch_ws(arr, len(problems), ws.ptr(), ws.nbytes(), _stream(dev)))
    return [p[2] for p in problems]


def lmhead_argmax(w: torch.Tensor, x: torch.Tensor, M: int, K: int, out_index: torch.Tensor | None = None,
                  out_value: torch.Tensor | None = None, ws: Workspace | None = None):
    """Fused Q8_0 LM head + argmax. Returns (index int32[1], value float32[1]) device tensors."""
    _need_cuda(w, x, out_index, out_value)
    out_index = out_index if out_index is not None else torch.empty(1, dtype=torch.int32, device=x.device)
    out_value = out_value if out_value is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    need = int(lib().lmhead_argmax_workspace_bytes(M, K))
    ws = _ws(ws, need, x.device)
    _check("lmhead_argmax", lib().lmhead_argmax(_ptr(w), _ptr(x), M, K, ws.ptr(), ws.nbytes(), _ptr(out_index),
                                                  _ptr(out_value), _stream(x.device)))
    return out_index, out_value


def lmhead_argmax_noalloc(w: torch.Tensor, x: torch.Tensor, M: int, K: int, out_index: torch.Tensor | None = None,
                          out_value: torch.Tensor | None = None):
    """lmhead_argmax with the partials in the library's own per-GPU array (no
    workspace; calls on one GPU must not overlap). Returns (index, value) tensors."""
    _need_cuda(w, x, out_index, out_value)
    out_index = out_index if out_index is not None else torch.empty(1, dtype=torch.int32, device=x.device)
    out_value = out_value if out_value is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    _check("lmhead_argmax_noalloc", lib().lmhead_argmax_noalloc(_ptr(w), _ptr(x), M, K, _ptr(out_index),
                                                                _ptr(out_value), _stream(x.device)))
    return out_index, out_value


def lmhead_argmax_verify(w: torch.Tensor, X: torch.Tensor, M: int, K: int, out_index: torch.Tensor | None = None,
                         out_value: torch.Tensor | None = None, ws: Workspace | None = None):
    """Batched greedy verification on a Q8_0 LM head. X: fp32 (N, ldx), row n = column n.
    Returns (index int32[N], value float32[N]) device tensors."""
    _need_cuda(w, X, out_index, out_value)
    N, ldx = X.shape
    if X.stride(1) != 1 or X.stride(0) != ldx:
        raise ValueError("X must be a contiguous (N, ldx) tensor")
    oi = out_index if out_index is not None else torch.empty(N, dtype=torch.int32, device=X.device)
    ov = out_value if out_value is not None else torch.empty(N, dtype=torch.float32, device=X.device)
    need = int(lib().lmhead_argmax_verify_workspace_bytes(M, K, N))
    ws = _ws(ws, need, X.device)
    _check("lmhead_argmax_verify", lib().lmhead_argmax_verify(_ptr(w), _ptr(X), ldx, M, K, N, ws.ptr(), ws.nbytes(),
                                                              _ptr(oi), _ptr(ov), _stream(X.device)))
    return oi, ov


def lmhead_argmax_verify_q8_1(w: torch.Tensor, xq: torch.Tensor, M: int, K: int, N: int,
                              out_index: torch.Tensor | None = None, out_value: torch.Tensor | None = None,
                              ws: Workspace | None = None):
    """Batched greedy verification on a Q8_0 LM head against N <= 8 quantized columns
    (quantize_q8_1_columns). Returns (index int32[N], value float32[N]) device tensors."""
    _need_cuda(w, xq, out_index, out_value)
    oi = out_index if out_index is not None else torch.empty(N, dtype=torch.int32, device=xq.device)
    ov = out_value if out_value is not None else torch.empty(N, dtype=torch.float32, device=xq.device)
    need = int(lib().lmhead_argmax_verify_q8_1_workspace_bytes(M, K, N))
    ws = _ws(ws, need, xq.device)
    _check("lmhead_argmax_verify_q8_1",
           lib().lmhead_argmax_verify_q8_1(_ptr(w), _ptr(xq), M, K, N, ws.ptr(), ws.nbytes(), _ptr(oi), _ptr(ov),
                                           _stream(xq.device)))
    return oi, ov


# ------------------------------------------------------------------ top-k / log-softmax / sampling
class TopK:
    """Device outputs of a top-k call: index[k] (int32), logit[k], logprob[k], lse[1]
    and, when a sampler was given, token[1] (int32)."""

    def __init__(self, k: int, device, sample: bool):
        self.index = torch.empty(k, dtype=torch.int32, device=device)
        self.logit = torch.empty(k, dtype=torch.float32, device=device)
        self.logprob = torch.empty(k, dtype=torch.float32, device=device)
        self.lse = torch.empty(1, dtype=torch.float32, device=device)
        self.token = torch.empty(1, dtype=torch.int32, device=device) if sample else None

    def _c(self) -> _TopkOut:
        return _TopkOut(_ptr(self.index), _ptr(self.logit), _ptr(self.logprob), _ptr(self.lse), _ptr(self.token))


def _sampler(sampler):
    """sampler: None or (temperature, top_p, min_p, u) with u a 1-element fp32 device tensor."""
    if sampler is None:
        return None
    T, top_p, min_p, u = sampler
    _need_cuda(u)
    if u.dtype != torch.float32 or u.numel() < 1:
        raise ValueError("u must be a float32 device tensor holding one uniform number")
    return ctypes.pointer(_Sampler(T, top_p, min_p, _ptr(u)))


def logits_topk(logits: torch.Tensor, k: int, sampler=None, ws: Workspace | None = None,
                out: TopK | None = None) -> TopK:
    """Top-k rows, log-softmax and (optionally) one sampled token of an fp32 logit
    vector on the device."""
    _need_cuda(logits)
    M = logits.numel()
    out = out if out is not None else TopK(k, logits.device, sampler is not None)
    need = int(lib().logits_topk_workspace_bytes(M))
    ws = _ws(ws, need, logits.device)
    oc = out._c()
    _check("logits_topk", lib().logits_topk(_ptr(logits), M, k, _sampler(sampler), ws.ptr(), ws.nbytes(),
                                            ctypes.byref(oc), _stream(logits.device)))
    return out


def lmhead_topk(w: torch.Tensor, x: torch.Tensor, M: int, K: int, k: int, logits: torch.Tensor | None = None,
                sampler=None, ws: Workspace | None = None, out: TopK | None = None):
    """Q8_0 LM head fused with top-k, log-softmax and sampling. Returns (TopK, logits);
    the logits stay in device memory."""
    _need_cuda(w, x, logits)
    logits = logits if logits is not None else torch.empty(M, dtype=torch.float32, device=x.device)
    out = out if out is not None else TopK(k, x.device, sampler is not None)
    need = int(lib().lmhead_topk_workspace_bytes(M, K))
    ws = _ws(ws, need, x.device)
    oc = out._c()
    _check("lmhead_topk", lib().lmhead_topk(_ptr(w), _ptr(x), M, K, k, _ptr(logits), _sampler(sampler), ws.ptr(),
                                            ws.nbytes(), ctypes.byref(oc), _stream(x.device)))
    return out, logits
