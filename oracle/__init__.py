"""ctypes binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its Python binding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.or_half_to_double.restype = ctypes.c_double
        L.or_half_to_double.argtypes = [ctypes.c_uint16]
        L.or_q4k_unpack_scales.argtypes = [_P, _P, _P]
        L.or_q4k_dequant_block.argtypes = [_P, _P]
        L.or_q8_0_dequant_block.argtypes = [_P, _P]
        L.or_q6k_dequant_block.argtypes = [_P, _P]
        L.or_q4k_dequant_row.argtypes = [_P, _I64, _P]
        L.or_q8_0_dequant_row.argtypes = [_P, _I64, _P]
        L.or_q6k_dequant_row.argtypes = [_P, _I64, _P]
        for name in ("or_gemv_q4k", "or_gemv_q8_0", "or_gemv_q6k"):
            getattr(L, name).argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P]
        L.or_gemv_q4k_factored.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.or_gemm_q4k.argtypes = [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _P, _P]
        L.or_argmax.restype = _I64
        L.or_argmax.argtypes = [_P, _I64]
        L.or_num_threads.restype = ctypes.c_int
        L.or_set_num_threads.argtypes = [ctypes.c_int]
        L.or_quantize_q8_1.argtypes = [_P, _I64, _P, _P, _P]
        L.or_gemv_q4k_q8_1.argtypes = [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P]
        L.or_gemv_q8_0_q8_1.argtypes = [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P]
        L.or_topk.argtypes = [_P, _I64, ctypes.c_int, _P]
        L.or_logsumexp.restype = ctypes.c_double
        L.or_logsumexp.argtypes = [_P, _I64]
        L.or_sample_topk.restype = ctypes.c_int
        L.or_sample_topk.argtypes = [_P, ctypes.c_int] + [ctypes.c_double] * 4
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u8(W) -> np.ndarray:
    W = np.ascontiguousarray(W)
    if W.dtype != np.uint8:
        raise TypeError("weights must be uint8 block bytes")
    return W


def _rows(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= M):
        raise IndexError("row index out of range")
    return r, r.size


def half_to_double(bits: int) -> float:
    return lib().or_half_to_double(int(bits) & 0xFFFF)


def q4k_unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    s = np.ascontiguousarray(s12, dtype=np.uint8)
    assert s.size == 12
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    lib().or_q4k_unpack_scales(_ptr(s), _ptr(sc), _ptr(m))
    return sc, m


def q4k_dequant_block(blk) -> np.ndarray:
    b = np.ascontiguousarray(blk, dtype=np.uint8)
    assert b.size == 144
    w = np.zeros(256, np.float64)
    lib().or_q4k_dequant_block(_ptr(b), _ptr(w))
    return w


def q8_0_dequant_block(blk) -> np.ndarray:
    b = np.ascontiguousarray(blk, dtype=np.uint8)
    assert b.size == 34
    w = np.zeros(32, np.float64)
    lib().or_q8_0_dequant_block(_ptr(b), _ptr(w))
    return w


def q6k_dequant_block(blk) -> np.ndarray:
    b = np.ascontiguousarray(blk, dtype=np.uint8)
    assert b.size == 210
    w = np.zeros(256, np.float64)
    lib().or_q6k_dequant_block(_ptr(b), _ptr(w))
    return w


def q6k_dequant(W, M: int, K: int) -> np.ndarray:
    W = _u8(W)
    assert W.size == M * (K // 256) * 210
    out = np.zeros((M, K), np.float64)
    for r in range(M):
        lib().or_q6k_dequant_row(_ptr(W.reshape(M, -1)[r]), K, _ptr(out[r]))
    return out


def q4k_dequant(W, M: int, K: int) -> np.ndarray:
    W = _u8(W)
    assert W.size == M * (K // 256) * 144
    out = np.zeros((M, K), np.float64)
    for r in range(M):
        lib().or_q4k_dequant_row(_ptr(W.reshape(M, -1)[r]), K, _ptr(out[r]))
    return out


def q8_0_dequant(W, M: int, K: int) -> np.ndarray:
    W = _u8(W)
    assert W.size == M * (K // 32) * 34
    out = np.zeros((M, K), np.float64)
    for r in range(M):
        lib().or_q8_0_dequant_row(_ptr(W.reshape(M, -1)[r]), K, _ptr(out[r]))
    return out


def _gemv(fn, W, M, K, x, rows, row_bytes):
    W = _u8(W)
    if W.size != M * row_bytes:
        raise ValueError("weight bytes do not match M x K")
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size != K:
        raise ValueError("x length must be K")
    r, n = _rows(rows, M)
    y = np.zeros(n, np.float64)
    a = np.zeros(n, np.float64)
    fn(_ptr(W), M, K, _ptr(x), _ptr(r), n, _ptr(y), _ptr(a))
    return y, a


def gemv_q4k(W, M: int, K: int, x, rows=None):
    """fp64 y and sum|w*x| for the listed rows (all rows when rows is None)."""
    return _gemv(lib().or_gemv_q4k, W, M, K, x, rows, (K // 256) * 144)


def gemv_q8_0(W, M: int, K: int, x, rows=None):
    return _gemv(lib().or_gemv_q8_0, W, M, K, x, rows, (K // 32) * 34)


def gemv_q6k(W, M: int, K: int, x, rows=None):
    return _gemv(lib().or_gemv_q6k, W, M, K, x, rows, (K // 256) * 210)


def gemv_q4k_factored(W, M: int, K: int, x, rows=None) -> np.ndarray:
    W = _u8(W)
    x = np.ascontiguousarray(x, dtype=np.float32)
    r, n = _rows(rows, M)
    y = np.zeros(n, np.float64)
    lib().or_gemv_q4k_factored(_ptr(W), M, K, _ptr(x), _ptr(r), n, _ptr(y))
    return y


def gemm_q4k(W, M: int, K: int, X_cols, rows=None):
    """X_cols: float32 (N, K), column n of the K x N operand. Returns Y, A of shape (N, nrows)."""
    W = _u8(W)
    X = np.ascontiguousarray(X_cols, dtype=np.float32)
    N = X.shape[0]
    assert X.shape[1] == K
    r, n = _rows(rows, M)
    Y = np.zeros((N, n), np.float64)
    A = np.zeros((N, n), np.float64)
    lib().or_gemm_q4k(_ptr(W), M, K, _ptr(X), K, N, _ptr(r), n, _ptr(Y), _ptr(A))
    return Y, A


def argmax(y) -> int:
    y = np.ascontiguousarray(y, dtype=np.float64)
    return int(lib().or_argmax(_ptr(y), y.size))


def quantize_q8_1(x):
    """Q8_1-style activations: (d float32[K/32], q int8[K], s int16[K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = x.size
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    d = np.empty(K // 32, np.float32)
    q = np.empty(K, np.int8)
    s = np.empty(K // 32, np.int16)
    lib().or_quantize_q8_1(_ptr(x), K, _ptr(d), _ptr(q), _ptr(s))
    return d, q, s


def gemv_q4k_q8_1(W, M: int, K: int, d, q, rows=None):
    """y = W xq with xq = d[k/32] * q[k]; returns (y, sum|w*xq|) in fp64."""
    W = _u8(W)
    d = np.ascontiguousarray(d, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.int8)
    r, n = _rows(rows, M)
    y = np.zeros(n, np.float64)
    a = np.zeros(n, np.float64)
    lib().or_gemv_q4k_q8_1(_ptr(W), M, K, _ptr(d), _ptr(q), _ptr(r), n, _ptr(y), _ptr(a))
    return y, a


def gemv_q8_0_q8_1(W, M: int, K: int, d, q, rows=None):
    """y = W xq for a Q8_0 matrix W and xq = d[k/32] * q[k]; returns (y, sum|w*xq|) in fp64."""
    W = _u8(W)
    if W.size != M * (K // 32) * 34:
        raise ValueError("weight bytes do not match M x K")
    d = np.ascontiguousarray(d, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.int8)
    r, n = _rows(rows, M)
    y = np.zeros(n, np.float64)
    a = np.zeros(n, np.float64)
    lib().or_gemv_q8_0_q8_1(_ptr(W), M, K, _ptr(d), _ptr(q), _ptr(r), n, _ptr(y), _ptr(a))
    return y, a


def topk(z, k: int) -> np.ndarray:
    """Indices of the k best entries, best first (larger value, then lower index;
    NaN counts as -inf)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    if not 1 <= k <= z.size:
        raise ValueError("need 1 <= k <= len(z)")
    out = np.empty(k, np.int64)
    lib().or_topk(_ptr(z), z.size, k, _ptr(out))
    return out


def logsumexp(z) -> float:
    z = np.ascontiguousarray(z, dtype=np.float64)
    return float(lib().or_logsumexp(_ptr(z), z.size))


def sample_topk(z_sorted, temperature: float, top_p: float, min_p: float, u: float) -> int:
    """Position drawn by the sampler chain over the k best logits (best first)."""
    z = np.ascontiguousarray(z_sorted, dtype=np.float64)
    return int(lib().or_sample_topk(_ptr(z), z.size, temperature, top_p, min_p, u))


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the OpenMP loops over rows in later calls (the results do not
    depend on it: each row is computed by one thread, in the same order)."""
    lib().or_set_num_threads(int(n))


def tolerance(a: np.ndarray) -> np.ndarray:
    """Per-output bound |y_gpu - y_ref| <= 1e-3 * sum|w*x| + 1e-6."""
    return 1e-3 * np.asarray(a) + 1e-6
