"""Shared helpers of the GPU parity tests: upload + pack, the oracle comparison
with the |y_gpu - y_ref| <= 1e-3 * sum|w*x| + 1e-6 bound, and case logging."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import quantized_gemv_argmax_amd as qg

DEV = "cuda:0"


def case(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def packed_q4k(W: np.ndarray, M: int, K: int) -> torch.Tensor:
    canon = to_dev(W.reshape(-1))
    return qg.pack_q4k(canon, M, K)


def packed_q8_0(W: np.ndarray, M: int, K: int) -> torch.Tensor:
    canon = to_dev(W.reshape(-1))
    return qg.pack_q8_0(canon, M, K)


def assert_within(y_gpu, y_ref, a_ref, what: str) -> float:
    """Element-wise bound check; returns the worst |err| / tol ratio."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = oracle.tolerance(a_ref)
    bad = np.flatnonzero(~(err <= tol))
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} outputs out of tolerance; first at {i}: gpu={y_gpu[i]!r} "
                             f"ref={y_ref[i]!r} err={err[i]:.3e} tol={tol[i]:.3e}")
    return float((err / tol).max()) if err.size else 0.0


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """First and last tiles' edge rows plus n random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 65, M // 2, M - 65, M - 64, M - 2, M - 1]
    rows = np.concatenate([np.array([r for r in fixed if 0 <= r < M]), rng.integers(0, M, n)])
    return np.unique(rows)
