"""GPU parity at the size limits of every entry point: the largest K the C ABI
accepts (2^24, one row of 64 Mi weights), long K walks through the pipelined
loops, and the largest-M shapes (vocabulary-sized outputs), each against the
fp64 oracle with the same bounds as the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, assert_within, case, packed_q4k, packed_q8_0, sample_rows, to_dev
from tests.test_gpu_q8_0_lmhead import check_argmax, check_verify

pytestmark = pytest.mark.gpu

K_MAX = 1 << 24


@pytest.mark.parametrize("M,K", [(3, K_MAX), (40, 262144)])
def test_q4k_gemv_long_k(M, K):
    W = workloads.q4k_blocks(M, K, key=(70, M, K))
    x = workloads.x_vector(K, key=(70, M, K))
    case(f"qgemv_q4k M={M} K={K}")
    y = qg.qgemv_q4k(packed_q4k(W, M, K), to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q4k(W, M, K, x)
    assert_within(y, yr, ar, f"q4k M={M} K={K}")


def test_q4k_gemv_vocab_rows():
    # the output head of a Q4_K model: 152064 rows, sampled against the oracle
    M, K = 152064, 3584
    W = workloads.q4k_blocks(M, K, key=(71,))
    x = workloads.x_vector(K, key=(71,))
    rows = sample_rows(M, 1500, seed=71)
    case(f"qgemv_q4k M={M} K={K}")
    y = qg.qgemv_q4k(packed_q4k(W, M, K), to_dev(x), M, K).cpu().numpy()[rows]
    yr, ar = oracle.gemv_q4k(W, M, K, x, rows=rows)
    assert_within(y, yr, ar, "q4k vocab rows")


@pytest.mark.parametrize("M,K", [(3, K_MAX), (17, 1 << 20)])
def test_q8_0_gemv_long_k(M, K):
    W = workloads.q8_0_blocks(M, K, key=(72, M, K))
    x = workloads.x_vector(K, key=(72, M, K))
    case(f"qgemv_q8_0 M={M} K={K}")
    y = qg.qgemv_q8_0(packed_q8_0(W, M, K), to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    assert_within(y, yr, ar, f"q8_0 M={M} K={K}")


def test_q8_0_gemv_long_k_with_tail_blocks():
    # K/32 not a multiple of 8: the canonical tail blocks after the macro-blocks
    M, K = 5, (1 << 20) + 96
    W = workloads.q8_0_blocks(M, K, key=(73,))
    x = workloads.x_vector(K, key=(73,))
    case(f"qgemv_q8_0 M={M} K={K}")
    y = qg.qgemv_q8_0(packed_q8_0(W, M, K), to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    assert_within(y, yr, ar, f"q8_0 tail M={M} K={K}")


@pytest.mark.parametrize("M,K", [(3, K_MAX), (20, 1 << 20)])
def test_q6k_gemv_long_k(M, K):
    W = workloads.q6k_blocks(M, K, key=(74, M, K))
    x = workloads.x_vector(K, key=(74, M, K))
    case(f"qgemv_q6k M={M} K={K}")
    y = qg.qgemv_q6k(qg.pack_q6k(to_dev(W.reshape(-1)), M, K), to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q6k(W, M, K, x)
    assert_within(y, yr, ar, f"q6k M={M} K={K}")


@pytest.mark.parametrize("M,K", [(3, K_MAX), (20, 1 << 20)])
def test_q4k_q8_1_long_k(M, K):
    W = workloads.q4k_blocks(M, K, key=(75, M, K))
    x = workloads.x_vector(K, key=(75, M, K))
    case(f"qgemv_q4k_q8_1 M={M} K={K}")
    xq = qg.quantize_q8_1(to_dev(x))
    y = qg.qgemv_q4k_q8_1(packed_q4k(W, M, K), xq, M, K).cpu().numpy()
    d, q, _ = oracle.quantize_q8_1(x)
    yq, aq = oracle.gemv_q4k_q8_1(W, M, K, d, q)
    assert np.all(np.abs(y - yq) <= 1e-5 * aq + 1e-6)
    yr, ar = oracle.gemv_q4k(W, M, K, x)
    assert_within(y, yr, ar, f"q4k_q8_1 vs fp32 activations M={M} K={K}")


@pytest.mark.parametrize("N", [5, 32])
def test_smalln_long_k(N):
    M, K = 20, 1 << 20
    W = workloads.q4k_blocks(M, K, key=(76, N))
    X = workloads.x_columns(K, N, key=(76, N))
    case(f"qgemm_q4k_smalln M={M} K={K} N={N}")
    Y = qg.qgemm_q4k_smalln(packed_q4k(W, M, K), to_dev(X), M, K).cpu().numpy()[:, :M]
    Yr, Ar = oracle.gemm_q4k(W, M, K, X)
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"smalln long K col {n}")


def test_lmhead_argmax_long_k():
    M, K = 100, 1 << 20
    W = workloads.q8_0_blocks(M, K, key=(77,))
    x = workloads.x_vector(K, key=(77,))
    check_argmax(W, M, K, x, "long K")


def test_verify_long_k():
    M, K, N = 100, 1 << 20, 5
    W = workloads.q8_0_blocks(M, K, key=(78,))
    X = workloads.x_columns(K, N, key=(78,))
    check_verify(W, M, K, X, "long K")


def test_topk_largest_vocabulary_and_k():
    M = qg.QG_TOPK_MAX_ROWS if hasattr(qg, "QG_TOPK_MAX_ROWS") else 262144
    z = (np.random.default_rng(79).standard_normal(M) * 2).astype(np.float32)
    case(f"logits_topk M={M} k=64")
    out = qg.logits_topk(to_dev(z), 64)
    torch.cuda.synchronize()
    assert out.index.cpu().tolist() == oracle.topk(z.astype(np.float64), 64).tolist()
