"""GPU parity of the int8-activation small-N product (qgemm_q4k_q8_1_smalln, N <= 8
quantized columns, one pass over the weights): per column against the oracle's
product with the same quantized activations (tight bound: the integer dots are
exact, only the per-sub-block float scaling rounds: 1e-5 * sum|w xq| + 1e-6, as for
qgemv_q4k_q8_1), bit for bit against qgemv_q4k_q8_1 of each column where that kernel
also runs four wavefronts per tile (K >= 2304), and at the decode shapes against
the fp32-activation product within 1e-3 * sum|w x| + 1e-6."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, assert_within, case, packed_q4k, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def quantized_columns(X):
    """Device buffer of the N quantized columns, and per column the oracle's view
    (scales d and quants q as the GPU wrote them)."""
    N, K = X.shape
    xq = qg.quantize_q8_1_columns(to_dev(X))
    nb = qg.q8_1_bytes(K)
    views = []
    for n in range(N):
        d, q, _ = qg.q8_1_views(xq[n * nb:(n + 1) * nb], K)
        views.append((d.cpu().numpy(), q.cpu().numpy()))
    torch.cuda.synchronize()
    return xq, views


def check_columns(W, M, K, X, Y, views, rows=None):
    for n in range(X.shape[0]):
        d, q = views[n]
        yq, aq = oracle.gemv_q4k_q8_1(W, M, K, d, q, rows=rows)
        y = Y[n] if rows is None else Y[n][rows]
        bad = ~(np.abs(y - yq) <= 1e-5 * aq + 1e-6)
        assert not bad.any(), f"M={M} K={K} col {n}: {int(bad.sum())} outputs beyond 1e-5 * sum|w xq|"


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("M,K", [(200, 512), (65, 3328), (48, 9984), (1, 256)])
def test_int8_smalln_shapes(M, K, N):
    W = workloads.q4k_blocks(M, K, key=(45, M, K, N))
    X = workloads.x_columns(K, N, key=(45, M, K, N))
    case(f"qgemm_q4k_q8_1_smalln M={M} K={K} N={N}")
    wp = packed_q4k(W, M, K)
    xq, views = quantized_columns(X)
    Y = qg.qgemm_q4k_q8_1_smalln(wp, xq, M, K, N)
    torch.cuda.synchronize()
    check_columns(W, M, K, X, Y.cpu().numpy()[:, :M], views)


@pytest.mark.parametrize("M,K", [(3584, 3584), (3584, 18944), (700, 2304)])
def test_int8_smalln_columns_bit_exact_with_gemv(M, K):
    N = 5
    W = workloads.q4k_blocks(M, K, key=(46, M, K))
    X = workloads.x_columns(K, N, key=(46, M, K))
    case(f"int8 small-N vs qgemv_q4k_q8_1 M={M} K={K} N={N}")
    wp = packed_q4k(W, M, K)
    xq, views = quantized_columns(X)
    Y = qg.qgemm_q4k_q8_1_smalln(wp, xq, M, K, N)
    nb = qg.q8_1_bytes(K)
    torch.cuda.synchronize()
    for n in range(N):
        y = qg.qgemv_q4k_q8_1(wp, xq[n * nb:(n + 1) * nb], M, K)
        torch.cuda.synchronize()
        assert np.array_equal(Y[n, :M].cpu().numpy(), y.cpu().numpy()), f"column {n}"
    rows = sample_rows(M, 64, seed=K)
    Yc = Y.cpu().numpy()[:, :M]
    check_columns(W, M, K, X, Yc, views, rows=rows)
    # the quantization stays within the fp32-activation bound at these shapes
    Yr, Ar = oracle.gemm_q4k(W, M, K, X, rows=rows)
    for n in range(N):
        assert_within(Yc[n][rows], Yr[n], Ar[n], f"int8 small-N vs fp32 product M={M} K={K} col {n}")


def test_int8_smalln_batch_mixed_columns():
    # one launch over problems with different N and padded output rows; the padding
    # stays untouched
    shapes = [(530, 4096, 8), (77, 256, 1), (16, 3584, 5), (1000, 1280, 3), (33, 18944, 2)]
    probs, refs = [], []
    for i, (M, K, N) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(47, i))
        X = workloads.x_columns(K, N, key=(47, i, N))
        xq, views = quantized_columns(X)
        Y = torch.full((N, (M + 3) // 4 * 4 + 4), float("nan"), device=DEV)
        probs.append((packed_q4k(W, M, K), xq, Y, M, K))
        refs.append((W, X, views))
    case("qgemm_q4k_q8_1_smalln_batch, mixed N")
    qg.qgemm_q4k_q8_1_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, xq, Y, M, K), (W, X, views) in zip(probs, refs):
        Yc = Y.cpu().numpy()
        assert np.all(np.isnan(Yc[:, M:])), "padding rows were written"
        check_columns(W, M, K, X, Yc[:, :M], views)


def test_int8_smalln_validation():
    W = workloads.q4k_blocks(64, 512, key=(48,))
    wp = packed_q4k(W, 64, 512)
    xq = torch.zeros(9 * qg.q8_1_bytes(512), dtype=torch.uint8, device=DEV)
    with pytest.raises(qg.QGError) as e:  # more than eight columns
        qg.qgemm_q4k_q8_1_smalln(wp, xq, 64, 512, 9)
    assert e.value.status == 2
    with pytest.raises(qg.QGError) as e:  # K not a multiple of 256
        qg.qgemm_q4k_q8_1_smalln(wp, xq, 64, 500, 2)
    assert e.value.status == 2
