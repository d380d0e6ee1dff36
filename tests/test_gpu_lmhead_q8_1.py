"""GPU parity of the LM-head batched verification on int8 activations
(lmhead_argmax_verify_q8_1): per column against the oracle's Q8_0 product with the
same quantized activations (scales and quants as the GPU wrote them). The block
products are exact integers and only the per-block fp32 scaling and the fp32
summation round, so the logit tolerance is 1e-5 * sum|w xq| + 1e-6 (as for the
int8-activation Q4_K products). Argmax rule as for the fp32-activation LM head:
when the oracle's top-2 gap exceeds the tolerance the index must be the oracle's,
otherwise one whose oracle logit lies within tolerance of the maximum; the value
returned must be within tolerance of the oracle logit of the returned index."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, case, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu


def quantized_columns(X):
    N, K = X.shape
    xq = qg.quantize_q8_1_columns(to_dev(X))
    nb = qg.q8_1_bytes(K)
    views = []
    for n in range(N):
        d, q, _ = qg.q8_1_views(xq[n * nb:(n + 1) * nb], K)
        views.append((d.cpu().numpy(), q.cpu().numpy()))
    torch.cuda.synchronize()
    return xq, views


def check_verify_q8_1(W, M, K, X, what, ws=None):
    N = X.shape[0]
    case(f"lmhead_argmax_verify_q8_1 {what} M={M} K={K} N={N}")
    wp = packed_q8_0(W, M, K)
    xq, views = quantized_columns(X)
    idx, val = qg.lmhead_argmax_verify_q8_1(wp, xq, M, K, N, ws=ws)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    exact = 0
    for n in range(N):
        d, q = views[n]
        yr, ar = oracle.gemv_q8_0_q8_1(W, M, K, d, q)
        tol = 1e-5 * ar + 1e-6
        gi, ri = int(idx[n]), oracle.argmax(yr)
        assert 0 <= gi < M, (what, n, gi)
        srt = np.sort(yr)
        gap = srt[-1] - srt[-2] if M > 1 else np.inf
        if gap > tol[ri]:
            assert gi == ri, (what, n, gi, ri, gap)
        else:
            assert yr[gi] >= yr[ri] - tol[gi] - tol[ri], (what, n, gi, ri)
        assert abs(float(val[n]) - yr[gi]) <= tol[gi], (what, n, float(val[n]), yr[gi], tol[gi])
        exact += gi == ri
    return exact


@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (200, 256, 5), (1000, 3584, 5), (4097, 512, 8), (63, 1024, 3),
                                   (3000, 768, 2), (17, 4096, 7), (16, 18944, 4), (250, 1280, 6)])
def test_verify_q8_1_small(M, K, N):
    W = workloads.q8_0_blocks(M, K, key=(60, M, K))
    X = workloads.x_columns(K, N, key=(60, M, K, N))
    check_verify_q8_1(W, M, K, X, "small")


@pytest.mark.parametrize("cfg", ["1,0", "4,0"])
@pytest.mark.parametrize("N", [1, 5, 8])
def test_verify_q8_1_launch_shapes(cfg, N):
    # one and four wavefronts per tile, with half macro-block counts that do not
    # divide evenly among the K-groups (K = 2816: 22 halves) and a ragged last tile
    qg.launch_override(verify_waves=int(cfg.split(",")[0])).set()
    M, K = 1000, 2816
    W = workloads.q8_0_blocks(M, K, key=(61, M))
    X = workloads.x_columns(K, N, key=(61, N))
    check_verify_q8_1(W, M, K, X, f"shape {cfg}")


def test_verify_q8_1_constructed_ties_per_column():
    # constant-quant rows, column n = (n + 1) * ones (quantized exactly: scale
    # (n + 1) / 127, quants 127): logit_{r,n} = d K c_r (n + 1) up to the scale's
    # rounding, the same for tied rows; rows 1, 3, 4 tie for the maximum, so every
    # column returns 1
    K, N = 512, 5
    c = np.array([5, 9, -3, 9, 9, 0, 8] * 20)
    M = len(c)
    W = np.stack([np.concatenate([enc.q8_0_block(0x3400, [cr] * 32) for _ in range(K // 32)]) for cr in c])
    X = np.stack([np.full(K, n + 1, np.float32) for n in range(N)])
    case("lmhead_argmax_verify_q8_1 ties")
    xq, views = quantized_columns(X)
    idx, val = qg.lmhead_argmax_verify_q8_1(packed_q8_0(W, M, K), xq, M, K, N)
    assert idx.cpu().tolist() == [1] * N
    for n in range(N):
        yr, ar = oracle.gemv_q8_0_q8_1(W, M, K, *views[n])
        assert abs(float(val[n].item()) - yr[1]) <= 1e-5 * ar[1]


def test_verify_q8_1_winner_in_last_ragged_tile_and_nan_rows():
    # the unique maximum sits in the last row of a ragged tile; a row of NaN
    # scales (fp16 0x7e00) never wins
    M, K, N = 16 * 9 + 3, 256, 4
    W = workloads.q8_0_blocks(M, K, key=(62,)).reshape(M, -1).copy()
    big = np.concatenate([enc.q8_0_block(0x4400, [100] * 32) for _ in range(K // 32)])
    nan = np.concatenate([enc.q8_0_block(0x7E00, [1] * 32) for _ in range(K // 32)])
    W[M - 1] = big
    W[5] = nan
    X = np.abs(workloads.x_columns(K, N, key=(62, 1))) + 0.5
    case("lmhead_argmax_verify_q8_1 ragged winner, NaN row")
    xq, _ = quantized_columns(X)
    idx, _ = qg.lmhead_argmax_verify_q8_1(packed_q8_0(W.reshape(-1), M, K), xq, M, K, N)
    assert idx.cpu().tolist() == [M - 1] * N


def test_verify_q8_1_vocab_152064_n5_matches_fp32_verify():
    """Full LM-head shape, five columns in one pass, the workspace left zero; the
    indices also agree with the fp32-activation verification wherever the
    fp32 oracle's top-2 gap exceeds the activation-quantization error bound."""
    M, K, N = workloads.VOCAB, workloads.HIDDEN, 5
    W = workloads.q8_0_blocks(M, K, key=(4, 0))
    X = workloads.x_columns(K, N, key=(4, 3))
    ws = qg.Workspace(DEV)
    exact = check_verify_q8_1(W, M, K, X, "vocab", ws=ws)
    assert int(ws.buf.count_nonzero()) == 0
    print(f"exact-match rate against the int8-activation oracle {exact}/{N}")
    wp = packed_q8_0(W, M, K)
    i32, _ = qg.lmhead_argmax_verify(wp, to_dev(X), M, K)
    xq, _ = quantized_columns(X)
    i8, _ = qg.lmhead_argmax_verify_q8_1(wp, xq, M, K, N)
    torch.cuda.synchronize()
    agree = 0
    for n in range(N):
        yr, ar = oracle.gemv_q8_0(W, M, K, X[n])
        srt = np.sort(yr)
        same = int(i8[n]) == int(i32[n])
        agree += same
        if srt[-1] - srt[-2] > 2.1 * oracle.tolerance(ar).max():
            assert same, n
    print(f"int8 and fp32 activations pick the same token in {agree}/{N} columns")
