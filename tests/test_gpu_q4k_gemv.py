"""GPU parity of the Q4_K GEMV (and its repack) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, assert_within, case, packed_q4k, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def run_q4k(M, K, key, rows=None, x=None):
    W = workloads.q4k_blocks(M, K, key=key)
    x = workloads.x_vector(K, key=key) if x is None else x
    case(f"qgemv_q4k M={M} K={K} key={key}")
    wp = packed_q4k(W, M, K)
    y = qg.qgemv_q4k(wp, to_dev(x), M, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    yr, ar = oracle.gemv_q4k(W, M, K, x, rows=rows)
    return (y if rows is None else y[rows]), yr, ar


@pytest.mark.parametrize("M,K", [(1, 256), (3, 256), (63, 512), (64, 256), (65, 512), (200, 3584),
                                 (512, 3584), (130, 18944), (700, 1024), (129, 4096)])
def test_small_and_ragged_shapes(M, K):
    y, yr, ar = run_q4k(M, K, key=(10, M, K))
    assert_within(y, yr, ar, f"q4k M={M} K={K}")


def test_config1_4096x4096_all_rows():
    y, yr, ar = run_q4k(4096, 4096, key=(1, 0))
    r = assert_within(y, yr, ar, "q4k 4096x4096")
    print("max err/tol", r)


@pytest.mark.parametrize("name,M,K", [m for m in workloads.LAYER_MATRICES])
def test_7b_layer_shapes_all_rows(name, M, K):
    y, yr, ar = run_q4k(M, K, key=(3, 0, workloads.LAYER_MATRICES.index((name, M, K))))
    assert_within(y, yr, ar, f"q4k {name}")


def test_closed_form_blocks_exact():
    # rows made of the hand-built blocks A, B, C; with x = 1 every output is the
    # block sums, exact in fp32 (integers and multiples of 2^-6 far below 2^24)
    G = enc.golden()
    M, K = 70, 768
    rows = []
    for r in range(M):
        names = [["A", "B", "C"][(r + b) % 3] for b in range(3)]
        rows.append(np.concatenate([G[n]["block"] for n in names]))
    W = np.stack(rows)
    expect = np.array([sum(G[["A", "B", "C"][(r + b) % 3]]["sum"] for b in range(3)) for r in range(M)])
    case("qgemv_q4k closed-form blocks")
    wp = packed_q4k(W, M, K)
    y = qg.qgemv_q4k(wp, to_dev(np.ones(K, np.float32)), M, K).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), expect)
    # x = e_k picks column k: exact weights
    for k in (0, 37, 255, 256 + 15, 512 + 96, 767):
        e = np.zeros(K, np.float32)
        e[k] = 1
        y = qg.qgemv_q4k(wp, to_dev(e), M, K).cpu().numpy()
        wref = oracle.q4k_dequant(W, M, K)[:, k]
        assert np.array_equal(y.astype(np.float64), wref), k


def test_zero_scales_give_exact_zero():
    M, K = 130, 1024
    W = workloads.q4k_blocks(M, K, key=(11,)).reshape(M, K // 256, 144).copy()
    W[:, :, 0:4] = 0
    case("qgemv_q4k zero scales")
    wp = packed_q4k(W.reshape(M, -1), M, K)
    y = qg.qgemv_q4k(wp, to_dev(workloads.x_vector(K, key=(11,))), M, K).cpu().numpy()
    assert np.all(y == 0)


def test_deterministic():
    M, K = 3584, 3584
    W = workloads.q4k_blocks(M, K, key=(12,))
    x = to_dev(workloads.x_vector(K, key=(12,)))
    case("qgemv_q4k determinism")
    wp = packed_q4k(W, M, K)
    y1 = qg.qgemv_q4k(wp, x, M, K).clone()
    y2 = qg.qgemv_q4k(wp, x, M, K).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_pack_is_a_permutation():
    M, K = 131, 768
    W = workloads.q4k_blocks(M, K, key=(13,))
    case("qg_pack_q4k permutation")
    p = packed_q4k(W, M, K).cpu().numpy()
    assert p.size == W.size
    assert np.array_equal(np.sort(p), np.sort(W.reshape(-1)))
    # segment 0 of super-block 0 of row i of tile 0 is bytes 0..15 of that row
    assert np.array_equal(p[16 * 5:16 * 6], W[5, :16])
    # segment 1 of super-block 0 of row 3 of tile 0 (16 rows): offset (1 * 16 + 3) * 16
    assert np.array_equal(p[16 * 19:16 * 20], W[3, 16:32])


def test_batch_matches_oracle_per_problem():
    # the attention-input stage of a 7B layer: Wq, Wk, Wv in one launch, plus a ragged problem
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (77, 768)]
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(14, i))
        x = workloads.x_vector(K, key=(14, i))
        probs.append((packed_q4k(W, M, K), to_dev(x), torch.empty(M, device=DEV), M, K))
        refs.append(oracle.gemv_q4k(W, M, K, x))
    case("qgemv_q4k_batch")
    qg.qgemv_q4k_batch(probs)
    torch.cuda.synchronize()
    for (w, x, y, M, K), (yr, ar) in zip(probs, refs):
        assert_within(y.cpu().numpy(), yr, ar, f"batch M={M} K={K}")
