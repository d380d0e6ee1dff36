"""GPU parity of the Q6_K GEMV (and its repack) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, assert_within, case, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def packed_q6k(W: np.ndarray, M: int, K: int) -> torch.Tensor:
    return qg.pack_q6k(to_dev(W.reshape(-1)), M, K)


def run_q6k(M, K, key, rows=None, x=None):
    W = workloads.q6k_blocks(M, K, key=key)
    x = workloads.x_vector(K, key=key) if x is None else x
    case(f"qgemv_q6k M={M} K={K} key={key}")
    wp = packed_q6k(W, M, K)
    y = qg.qgemv_q6k(wp, to_dev(x), M, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    yr, ar = oracle.gemv_q6k(W, M, K, x, rows=rows)
    return (y if rows is None else y[rows]), yr, ar


# one super-block (MODE 0 with idle K-groups), several per K-group (pair loop,
# odd and even counts), ragged last tiles, and the 7B Q6_K shapes
@pytest.mark.parametrize("M,K", [(1, 256), (3, 256), (15, 512), (16, 256), (17, 768), (63, 4096),
                                 (200, 3584), (130, 18944), (700, 1024), (129, 9216), (512, 3584)])
def test_small_and_ragged_shapes(M, K):
    y, yr, ar = run_q6k(M, K, key=(20, M, K))
    assert_within(y, yr, ar, f"q6k M={M} K={K}")


def test_ffn_down_3584x18944_all_rows():
    y, yr, ar = run_q6k(3584, 18944, key=(21,))
    print("max err/tol", assert_within(y, yr, ar, "q6k ffn_down"))


def test_output_head_152064x3584_sampled_rows():
    M, K = 152064, 3584
    rows = sample_rows(M, 1500, seed=22)
    y, yr, ar = run_q6k(M, K, key=(22,), rows=rows)
    print("max err/tol", assert_within(y, yr, ar, "q6k output head"))


def _golden_matrix(M, nbk):
    G = enc.golden_q6k()
    names = sorted(G)
    rows, sums = [], []
    for r in range(M):
        pick = [names[(r + b) % len(names)] for b in range(nbk)]
        rows.append(np.concatenate([G[n]["block"] for n in pick]))
        sums.append(sum(G[n]["sum"] for n in pick))
    return G, names, np.stack(rows), np.array(sums)


def test_golden_blocks_closed_form_exact():
    # rows made of the hand-derived blocks; with x = 1 each output is the sum of
    # its blocks' weights, exact in fp32 (small integers and halves)
    M, nbk = 37, 3
    K = 256 * nbk
    G, names, W, expect = _golden_matrix(M, nbk)
    case("qgemv_q6k golden blocks")
    wp = packed_q6k(W, M, K)
    y = qg.qgemv_q6k(wp, to_dev(np.ones(K, np.float32)), M, K).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), expect)
    # x = e_k picks column k: the listed weights of the golden blocks, exactly
    for r in (0, 1, 17, 36):
        for b in range(nbk):
            g = G[names[(r + b) % len(names)]]
            for k, wv in g["w"].items():
                e = np.zeros(K, np.float32)
                e[256 * b + k] = 1
                y = qg.qgemv_q6k(wp, to_dev(e), M, K).cpu().numpy()
                assert y[r] == wv, (r, b, k, y[r], wv)


def test_unit_columns_exact():
    # every weight d * sc * (q - 32) is exact in fp32 (11-bit d times a 13-bit
    # integer), and x = e_k makes the product that weight
    M, K = 40, 512
    W = workloads.q6k_blocks(M, K, key=(23,))
    wref = oracle.q6k_dequant(W, M, K)
    case("qgemv_q6k unit columns")
    wp = packed_q6k(W, M, K)
    for k in (0, 1, 15, 16, 31, 32, 63, 64, 95, 127, 128, 191, 255, 256, 300, 383, 448, 511):
        e = np.zeros(K, np.float32)
        e[k] = 1
        y = qg.qgemv_q6k(wp, to_dev(e), M, K).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), wref[:, k]), k


def test_encoded_weights_match():
    # blocks written by the independent encoder from random parameters: the GPU
    # result matches the product with the parameter-built weights
    rng = np.random.default_rng(24)
    M, nbk = 19, 2
    K = 256 * nbk
    rows, wrows = [], []
    for _ in range(M):
        blks, ws = [], []
        for _ in range(nbk):
            d = np.float16(rng.uniform(0.001, 0.05))
            sc = rng.integers(-128, 128, 16)
            q = rng.integers(0, 64, 256)
            blks.append(enc.q6k_block(int(d.view(np.uint16)), sc, q))
            ws.append(enc.q6k_weights(float(d), sc, q))
        rows.append(np.concatenate(blks))
        wrows.append(np.concatenate(ws))
    W, Wf = np.stack(rows), np.stack(wrows)
    x = workloads.x_vector(K, key=(24,))
    case("qgemv_q6k encoder blocks")
    y = qg.qgemv_q6k(packed_q6k(W, M, K), to_dev(x), M, K).cpu().numpy()
    yr = Wf @ x.astype(np.float64)
    assert_within(y, yr, np.abs(Wf) @ np.abs(x.astype(np.float64)), "q6k encoder")


def test_zero_d_gives_exact_zero():
    M, K = 70, 1024
    W = workloads.q6k_blocks(M, K, key=(25,)).reshape(M, K // 256, 210).copy()
    W[:, :, 208:210] = 0
    case("qgemv_q6k zero d")
    y = qg.qgemv_q6k(packed_q6k(W.reshape(M, -1), M, K), to_dev(workloads.x_vector(K, key=(25,))), M, K)
    assert torch.all(y == 0)


def test_deterministic():
    M, K = 3584, 18944
    W = workloads.q6k_blocks(M, K, key=(26,))
    x = to_dev(workloads.x_vector(K, key=(26,)))
    case("qgemv_q6k determinism")
    wp = packed_q6k(W, M, K)
    y1 = qg.qgemv_q6k(wp, x, M, K).clone()
    y2 = qg.qgemv_q6k(wp, x, M, K).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("cfg", ["1", "2", "4", "8"])
def test_launch_shapes(cfg):
    # every wavefront count per workgroup, in both the single-super-block and
    # the pair-loop forms
    qg.launch_override(gemv_waves=int(cfg)).set()
    for M, K in [(35, 1024), (33, 9472)]:
        y, yr, ar = run_q6k(M, K, key=(27, M, int(cfg)))
        assert_within(y, yr, ar, f"q6k cfg={cfg} M={M} K={K}")


@pytest.mark.parametrize("M,K", [(5, 512), (37, 768)])
def test_pack_layout(M, K):
    W = workloads.q6k_blocks(M, K, key=(28, M))
    case(f"qg_pack_q6k layout M={M}")
    p = packed_q6k(W, M, K).cpu().numpy()
    assert p.size == W.size
    assert np.array_equal(np.sort(p), np.sort(W.reshape(-1)))
    nb = K // 256
    for t in range((M + 15) // 16):
        rt = min(16, M - 16 * t)
        base = t * 16 * nb * 210
        for i in range(rt):
            r = 16 * t + i
            for b in range(nb):
                for s in range(13):
                    o = base + ((b * 13 + s) * rt + i) * 16
                    assert np.array_equal(p[o:o + 16], W[r, b * 210 + 16 * s:b * 210 + 16 * s + 16]), (r, b, s)
                o = base + nb * 13 * rt * 16 + (b * rt + i) * 2
                assert np.array_equal(p[o:o + 2], W[r, b * 210 + 208:b * 210 + 210]), (r, b)
