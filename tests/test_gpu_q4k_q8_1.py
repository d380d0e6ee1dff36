"""GPU parity of the int8-activation path: qg_quantize_q8_1 against the oracle's
quantization (bit-exact: both take the integer decisions in float32), and
qgemv_q4k_q8_1 against the oracle's product with the same quantized activations
(tight bound: the integer dot products are exact, only the per-sub-block float
scaling rounds: 1e-5 * sum|w xq| + 1e-6, about ten times the worst fp32 rounding
of those scalings and sums) and, at K >= 3584 (the decode shapes), against the
fp32-activation product within the usual 1e-3 * sum|w x| + 1e-6 bound."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, assert_within, case, packed_q4k, to_dev
from tests.test_oracle_pins import _golden_q8_1

pytestmark = pytest.mark.gpu


def gpu_quantize(x):
    K = x.size
    xq = qg.quantize_q8_1(to_dev(x))
    d, q, s = qg.q8_1_views(xq, K)
    torch.cuda.synchronize()
    return xq, d.cpu().numpy(), q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("K,scale", [(256, 1.0), (3584, 1.0), (18944, 1e-3), (4096, 300.0), (512, 0.0)])
def test_quantize_bit_exact(K, scale):
    x = (workloads.x_vector(K, key=(60, K)) * scale).astype(np.float32)
    case(f"qg_quantize_q8_1 K={K} scale={scale}")
    _, d, q, bs = gpu_quantize(x)
    dr, qr, bsr = oracle.quantize_q8_1(x)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))
    assert np.array_equal(q, qr)
    assert np.array_equal(bs, bsr)


def test_quantize_golden_blocks():
    G = _golden_q8_1()
    x = np.concatenate([G[n]["x"] for n in ("A", "B", "C")])
    case("qg_quantize_q8_1 golden blocks")
    _, d, q, s = gpu_quantize(x)
    for b, n in enumerate(("A", "B", "C")):
        assert d[8 * b:8 * b + 8].astype(np.float64).tolist() == G[n]["d"]
        assert q[256 * b:256 * b + 256].astype(np.int64).tolist() == G[n]["q"].tolist()
        assert s[8 * b:8 * b + 8].astype(np.int64).tolist() == G[n]["s"]


def run(M, K, key, x=None):
    W = workloads.q4k_blocks(M, K, key=key)
    x = workloads.x_vector(K, key=key) if x is None else x
    case(f"qgemv_q4k_q8_1 M={M} K={K} key={key}")
    wp = packed_q4k(W, M, K)
    xq, d, q, _ = gpu_quantize(x)
    y = qg.qgemv_q4k_q8_1(wp, xq, M, K).cpu().numpy()
    yq, aq = oracle.gemv_q4k_q8_1(W, M, K, d, q)
    assert np.all(np.abs(y - yq) <= 1e-5 * aq + 1e-6), f"M={M} K={K}: {np.max(np.abs(y - yq) / (1e-5 * aq + 1e-6))}"
    yf, af = oracle.gemv_q4k(W, M, K, x)
    return y, yf, af


@pytest.mark.parametrize("M,K", [(1, 256), (3, 256), (63, 512), (65, 512), (200, 3584), (130, 18944),
                                 (700, 1024), (129, 4096), (4096, 4096)])
def test_shapes(M, K):
    y, yf, af = run(M, K, key=(61, M, K))
    r = np.max(np.abs(y - yf) / oracle.tolerance(af))
    print(f"M={M} K={K}: max |y - y(fp32 x)| / tol = {r:.3f}")
    if K >= 3584:
        assert_within(y, yf, af, f"q4k_q8_1 M={M} K={K} vs fp32 activations")


@pytest.mark.parametrize("name,M,K", [m for m in workloads.LAYER_MATRICES])
def test_7b_layer_shapes_all_rows(name, M, K):
    y, yf, af = run(M, K, key=(62, workloads.LAYER_MATRICES.index((name, M, K))))
    print(name, "max err/tol vs fp32 activations", assert_within(y, yf, af, f"q4k_q8_1 {name}"))


def test_exact_integer_case():
    # d = 1, dmin = 0, unit sub-scales and activations k/8 with 127/8 in every block
    # of 32: y = (Q @ k) / 8 exactly
    M, K = 21, 768
    rng = np.random.default_rng(63)
    Q = rng.integers(0, 16, (M, K))
    W = np.stack([np.concatenate([enc.q4k_block(0x3C00, 0, [1] * 8, [0] * 8, Q[r, 256 * b:256 * b + 256])
                                  for b in range(K // 256)]) for r in range(M)])
    k = rng.integers(-127, 128, K)
    k[::32] = 127
    case("qgemv_q4k_q8_1 exact integer case")
    xq = qg.quantize_q8_1(to_dev((k / 8).astype(np.float32)))
    y = qg.qgemv_q4k_q8_1(packed_q4k(W, M, K), xq, M, K).cpu().numpy()
    assert np.array_equal(y.astype(np.float64) * 8, (Q @ k).astype(np.float64))


def test_zero_activations_give_zero():
    M, K = 100, 1024
    W = workloads.q4k_blocks(M, K, key=(64,))
    case("qgemv_q4k_q8_1 zero x")
    xq = qg.quantize_q8_1(torch.zeros(K, device=DEV))
    y = qg.qgemv_q4k_q8_1(packed_q4k(W, M, K), xq, M, K)
    assert torch.all(y == 0)


@pytest.mark.parametrize("cfg", ["1", "2", "4", "8"])
def test_launch_shapes(cfg):
    qg.launch_override(gemv_waves=int(cfg)).set()
    for M, K in [(35, 1024), (33, 9472)]:
        run(M, K, key=(65, M, int(cfg)))


def test_deterministic():
    M, K = 3584, 18944
    W = workloads.q4k_blocks(M, K, key=(66,))
    wp = packed_q4k(W, M, K)
    case("qgemv_q4k_q8_1 determinism")
    xq = qg.quantize_q8_1(to_dev(workloads.x_vector(K, key=(66,))))
    y1 = qg.qgemv_q4k_q8_1(wp, xq, M, K).clone()
    y2 = qg.qgemv_q4k_q8_1(wp, xq, M, K).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_batch_matches_single_calls():
    # the attention-input stage (Wq, Wk, Wv on one quantized x) and a ragged problem
    # with its own activations, in one launch; each output matches the oracle's
    # quantized product, and the three 3584-column ones equal their single calls bit
    # for bit (same launch shape, same per-row arithmetic)
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (77, 768)]
    x0 = workloads.x_vector(3584, key=(67, 0))
    xq0 = qg.quantize_q8_1(to_dev(x0))
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(67, i))
        if K == 3584:
            xq, x = xq0, x0
        else:
            x = workloads.x_vector(K, key=(67, i))
            xq = qg.quantize_q8_1(to_dev(x))
        probs.append((packed_q4k(W, M, K), xq, torch.full((M,), float("nan"), device=DEV), M, K))
        refs.append((W, x))
    case("qgemv_q4k_q8_1_batch")
    qg.qgemv_q4k_q8_1_batch(probs)
    torch.cuda.synchronize()
    for (w, xq, y, M, K), (W, x) in zip(probs, refs):
        if K == 3584:
            single = qg.qgemv_q4k_q8_1(w, xq, M, K)
            torch.cuda.synchronize()
            assert torch.equal(y, single), f"M={M} K={K}"
        d, q, _ = oracle.quantize_q8_1(x)
        yq, aq = oracle.gemv_q4k_q8_1(W, M, K, d, q)
        assert np.all(np.abs(y.cpu().numpy() - yq) <= 1e-5 * aq + 1e-6)
