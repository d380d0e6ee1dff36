"""GPU parity in the launch configuration bench.py times: one layer of the 7B decode
step with the benchmark's seeded weights and activations, launched as the benchmark
launches it (one grouped launch per dependency stage: {q,k,v}, {o}, {gate,up},
{down}), for the fp32-activation GEMV (every row of all seven matrices), the int8-
activation GEMV and N = 5 verify product, and the small-N verify product at N = 5, N = 32
and N = 2 (sampled rows)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, assert_within, case, packed_q4k, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _layer(L):
    mats = []
    for i, (name, M, K) in enumerate(workloads.LAYER_MATRICES):
        W = workloads.q4k_blocks(M, K, key=(3, L, i))
        mats.append((name, W, packed_q4k(W, M, K), M, K))
    return mats


@pytest.mark.parametrize("L", [0, 27])
def test_decode_step_layer_as_timed(L):
    mats = _layer(L)
    xs = [workloads.x_vector(K, key=(3, L, i)) for i, (_, _, _, M, K) in enumerate(mats)]
    ys = [torch.full((M,), float("nan"), device=DEV) for (_, _, _, M, _) in mats]
    case(f"qgemv_q4k_batch, layer {L} of the decode step, stage by stage")
    for st in workloads.LAYER_STAGES:
        qg.qgemv_q4k_batch([(mats[i][2], to_dev(xs[i]), ys[i], mats[i][3], mats[i][4]) for i in st])
    torch.cuda.synchronize()
    for i, (name, W, _, M, K) in enumerate(mats):
        yr, ar = oracle.gemv_q4k(W, M, K, xs[i])
        assert_within(ys[i].cpu().numpy(), yr, ar, f"layer {L} {name}")


def test_int8_decode_step_layer_as_timed():
    L = 0
    mats = _layer(L)
    xqs, refs = [], []
    for i, (name, W, _, M, K) in enumerate(mats):
        x = workloads.x_vector(K, key=(3, L, i))
        xq = qg.quantize_q8_1(to_dev(x))
        d, q, _ = (t.cpu().numpy() for t in qg.q8_1_views(xq, K))
        rows = sample_rows(M, 256, seed=M + i)
        refs.append((rows, oracle.gemv_q4k_q8_1(W, M, K, d, q, rows=rows)))
        xqs.append(xq)
    ys = [torch.full((M,), float("nan"), device=DEV) for (_, _, _, M, _) in mats]
    case("qgemv_q4k_q8_1_batch, layer 0 of the decode step, stage by stage")
    for st in workloads.LAYER_STAGES:
        qg.qgemv_q4k_q8_1_batch([(mats[i][2], xqs[i], ys[i], mats[i][3], mats[i][4]) for i in st])
    torch.cuda.synchronize()
    for i, (name, W, _, M, K) in enumerate(mats):
        rows, (yr, ar) = refs[i]
        y = ys[i].cpu().numpy()[rows]
        assert np.all(np.abs(y - yr) <= 1e-5 * ar + 1e-6), f"int8 layer 0 {name}"


def test_int8_verify_step_layer_as_timed():
    # the N = 5 verify step on int8 activations, as the benchmark launches it
    L, N = 0, 5
    mats = _layer(L)
    xqs, refs = [], []
    for i, (name, W, _, M, K) in enumerate(mats):
        X = workloads.x_columns(K, N, key=(5, L, i, N))
        xq = qg.quantize_q8_1_columns(to_dev(X))
        nb = qg.q8_1_bytes(K)
        rows = sample_rows(M, 96, seed=M + K + i)
        cols = []
        for n in range(N):
            d, q, _ = (t.cpu().numpy() for t in qg.q8_1_views(xq[n * nb:(n + 1) * nb], K))
            cols.append(oracle.gemv_q4k_q8_1(W, M, K, d, q, rows=rows))
        refs.append((rows, cols))
        xqs.append(xq)
    Ys = [torch.full((N, (M + 3) // 4 * 4), float("nan"), device=DEV) for (_, _, _, M, _) in mats]
    case("qgemm_q4k_q8_1_smalln_batch N=5, layer 0 of the verify step, stage by stage")
    for st in workloads.LAYER_STAGES:
        qg.qgemm_q4k_q8_1_smalln_batch([(mats[i][2], xqs[i], Ys[i], mats[i][3], mats[i][4]) for i in st])
    torch.cuda.synchronize()
    for i, (name, W, _, M, K) in enumerate(mats):
        rows, cols = refs[i]
        Y = Ys[i].cpu().numpy()[:, :M][:, rows]
        for n, (yr, ar) in enumerate(cols):
            assert np.all(np.abs(Y[n] - yr) <= 1e-5 * ar + 1e-6), f"int8 verify layer 0 {name} col {n}"


@pytest.mark.parametrize("N", [5, 32, 2])
def test_verify_step_layer_as_timed(N):
    L = 0
    mats = _layer(L)
    Xs = [workloads.x_columns(K, N, key=(5, L, i, N)) for i, (_, _, _, M, K) in enumerate(mats)]
    Ys = [torch.full((N, (M + 3) // 4 * 4), float("nan"), device=DEV) for (_, _, _, M, _) in mats]
    case(f"qgemm_q4k_smalln_batch N={N}, layer 0 of the verify step, stage by stage")
    for st in workloads.LAYER_STAGES:
        qg.qgemm_q4k_smalln_batch([(mats[i][2], to_dev(Xs[i]), Ys[i], mats[i][3], mats[i][4]) for i in st])
    torch.cuda.synchronize()
    for i, (name, W, _, M, K) in enumerate(mats):
        rows = sample_rows(M, 160, seed=M + K + N)
        Yr, Ar = oracle.gemm_q4k(W, M, K, Xs[i], rows=rows)
        Y = Ys[i].cpu().numpy()[:, :M][:, rows]
        for n in range(N):
            assert_within(Y[n], Yr[n], Ar[n], f"verify N={N} {name} col {n}")
