"""GPU parity of the Q8_0 GEMV and the fused LM-head argmax against the oracle.

Argmax rule: when the oracle's top-2 gap exceeds the float tolerance of the
winning row, the GPU index must equal the oracle's; otherwise it must be one of
the rows whose oracle logit lies within tolerance of the maximum. The value
returned must be within tolerance of the oracle logit of the returned index.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, assert_within, case, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 32), (5, 64), (64, 256), (65, 288), (130, 4096), (200, 928),
                                 (11008, 4096), (4096, 11008), (333, 3584)])
def test_q8_0_gemv(M, K):
    W = workloads.q8_0_blocks(M, K, key=(20, M, K))
    x = workloads.x_vector(K, key=(20, M, K))
    case(f"qgemv_q8_0 M={M} K={K}")
    wp = packed_q8_0(W, M, K)
    y = qg.qgemv_q8_0(wp, to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    assert_within(y, yr, ar, f"q8_0 M={M} K={K}")


def test_q8_0_integer_exact():
    # d = 1, integer x: every partial sum is an integer below 2^24 -> exact
    rng = np.random.default_rng(21)
    M, K = 70, 512
    Q = rng.integers(-127, 128, (M, K))
    W = np.stack([np.concatenate([enc.q8_0_block(0x3C00, Q[r, 32 * b:32 * (b + 1)]) for b in range(K // 32)])
                  for r in range(M)])
    xi = rng.integers(-20, 21, K)
    case("qgemv_q8_0 integer exact")
    y = qg.qgemv_q8_0(packed_q8_0(W, M, K), to_dev(xi.astype(np.float32)), M, K).cpu().numpy()
    assert np.array_equal(y.astype(np.int64), Q @ xi)


def check_argmax(W, M, K, x, what):
    case(f"lmhead_argmax {what} M={M} K={K}")
    wp = packed_q8_0(W, M, K)
    idx, val = qg.lmhead_argmax(wp, to_dev(x), M, K)
    torch.cuda.synchronize()
    gi, gv = int(idx.item()), float(val.item())
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    ri = oracle.argmax(yr)
    tol = oracle.tolerance(ar)
    srt = np.sort(yr)
    gap = srt[-1] - srt[-2] if M > 1 else np.inf
    if gap > tol[ri]:
        assert gi == ri, (what, gi, ri, gap)
    else:
        assert yr[gi] >= yr[ri] - tol[gi] - tol[ri], (what, gi, ri)
    assert abs(gv - yr[gi]) <= tol[gi], (what, gv, yr[gi])
    return gi, ri, gap


@pytest.mark.parametrize("M,K", [(1, 32), (63, 64), (64, 256), (1000, 3584), (4097, 928)])
def test_lmhead_small(M, K):
    W = workloads.q8_0_blocks(M, K, key=(22, M, K))
    x = workloads.x_vector(K, key=(22, M, K))
    check_argmax(W, M, K, x, "small")


def test_lmhead_constructed_ties_lowest_index():
    # constant-quant rows with x = 1: logit_r = d * K * c_r; the maximum is tied
    K = 256
    c = np.array([5, 9, -3, 9, 9, 0, 8] * 20)  # ties at 9: first at index 1
    M = len(c)
    W = np.stack([np.concatenate([enc.q8_0_block(0x3400, [cr] * 32) for _ in range(K // 32)]) for cr in c])
    case("lmhead_argmax ties")
    idx, val = qg.lmhead_argmax(packed_q8_0(W, M, K), to_dev(np.ones(K, np.float32)), M, K)
    assert int(idx.item()) == 1
    assert float(val.item()) == 0.25 * K * 9


def test_lmhead_winner_in_last_ragged_tile():
    K = 64
    c = np.zeros(200, int)
    c[199] = 7
    c[130] = 6
    W = np.stack([np.concatenate([enc.q8_0_block(0x3C00, [cr] * 32) for _ in range(K // 32)]) for cr in c])
    case("lmhead_argmax last tile")
    idx, val = qg.lmhead_argmax(packed_q8_0(W, 200, K), to_dev(np.ones(K, np.float32)), 200, K)
    assert int(idx.item()) == 199 and float(val.item()) == 7 * K


def test_lmhead_vocab_152064_with_resampling():
    """Full LM-head shape; x is redrawn while the oracle's top-2 gap is below 1e-3."""
    M, K = workloads.VOCAB, workloads.HIDDEN
    W = workloads.q8_0_blocks(M, K, key=(4, 0))
    case("lmhead_argmax 152064x3584 pack")
    wp = packed_q8_0(W, M, K)
    exact = 0
    trials = 16
    worst = 0.0  # largest |out_value - y_ref[id]| / tol over the trials
    for t in range(trials):
        r = 0
        while True:
            x = workloads.x_vector(K, key=(4, 1, t, r))
            yr, ar = oracle.gemv_q8_0(W, M, K, x)
            s = np.sort(yr)
            if s[-1] - s[-2] >= 1e-3:
                break
            r += 1
        case(f"lmhead_argmax 152064x3584 trial {t} resample {r}")
        idx, val = qg.lmhead_argmax(wp, to_dev(x), M, K)
        gi, gv = int(idx.item()), float(val.item())
        ri = oracle.argmax(yr)
        tol = oracle.tolerance(ar)
        if s[-1] - s[-2] > tol[ri]:
            assert gi == ri
        else:  # within the tolerance band any row that could be the maximum will do
            assert yr[gi] >= yr[ri] - tol[gi] - tol[ri]
        assert abs(gv - yr[gi]) <= tol[gi]
        worst = max(worst, abs(gv - yr[gi]) / tol[gi])
        exact += gi == ri
    print(f"exact-match rate {exact}/{trials}, largest out_value error {worst:.4f} of the tolerance")


def test_lmhead_leaves_workspace_zero():
    # the partial (max, index) pairs are cleared by the reduction, so a workspace
    # shared with the small-N product (which needs idle, zero slots) stays valid
    M, K = 5000, 512
    W = workloads.q8_0_blocks(M, K, key=(23,))
    x = workloads.x_vector(K, key=(23,))
    ws = qg.Workspace(DEV)
    case("lmhead_argmax workspace left zero")
    wp = packed_q8_0(W, M, K)
    for _ in range(2):
        idx, _ = qg.lmhead_argmax(wp, to_dev(x), M, K, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.buf.count_nonzero()) == 0
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    gi, ri = int(idx.item()), oracle.argmax(yr)
    tol = oracle.tolerance(ar)
    assert gi == ri or yr[gi] >= yr[ri] - tol[gi] - tol[ri]


def check_verify(W, M, K, X, what, ws=None):
    """lmhead_argmax_verify against the oracle, column by column (same band rule
    as the single-column LM head)."""
    N = X.shape[0]
    case(f"lmhead_argmax_verify {what} M={M} K={K} N={N}")
    wp = packed_q8_0(W, M, K)
    idx, val = qg.lmhead_argmax_verify(wp, to_dev(X), M, K, ws=ws)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    exact = 0
    for n in range(N):
        yr, ar = oracle.gemv_q8_0(W, M, K, X[n])
        gi, ri = int(idx[n]), oracle.argmax(yr)
        tol = oracle.tolerance(ar)
        srt = np.sort(yr)
        gap = srt[-1] - srt[-2] if M > 1 else np.inf
        if gap > tol[ri]:
            assert gi == ri, (what, n, gi, ri, gap)
        else:
            assert yr[gi] >= yr[ri] - tol[gi] - tol[ri], (what, n, gi, ri)
        assert abs(float(val[n]) - yr[gi]) <= tol[gi], (what, n, float(val[n]), yr[gi])
        exact += gi == ri
    return exact


@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (200, 256, 5), (1000, 3584, 5), (4097, 512, 17), (63, 1024, 32),
                                   (3000, 768, 16)])
def test_verify_small(M, K, N):
    W = workloads.q8_0_blocks(M, K, key=(24, M, K))
    X = workloads.x_columns(K, N, key=(24, M, K, N))
    check_verify(W, M, K, X, "small")


def test_verify_constructed_ties_per_column():
    # constant-quant rows, column n = (n + 1) * ones: logit_{r,n} = d K c_r (n + 1);
    # the maximum is tied between rows 1, 3, 4: every column must return 1
    K, N = 256, 5
    c = np.array([5, 9, -3, 9, 9, 0, 8] * 20)
    M = len(c)
    W = np.stack([np.concatenate([enc.q8_0_block(0x3400, [cr] * 32) for _ in range(K // 32)]) for cr in c])
    X = np.stack([np.full(K, n + 1, np.float32) for n in range(N)])
    case("lmhead_argmax_verify ties")
    idx, val = qg.lmhead_argmax_verify(packed_q8_0(W, M, K), to_dev(X), M, K)
    assert idx.cpu().tolist() == [1] * N
    assert val.cpu().tolist() == [0.25 * K * 9 * (n + 1) for n in range(N)]


def test_verify_vocab_152064_n5():
    """Full LM-head shape, five columns in one pass; a column is redrawn while its
    oracle top-2 gap is below 1e-3. The workspace is left zero."""
    M, K, N = workloads.VOCAB, workloads.HIDDEN, 5
    W = workloads.q8_0_blocks(M, K, key=(4, 0))
    cols = []
    for n in range(N):
        r = 0
        while True:
            x = workloads.x_vector(K, key=(4, 2, n, r))
            s = np.sort(oracle.gemv_q8_0(W, M, K, x)[0])
            if s[-1] - s[-2] >= 1e-3:
                break
            r += 1
        cols.append(x)
    ws = qg.Workspace(DEV)
    exact = check_verify(W, M, K, np.stack(cols), "vocab", ws=ws)
    assert int(ws.buf.count_nonzero()) == 0
    print(f"exact-match rate {exact}/{N}")


@pytest.mark.parametrize("cfg", ["8,1", "8,2", "8,4", "4,2", "4,4"])
@pytest.mark.parametrize("N", [5, 20])
def test_verify_launch_shapes(cfg, N):
    # every (wavefronts, tiles per workgroup) shape of the matrix-core form, with a
    # tile count that is not a multiple of the tiles per workgroup and a ragged last
    # tile
    w, tw = (int(v) for v in cfg.split(","))
    qg.launch_override(verify_form=qg.FORM_VERIFY_MFMA, verify_waves=w, verify_tiles=tw).set()
    M, K = 1000, 1024
    W = workloads.q8_0_blocks(M, K, key=(25, M))
    X = workloads.x_columns(K, N, key=(25, N))
    check_verify(W, M, K, X, f"shape {cfg}")


@pytest.mark.parametrize("cfg", ["1,0", "4,0"])
@pytest.mark.parametrize("N", [1, 3, 6])
def test_verify_vector_alu_form_shapes(cfg, N):
    # the vector-ALU form (N <= 6): one and four wavefronts per tile, half
    # macro-block counts that do not divide among the K-groups (K = 2816: 22
    # halves), a ragged last tile; the workspace (partials, fp16 pairs and block
    # sums) is left zero
    qg.launch_override(verify_form=qg.FORM_VERIFY_DOT, verify_waves=int(cfg.split(",")[0])).set()
    M, K = 1000, 2816
    W = workloads.q8_0_blocks(M, K, key=(26, M))
    X = workloads.x_columns(K, N, key=(26, N))
    ws = qg.Workspace(DEV)
    check_verify(W, M, K, X, f"vector-ALU form {cfg}", ws=ws)
    assert int(ws.buf.count_nonzero()) == 0


@pytest.mark.parametrize("N", [1, 2, 5, 8, 9, 12, 16])
def test_verify_streamed_form_shapes(N):
    # the streamed form (grid of resident workgroups walking tiles in rounds of
    # two), in its 8-column and 16-column instances: one tile (a single round of
    # one tile), one macro-block, a ragged last tile, walks of many tiles with
    # K = 4096 (its largest); the workspace is left zero
    qg.launch_override(verify_form=qg.FORM_VERIFY_STREAM).set()
    for key, (M, K) in enumerate([(16, 256), (33, 768), (1000, 2816), (20000, 4096)]):
        W = workloads.q8_0_blocks(M, K, key=(28, M))
        X = workloads.x_columns(K, N, key=(28, N, key))
        ws = qg.Workspace(DEV)
        check_verify(W, M, K, X, f"streamed form M={M} K={K} N={N}", ws=ws)
        assert int(ws.buf.count_nonzero()) == 0


def test_verify_forms_agree_on_ldx_padding():
    # X with ldx > K (padding columns of NaN never read) through both forms
    M, K, N, ldx = 500, 1024, 4, 1100
    W = workloads.q8_0_blocks(M, K, key=(27,))
    X = workloads.x_columns(K, N, key=(27,))
    Xp = np.full((N, ldx), np.nan, np.float32)
    Xp[:, :K] = X
    wp = packed_q8_0(W, M, K)
    case("lmhead_argmax_verify ldx padding, both forms")
    i_dot, v_dot = qg.lmhead_argmax_verify(wp, to_dev(Xp), M, K)
    with qg.launch_override(verify_form=qg.FORM_VERIFY_MFMA):
        i_mma, v_mma = qg.lmhead_argmax_verify(wp, to_dev(Xp), M, K)
    with qg.launch_override(verify_form=qg.FORM_VERIFY_DOT):
        i_vd, v_vd = qg.lmhead_argmax_verify(wp, to_dev(Xp), M, K)
    torch.cuda.synchronize()
    for n in range(N):
        yr, ar = oracle.gemv_q8_0(W, M, K, X[n])
        tol = oracle.tolerance(ar)
        for gi, gv in ((int(i_dot[n]), float(v_dot[n])), (int(i_mma[n]), float(v_mma[n])),
                       (int(i_vd[n]), float(v_vd[n]))):
            ri = oracle.argmax(yr)
            assert yr[gi] >= yr[ri] - tol[gi] - tol[ri], n
            assert abs(gv - yr[gi]) <= tol[gi], n
