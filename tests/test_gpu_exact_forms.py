"""Exact edge cases through every kernel form (each forced with the launch
override), compared bit for bit with the oracle where every intermediate value
is representable:

* Q4_K small-N product, all four forms (register-staged, chunked-LDS and
  single-pass-LDS matrix-core forms, vector-ALU dot form) and the automatic
  choice: rows of the hand-derived golden blocks A/B/C, min-only rows (q = 0),
  rows with d = dmin = 0 and rows of random quants with few-bit scales, against
  activation columns of ones and of unit vectors e_k;
* the same for the int8-activation Q4_K products (columns 127 * e_k and 127 * 1,
  whose Q8_1 quantization is exact);
* the Q8_0 LM-head verification in its matrix-core, vector-ALU and int8 forms,
  with d = 1, integer quants and integer activations: integer-exact logits, the
  expected token ids (first maximum, including planted ties) and their values;
* Q8_0 rows whose quants are all zero give exactly 0 for N(0, 1) activations
  (the quants are taken as signed fp16 values, so no bias term has to cancel),
  and rows with d = 0 give 0 in every form.
The pins are the definitions of the fused scale x int products (dotLLM README, Key
Features) and of the argmax (first maximum)."""
import functools

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests import blockenc as enc
from tests.gpu_helpers import DEV, case, packed_q4k, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu

FORMS = {"auto": qg.FORM_AUTO, "regs": qg.FORM_SMALLN_REGS, "lds": qg.FORM_SMALLN_LDS,
         "lds1": qg.FORM_SMALLN_LDS1, "dot": qg.FORM_SMALLN_DOT, "stream": qg.FORM_SMALLN_STREAM,
         "walk": qg.FORM_SMALLN_WALK, "split": qg.FORM_SMALLN_SPLIT, "slice": qg.FORM_SMALLN_SLICE,
         "slice1": qg.FORM_SMALLN_SLICE}  # slice1: the slice form without a workspace (no K slices)


@functools.lru_cache(maxsize=None)
def exact_q4k_rows(M: int, K: int, seed: int, small: bool = False) -> np.ndarray:
    """M rows of K/256 Q4_K blocks, four kinds by r % 4: golden blocks A/B/C;
    min-only (q = 0, random 6-bit sc, m); d = dmin = 0 (random sc, m, q); random
    sc, m, q. Every d and dmin has one or two significant bits, so every product
    of a scale with an integer is exact in fp32. With small=True (for activations
    of 127): golden A/C only, d = dmin = 1/2 and sc < 8, m < 16 in the random
    rows, which keeps every partial sum of 127-scaled products below 2^23."""
    G = enc.golden()
    rng = np.random.default_rng(seed)
    nb = K // 256
    rows = []
    for r in range(M):
        kind = r % 4
        blocks = []
        for b in range(nb):
            if kind == 0:
                names = ["A", "C"] if small else ["A", "B", "C"]
                blocks.append(G[names[(r + b) % len(names)]]["block"])
                continue
            sc = rng.integers(0, 8 if small else 64, 8)
            m = rng.integers(0, 16 if small else 64, 8)
            q = rng.integers(0, 16, 256)
            if kind == 1:    # d = 1/64 (or 1/2), dmin = 3/128 (or 1/2)
                blocks.append(enc.q4k_block(0x3800 if small else 0x2400, 0x3800 if small else 0x2600, sc, m,
                                            np.zeros(256, int)))
            elif kind == 2:
                blocks.append(enc.q4k_block(0x0000, 0x0000, sc, m, q))
            else:            # d = 1/32 (or 1/2), dmin = 1/64 (or 1/2)
                blocks.append(enc.q4k_block(0x3800 if small else 0x2800, 0x3800 if small else 0x2400, sc, m, q))
        rows.append(np.concatenate(blocks))
    return np.stack(rows)


def exact_columns(K: int, N: int, scale: float = 1.0, ones: bool = True) -> np.ndarray:
    """Column n: all `scale` for n % 3 == 0 (if ones), else scale * e_k with k
    running over the first and last positions of sub-blocks and super-blocks and
    inner positions."""
    pos = [K - 1, 0, 31, 32, 255, 256 % K, 511 % K, 37, 100, K // 2, K - 256, K - 33, 129]
    X = np.zeros((N, K), np.float32)
    j = 0
    for n in range(N):
        if ones and n % 3 == 0:
            X[n] = scale
        else:
            X[n, pos[j % len(pos)]] = scale
            j += 1
    return X


def row_quanta(Wd: np.ndarray) -> np.ndarray:
    """Per row, the largest power of two that divides every weight (1 for zero rows)."""
    q = np.ones(Wd.shape[0])
    for r in range(Wd.shape[0]):
        nz = Wd[r][Wd[r] != 0]
        e = 10
        while nz.size and np.any(np.mod(nz, 2.0 ** e) != 0):
            e -= 1
        q[r] = 2.0 ** e
    return q


def check_exact(Y, W, M, K, X, what):
    """Y (N, M) equal to W_deq X bit for bit. The data are built so that every
    partial sum the kernels form is a multiple of the row's quantum with fewer
    than 24 significant bits (asserted), so any fp32 summation order is exact."""
    Wd = oracle.q4k_dequant(W, M, K)
    quanta = row_quanta(Wd)
    for n in range(X.shape[0]):
        xs = X[n].astype(np.float64)
        assert np.all(np.mod(xs, 1) == 0)
        assert np.all(np.abs(Wd) @ np.abs(xs) < 2.0 ** 24 * quanta), what
        ref = Wd @ xs
        got = Y[n].astype(np.float64)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, f"{what} col {n}: {bad.size} rows differ; first {bad[0]}: {got[bad[0]]!r} vs {ref[bad[0]]!r}"


SMALLN_CASES = [("auto", N) for N in (1, 2, 3, 4, 5, 8, 9, 16, 17, 32)] + \
               [("regs", N) for N in (5, 17, 32)] + [("lds", N) for N in (5, 17, 32)] + \
               [("lds1", N) for N in (5, 8)] + [("dot", N) for N in (1, 5, 8)] + \
               [("stream", N) for N in (1, 5, 8)] + [("walk", N) for N in (1, 5, 16, 17, 32)] + \
               [("split", N) for N in (1, 5, 17, 32)] + [("slice", N) for N in (1, 4, 5, 8, 16)] + \
               [("slice1", N) for N in (1, 5, 8, 16)]


@pytest.mark.parametrize("form,N", SMALLN_CASES)
@pytest.mark.parametrize("M,K", [(70, 768), (37, 9984), (300, 3840)])
def test_smalln_exact(form, N, M, K):
    if form in ("lds1", "stream") and K > 4096:
        pytest.skip("the single-pass forms take K <= 4096")
    W = exact_q4k_rows(M, K, seed=M + K)
    X = exact_columns(K, N)
    wp = packed_q4k(W, M, K)
    case(f"qgemm_q4k_smalln exact form={form} M={M} K={K} N={N}")
    with qg.launch_override(smalln_form=FORMS[form]):
        if form in ("split", "slice"):
            Y = torch.empty((N, (M + 3) // 4 * 4), device="cuda:0")
            qg.qgemm_q4k_smalln_batch_ws([(wp, to_dev(X), Y, M, K)])
        else:
            Y = qg.qgemm_q4k_smalln(wp, to_dev(X), M, K)
    torch.cuda.synchronize()
    check_exact(Y.cpu().numpy()[:, :M], W, M, K, X, f"{form} M={M} K={K} N={N}")


@pytest.mark.parametrize("N", [3, 5, 8])
def test_smalln_exact_many_tiles(N):
    # a batch of more than 1024 tiles on short K: the automatic choice takes the
    # streamed form with one 16-wavefront workgroup per CU walking up to ten tiles
    M, K = 16400, 768
    W = exact_q4k_rows(M, K, seed=11)
    X = exact_columns(K, N)
    case(f"qgemm_q4k_smalln exact many tiles M={M} K={K} N={N}")
    Y = qg.qgemm_q4k_smalln(packed_q4k(W, M, K), to_dev(X), M, K)
    torch.cuda.synchronize()
    check_exact(Y.cpu().numpy()[:, :M], W, M, K, X, f"many tiles N={N}")


@pytest.mark.parametrize("form,N", [("auto", 5), ("auto", 32), ("regs", 5), ("regs", 32), ("lds", 5),
                                    ("lds", 32), ("lds1", 5), ("dot", 5), ("stream", 5),
                                    ("walk", 5), ("walk", 32), ("slice1", 5)])
def test_smalln_zero_scales_exact_zero_random_x(form, N):
    # d = dmin = 0 in every block: exactly 0 whatever the activations
    M, K = 100, 3584
    W = workloads.q4k_blocks(M, K, key=(95,)).reshape(M, K // 256, 144).copy()
    W[:, :, 0:4] = 0
    W = W.reshape(M, -1)
    X = workloads.x_columns(K, N, key=(95, N))
    case(f"qgemm_q4k_smalln zero scales form={form} N={N}")
    with qg.launch_override(smalln_form=FORMS[form]):
        Y = qg.qgemm_q4k_smalln(packed_q4k(W, M, K), to_dev(X), M, K)
    torch.cuda.synchronize()
    assert torch.all(Y[:, :M] == 0)


@pytest.mark.parametrize("M,K", [(70, 768), (37, 9984)])
def test_gemv_exact(M, K):
    W = exact_q4k_rows(M, K, seed=7 * M + K)
    X = exact_columns(K, 7)
    wp = packed_q4k(W, M, K)
    case(f"qgemv_q4k exact M={M} K={K}")
    Y = np.stack([qg.qgemv_q4k(wp, to_dev(X[n]), M, K).cpu().numpy() for n in range(X.shape[0])])
    check_exact(Y, W, M, K, X, f"gemv M={M} K={K}")


@pytest.mark.parametrize("N", [1, 3, 5, 8])
@pytest.mark.parametrize("M,K", [(70, 768), (37, 9984)])
def test_int8_products_exact(M, K, N):
    # columns 127 * e_k and 127 * 1: every 32-block's scale is exactly 1 (blocks
    # without a nonzero get scale 0) and the int8 codes equal the activations
    W = exact_q4k_rows(M, K, seed=3 * M + K, small=True)
    X = exact_columns(K, N, scale=127.0, ones=K <= 768)
    wp = packed_q4k(W, M, K)
    case(f"int8-activation products exact M={M} K={K} N={N}")
    xq = qg.quantize_q8_1_columns(to_dev(X))
    nb = qg.q8_1_bytes(K)
    for n in range(N):
        d, q, _ = (t.cpu().numpy() for t in qg.q8_1_views(xq[n * nb:(n + 1) * nb], K))
        assert np.array_equal(q.astype(np.float32), X[n]) and set(np.unique(d)) <= {0.0, 1.0}
    Y = qg.qgemm_q4k_q8_1_smalln(wp, xq, M, K, N).cpu().numpy()[:, :M]
    check_exact(Y, W, M, K, X, f"int8 smalln M={M} K={K} N={N}")
    y0 = qg.qgemv_q4k_q8_1(wp, xq[:nb], M, K).cpu().numpy()
    check_exact(y0[None], W, M, K, X[:1], f"int8 gemv M={M} K={K}")


# ---------------------------------------------------------------- Q8_0 LM head
@functools.lru_cache(maxsize=None)
def integer_head(M: int, K: int, seed: int, qmax: int = 127):
    """Q8_0 rows with d = 1 and integer quants in [-qmax, qmax]; rows 5, 21, ...
    (r % 16 == 5) have all-zero quants and rows r % 16 == 9 have d = 0."""
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(M):
        blocks = []
        for b in range(K // 32):
            q = rng.integers(-qmax, qmax + 1, 32)
            if r % 16 == 5:
                q[:] = 0
            blocks.append(enc.q8_0_block(0x0000 if r % 16 == 9 else 0x3C00, q))
        rows.append(np.concatenate(blocks))
    return np.stack(rows)


def plant_tie(W, X0, M, K):
    """Copy the row with the largest logit for column 0 to a lower index in
    another tile, so that column 0 has two exact maxima."""
    Wd = oracle.q8_0_dequant(W, M, K)
    best = int(np.argmax(Wd @ X0.astype(np.float64)))
    low = (best - 1000) % M if best >= 1000 else (best + 17) % M
    W = W.copy()
    W[low] = W[best]
    return W


def expected_ids(W, M, K, X):
    Wd = oracle.q8_0_dequant(W, M, K)
    L = Wd @ X.T.astype(np.float64)  # (M, N), exact integers
    assert np.abs(L).max() < 2 ** 24
    ids = [oracle.argmax(L[:, n]) for n in range(X.shape[0])]
    return np.array(ids), np.array([L[ids[n], n] for n in range(X.shape[0])]), L


@pytest.mark.parametrize("form,N,W_,TW", [("mfma", 5, 4, 4), ("mfma", 5, 8, 1), ("mfma", 9, 8, 2),
                                          ("mfma", 20, 4, 1), ("mfma", 32, 4, 2), ("dot", 1, 1, 0),
                                          ("dot", 5, 1, 0), ("dot", 6, 4, 0), ("auto", 5, 0, 0),
                                          ("auto", 17, 0, 0), ("stream", 1, 0, 0), ("stream", 5, 0, 0),
                                          ("stream", 8, 0, 0), ("stream", 9, 0, 0), ("stream", 16, 0, 0),
                                          ("auto", 12, 0, 0)])
def test_verify_integer_exact(form, N, W_, TW):
    M, K = 5000, 1536
    rng = np.random.default_rng(N)
    X = rng.integers(-3, 4, (N, K)).astype(np.float32)
    W = plant_tie(integer_head(M, K, seed=91), X[0], M, K)
    ids, vals, L = expected_ids(W, M, K, X)
    assert np.sum(L[:, 0] == vals[0]) >= 2  # the planted tie
    wp = packed_q8_0(W, M, K)
    ov = {"verify_form": {"mfma": qg.FORM_VERIFY_MFMA, "dot": qg.FORM_VERIFY_DOT, "auto": 0,
                          "stream": qg.FORM_VERIFY_STREAM}[form],
          "verify_waves": W_, "verify_tiles": TW}
    ws = qg.Workspace(DEV)
    case(f"lmhead_argmax_verify integer form={form} N={N} W={W_} TW={TW}")
    with qg.launch_override(**ov):
        idx, val = qg.lmhead_argmax_verify(wp, to_dev(X), M, K, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ids)
    assert np.array_equal(val.cpu().numpy().astype(np.float64), vals)
    assert int(ws.buf.count_nonzero()) == 0


@pytest.mark.parametrize("N,W_", [(1, 1), (5, 1), (5, 4), (8, 4)])
def test_verify_q8_1_integer_exact(N, W_):
    # int8 columns with a +-127 in every 32-block: scale 1, codes equal to x
    M, K = 5000, 1536
    rng = np.random.default_rng(100 + N)
    X = rng.integers(-127, 128, (N, K)).astype(np.float32)
    X[:, ::32] = 127 * np.sign(X[:, ::32] + 0.5)
    W = plant_tie(integer_head(M, K, seed=92, qmax=15), X[0], M, K)
    ids, vals, _ = expected_ids(W, M, K, X)
    wp = packed_q8_0(W, M, K)
    case(f"lmhead_argmax_verify_q8_1 integer N={N} W={W_}")
    xq = qg.quantize_q8_1_columns(to_dev(X))
    with qg.launch_override(verify_waves=W_):
        idx, val = qg.lmhead_argmax_verify_q8_1(wp, xq, M, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ids)
    assert np.array_equal(val.cpu().numpy().astype(np.float64), vals)


@pytest.mark.parametrize("gw", [0, 1, 2, 4, 8])
def test_lmhead_and_gemv_integer_exact(gw):
    M, K = 3000, 1280  # K / 32 = 40: five macro-blocks, no tail
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, K).astype(np.float32)
    W = plant_tie(integer_head(M, K, seed=93), x, M, K)
    ids, vals, L = expected_ids(W, M, K, x[None])
    wp = packed_q8_0(W, M, K)
    case(f"lmhead_argmax / qgemv_q8_0 integer gemv_waves={gw}")
    with qg.launch_override(gemv_waves=gw):
        idx, val = qg.lmhead_argmax(wp, to_dev(x), M, K)
        y = qg.qgemv_q8_0(wp, to_dev(x), M, K)
    torch.cuda.synchronize()
    assert int(idx.item()) == ids[0] and float(val.item()) == vals[0]
    assert np.array_equal(y.cpu().numpy().astype(np.float64), L[:, 0])


@pytest.mark.parametrize("M,K", [(300, 4096), (77, 4000), (1000, 3584)])
def test_q8_0_zero_quant_rows_exact_zero_random_x(M, K):
    # all-zero quants with N(0, 1) activations: every product is an exact zero,
    # so y = 0 exactly (K = 4000 also runs the canonical-form tail blocks)
    W = workloads.q8_0_blocks(M, K, key=(94, M)).reshape(M, K // 32, 34).copy()
    W[1::3, :, 2:] = 0
    W = W.reshape(M, -1)
    x = workloads.x_vector(K, key=(94, K))
    wp = packed_q8_0(W, M, K)
    case(f"qgemv_q8_0 zero-quant rows M={M} K={K}")
    for gw in (0, 1, 4):
        with qg.launch_override(gemv_waves=gw):
            y = qg.qgemv_q8_0(wp, to_dev(x), M, K).cpu().numpy()
        assert np.all(y[1::3] == 0), gw
        yr, ar = oracle.gemv_q8_0(W, M, K, x)
        tol = oracle.tolerance(ar)
        assert np.all(np.abs(y - yr) <= tol), gw


def test_q8_0_small_quants_bound():
    # quants in {-1, 0, 1}: sum|w x| is small, and the product must stay within
    # 1e-3 sum|w x| + 1e-6 of the oracle (no error term proportional to sum|x|)
    M, K = 2000, 3584
    rng = np.random.default_rng(96)
    W = workloads.q8_0_blocks(M, K, key=(96,)).reshape(M, K // 32, 34).copy()
    W[:, :, 2:] = rng.integers(-1, 2, (M, K // 32, 32)).astype(np.int8).view(np.uint8)
    W = W.reshape(M, -1)
    x = workloads.x_vector(K, key=(96, 1))
    case("qgemv_q8_0 small quants")
    y = qg.qgemv_q8_0(packed_q8_0(W, M, K), to_dev(x), M, K).cpu().numpy()
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    err = np.abs(y - yr)
    assert np.all(err <= oracle.tolerance(ar))
    # the error is the fp16 rounding of x and fp32 summation: far below the bound
    assert float((err / oracle.tolerance(ar)).max()) < 0.05
