"""GPU parity of the small-N Q4_K product (verify / prefill tile) against the oracle,
per (row, column), plus the invariant that column n equals the GEMV of x_n."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import assert_within, case, packed_q4k, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def run_smalln(M, K, N, key, rows=None):
    W = workloads.q4k_blocks(M, K, key=key)
    X = workloads.x_columns(K, N, key=key)
    case(f"qgemm_q4k_smalln M={M} K={K} N={N} key={key}")
    wp = packed_q4k(W, M, K)
    Y = qg.qgemm_q4k_smalln(wp, to_dev(X), M, K)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()[:, :M]
    Yr, Ar = oracle.gemm_q4k(W, M, K, X, rows=rows)
    if rows is not None:
        Y = Y[:, rows]
    return W, X, wp, Y, Yr, Ar


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 9, 16, 17, 32])
@pytest.mark.parametrize("M,K", [(200, 512), (65, 768), (1, 256)])
def test_smalln_small(M, K, N):
    _, _, _, Y, Yr, Ar = run_smalln(M, K, N, key=(30, M, K, N))
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"smalln M={M} K={K} N={N} col {n}")


@pytest.mark.parametrize("N", [5, 32])
@pytest.mark.parametrize("name,M,K", [m for m in workloads.LAYER_MATRICES])
def test_smalln_7b_shapes(name, M, K, N):
    rows = sample_rows(M, 192, seed=M + K + N)
    _, _, _, Y, Yr, Ar = run_smalln(M, K, N, key=(5, 0, workloads.LAYER_MATRICES.index((name, M, K)), N), rows=rows)
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"smalln {name} N={N} col {n}")


@pytest.mark.parametrize("N", [5, 32])
def test_columns_match_gemv(N):
    M, K = 3584, 3584
    W, X, wp, Y, Yr, Ar = run_smalln(M, K, N, key=(31, N), rows=np.arange(0, M, 7))
    for n in range(N):
        y = qg.qgemv_q4k(wp, to_dev(X[n]), M, K).cpu().numpy()
        # both within tolerance of the same oracle column, hence within 2 tol of each other
        tol = oracle.tolerance(Ar[n])
        assert np.all(np.abs(y[::7] - Y[n]) <= 2 * tol)


def test_padded_leading_dimensions():
    M, K, N = 130, 512, 5
    W = workloads.q4k_blocks(M, K, key=(32,))
    X = workloads.x_columns(K, N, key=(32,))
    ldx, ldy = K + 12, M + 10
    Xp = np.zeros((N, ldx), np.float32)
    Xp[:, :K] = X
    case("qgemm_q4k_smalln padded ld")
    wp = packed_q4k(W, M, K)
    Yd = torch.full((N, ldy), 123.0, device="cuda:0")
    qg.qgemm_q4k_smalln(wp, to_dev(Xp), M, K, Y=Yd)
    Y = Yd.cpu().numpy()
    assert np.all(Y[:, M:] == 123.0)  # padding untouched
    Yr, Ar = oracle.gemm_q4k(W, M, K, X)
    for n in range(N):
        assert_within(Y[n, :M], Yr[n], Ar[n], f"padded col {n}")


def test_batch_mixed_problems():
    # the attention-input stage with N=5, plus ragged problems with other N in the
    # same launch (the launch uses the widest column count of the batch)
    shapes = [(3584, 3584, 5), (512, 3584, 5), (512, 3584, 5), (77, 768, 3), (33, 512, 17)]
    probs, refs = [], []
    for i, (M, K, N) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(33, i))
        X = workloads.x_columns(K, N, key=(33, i))
        Y = torch.full((N, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X, rows=np.arange(0, M, 5)))
    case("qgemm_q4k_smalln_batch mixed")
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, X, Y, M, K), (Yr, Ar) in zip(probs, refs):
        Yc = Y.cpu().numpy()[:, :M][:, ::5]
        for n in range(X.shape[0]):
            assert_within(Yc[n], Yr[n], Ar[n], f"batch M={M} K={K} col {n}")


@pytest.mark.parametrize("cfg", ["1,1", "2,2", "4,4", "8,1", "8,2", "4,2"])
@pytest.mark.parametrize("N", [5, 32])
def test_launch_shapes(cfg, N):
    # every (wavefronts, tiles per wavefront) shape of the register-staged form, on a
    # batch whose tile counts are not multiples of the tiles per wavefront and whose K
    # ranges leave some wavefronts with an odd number of units (or none)
    w, tw = (int(v) for v in cfg.split(","))
    qg.launch_override(smalln_form=qg.FORM_SMALLN_REGS, smalln_waves=w, smalln_tiles=tw).set()
    shapes = [(530, 1024), (77, 256), (16, 768), (1000, 512)]
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(34, i))
        X = workloads.x_columns(K, N, key=(34, i, N))
        Y = torch.full((N, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X))
    case(f"qgemm_q4k_smalln_batch cfg={cfg} N={N}")
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, X, Y, M, K), (Yr, Ar) in zip(probs, refs):
        Yc = Y.cpu().numpy()[:, :M]
        for n in range(N):
            assert_within(Yc[n], Yr[n], Ar[n], f"cfg {cfg} M={M} K={K} col {n}")


# LDS-staged form (producer wavefronts stage the activations per chunk of super-blocks,
# consumer wavefronts keep their weight loads chunks ahead): forced on shapes whose
# super-block counts leave a short last chunk (nb % 8, nb % 4 != 0), a single chunk
# (nb = 1), ragged tiles, and column counts on both sides of 16.
@pytest.mark.parametrize("N", [1, 3, 5, 16, 17, 32])
@pytest.mark.parametrize("M,K", [(200, 512), (65, 3328), (16, 256), (530, 9984)])
def test_lds_form_shapes(M, K, N):
    qg.launch_override(smalln_form=qg.FORM_SMALLN_LDS).set()
    rows = None if M * K <= 200 * 3328 else sample_rows(M, 96, seed=M + N)
    _, _, _, Y, Yr, Ar = run_smalln(M, K, N, key=(36, M, K, N), rows=rows)
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"lds form M={M} K={K} N={N} col {n}")


@pytest.mark.parametrize("cfg", ["1,2", "1,3", "1,4", "2,2", "2,3", "2,4"])
@pytest.mark.parametrize("N", [5, 32])
def test_lds_form_launch_shapes(cfg, N):
    # every (tiles per workgroup, queue depth) the launcher accepts, on a batch whose
    # tile counts are not multiples of the tiles per workgroup (a depth of 4 is taken
    # up to 16 columns only; above, the launcher keeps its default depth)
    tw, depth = (int(v) for v in cfg.split(","))
    qg.launch_override(smalln_form=qg.FORM_SMALLN_LDS, smalln_tiles=tw, smalln_depth=depth).set()
    shapes = [(530, 2304), (77, 256), (16, 768), (1000, 1280)]
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(37, i))
        X = workloads.x_columns(K, N, key=(37, i, N))
        Y = torch.full((N, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X))
    case(f"qgemm_q4k_smalln_batch lds cfg={cfg} N={N}")
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    first = [p[2].clone() for p in probs]
    qg.qgemm_q4k_smalln_batch(probs)  # deterministic: the same bits on a second call
    torch.cuda.synchronize()
    for (w, X, Y, M, K), Y0, (Yr, Ar) in zip(probs, first, refs):
        assert torch.equal(Y[:, :M], Y0[:, :M])
        Yc = Y.cpu().numpy()[:, :M]
        for n in range(N):
            assert_within(Yc[n], Yr[n], Ar[n], f"lds cfg {cfg} M={M} K={K} col {n}")


def test_lds_form_padded_and_mixed_columns():
    # padded leading dimensions and problems with different column counts in one
    # launch (LDS rows sized for the widest)
    qg.launch_override(smalln_form=qg.FORM_SMALLN_LDS).set()
    shapes = [(130, 2048, 5, 12, 10), (40, 1024, 2, 4, 8), (33, 512, 9, 0, 3)]
    probs, refs = [], []
    for i, (M, K, N, px, py) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(38, i))
        X = workloads.x_columns(K, N, key=(38, i))
        Xp = np.zeros((N, K + px), np.float32)
        Xp[:, :K] = X
        Y = torch.full((N, M + py), 123.0, device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(Xp), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X))
    case("qgemm_q4k_smalln_batch lds padded / mixed N")
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, X, Y, M, K), (Yr, Ar) in zip(probs, refs):
        Yc = Y.cpu().numpy()
        assert np.all(Yc[:, M:] == 123.0)
        for n in range(X.shape[0]):
            assert_within(Yc[n, :M], Yr[n], Ar[n], f"lds padded M={M} K={K} col {n}")


@pytest.mark.parametrize("N", [1, 5, 17, 32])
@pytest.mark.parametrize("M,K", [(200, 512), (65, 3328), (48, 9984)])
def test_register_form_shapes(M, K, N):
    # the register-staged form (activations in registers, wavefronts splitting K in
    # 64-weight units)
    qg.launch_override(smalln_form=qg.FORM_SMALLN_REGS).set()
    _, _, _, Y, Yr, Ar = run_smalln(M, K, N, key=(40, M, K, N))
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"register form M={M} K={K} N={N} col {n}")


@pytest.mark.parametrize("tw", ["1", "2"])
def test_single_pass_form(tw):
    # short-K single-pass form (all activations in LDS, every super-block of a row
    # in flight at once): the largest K it takes (4096: sixteen super-blocks, two
    # per wavefront), one super-block, N from 1 to its limit of 8 in one launch,
    # ragged tiles and tile counts not a multiple of the tiles per workgroup
    qg.launch_override(smalln_form=qg.FORM_SMALLN_LDS1, smalln_tiles=int(tw)).set()
    shapes = [(530, 4096, 8), (77, 256, 1), (16, 3584, 5), (1000, 1280, 3), (33, 768, 2)]
    probs, refs = [], []
    for i, (M, K, N) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(39, i))
        X = workloads.x_columns(K, N, key=(39, i, N))
        Y = torch.full((N, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X))
    case(f"qgemm_q4k_smalln_batch single-pass TW={tw}")
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    first = [p[2].clone() for p in probs]
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, X, Y, M, K), Y0, (Yr, Ar) in zip(probs, first, refs):
        assert torch.equal(Y[:, :M], Y0[:, :M])
        Yc = Y.cpu().numpy()[:, :M]
        for n in range(X.shape[0]):
            assert_within(Yc[n], Yr[n], Ar[n], f"single-pass TW={tw} M={M} K={K} col {n}")


def test_streamed_form():
    # streamed single-pass form (workgroups walk up to five tiles each, per-tile
    # sums parked in LDS): ragged tiles, one super-block, K = 4096, N from 1 to 8,
    # and batches of more tiles than the grid has workgroups, so that walks of one
    # to five tiles occur (3125 tiles of one super-block; 1250 + 20 tiles of two)
    qg.launch_override(smalln_form=qg.FORM_SMALLN_STREAM).set()
    batches = [[(530, 4096, 8), (77, 256, 1), (16, 3584, 5), (1000, 1280, 3), (33, 768, 2)],
               [(50000, 256, 5)],
               [(20000, 512, 5), (317, 512, 5)],
               [(18944, 3584, 5), (18944, 3584, 5)]]
    for bi, shapes in enumerate(batches):
        probs, refs = [], []
        for i, (M, K, N) in enumerate(shapes):
            W = workloads.q4k_blocks(M, K, key=(43, bi, i))
            X = workloads.x_columns(K, N, key=(43, bi, i, N))
            Y = torch.full((N, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
            rows = sample_rows(M, 256, seed=M + i) if M * K > 1 << 24 else None
            probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
            refs.append((rows, oracle.gemm_q4k(W, M, K, X, rows=rows)))
        case(f"qgemm_q4k_smalln_batch streamed batch {bi}: {shapes}")
        qg.qgemm_q4k_smalln_batch(probs)
        torch.cuda.synchronize()
        first = [p[2].clone() for p in probs]
        qg.qgemm_q4k_smalln_batch(probs)
        torch.cuda.synchronize()
        for (w, X, Y, M, K), Y0, (rows, (Yr, Ar)) in zip(probs, first, refs):
            assert torch.equal(Y[:, :M], Y0[:, :M]), "streamed form not deterministic"
            assert not torch.isnan(Y[:, :M]).any(), "streamed form left outputs unwritten"
            Yc = Y.cpu().numpy()[:, :M]
            if rows is not None:
                Yc = Yc[:, rows]
            for n in range(X.shape[0]):
                assert_within(Yc[n], Yr[n], Ar[n], f"streamed M={M} K={K} col {n}")


@pytest.mark.parametrize("N", [1, 5, 16, 17, 32])
def test_walk_form(N):
    # chunked walk form (one workgroup per CU walking up to ten tiles, K in chunks
    # of four super-blocks for N <= 16, two above): chunk counts with a ragged last
    # chunk (K = 768, 3328, 9984), one super-block, ragged tiles, walks of one to
    # ten tiles (30000 rows: 1875 tiles), two problems of different K in one batch
    qg.launch_override(smalln_form=qg.FORM_SMALLN_WALK).set()
    batches = [[(530, 768, N), (77, 256, N), (1000, 3328, N)],
               [(30000, 512, N)],
               [(4000, 9984, N), (3001, 1280, N)]]
    for bi, shapes in enumerate(batches):
        probs, refs = [], []
        for i, (M, K, n_) in enumerate(shapes):
            W = workloads.q4k_blocks(M, K, key=(44, bi, i))
            X = workloads.x_columns(K, n_, key=(44, bi, i, n_))
            Y = torch.full((n_, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
            rows = sample_rows(M, 192, seed=M + i) if M * K * n_ > 1 << 26 else None
            probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
            refs.append((rows, oracle.gemm_q4k(W, M, K, X, rows=rows)))
        case(f"qgemm_q4k_smalln_batch walk N={N} batch {bi}: {shapes}")
        qg.qgemm_q4k_smalln_batch(probs)
        torch.cuda.synchronize()
        first = [p[2].clone() for p in probs]
        qg.qgemm_q4k_smalln_batch(probs)
        torch.cuda.synchronize()
        for (w, X, Y, M, K), Y0, (rows, (Yr, Ar)) in zip(probs, first, refs):
            assert torch.equal(Y[:, :M], Y0[:, :M]), "walk form not deterministic"
            assert not torch.isnan(Y[:, :M]).any(), "walk form left outputs unwritten"
            Yc = Y.cpu().numpy()[:, :M]
            if rows is not None:
                Yc = Yc[:, rows]
            for n in range(X.shape[0]):
                assert_within(Yc[n], Yr[n], Ar[n], f"walk M={M} K={K} col {n}")


def run_split(N, form, batches, key, what):
    """Batches of problems through qgemm_q4k_smalln_batch_ws with a forced K-slice
    form: nine calls on one workspace give bit-identical results, leave the
    arrival counters zero and match the oracle per (row, column)."""
    qg.launch_override(smalln_form=form).set()
    for bi, shapes in enumerate(batches):
        probs, refs = [], []
        for i, (M, K, n_) in enumerate(shapes):
            W = workloads.q4k_blocks(M, K, key=(key, bi, i))
            X = workloads.x_columns(K, n_, key=(key, bi, i, n_))
            Y = torch.full((n_, (M + 3) // 4 * 4), float("nan"), device="cuda:0")
            rows = sample_rows(M, 192, seed=M + i) if M * K * n_ > 1 << 26 else None
            probs.append((packed_q4k(W, M, K), to_dev(X), Y, M, K))
            refs.append((rows, oracle.gemm_q4k(W, M, K, X, rows=rows)))
        need = qg.qgemm_q4k_smalln_batch_workspace_bytes(probs)
        case(f"qgemm_q4k_smalln_batch_ws {what} N={N} batch {bi}: {shapes}, workspace {need}")
        assert need > 0
        ws = qg.Workspace("cuda:0", need)  # zero-filled: the arrival counters start at 0
        qg.qgemm_q4k_smalln_batch_ws(probs, ws)
        torch.cuda.synchronize()
        first = [p[2].clone() for p in probs]
        # repeated calls on the same workspace: the counters return to zero and the
        # slice sums never read a stale partial (bit-identical results every time)
        for rep in range(8):
            for p_ in probs:
                p_[2].fill_(float("nan"))
            qg.qgemm_q4k_smalln_batch_ws(probs, ws)
            torch.cuda.synchronize()
            for p_, Y0 in zip(probs, first):
                assert torch.equal(p_[2][:, :p_[3]], Y0[:, :p_[3]]), f"{what} form differs on call {rep + 2}"
        assert int(ws.buf[:4096].ne(0).sum()) == 0, "arrival counters not returned to zero"
        for (w, X, Y, M, K), Y0, (rows, (Yr, Ar)) in zip(probs, first, refs):
            assert torch.equal(Y[:, :M], Y0[:, :M]), f"{what} form not deterministic"
            assert not torch.isnan(Y[:, :M]).any(), f"{what} form left outputs unwritten"
            Yc = Y.cpu().numpy()[:, :M]
            if rows is not None:
                Yc = Yc[:, rows]
            for n in range(X.shape[0]):
                assert_within(Yc[n], Yr[n], Ar[n], f"{what} M={M} K={K} col {n}")


@pytest.mark.parametrize("N", [1, 5, 16, 17, 32])
def test_split_walk_form(N):
    # the walk form over tile groups and K slices (with a workspace): slices of one
    # to many super-blocks, a ragged last slice, problems left with one slice next
    # to sliced ones in one batch, ragged tiles; partial sums added in slice order
    batches = [[(530, 768, N), (77, 256, N), (1000, 3328, N)],
               [(3584, 18944, N)],
               [(33, 9984, N), (3001, 1280, N)]]
    run_split(N, qg.FORM_SMALLN_SPLIT, batches, 45, "split walk")


@pytest.mark.parametrize("N", [1, 4, 5, 8, 9, 16])
def test_slice_form(N):
    # tile groups and K slices with each slice's activations staged whole: the 7B
    # down projection (slices of 18 and 19 super-blocks), slices of one to a few
    # super-blocks next to unsliced problems, ragged tiles and tile groups; where N
    # times a slice's super-blocks exceeds 160 (N = 9 and 16 on the down
    # projection) the batch goes to the K-sliced walk instead
    batches = [[(3584, 18944, N)],
               [(530, 768, N), (77, 256, N), (1000, 3328, N)],
               [(33, 9984, N), (3001, 1280, N)],
               [(1234, 4608, N), (64, 2560, N)]]
    run_split(N, qg.FORM_SMALLN_SLICE, batches, 46, "slice")


@pytest.mark.parametrize("N", [5, 12, 16, 32])
def test_batch_ws_7b_stages(N):
    # the workspace entry point with the automatic choice on the 7B decode stages
    # (per column count it picks the streamed form, the slice form with or without
    # K slices, the K-sliced walk or the walk; at N = 12 and 16 the q/k/v and o
    # stages take the slice form over K slices): sampled rows
    for si, stage in enumerate(workloads.LAYER_STAGES):
        probs, refs = [], []
        for mi in stage:
            name, M, K = workloads.LAYER_MATRICES[mi]
            W = workloads.q4k_blocks(M, K, key=(46, mi, N))
            X = workloads.x_columns(K, N, key=(46, mi, N, 1))
            rows = sample_rows(M, 96, seed=M + K + N)
            probs.append((packed_q4k(W, M, K), to_dev(X), torch.full((N, (M + 3) // 4 * 4), float("nan"),
                                                                     device="cuda:0"), M, K))
            refs.append((rows, oracle.gemm_q4k(W, M, K, X, rows=rows)))
        case(f"qgemm_q4k_smalln_batch_ws 7B stage {si} N={N}")
        qg.qgemm_q4k_smalln_batch_ws(probs)
        torch.cuda.synchronize()
        for (w, X, Y, M, K), (rows, (Yr, Ar)) in zip(probs, refs):
            Yc = Y.cpu().numpy()[:, :M][:, rows]
            for n in range(N):
                assert_within(Yc[n], Yr[n], Ar[n], f"ws stage {si} M={M} K={K} col {n}")


def test_ws_shared_across_shapes():
    # one workspace for batches whose K-sliced plans differ (the 7B down projection at
    # N = 5: 56 tile groups; q/k/v at N = 12: 72; o at N = 32: 28 in the walk form):
    # the counters sit in a fixed block, so one batch's partial sums never land on
    # another's counters, and every call writes all its outputs, bit-identical to a
    # call on a fresh workspace
    batches = [[(3584, 18944, 5)], [(3584, 3584, 12), (512, 3584, 12), (512, 3584, 12)], [(3584, 3584, 32)]]
    runs = []
    for bi, shapes in enumerate(batches):
        probs = []
        for i, (M, K, N) in enumerate(shapes):
            W = workloads.q4k_blocks(M, K, key=(47, bi, i))
            X = workloads.x_columns(K, N, key=(47, bi, i, N))
            probs.append((packed_q4k(W, M, K), to_dev(X), torch.full((N, (M + 3) // 4 * 4), float("nan"),
                                                                     device="cuda:0"), M, K))
        need = qg.qgemm_q4k_smalln_batch_workspace_bytes(probs)
        assert need > 0, shapes
        case(f"qgemm_q4k_smalln_batch_ws fresh workspace, batch {bi}: {shapes}")
        qg.qgemm_q4k_smalln_batch_ws(probs, qg.Workspace("cuda:0", need))
        torch.cuda.synchronize()
        runs.append((probs, need, [p[2].clone() for p in probs]))
    shared = qg.Workspace("cuda:0", max(r[1] for r in runs))
    for step, bi in enumerate([0, 1, 2, 1, 0, 2, 1]):
        probs, _, ref = runs[bi]
        for p_ in probs:
            p_[2].fill_(float("nan"))
        case(f"qgemm_q4k_smalln_batch_ws shared workspace, call {step}: batch {bi}")
        qg.qgemm_q4k_smalln_batch_ws(probs, shared)
        torch.cuda.synchronize()
        for (w, X, Y, M, K), Y0 in zip(probs, ref):
            assert not torch.isnan(Y[:, :M]).any(), f"call {step}, batch {bi}: outputs left unwritten"
            assert torch.equal(Y[:, :M], Y0[:, :M]), f"call {step}, batch {bi}: differs from a fresh workspace"
    assert int(shared.buf[:4096].count_nonzero()) == 0, "arrival counters not returned to zero"


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("M,K", [(200, 512), (65, 3328), (48, 9984), (1, 256)])
def test_dot_form_shapes(M, K, N):
    # the vector-ALU dot-product form (N <= 8): one super-block per K-group (K up to
    # 4096) and the pipelined walk over several (K = 9984: 39 super-blocks, a
    # ragged last round), ragged tiles, a single row
    qg.launch_override(smalln_form=qg.FORM_SMALLN_DOT).set()
    _, _, _, Y, Yr, Ar = run_smalln(M, K, N, key=(41, M, K, N))
    for n in range(N):
        assert_within(Y[n], Yr[n], Ar[n], f"dot form M={M} K={K} N={N} col {n}")


@pytest.mark.parametrize("M,K", [(3584, 3584), (3584, 18944), (700, 2304)])
def test_dot_form_columns_bit_exact_with_gemv(M, K):
    # each column of the dot-product form repeats the single-column kernel's
    # arithmetic in the same order (four wavefronts per tile once K >= 2304), so it
    # equals qgemv_q4k of that column bit for bit
    qg.launch_override(smalln_form=qg.FORM_SMALLN_DOT).set()
    N = 5
    W = workloads.q4k_blocks(M, K, key=(42, M, K))
    X = workloads.x_columns(K, N, key=(42, M, K))
    case(f"dot form vs qgemv_q4k M={M} K={K} N={N}")
    wp = packed_q4k(W, M, K)
    Y = qg.qgemm_q4k_smalln(wp, to_dev(X), M, K)
    torch.cuda.synchronize()
    for n in range(N):
        y = qg.qgemv_q4k(wp, to_dev(X[n]), M, K)
        torch.cuda.synchronize()
        assert np.array_equal(Y[n, :M].cpu().numpy(), y.cpu().numpy()), f"column {n}"
    rows = sample_rows(M, 64, seed=K)
    Yr, Ar = oracle.gemm_q4k(W, M, K, X, rows=rows)
    Yc = Y.cpu().numpy()[:, :M]
    for n in range(N):
        assert_within(Yc[n, rows], Yr[n], Ar[n], f"dot form M={M} K={K} col {n}")


def test_dot_form_batch_mixed_columns():
    # one launch over problems with different N (the kernel is built for the largest;
    # smaller problems read zeros past their N and store only their own columns) and
    # padded leading dimensions; padding and columns past N stay untouched
    qg.launch_override(smalln_form=qg.FORM_SMALLN_DOT).set()
    shapes = [(530, 4096, 8), (77, 256, 1), (16, 3584, 5), (1000, 1280, 3), (33, 18944, 2)]
    probs, refs, Xs = [], [], []
    for i, (M, K, N) in enumerate(shapes):
        W = workloads.q4k_blocks(M, K, key=(43, i))
        X = workloads.x_columns(K, N, key=(43, i, N))
        ldx = K + 256
        Xp = np.full((N, ldx), np.nan, np.float32)
        Xp[:, :K] = X
        Y = torch.full((N, (M + 3) // 4 * 4 + 4), float("nan"), device="cuda:0")
        probs.append((packed_q4k(W, M, K), to_dev(Xp), Y, M, K))
        refs.append(oracle.gemm_q4k(W, M, K, X))
    case("qgemm_q4k_smalln_batch dot form, mixed N")
    # X rows are K + 256 long (NaN past K), Y rows longer than M: ldx > K, ldy > M
    qg.qgemm_q4k_smalln_batch(probs)
    torch.cuda.synchronize()
    for (w, Xd, Y, M, K), (Yr, Ar) in zip(probs, refs):
        Yc = Y.cpu().numpy()
        assert np.all(np.isnan(Yc[:, M:])), "padding rows were written"
        for n in range(Yc.shape[0]):
            assert_within(Yc[n, :M], Yr[n], Ar[n], f"dot batch M={M} K={K} col {n}")
