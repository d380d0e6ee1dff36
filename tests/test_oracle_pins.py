"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself:
hand-derived closed-form blocks, the IEEE binary16 definition checked exhaustively
against numpy, encode/decode round trips through independently written encoders,
integer special cases that reduce to numpy's integer matmul, linearity in x,
zero scales, and the argmax convention of numpy.argmax.

The definitions pinned: y = W x with W the dequantized block matrix (the plain
sequential dot product of "Building a Fully Custom C# LLM Runtime", VectorMath
sample, widened to fp64), the per-row bound sum|w*x|, and the greedy token choice
(first maximum) of "Why Local LLMs Don't Need C++ or Python", section 2.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import blockenc as enc

G = enc.golden()


# ---------------------------------------------------------------- fp16 decode
def test_fp16_decode_exhaustive_vs_numpy():
    L = oracle.lib()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([L.or_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp16_decode_closed_forms():
    # (-1)^s * 2^(e-15) * (1 + f/1024); subnormal 2^-14 * f/1024
    assert oracle.half_to_double(0x3C00) == 1.0
    assert oracle.half_to_double(0x3800) == 0.5
    assert oracle.half_to_double(0xC000) == -2.0
    assert oracle.half_to_double(0x7BFF) == 65504.0
    assert oracle.half_to_double(0x0001) == 2.0 ** -24
    assert oracle.half_to_double(0x03FF) == 1023 * 2.0 ** -24
    assert oracle.half_to_double(0x0400) == 2.0 ** -14
    assert oracle.half_to_double(0x8000) == 0.0 and np.signbit(oracle.half_to_double(0x8000))
    assert np.isinf(oracle.half_to_double(0x7C00))
    assert np.isnan(oracle.half_to_double(0x7E00))


# ---------------------------------------------------------------- scale fields
@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_scale_unpack_golden(name):
    g = G[name]
    sc, m = oracle.q4k_unpack_scales(g["block"][4:16])
    assert list(sc) == g["sc"]
    assert list(m) == g["m"]


def test_scale_pack_unpack_roundtrip():
    rng = np.random.default_rng(5)
    cases = [([0] * 8, [0] * 8), ([63] * 8, [63] * 8), ([15, 16, 31, 32, 47, 48, 62, 63], [16, 15, 48, 47, 0, 63, 32, 31])]
    cases += [(rng.integers(0, 64, 8), rng.integers(0, 64, 8)) for _ in range(200)]
    for sc, m in cases:
        s2, m2 = oracle.q4k_unpack_scales(enc.pack_scales(sc, m))
        assert list(s2) == [int(v) for v in sc] and list(m2) == [int(v) for v in m]


def test_scale_bytes_are_a_bijection():
    # every 12-byte pattern maps to distinct fields: flipping any single bit changes
    # exactly one field by a power of two
    base = np.zeros(12, np.uint8)
    sc0, m0 = oracle.q4k_unpack_scales(base)
    for byte in range(12):
        for bit in range(8):
            s = base.copy()
            s[byte] = 1 << bit
            sc, m = oracle.q4k_unpack_scales(s)
            diff = np.concatenate([sc - sc0, m - m0])
            nz = np.flatnonzero(diff)
            assert nz.size == 1 and diff[nz[0]] in (1, 2, 4, 8, 16, 32)


# ---------------------------------------------------------------- Q4_K blocks
@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_q4k_golden_blocks(name):
    g = G[name]
    w = oracle.q4k_dequant_block(g["block"])
    assert w.sum() == g["sum"]
    for i, v in g["w"].items():
        assert w[i] == v, (name, i, w[i], v)


def test_q4k_block_c_every_weight():
    # Block C: weight 64g+l (l<32) = l mod 16, weight 64g+32+l = g
    w = oracle.q4k_dequant_block(G["C"]["block"])
    i = np.arange(256)
    expect = np.where(i % 64 < 32, (i % 64) % 16, i // 64)
    assert np.array_equal(w, expect.astype(np.float64))


def test_q4k_golden_rows_and_ek_probes():
    # A row of K=512 = [block A, block B]; x = e_k returns weight k; x = 1 returns the sums.
    row = np.concatenate([G["A"]["block"], G["B"]["block"]])
    W = np.stack([row, row])  # two identical rows
    K = 512
    ones = np.ones(K, np.float32)
    y, a = oracle.gemv_q4k(W, 2, K, ones)
    assert np.all(y == G["A"]["sum"] + G["B"]["sum"])
    wa = oracle.q4k_dequant_block(G["A"]["block"])
    for k in (0, 37, 255, 256, 256 + 15, 511):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        y, a = oracle.gemv_q4k(W, 2, K, e)
        expect = G["A"]["w"].get(k) if k < 256 else G["B"]["w"].get(k - 256)
        if expect is None:
            expect = wa[k] if k < 256 else None
        if expect is not None:
            assert y[0] == expect and y[1] == expect
        assert a[0] == abs(y[0])


def test_q4k_encode_decode_random_blocks():
    rng = np.random.default_rng(11)
    for _ in range(100):
        d, dmin, sc, m, q = enc.random_q4k_params(rng)
        blk = enc.q4k_block(enc.half_bits(d), enc.half_bits(dmin), sc, m, q)
        w = oracle.q4k_dequant_block(blk)
        ref = enc.q4k_weights(d, dmin, sc, m, q)
        assert np.array_equal(w, ref)


def test_q4k_bruteforce_tiny_matrices():
    # M <= 4, K in {256, 512}: blocks encoded from chosen parameters, expected y from
    # the parameters with numpy's float64 matmul.
    rng = np.random.default_rng(12)
    for M, K in [(1, 256), (3, 256), (4, 512), (2, 512)]:
        nb = K // 256
        blocks, Wd = [], np.zeros((M, K))
        for r in range(M):
            row = []
            for b in range(nb):
                d, dmin, sc, m, q = enc.random_q4k_params(rng)
                row.append(enc.q4k_block(enc.half_bits(d), enc.half_bits(dmin), sc, m, q))
                Wd[r, 256 * b:256 * (b + 1)] = enc.q4k_weights(d, dmin, sc, m, q)
            blocks.append(np.concatenate(row))
        W = np.stack(blocks)
        x = rng.standard_normal(K).astype(np.float32)
        y, a = oracle.gemv_q4k(W, M, K, x)
        ref = Wd @ x.astype(np.float64)
        aref = np.abs(Wd * x.astype(np.float64)).sum(axis=1)
        assert np.allclose(y, ref, rtol=0, atol=1e-12 * aref.max())
        assert np.allclose(a, aref, rtol=1e-13, atol=0)


def test_q4k_integer_special_case_is_integer_matmul():
    # d = 1, dmin = 0, sc = 1: W is the quant matrix itself; with integer x the product
    # is an exact integer, compared with numpy's int64 matmul.
    rng = np.random.default_rng(13)
    M, K = 5, 768
    Q = rng.integers(0, 16, (M, K))
    W = np.stack([np.concatenate([enc.q4k_block(0x3C00, 0, [1] * 8, [0] * 8, Q[r, 256 * b:256 * (b + 1)])
                                  for b in range(K // 256)]) for r in range(M)])
    xi = rng.integers(-50, 51, K)
    y, _ = oracle.gemv_q4k(W, M, K, xi.astype(np.float32))
    assert np.array_equal(y, (Q @ xi).astype(np.float64))


def test_q4k_dense_vs_factored():
    M, K = 16, 1024
    W = workloads.q4k_blocks(M, K, key=(99, 1))
    x = workloads.x_vector(K, key=(99, 2))
    y, a = oracle.gemv_q4k(W, M, K, x)
    yf = oracle.gemv_q4k_factored(W, M, K, x)
    assert np.all(np.abs(y - yf) <= 1e-12 * a)


def test_q4k_linearity_in_x():
    rng = np.random.default_rng(14)
    M, K = 8, 512
    W = workloads.q4k_blocks(M, K, key=(98, 1))
    xa = rng.integers(-8, 9, K).astype(np.float32)
    xb = rng.integers(-8, 9, K).astype(np.float32)
    xc = (2.0 * xa - 3.0 * xb).astype(np.float32)  # exact in float32
    ya, aa = oracle.gemv_q4k(W, M, K, xa)
    yb, ab = oracle.gemv_q4k(W, M, K, xb)
    yc, ac = oracle.gemv_q4k(W, M, K, xc)
    assert np.all(np.abs(yc - (2 * ya - 3 * yb)) <= 1e-12 * (2 * aa + 3 * ab))


def test_q4k_zero_scales_give_zero():
    M, K = 4, 512
    W = workloads.q4k_blocks(M, K, key=(97, 1)).reshape(M, K // 256, 144).copy()
    x = workloads.x_vector(K, key=(97, 2))
    Z = W.copy()
    Z[:, :, 0:4] = 0  # d = dmin = 0
    y, a = oracle.gemv_q4k(Z.reshape(M, -1), M, K, x)
    assert np.all(y == 0) and np.all(a == 0)
    Z = W.copy()
    Z[:, :, 4:16] = 0  # sc = m = 0
    y, a = oracle.gemv_q4k(Z.reshape(M, -1), M, K, x)
    assert np.all(y == 0)


def test_q4k_min_term_alone():
    # q = 0 everywhere: w = -dmin*m[j]; with x = 1 the row sum is -32*dmin*sum(m)
    m = [3, 0, 63, 1, 17, 32, 5, 60]
    blk = enc.q4k_block(0x3C00, 0x3400, [7] * 8, m, np.zeros(256, int))  # dmin = 0.25
    y, _ = oracle.gemv_q4k(blk[None, :], 1, 256, np.ones(256, np.float32))
    assert y[0] == -32 * 0.25 * sum(m)


# ---------------------------------------------------------------- Q8_0 blocks
@pytest.mark.parametrize("name", ["Q8A", "Q8B", "Q8C"])
def test_q8_0_golden_blocks(name):
    g = G[name]
    w = oracle.q8_0_dequant_block(g["block"])
    assert w.sum() == g["sum"]
    for i, v in g["w"].items():
        assert w[i] == v


def test_q8_0_decodes_minus_128():
    blk = enc.q8_0_block(0x3C00, [-128] + [0] * 31)
    assert oracle.q8_0_dequant_block(blk)[0] == -128.0


def test_q8_0_integer_special_case_is_integer_matmul():
    rng = np.random.default_rng(15)
    M, K = 7, 320
    Q = rng.integers(-127, 128, (M, K))
    W = np.stack([np.concatenate([enc.q8_0_block(0x3C00, Q[r, 32 * b:32 * (b + 1)]) for b in range(K // 32)])
                  for r in range(M)])
    xi = rng.integers(-100, 101, K)
    y, a = oracle.gemv_q8_0(W, M, K, xi.astype(np.float32))
    assert np.array_equal(y, (Q @ xi).astype(np.float64))
    assert np.array_equal(a, (np.abs(Q) @ np.abs(xi)).astype(np.float64))


def test_q8_0_scaled_blocks_vs_params():
    rng = np.random.default_rng(16)
    M, K = 3, 256
    Wd = np.zeros((M, K))
    rows = []
    for r in range(M):
        row = []
        for b in range(K // 32):
            d = float(np.float16(rng.uniform(0.001, 0.02)))
            q = rng.integers(-127, 128, 32)
            row.append(enc.q8_0_block(enc.half_bits(d), q))
            Wd[r, 32 * b:32 * (b + 1)] = d * q
        rows.append(np.concatenate(row))
    W = np.stack(rows)
    x = rng.standard_normal(K).astype(np.float32)
    y, a = oracle.gemv_q8_0(W, M, K, x)
    aref = np.abs(Wd * x.astype(np.float64)).sum(1)
    assert np.allclose(y, Wd @ x.astype(np.float64), rtol=0, atol=1e-12 * aref.max())


def test_q8_0_zero_scale():
    W = workloads.q8_0_blocks(4, 128, key=(96, 1)).reshape(4, 4, 34).copy()
    W[:, :, 0:2] = 0
    y, a = oracle.gemv_q8_0(W.reshape(4, -1), 4, 128, workloads.x_vector(128, key=(96, 2)))
    assert np.all(y == 0)


# ---------------------------------------------------------------- rows subset, small N
# ---------------------------------------------------------------- Q6_K

def random_q6k_params(rng):
    d = float(np.float16(rng.uniform(0.001, 0.02)))
    sc = rng.integers(-128, 128, 16)
    q = rng.integers(0, 64, 256)
    return d, sc, q


@pytest.mark.parametrize("name", ["Q6A", "Q6B"])
def test_q6k_golden_blocks(name):
    g = enc.golden_q6k()[name]
    w = oracle.q6k_dequant_block(g["block"])
    assert w.sum() == g["sum"]
    for i, v in g["w"].items():
        assert w[i] == v, (name, i)


def test_q6k_encoder_reproduces_golden_bytes():
    # the golden bytes (hand-written rules) equal the encoder's output for the
    # parameters they were derived from
    G = enc.golden_q6k()
    i = np.arange(256)
    a = enc.q6k_block(0x3C00, np.arange(16) - 8, i % 64)
    assert np.array_equal(a, G["Q6A"]["block"])
    p, l = (i % 128) // 32, i % 32
    b = enc.q6k_block(0x3800, np.ones(16, int), 16 * p + (l & 15))
    assert np.array_equal(b, G["Q6B"]["block"])


def test_q6k_encode_decode_random_blocks():
    rng = np.random.default_rng(41)
    for _ in range(100):
        d, sc, q = random_q6k_params(rng)
        blk = enc.q6k_block(enc.half_bits(d), sc, q)
        assert np.array_equal(oracle.q6k_dequant_block(blk), enc.q6k_weights(d, sc, q))


def test_q6k_extreme_quants_and_scales():
    # q = 0 -> -32, q = 63 -> +31; scale -128 and 127
    sc = np.array([-128, 127] * 8)
    q = np.array([0, 63] * 128)
    blk = enc.q6k_block(0x3C00, sc, q)
    w = oracle.q6k_dequant_block(blk)
    j = np.arange(256) // 16
    assert np.array_equal(w, sc[j] * np.where(np.arange(256) % 2 == 0, -32.0, 31.0))


def test_q6k_zero_scale_gives_zero():
    rng = np.random.default_rng(42)
    _, sc, q = random_q6k_params(rng)
    assert np.all(oracle.q6k_dequant_block(enc.q6k_block(0, sc, q)) == 0)


def test_q6k_bruteforce_tiny_matrices():
    rng = np.random.default_rng(43)
    for M, K in [(1, 256), (3, 512), (4, 256)]:
        nb = K // 256
        blocks, Wd = [], np.zeros((M, K))
        for r in range(M):
            row = []
            for b in range(nb):
                d, sc, q = random_q6k_params(rng)
                row.append(enc.q6k_block(enc.half_bits(d), sc, q))
                Wd[r, 256 * b:256 * (b + 1)] = enc.q6k_weights(d, sc, q)
            blocks.append(np.concatenate(row))
        W = np.stack(blocks)
        x = rng.standard_normal(K).astype(np.float32)
        y, a = oracle.gemv_q6k(W, M, K, x)
        ref = Wd @ x.astype(np.float64)
        aref = np.abs(Wd * x.astype(np.float64)).sum(axis=1)
        assert np.allclose(y, ref, rtol=0, atol=1e-12 * aref.max())
        assert np.allclose(a, aref, rtol=1e-13, atol=0)


def test_row_subset_matches_full():
    M, K = 40, 512
    W = workloads.q4k_blocks(M, K, key=(95, 1))
    x = workloads.x_vector(K, key=(95, 2))
    y, a = oracle.gemv_q4k(W, M, K, x)
    rows = np.array([39, 0, 17, 17, 3])
    ys, as_ = oracle.gemv_q4k(W, M, K, x, rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(as_, a[rows])


def test_gemm_columns_equal_gemv():
    M, K, N = 9, 512, 5
    W = workloads.q4k_blocks(M, K, key=(94, 1))
    X = workloads.x_columns(K, N, key=(94, 2))
    Y, A = oracle.gemm_q4k(W, M, K, X)
    for n in range(N):
        y, a = oracle.gemv_q4k(W, M, K, X[n])
        assert np.array_equal(Y[n], y) and np.array_equal(A[n], a)


# ---------------------------------------------------------------- argmax
def test_argmax_matches_numpy_first_maximum():
    rng = np.random.default_rng(17)
    for n in (1, 2, 7, 1000):
        y = rng.standard_normal(n)
        assert oracle.argmax(y) == int(np.argmax(y))
    y = np.array([1.0, 5.0, 3.0, 5.0, 5.0])
    assert oracle.argmax(y) == 1 == int(np.argmax(y))
    assert oracle.argmax(np.full(9, -2.0)) == 0
    assert oracle.argmax(np.array([])) == -1


def test_argmax_on_constructed_lm_head():
    # Q8_0 rows with constant quant c_r and x = 1: logit_r = d * K * c_r (d = 1/4).
    K = 64
    c = np.array([3, -7, 12, 12, 0, 11, -127, 12])
    W = np.stack([np.concatenate([enc.q8_0_block(0x3400, [cr] * 32) for _ in range(K // 32)]) for cr in c])
    y, _ = oracle.gemv_q8_0(W, len(c), K, np.ones(K, np.float32))
    assert np.array_equal(y, 0.25 * K * c)
    assert oracle.argmax(y) == 2  # three-way tie at 12 -> lowest index


def test_tolerance_formula():
    a = np.array([0.0, 1.0, 1000.0])
    assert np.allclose(oracle.tolerance(a), [1e-6, 1e-3 + 1e-6, 1.0 + 1e-6])


# ---------------------------------------------------------------- sampling side
GOLDEN_SAMPLING = os.path.join(os.path.dirname(__file__), "golden", "sampling_cases.txt")


def _golden_sampling():
    out = []
    with open(GOLDEN_SAMPLING) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = (t.strip() for t in line.split("->"))
            kind, *fields = lhs.split()
            kv = dict(fl.split("=", 1) for fl in fields)
            z = kv.pop("z")
            if z.startswith("log:"):
                zz = np.log(np.array([float(v) for v in z[4:].split(",")]))
            else:
                zz = np.array([float(v) for v in z.split(",")])
            out.append((kind, zz, kv, rhs))
    return out


@pytest.mark.parametrize("case", _golden_sampling(), ids=lambda c: c[0])
def test_sampling_golden(case):
    kind, z, kv, rhs = case
    if kind == "topk":
        got = oracle.topk(z, int(kv["k"]))
        assert got.tolist() == [int(v) for v in rhs.split(",")]
    elif kind == "lse":
        want = float(rhs)
        got = oracle.logsumexp(z)
        assert (got == want) if np.isinf(want) else abs(got - want) <= 1e-14 * max(1.0, abs(want))
    else:
        got = oracle.sample_topk(z, float(kv["T"]), float(kv["top_p"]), float(kv["min_p"]), float(kv["u"]))
        assert got == int(rhs)


def test_topk_matches_python_sort_with_ties():
    rng = np.random.default_rng(40)
    for n, k in [(1, 1), (7, 3), (50, 50), (300, 20), (1000, 64)]:
        z = rng.integers(-5, 6, n).astype(np.float64)  # many ties
        z[rng.integers(0, n, max(1, n // 20))] = -np.inf
        want = sorted(range(n), key=lambda i: (-z[i], i))[:k]
        assert oracle.topk(z, k).tolist() == want


def test_logsumexp_against_scipy_and_shift():
    from scipy.special import logsumexp as sp_lse
    rng = np.random.default_rng(41)
    for n, s in [(1, 1.0), (10, 0.1), (1000, 3.0), (152064, 50.0)]:
        z = rng.standard_normal(n) * s
        a = oracle.logsumexp(z)
        assert abs(a - sp_lse(z)) <= 1e-12 * max(1.0, abs(a))
        # log-sum-exp commutes with a constant shift
        assert abs(oracle.logsumexp(z + 7.25) - (a + 7.25)) <= 1e-12 * max(1.0, abs(a))
        # the log-softmax exponentiates to a distribution
        assert abs(np.exp(z - a).sum() - 1.0) <= 1e-12 * n


def _sample_vectorized(z, T, top_p, min_p, u):
    """A second formulation: softmax probabilities, cumulative sums, searchsorted."""
    if T <= 0:
        return 0
    p = np.exp((z - z.max()) / T)
    p = p / p.sum()
    n = len(p) if top_p >= 1 else int(np.searchsorted(np.cumsum(p), top_p, side="left")) + 1
    n = min(n, len(p))
    keep = np.flatnonzero(p[:n] >= min_p * p[0])
    m = keep[-1] + 1
    c = np.cumsum(p[:m])
    return int(min(np.searchsorted(c, u * c[-1], side="right"), m - 1)), c / c[-1]


def test_sampler_matches_second_formulation():
    rng = np.random.default_rng(42)
    checked = 0
    for _ in range(400):
        k = int(rng.integers(1, 65))
        z = np.sort(rng.standard_normal(k) * rng.choice([0.3, 1.0, 4.0]))[::-1].copy()
        T = float(rng.choice([0.0, 0.5, 1.0, 1.7]))
        top_p = float(rng.choice([1.0, 0.9, 0.5, 0.05]))
        min_p = float(rng.choice([0.0, 0.05, 0.3]))
        u = float(rng.random())
        r = _sample_vectorized(z, T, top_p, min_p, u)
        if T <= 0:
            assert oracle.sample_topk(z, T, top_p, min_p, u) == 0
            continue
        j, cdf = r
        if np.min(np.abs(cdf - u)) < 1e-9:  # too close to a boundary to be a fair test
            continue
        assert oracle.sample_topk(z, T, top_p, min_p, u) == j
        checked += 1
    assert checked > 250


def test_sampler_inverse_cdf_counts_are_exact():
    # u on a uniform grid: each token is drawn exactly N * p times
    p = np.array([0.5, 0.25, 0.125, 0.125])
    z = np.log(p)
    N = 800
    counts = np.zeros(4, int)
    for i in range(N):
        counts[oracle.sample_topk(z, 1.0, 1.0, 0.0, (i + 0.5) / N)] += 1
    assert counts.tolist() == [400, 200, 100, 100]


# ---------------------------------------------------------------- int8 activations
GOLDEN_Q8_1 = os.path.join(os.path.dirname(__file__), "golden", "q8_1_activation_cases.txt")


def _golden_q8_1():
    f = {}
    for line in open(GOLDEN_Q8_1):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = (t.strip() for t in line.split("=", 1))
        name, attr = k.split(".")
        f.setdefault(name, {})[attr] = v
    out = {}
    i = np.arange(256)
    for name, fl in f.items():
        if "x_rule" in fl:
            x = eval(fl["x_rule"], {"i": i}).astype(np.float32)
            q = eval(fl["q_rule"], {"i": i}).astype(np.int64)
        else:
            x = np.zeros(256, np.float32)
            vals = [float(v) for v in fl["x_list"].split()]
            x[:len(vals)] = vals
            q = np.zeros(256, np.int64)
            qs = [int(v) for v in fl["q_list"].split()]
            q[:len(qs)] = qs
        out[name] = dict(x=x, d=[float(v) for v in fl["d"].split()], q=q, s=[int(v) for v in fl["s"].split()])
    return out


@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_q8_1_golden_blocks(name):
    g = _golden_q8_1()[name]
    d, q, s = oracle.quantize_q8_1(g["x"])
    assert d.astype(np.float64).tolist() == g["d"]
    assert q.astype(np.int64).tolist() == g["q"].tolist()
    assert s.astype(np.int64).tolist() == g["s"]


def test_q8_1_error_bound_and_extremes():
    rng = np.random.default_rng(50)
    x = (rng.standard_normal(32 * 300) * rng.choice([1e-3, 1.0, 300.0], 32 * 300)).astype(np.float32)
    d, q, s = oracle.quantize_q8_1(x)
    xb = x.reshape(-1, 32).astype(np.float64)
    qb = q.reshape(-1, 32).astype(np.float64)
    db = d.astype(np.float64)[:, None]
    # the largest magnitude of each block maps to +-127, every element within half a step
    assert np.all(np.abs(qb).max(axis=1) == 127)
    assert np.all(np.abs(xb - db * qb) <= db * (0.5 + 1e-5))
    assert np.array_equal(s.astype(np.int64), qb.sum(axis=1).astype(np.int64))


def test_q8_1_gemv_exact_when_quantization_is_exact():
    # activations that are multiples of 1/8 with 127/8 in every block quantize
    # without error, so the integer-activation product equals the fp32 one exactly
    M, K = 33, 768
    W = workloads.q4k_blocks(M, K, key=(51,))
    k = np.random.default_rng(51).integers(-127, 128, K)
    k[::32] = 127
    x = (k / 8).astype(np.float32)
    d, q, _ = oracle.quantize_q8_1(x)
    assert np.array_equal(q.astype(np.int64), k)
    y8, a8 = oracle.gemv_q4k_q8_1(W, M, K, d, q)
    y, a = oracle.gemv_q4k(W, M, K, x)
    assert np.array_equal(y8, y) and np.array_equal(a8, a)


def test_q8_1_gemv_integer_case_against_int64_matmul():
    # d = 1, dmin = 0, every sub-scale 1: weights are the 4-bit quants; activations
    # k/8 with 127/8 in every block: y = (Q @ k) / 8 exactly
    M, K = 9, 512
    rng = np.random.default_rng(52)
    Q = rng.integers(0, 16, (M, K))
    W = np.stack([np.concatenate([enc.q4k_block(0x3C00, 0, [1] * 8, [0] * 8, Q[r, 256 * b:256 * b + 256])
                                  for b in range(K // 256)]) for r in range(M)])
    k = rng.integers(-127, 128, K)
    k[::32] = -127
    d, q, _ = oracle.quantize_q8_1((k / 8).astype(np.float32))
    y, _ = oracle.gemv_q4k_q8_1(W, M, K, d, q)
    assert np.array_equal(y * 8, (Q @ k).astype(np.float64))


def test_q8_1_gemv_within_the_parity_tolerance_of_fp32_activations():
    # the quantization error (at most half a step per activation, the step set per
    # 32 activations) keeps the product inside 1e-3 * sum|w x| of the
    # fp32-activation product at the 7B decode shapes
    for M, K in [(64, 3584), (16, 18944)]:
        W = workloads.q4k_blocks(M, K, key=(53, K))
        x = workloads.x_vector(K, key=(53, K))
        d, q, _ = oracle.quantize_q8_1(x)
        y8, _ = oracle.gemv_q4k_q8_1(W, M, K, d, q)
        y, a = oracle.gemv_q4k(W, M, K, x)
        assert np.all(np.abs(y8 - y) <= oracle.tolerance(a))


def test_q8_0_q8_1_gemv_exact_when_quantization_is_exact():
    # LM head with integer activations: multiples of 1/8 with 127/8 in every block
    # quantize without error, so the product equals the fp32-activation Q8_0 product
    M, K = 41, 1024
    W = workloads.q8_0_blocks(M, K, key=(54,))
    k = np.random.default_rng(54).integers(-127, 128, K)
    k[5::32] = -127
    x = (k / 8).astype(np.float32)
    d, q, _ = oracle.quantize_q8_1(x)
    assert np.array_equal(q.astype(np.int64), k)
    y8, a8 = oracle.gemv_q8_0_q8_1(W, M, K, d, q)
    y, a = oracle.gemv_q8_0(W, M, K, x)
    assert np.array_equal(y8, y) and np.array_equal(a8, a)
    rows = np.array([40, 0, 17])
    yr, ar = oracle.gemv_q8_0_q8_1(W, M, K, d, q, rows=rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(ar, a[rows])


def test_q8_0_q8_1_gemv_integer_case_against_int64_matmul():
    # fp16 scale 1.0 in every weight block: weights are the int8 quants; activations
    # k/4 with 127/4 in every block: y = (Q @ k) / 4 exactly, signs of both kept
    M, K = 7, 320
    rng = np.random.default_rng(55)
    Q = rng.integers(-128, 128, (M, K))
    W = np.stack([np.concatenate([enc.q8_0_block(0x3C00, Q[r, 32 * b:32 * b + 32]) for b in range(K // 32)])
                  for r in range(M)])
    k = rng.integers(-127, 128, K)
    k[::32] = 127
    d, q, _ = oracle.quantize_q8_1((k / 4).astype(np.float32))
    y, a = oracle.gemv_q8_0_q8_1(W, M, K, d, q)
    assert np.array_equal(y * 4, (Q @ k).astype(np.float64))
    assert np.array_equal(a * 4, (np.abs(Q) @ np.abs(k)).astype(np.float64))


def test_q8_0_q8_1_gemv_within_the_parity_tolerance_of_fp32_activations():
    # at the LM-head width the activation quantization keeps the logits inside
    # 1e-3 * sum|w x| of the fp32-activation logits
    M, K = 96, 3584
    W = workloads.q8_0_blocks(M, K, key=(56,))
    x = workloads.x_vector(K, key=(56,))
    d, q, _ = oracle.quantize_q8_1(x)
    y8, _ = oracle.gemv_q8_0_q8_1(W, M, K, d, q)
    y, a = oracle.gemv_q8_0(W, M, K, x)
    assert np.all(np.abs(y8 - y) <= oracle.tolerance(a))
