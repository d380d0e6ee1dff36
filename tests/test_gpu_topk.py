"""GPU parity of top-k, log-softmax and the top-k sampler (logits_topk and the
fused Q8_0 LM head lmhead_topk) against the fp64 oracle.

The selection is compared exactly against the oracle's top-k of the same fp32
logits (the decision taken in the kernel's precision); the logits of the fused
head are compared with the oracle's GEMV within the GEMV tolerance. The
log-sum-exp bound 1e-5 + 2e-7 |lse| covers fp32 exponentials, a summation tree of
depth about 60 and the final logarithm and addition."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, assert_within, case, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu


def lse_tol(lse):
    return 1e-5 + 2e-7 * abs(lse)


def check_topk(z32: np.ndarray, out: qg.TopK, k: int, what: str):
    """GPU outputs against the oracle's top-k / log-sum-exp of the same fp32 values."""
    torch.cuda.synchronize()
    z = z32.astype(np.float64)
    idx = out.index.cpu().numpy()
    want = oracle.topk(z, k)
    assert idx.tolist() == want.tolist(), f"{what}: index {idx[:8]} vs {want[:8]}"
    zz = np.where(np.isnan(z), -np.inf, z)
    np.testing.assert_array_equal(out.logit.cpu().numpy().astype(np.float64), zz[want], err_msg=what)
    lse_ref = oracle.logsumexp(z)
    lse = float(out.lse.cpu().numpy()[0])
    if np.isinf(lse_ref):
        assert lse == lse_ref, what
    else:
        assert abs(lse - lse_ref) <= lse_tol(lse_ref), f"{what}: lse {lse} vs {lse_ref}"
        lp = out.logprob.cpu().numpy().astype(np.float64)
        ref = zz[want] - lse_ref
        fin = np.isfinite(ref)
        assert np.all(np.abs(lp[fin] - ref[fin]) <= lse_tol(lse_ref) + 2e-7 * np.abs(ref[fin])), what
        assert np.all(lp[~fin] == -np.inf), what


def logits_case(M, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        z = rng.integers(-3, 4, M).astype(np.float32)
    elif kind == "special":
        z = rng.standard_normal(M).astype(np.float32) * 3
        z[rng.integers(0, M, max(1, M // 7))] = -np.inf
        z[rng.integers(0, M, max(1, M // 11))] = np.nan
        z[rng.integers(0, M, max(1, M // 13))] = -0.0
        z[rng.integers(0, M, max(1, M // 13))] = 0.0
    else:
        z = (rng.standard_normal(M) * float(kind)).astype(np.float32)
    return z


@pytest.mark.parametrize("M,k", [(1, 1), (5, 5), (16, 3), (17, 17), (1000, 20), (4097, 64), (20000, 1),
                                 (152064, 20), (152064, 64), (262144, 40)])
@pytest.mark.parametrize("kind", ["0.05", "3", "60", "ties", "special"])
def test_logits_topk_exact(M, k, kind):
    z = logits_case(M, kind, seed=M * 7 + k)
    case(f"logits_topk M={M} k={k} kind={kind}")
    ws = qg.Workspace(DEV)
    out = qg.logits_topk(to_dev(z), k, ws=ws)
    check_topk(z, out, k, f"M={M} k={k} {kind}")
    assert int(ws.buf.count_nonzero()) == 0  # workspace left all-zero


def test_all_equal_and_all_minus_inf():
    case("logits_topk degenerate vectors")
    z = np.full(3000, 1.5, np.float32)  # every row ties: the lowest rows win
    out = qg.logits_topk(to_dev(z), 10)
    check_topk(z, out, 10, "all equal")
    assert out.index.cpu().tolist() == list(range(10))
    z = np.full(50, -np.inf, np.float32)
    out = qg.logits_topk(to_dev(z), 7)
    torch.cuda.synchronize()
    assert out.index.cpu().tolist() == list(range(7))
    assert float(out.lse.cpu()[0]) == -np.inf


def test_deterministic():
    z = logits_case(152064, "3", seed=5)
    zd = to_dev(z)
    case("logits_topk determinism")
    a = qg.logits_topk(zd, 64)
    b = qg.logits_topk(zd, 64)
    torch.cuda.synchronize()
    for f in ("index", "logit", "logprob", "lse"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


# ------------------------------------------------------------------ sampler
def sorted_topk_values(z32, k):
    z = np.where(np.isnan(z32.astype(np.float64)), -np.inf, z32.astype(np.float64))
    return z[oracle.topk(z, k)]


def boundary_distance(zs, T, top_p, min_p, u):
    """Distance of u from the nearest decision boundary of the oracle's draw."""
    if T <= 0:
        return 1.0
    q = np.exp((zs - zs[0]) / T)
    c = np.cumsum(q)
    n = len(q)
    if top_p < 1:
        n = int(np.argmax(c >= top_p * c[-1])) + 1
        if min(abs(c[:len(q)] / c[-1] - top_p)) < 1e-4:
            return 0.0
    m = int(np.flatnonzero(q[:n] >= min_p)[-1]) + 1
    if min_p > 0 and np.min(np.abs(q - min_p)) < 1e-4:
        return 0.0
    return float(np.min(np.abs(c[:m] / c[m - 1] - u)))


def test_sampler_matches_oracle():
    rng = np.random.default_rng(77)
    M = 5000
    ws = qg.Workspace(DEV)
    u_dev = torch.empty(1, device=DEV)
    checked = 0
    for trial in range(150):
        k = int(rng.integers(1, 65))
        z = (rng.standard_normal(M) * float(rng.choice([0.5, 2.0, 8.0]))).astype(np.float32)
        T = float(rng.choice([0.0, 0.3, 1.0, 2.5]))
        top_p = float(rng.choice([1.0, 0.95, 0.6, 0.1]))
        min_p = float(rng.choice([0.0, 0.02, 0.2]))
        u = float(np.float32(rng.random()))
        zs = sorted_topk_values(z, k)
        if boundary_distance(zs, T, top_p, min_p, u) < 1e-4:
            continue
        u_dev.fill_(u)
        case(f"sampler trial={trial} k={k} T={T} top_p={top_p} min_p={min_p} u={u}")
        out = qg.logits_topk(to_dev(z), k, sampler=(T, top_p, min_p, u_dev), ws=ws)
        torch.cuda.synchronize()
        pos = oracle.sample_topk(zs, T, top_p, min_p, u)
        want = int(oracle.topk(z.astype(np.float64), k)[pos])
        assert int(out.token.cpu()[0]) == want, (trial, k, T, top_p, min_p, u)
        checked += 1
    assert checked > 100


def test_sampler_inverse_cdf_counts():
    # probabilities .5, .25, .125, .125: the draw's boundaries (cumulative .5, .75,
    # .875, up to fp32 rounding) sit half a grid step from every u, so each token
    # is drawn exactly N p times
    p = np.array([0.5, 0.25, 0.125, 0.125])
    z = np.full(300, -np.inf, np.float32)
    z[[10, 200, 3, 77]] = np.log(p).astype(np.float32)
    zd = to_dev(z)
    u_dev = torch.empty(1, device=DEV)
    N = 64
    counts = {}
    case("sampler inverse-CDF counts")
    for i in range(N):
        u_dev.fill_((i + 0.5) / N)
        out = qg.logits_topk(zd, 4, sampler=(1.0, 1.0, 0.0, u_dev))
        t = int(out.token.cpu()[0])
        counts[t] = counts.get(t, 0) + 1
    assert counts == {10: 32, 200: 16, 3: 8, 77: 8}


def test_greedy_and_filters_pick_the_top():
    z = logits_case(10000, "3", seed=9)
    zd = to_dev(z)
    u_dev = torch.full((1,), 0.999, device=DEV)
    top = int(oracle.topk(z.astype(np.float64), 1)[0])
    case("sampler greedy / narrow filters")
    for T, top_p, min_p in [(0.0, 1.0, 0.0), (-1.0, 0.5, 0.3), (1.0, 1e-6, 0.0), (1.0, 1.0, 1.0)]:
        out = qg.logits_topk(zd, 20, sampler=(T, top_p, min_p, u_dev))
        torch.cuda.synchronize()
        assert int(out.token.cpu()[0]) == top, (T, top_p, min_p)
    out = qg.logits_topk(zd, 1, sampler=(1.0, 1.0, 0.0, u_dev))
    torch.cuda.synchronize()
    assert int(out.token.cpu()[0]) == top


# ------------------------------------------------------------------ fused LM head
def run_head(M, K, k, key, xscale=1.0, sampler=None):
    W = workloads.q8_0_blocks(M, K, key=key)
    x = (workloads.x_vector(K, key=key) * xscale).astype(np.float32)
    wp = packed_q8_0(W, M, K)
    xd = to_dev(x)
    ws = qg.Workspace(DEV)
    case(f"lmhead_topk M={M} K={K} k={k} key={key}")
    out, logits = qg.lmhead_topk(wp, xd, M, K, k, sampler=sampler, ws=ws)
    y = qg.qgemv_q8_0(wp, xd, M, K)
    torch.cuda.synchronize()
    assert int(ws.buf.count_nonzero()) == 0
    # the fused kernel's logits are the GEMV's, bit for bit
    assert torch.equal(logits, y)
    lg = logits.cpu().numpy()
    # selection and normalization exact / within fp32 bounds on those logits
    check_topk(lg, out, k, f"head M={M}")
    # and the logits themselves match the fp64 oracle within the GEMV tolerance
    yr, ar = oracle.gemv_q8_0(W, M, K, x)
    assert_within(lg, yr, ar, f"head logits M={M}")
    # log-sum-exp is 1-Lipschitz in the max norm: within the largest logit bound
    lse = float(out.lse.cpu()[0])
    assert abs(lse - oracle.logsumexp(yr)) <= oracle.tolerance(ar).max() + lse_tol(lse)
    return out, lg


@pytest.mark.parametrize("M,K,k,xs", [(1000, 512, 20, 0.05), (777, 4096, 64, 0.02), (16, 256, 16, 1.0),
                                      (5003, 3584, 5, 0.01)])
def test_lmhead_topk_small(M, K, k, xs):
    run_head(M, K, k, key=(30, M, K), xscale=xs)


def test_lmhead_topk_vocab_152064x3584():
    for t, xs in enumerate([1.0, 0.003]):
        run_head(152064, 3584, 20, key=(31, t), xscale=xs)


def test_lmhead_topk_with_sampler():
    u_dev = torch.full((1,), 0.37, device=DEV)
    out, lg = run_head(4000, 1024, 40, key=(32,), xscale=0.01, sampler=(0.8, 0.9, 0.01, u_dev))
    zs = sorted_topk_values(lg, 40)
    if boundary_distance(zs, 0.8, 0.9, 0.01, 0.37) >= 1e-4:
        pos = oracle.sample_topk(zs, 0.8, 0.9, 0.01, float(np.float32(0.37)))
        assert int(out.token.cpu()[0]) == int(out.index.cpu()[pos])
