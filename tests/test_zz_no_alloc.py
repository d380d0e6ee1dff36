"""lmhead_argmax_noalloc (the entry point for callers that cannot allocate: its
partials live in the library's own per-GPU array) against lmhead_argmax with a
caller workspace, through the C ABI: two calls in a row, the second on a smaller
head, each bit for bit equal to the workspace form (same kernels, same order)
and within the oracle's argmax band. Collected last, so it also runs after every
other test in the same process."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, case, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu


def _call_both(wp, x, M, K):
    L = qg.lib()
    stream = torch.cuda.current_stream().cuda_stream
    oi = torch.full((2,), -7, dtype=torch.int32, device=DEV)
    ov = torch.full((2,), float("nan"), device=DEV)
    nbytes = int(L.lmhead_argmax_workspace_bytes(M, K))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    st = L.lmhead_argmax(wp.data_ptr(), x.data_ptr(), M, K, ws.data_ptr(), nbytes, oi.data_ptr(), ov.data_ptr(),
                         stream)
    assert st == 0, qg.last_error()
    st = L.lmhead_argmax_noalloc(wp.data_ptr(), x.data_ptr(), M, K, oi.data_ptr() + 4, ov.data_ptr() + 4, stream)
    assert st == 0, qg.last_error()
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    return oi.cpu().numpy(), ov.cpu().numpy()


@pytest.mark.parametrize("shapes", [[(152064, 3584), (20000, 1024)], [(524288, 512), (1000, 256)]])
def test_noalloc_matches_workspace_form(shapes):
    for t, (M, K) in enumerate(shapes):
        W = workloads.q8_0_blocks(M, K, key=(97, M, K))
        x = workloads.x_vector(K, key=(97, t, K))
        case(f"lmhead_argmax_noalloc M={M} K={K} (call {t + 1})")
        wp = packed_q8_0(W, M, K)
        idx, val = _call_both(wp, to_dev(x), M, K)
        assert idx[0] == idx[1] and val[0].tobytes() == val[1].tobytes(), (idx, val)
        yr, ar = oracle.gemv_q8_0(W, M, K, x)
        ri, gi = oracle.argmax(yr), int(idx[1])
        tol = oracle.tolerance(ar)
        assert gi == ri or yr[gi] >= yr[ri] - tol[gi] - tol[ri]
        assert abs(float(val[1]) - yr[gi]) <= tol[gi]
        del wp
        torch.cuda.empty_cache()


def test_noalloc_rejects_oversized_head():
    L = qg.lib()
    oi = torch.empty(1, dtype=torch.int32, device=DEV)
    st = L.lmhead_argmax_noalloc(0x10000, 0x20000, 524289, 512, oi.data_ptr(), None, None)
    assert st == 2 and "524288" in qg.last_error()
